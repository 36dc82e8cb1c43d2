// Cross-lane reductions of a 64-lane wave on gfx950 without LDS round
// trips: DPP row rotations inside each 16-lane row, and the gfx950 lane-swap
// instructions (v_permlane16_swap / v_permlane32_swap, plain VALU) across
// the four rows.  permlane16_swap(x, x) returns, in every lane, the values of
// its row pair (rows 2k, 2k+1) at the same column; permlane32_swap(x, x)
// those of lanes l mod 32 and l mod 32 + 32.  Every lane of a reduced group
// ends with the same value (each step combines a pair symmetrically).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {
namespace lanes {

// x of lane (row, (c - N) mod 16): DPP rotation by N inside each 16-lane row
template <int N>
__device__ inline float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}

struct Max {
  __device__ static float f(float a, float b) { return fmaxf(a, b); }
};
struct Sum {
  __device__ static float f(float a, float b) { return a + b; }
};

// over the four lanes c, c + 16, c + 32, c + 48 (the four rows at column c):
// ((row 0 op row 1) op (row 2 op row 3)) in every lane
template <class Op>
__device__ inline float across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = Op::f(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return Op::f(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// over the whole wave
template <class Op>
__device__ inline float wave_all(float x) {
  x = Op::f(x, row_ror<8>(x));
  x = Op::f(x, row_ror<4>(x));
  x = Op::f(x, row_ror<2>(x));
  x = Op::f(x, row_ror<1>(x));
  return across_rows<Op>(x);
}

}  // namespace lanes
}  // namespace kvq
