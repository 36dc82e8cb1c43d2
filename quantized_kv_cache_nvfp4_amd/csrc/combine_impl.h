// Device routines of the split combine, shared by the standalone combine
// kernel and the fused decode so that both paths give identical bits.
// Combine rule (Model-Optimizer PR #1832, Testing section: the partials of
// the s splits are merged): LSE = M + log(sum_j exp(lse_j - M)), M the max;
// o = sum_j exp(lse_j - M) o_j / sum_j exp(lse_j - M); -inf splits skipped.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"
#include "wave_reduce.h"

namespace kvq {

// Loads of partials: COHERENT reads at device scope (past this XCD's L2),
// for partials that other work-groups of the same launch have just written.
template <bool COHERENT>
__device__ inline float ld_part(const float* p) {
  if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

__device__ inline uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round half to even (finite inputs)
  return static_cast<uint16_t>(u >> 16);
}

// E4M3 code of fp32 r: hardware round-to-nearest-even conversion after
// clamping to +-448 (the hardware convert does not saturate on its own)
__device__ inline uint8_t f32_to_e4m3_sat(float r) {
  r = fminf(fmaxf(r, -448.0f), 448.0f);
  return static_cast<uint8_t>(__builtin_amdgcn_cvt_pk_fp8_f32(r, 0.0f, 0, false) & 0xFF);
}

// out[idx] = o as fp32, bf16 (RNE) or E4M3(o / osc) (saturating)
__device__ inline void store_out(void* out, int dt, int64_t idx, float o, float osc) {
  if (dt == KVQ_F32) static_cast<float*>(out)[idx] = o;
  else if (dt == KVQ_BF16) static_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(o);
  else static_cast<uint8_t*>(out)[idx] = f32_to_e4m3_sat(o / osc);
}

// Wave-wide split weights (s <= 64): lane j < s returns w_j = exp(lse_j - M)
// (0 for the other lanes); every lane receives 1/sum_j w_j in inv and the
// merged LSE in lse_m.  Must be called by a whole wave.
template <bool COHERENT>
__device__ inline float wave_split_weight(const float* lse, int s, float& inv, float& lse_m) {
  const int lane = threadIdx.x & 63;
  const float lj = lane < s ? ld_part<COHERENT>(lse + lane) : -INFINITY;
  const float M = lanes::wave_all<lanes::Max>(lj);
  const float wj = (M == -INFINITY || lj == -INFINITY) ? 0.0f : __expf(lj - M);
  const float sum = lanes::wave_all<lanes::Sum>(wj);
  inv = sum > 0.0f ? 1.0f / sum : 0.0f;
  lse_m = sum > 0.0f ? M + __logf(sum) : -INFINITY;
  return wj;
}

// Merge of columns [d_lo, d_hi) of one (request, head) by one wave: po = its
// partials [s][Dv], out element i of the head = out[oidx + i]; lse_out (may
// be null) receives the merged LSE.  The partial loads of the
// lane's columns (lane, lane + 64) for all s splits are issued before the
// weights are computed, so the merge costs one memory round trip per 128
// columns (64 when s > 32).  Splits j >= s read split s - 1 and get weight 0 (lane j's
// weight), which leaves every sum unchanged, so N (16, 32 or 64) does not
// change the result.  Four accumulators (j mod 4).  (For N = 64 one column
// per pass.)
template <bool COHERENT, int N>
__device__ __attribute__((always_inline)) inline void combine_head_n(const float* lse, const float* po, int s, int Dv, int d_lo, int d_hi, void* out,
                                      int dt, int64_t oidx, float osc, float* lse_out) {
  constexpr int C = N <= 32 ? 2 : 1;   // columns per lane per pass (at most 64 loads in flight)
  const int lane = threadIdx.x & 63;
  float inv = 0.0f, lse_m = -INFINITY, w = 0.0f;
  for (int d0 = d_lo; d0 < d_hi; d0 += 64 * C) {
    float v[C][N];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int d = d0 + lane + 64 * c;
      if (d < d_hi) {
#pragma unroll
        for (int j = 0; j < N; ++j) v[c][j] = ld_part<COHERENT>(po + static_cast<int64_t>(j < s ? j : s - 1) * Dv + d);
      }
    }
    if (d0 == d_lo) w = wave_split_weight<COHERENT>(lse, s, inv, lse_m);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int d = d0 + lane + 64 * c;
      if (d < d_hi) {
        float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < N; ++j) a[j & 3] += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j)) * v[c][j];
        store_out(out, dt, oidx + d, ((a[0] + a[1]) + (a[2] + a[3])) * inv, osc);
      }
    }
  }
  if (lane == 0 && lse_out != nullptr) *lse_out = lse_m;
}

// (always inlined: called as a function from the fused decode kernel it
// would run on a stack in scratch memory)
template <bool COHERENT>
__device__ __attribute__((always_inline)) inline void combine_head(const float* lse, const float* po, int s, int Dv, int d_lo, int d_hi, void* out,
                                    int dt, int64_t oidx, float osc, float* lse_out) {
  if (s <= 16) combine_head_n<COHERENT, 16>(lse, po, s, Dv, d_lo, d_hi, out, dt, oidx, osc, lse_out);
  else if (s <= 32) combine_head_n<COHERENT, 32>(lse, po, s, Dv, d_lo, d_hi, out, dt, oidx, osc, lse_out);
  else combine_head_n<COHERENT, 64>(lse, po, s, Dv, d_lo, d_hi, out, dt, oidx, osc, lse_out);
}

}  // namespace kvq
