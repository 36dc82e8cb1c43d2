// FP8 matrix-core accumulation probe: the error of gfx950's FP8 E4M3
// 16x16x32 MFMA against the exact sum of its products, which bounds the
// score error of the FP8-query prefill (Q.K^T on FP8 codes).  Products of
// two E4M3 values are exact in fp32, but the instruction adds its 32
// products at a precision below fp32's when their magnitudes spread widely,
// so the prefill's tolerance carries a term proportional to sum |q_k k_k|;
// this probe lets a test measure that term on the device.  A measurement
// aid built into libkvq_probe.so, not part of the kvq C ABI.
//
//   kvq_probe_mfma_fp8(a, b, n, chain, c, stream)
//     a, b   device uint8[n][512] (8-byte aligned): operand tiles.  Tile j
//            of a is the 16 x 32 E4M3 matrix A_j, A_j[i][k] at byte
//            8 (16 (k / 8) + i) + k % 8 of the tile; tile j of b holds the
//            32 x 16 matrix B_j, B_j[k][m] at byte 8 (16 (k / 8) + m) + k % 8.
//     chain  1, 2, 4 or 8 tiles accumulated per result (n % chain == 0),
//            the way the prefill chains 4 instructions over head_dim 128.
//     c      device float[n / chain][16][16] (4-byte aligned):
//            c[g][i][m] = sum over the chain's tiles j of (A_j B_j)[i][m],
//            as the matrix core computes it from zero.
//   Returns 0, or 1 for bad arguments, 2 for a launch error.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// one wave per chain group; lane l holds row l % 16 (A) / column l % 16 (B)
// of k-slice l / 16, and result rows 4 (l / 16) .. + 3 of column l % 16
__global__ void __launch_bounds__(64) k_mfma_fp8_probe(const long* __restrict__ a, const long* __restrict__ b,
                                                       int chain, float* __restrict__ c) {
  const int l = threadIdx.x, grp = blockIdx.x;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < chain; ++j) {
    const int64_t t = static_cast<int64_t>(grp) * chain + j;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a[t * 64 + l], b[t * 64 + l], acc, 0, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) c[static_cast<int64_t>(grp) * 256 + (4 * (l >> 4) + e) * 16 + (l & 15)] = acc[e];
}

}  // namespace

extern "C" int kvq_probe_mfma_fp8(const uint8_t* a, const uint8_t* b, int32_t n, int32_t chain, float* c,
                                  void* stream) {
  if (a == nullptr || b == nullptr || c == nullptr || n <= 0 || n > (1 << 20) ||
      (chain != 1 && chain != 2 && chain != 4 && chain != 8) || n % chain != 0 ||
      reinterpret_cast<uintptr_t>(a) % 8 != 0 || reinterpret_cast<uintptr_t>(b) % 8 != 0 ||
      reinterpret_cast<uintptr_t>(c) % 4 != 0)
    return 1;
  hipLaunchKernelGGL(k_mfma_fp8_probe, dim3(n / chain), dim3(64), 0, static_cast<hipStream_t>(stream),
                     reinterpret_cast<const long*>(a), reinterpret_cast<const long*>(b), chain, c);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
