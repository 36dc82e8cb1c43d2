// Combine of split-KV partials (Model-Optimizer PR #1832 "Add quant+sparse
// attention for vLLM serving", Testing section: a small combine kernel
// merges the s partials of each (request, head)), with the output written as
// fp32, bf16 (round to nearest even) or FP8 E4M3 with an output scale (vLLM
// PR #15734, item 1: the attention output kept in FP8 for the next layer).
//
// LSE = M + log(sum_j exp(lse_j - M)), M = max_j lse_j; o = sum_j
// exp(lse_j - LSE) o_j.  Splits with lse_j = -inf are skipped; if all are,
// o = 0 and LSE = -inf.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 128;

__device__ inline uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round half to even (finite inputs)
  return static_cast<uint16_t>(u >> 16);
}

// E4M3 code of fp32 r: hardware round-to-nearest-even conversion after
// clamping to +-448 (the hardware convert does not saturate on its own)
__device__ inline uint8_t f32_to_e4m3_sat(float r) {
  r = fminf(fmaxf(r, -448.0f), 448.0f);
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(r, 0.0f, 0, false);
  return static_cast<uint8_t>(w & 0xFF);
}

// grid: (B*Hq); block: 128 threads striding over Dv
__global__ void __launch_bounds__(kThreads) k_combine(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                                      int Dv, int s, void* __restrict__ out, int out_dtype,
                                                      const float* __restrict__ out_scale, float* __restrict__ lse_out) {
  const int64_t bh = blockIdx.x;
  const float* lse = part_lse + bh * s;
  float M = -INFINITY;
  for (int j = 0; j < s; ++j) M = fmaxf(M, lse[j]);
  float wsum = 0.0f;
  if (M != -INFINITY)
    for (int j = 0; j < s; ++j) wsum += (lse[j] == -INFINITY) ? 0.0f : __expf(lse[j] - M);
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  const float osc = (out_dtype == KVQ_FP8E4M3) ? *out_scale : 1.0f;
  for (int d = threadIdx.x; d < Dv; d += kThreads) {
    float acc = 0.0f;
    if (M != -INFINITY)
      for (int j = 0; j < s; ++j) {
        if (lse[j] == -INFINITY) continue;
        acc += __expf(lse[j] - M) * part_o[(bh * s + j) * Dv + d];
      }
    const float o = acc * inv;
    if (out_dtype == KVQ_F32) static_cast<float*>(out)[bh * Dv + d] = o;
    else if (out_dtype == KVQ_BF16) static_cast<uint16_t*>(out)[bh * Dv + d] = f32_to_bf16_rne(o);
    else static_cast<uint8_t*>(out)[bh * Dv + d] = f32_to_e4m3_sat(o / osc);
  }
  if (threadIdx.x == 0 && lse_out != nullptr) lse_out[bh] = (M == -INFINITY) ? -INFINITY : M + __logf(wsum);
}

}  // namespace

hipError_t launch_combine(const float* part_o, const float* part_lse, int B, int Hq, int Dv, int s, void* out,
                          int out_dtype, const float* out_scale, float* lse_out, hipStream_t st) {
  hipLaunchKernelGGL(k_combine, dim3(B * Hq), dim3(kThreads), 0, st, part_o, part_lse, Dv, s, out, out_dtype, out_scale,
                     lse_out);
  return hipGetLastError();
}

}  // namespace kvq
