// Device routines of the split combine, shared by the standalone combine
// kernel and the fused decode so that both paths give identical bits.
// Combine rule (Model-Optimizer PR #1832, Testing section: the partials of
// the s splits are merged): LSE = M + log(sum_j exp(lse_j - M)), M the max;
// o = sum_j exp(lse_j - M) o_j / sum_j exp(lse_j - M); -inf splits skipped.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

// w[j] = exp(lse_j - M); returns 1/sum in inv and the merged LSE in lse_m.
__device__ inline void split_weights(const float* lse, int s, float* w, float& inv, float& lse_m) {
  float M = -INFINITY;
  for (int j = 0; j < s; ++j) M = fmaxf(M, lse[j]);
  float sum = 0.0f;
  for (int j = 0; j < s; ++j) {
    const float lj = lse[j];
    const float wj = (M == -INFINITY || lj == -INFINITY) ? 0.0f : __expf(lj - M);
    w[j] = wj;
    sum += wj;
  }
  inv = sum > 0.0f ? 1.0f / sum : 0.0f;
  lse_m = sum > 0.0f ? M + __logf(sum) : -INFINITY;
}

// sum_j w[j] * po[j * stride] with four independent accumulators (so the
// loads are in flight together), times inv.
__device__ inline float combine_column(const float* po, int64_t stride, const float* w, int s, float inv) {
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
  int j = 0;
  for (; j + 4 <= s; j += 4) {
    a0 += w[j] * po[(j + 0) * stride];
    a1 += w[j + 1] * po[(j + 1) * stride];
    a2 += w[j + 2] * po[(j + 2) * stride];
    a3 += w[j + 3] * po[(j + 3) * stride];
  }
  for (; j < s; ++j) a0 += w[j] * po[j * stride];
  return ((a0 + a1) + (a2 + a3)) * inv;
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

}  // namespace kvq
