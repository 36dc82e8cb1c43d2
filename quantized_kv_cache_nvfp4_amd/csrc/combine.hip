// Combine of split-KV partials (Model-Optimizer PR #1832 "Add quant+sparse
// attention for vLLM serving", Testing section: the per-split results of
// each (request, head) are merged by a separate small kernel), with the output written as
// fp32, bf16 (round to nearest even) or FP8 E4M3 with an output scale (vLLM
// PR #15734, item 1: the attention output kept in FP8 for the next layer).
//
// LSE = M + log(sum_j exp(lse_j - M)), M = max_j lse_j; o = sum_j
// exp(lse_j - LSE) o_j.  Splits with lse_j = -inf are skipped; if all are,
// o = 0 and LSE = -inf.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

#include "combine_impl.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;   // 4 waves, each merging one column slice of one (request, head)
constexpr int kSlice = 128;     // columns per wave: wide heads (the 512-wide MLA latent) spread over several waves

// grid: ceil(B*Hq*nsl / 4), nsl = ceil(Dv / kSlice); wave -> (request, head) bh, slice sl
__global__ void __launch_bounds__(kThreads) k_combine(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                                      int nbh, int nsl, int Dv, int s, void* __restrict__ out,
                                                      int out_dtype, const float* __restrict__ out_scale,
                                                      float* __restrict__ lse_out) {
  const int64_t wv = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (wv >= static_cast<int64_t>(nbh) * nsl) return;   // whole waves leave together
  const int64_t bh = wv / nsl;
  const int sl = static_cast<int>(wv - bh * nsl);
  const int d_lo = sl * kSlice, d_hi = d_lo + kSlice < Dv ? d_lo + kSlice : Dv;
  const float osc = (out_dtype == KVQ_FP8E4M3) ? *out_scale : 1.0f;
  float* const lo = (lse_out != nullptr && sl == 0) ? lse_out + bh : nullptr;
  // up to 8 splits: loads of those splits only (the same sums: the extra
  // terms of the wider forms add +0 in the same order)
  if (s <= 8) combine_head_n<false, 8>(part_lse + bh * s, part_o + bh * s * Dv, s, Dv, d_lo, d_hi, out, out_dtype, bh * Dv, osc, lo);
  else combine_head<false>(part_lse + bh * s, part_o + bh * s * Dv, s, Dv, d_lo, d_hi, out, out_dtype, bh * Dv, osc, lo);
}

}  // namespace

hipError_t launch_combine(const float* part_o, const float* part_lse, int B, int Hq, int Dv, int s, void* out,
                          int out_dtype, const float* out_scale, float* lse_out, hipStream_t st) {
  const int nbh = B * Hq;
  const int nsl = (Dv + kSlice - 1) / kSlice;
  const int64_t waves = static_cast<int64_t>(nbh) * nsl;
  hipLaunchKernelGGL(k_combine, dim3(static_cast<unsigned>((waves + kThreads / 64 - 1) / (kThreads / 64))), dim3(kThreads),
                     0, st, part_o, part_lse, nbh, nsl, Dv, s, out, out_dtype, out_scale, lse_out);
  return hipGetLastError();
}

}  // namespace kvq
