// Split-KV flash decode over an NVFP4 or FP8 E4M3 KV cache, GQA / MHA layout,
// for gfx950 (wave64, MFMA 16x16x32 f16).
//
// Method: Model-Optimizer PR #1832 "Add quant+sparse attention for vLLM
// serving", Testing section: the KV sequence of one (request, head) is cut
// into s contiguous chunks; each program keeps a running max and denominator
// of the softmax over its chunk and accumulates the probability-weighted V,
// and a separate step merges the per-split results.  Cache formats: Model-Optimizer
// PR #714 Testing section (NVFP4: E2M1 codes, E4M3 scale per 16 elements
// along head_dim, per-tensor fp32 scale) and compressed-tensors PR #436
// kv_cache_scheme (per-tensor FP8 E4M3).
//
// Design for CDNA4 (not a translation of the pages' Triton kernel):
//  * one work-group = 4 waves = one chunk of one (request, kv head); the
//    waves take interleaved tiles of the chunk and are merged through LDS.
//  * loads go through buffer resources sized to the chunk: tokens past its
//    end read zeros in hardware, no per-lane clamping or address math.
//  * dequantization happens in registers: E2M1 -> f16 with the hardware
//    convert (exact), times the E4M3 block scale (an exact f16 product:
//    at most 5 significant bits, inside f16's normal range); the per-tensor
//    scale is applied in fp32 after the contraction.
//  * Q.K^T and P.V run on MFMA 16x16x32 f16.  The query group is narrow
//    (G = Hq/Hkv query heads share a kv head), so the 16 MFMA columns are
//    filled with (sub-tile, head) pairs: sub-tile u of 16 tokens only
//    meets the Q columns of its own row group (block-diagonal B operand), so
//    one 16x16 score tile holds 16*16/G tokens x G heads with no padding.
//    Each of the 16 rows keeps its own denominator and accumulators; the rows
//    of one head share one running maximum (the maxima are taken over all of
//    the head's rows), so at the end of the chunk they add up unweighted and
//    only the 4 waves' states are merged, with weights.
//  * Q.K^T contracts over head_dim, and the order of that contraction is
//    free: lane group g owns a contiguous quarter of head_dim, so each lane
//    reads its K codes with one 128-bit load per token.  P.V contracts over
//    tokens: with the TOKEN4 V layout one byte holds one element of two
//    consecutive tokens, so the hardware convert yields the token-contiguous
//    MFMA operand directly; with row-major V, 2x2 blocks of f16 are
//    transposed in registers (v_perm_b32).
//  * the softmax works on groups of 4 tiles: one row maximum and at most
//    one rescale of the accumulators per group.
//  * fp32 queries are split into f16 hi + lo parts and P is split the same
//    way (two MFMAs each) for the fp32-accuracy path.
//  * FP8 probabilities (vLLM PR #15734 "[Quantization][FP8] Add support for
//    FP8 models with input_scale for output projection and QK
//    quantization", item 2: softmax(QK^T) quantized to FP8 with a
//    probability scale inside the attention loop), read as the normalized
//    probabilities P = softmax over the whole sequence, so the quantized
//    P~ = E4M3(P / prob_scale) * prob_scale do not depend on the split or
//    the tile order.  P needs the global max and denominator, hence two
//    passes over the same chunking: pass 1 (PM = 1) computes the scores
//    from K only, spills them (fp32, log2 units) and writes each split's
//    log-sum-exp to the partial lse array; pass 2 (PM = 2) reads the
//    spilled scores of its chunk and the s split lse values of its heads,
//    forms P, quantizes it and accumulates P~ . V from V only.  Its partial
//    is o_j = sum_t P~_t V_t / w_j with w_j = exp(lse_j - LSE) the split's
//    share of the softmax mass, so that the ordinary combine (weights w_j)
//    returns sum_t P~_t V_t, not renormalized.
//
// The kernel template lives in decode_gqa_kernel.h; its instantiations are
// split over one source per (cache format, head_dim).  This file holds the
// entry points used by the C ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_gqa_kernel.h"

namespace kvq {

namespace {

hipError_t dispatch(int pm, const kvq_decode_args& a, const DecodePlan& p, const gqa::FusedOut* fo, hipStream_t st) {
  if (a.kv_format == KVQ_NVFP4)
    return a.D == 128 ? gqa_dispatch_nvfp4_d128(pm, a, p, fo, st) : gqa_dispatch_nvfp4_d64(pm, a, p, fo, st);
  return a.D == 128 ? gqa_dispatch_fp8_d128(pm, a, p, fo, st) : gqa_dispatch_fp8_d64(pm, a, p, fo, st);
}

}  // namespace

int gqa_tile_tokens(int G) {
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return 0;
  const int nsub = 16 / G;
  return 16 * (nsub < 2 ? 2 : nsub);
}

const char* gqa_unsupported(const kvq_decode_args& a) {
  if (a.kv_format != KVQ_NVFP4 && a.kv_format != KVQ_FP8E4M3) return "cache format must be NVFP4 or FP8E4M3";
  const int G = a.Hq / a.Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return "query group G = Hq / Hkv must be 1, 2, 4, 8 or 16";
  if (a.D != 64 && a.D != 128) return "head_dim must be 64 or 128";
  if (a.q_dtype != KVQ_BF16 && a.q_dtype != KVQ_F32 && a.q_dtype != KVQ_FP8E4M3)
    return "queries must be BF16, F32 or FP8E4M3";
  if (a.D == 128 && a.v_layout != KVQ_PLANE_TOKEN4) return "V planes at head_dim 128 are decoded in the TOKEN4 layout";
  if (a.D == 64) {
    if (a.v_layout != KVQ_PLANE_ROWS) return "V planes at head_dim 64 are decoded in the row layout";
    if (a.block_table != nullptr) return "paged planes are decoded at head_dim 128";
    if (a.new_k != nullptr) return "the fused append is implemented at head_dim 128";
    if (a.q_dtype == KVQ_FP8E4M3) return "FP8 queries are decoded at head_dim 128";
  }
  if (a.q_dtype == KVQ_F32 && a.block_table != nullptr) return "fp32 queries are decoded over contiguous planes";
  return nullptr;
}

hipError_t launch_decode_gqa(const kvq_decode_args& a, const DecodePlan& p, hipStream_t st) {
  return dispatch(0, a, p, nullptr, st);
}

hipError_t launch_decode_fp8p(const kvq_decode_args& a, const DecodePlan& p, hipStream_t st) {
  hipError_t e = dispatch(1, a, p, nullptr, st);   // scores + split lse
  if (e == hipSuccess) e = dispatch(2, a, p, nullptr, st);   // quantized P . V
  return e;
}

hipError_t launch_decode_gqa_fused(const kvq_decode_args& a, const DecodePlan& p, void* out, int out_dtype,
                                   const float* out_scale, float* lse_out, int* counters, hipStream_t st) {
  gqa::FusedOut fo{out, out_dtype, out_scale, lse_out, counters};
  return dispatch(0, a, p, &fo, st);
}

}  // namespace kvq
