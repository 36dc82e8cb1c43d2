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
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "combine_impl.h"
#include "decode_common.h"
#include "kvq_internal.h"
#include "pack_codec.h"
#include "wave_reduce.h"

namespace kvq {
namespace gqa {

using namespace dec;

// K and V plane loads with a cache policy (the buffer loads' auxiliary
// operand): the non-temporal hint (2) or none (0).  Measured on the bench
// shapes: the NVFP4 GQA 32K split kernel 15.9 -> 14.6 us and the MHA 32K one
// 29.6 -> 27.6 us with the hint on both planes; the FP8 ragged B = 64 kernel
// 64.1 -> 74.5 us with it on both, 64.1 -> 62.7 us on K alone (V alone
// 66.3 us), while its FP8-P pass 1, which reads K alone, went 84.5 -> 86.5 us
// with it.  So NVFP4 planes take the hint, FP8 K planes only in attention
// with exact probabilities, FP8 V planes never.
template <int KVF, int PM>
constexpr int k_load_policy() { return (KVF == KVQ_NVFP4 || PM == 0) ? 2 : 0; }
template <int KVF>
constexpr int v_load_policy() { return KVF == KVQ_NVFP4 ? 2 : 0; }
template <int CP>
__device__ inline u32x4 ld128_p(Rsrc r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP));
}
template <int CP>
__device__ inline u32x2 ld64_p(Rsrc r, int off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CP));
}
template <int CP>
__device__ inline uint32_t ld32_p(Rsrc r, int off) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP));
}
template <int CP>
__device__ inline uint32_t ld16_p(Rsrc r, int off) {
  return static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, CP));
}
template <int CP>
__device__ inline uint32_t ld8_p(Rsrc r, int off) {
  return static_cast<uint8_t>(__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, CP));
}

#ifndef KVQ_GQA_WAVES
#define KVQ_GQA_WAVES 4
#endif
constexpr int kWaves = KVQ_GQA_WAVES;   // waves per work-group
constexpr int kThreads = 64 * kWaves;

// ------------------------------------------------------------------ traits
template <int KVF, int D>
struct Geo {
  static constexpr bool kFp4 = (KVF == KVQ_NVFP4);
  static constexpr int kRowBytes = kFp4 ? D / 2 : D;   // code bytes per token row
  static constexpr int kScaleBytes = D / 16;            // NVFP4 scale bytes per row
  static constexpr int kQkJ = D / 32;                   // QK MFMAs per sub-tile
  static constexpr int kPvJ = D / 16;                   // PV MFMAs (output column blocks)
  static constexpr int kQkElems = D / 4;                // head_dim elements per lane (QK)
  static constexpr int kPvElems = D / 16;               // head_dim elements per lane (PV)
  static constexpr int kKWords = kFp4 ? D / 32 : D / 16;  // K code dwords per lane per token
  static constexpr int kVBytes = kFp4 ? kPvElems / 2 : kPvElems;  // V code bytes per lane per token
};

// dequantized K operand of QK MFMA j for this lane (8 consecutive elements)
template <int KVF, int D>
__device__ inline f16x8 k_operand(const uint32_t* kw, uint32_t ks, int j) {
  if constexpr (KVF == KVQ_NVFP4) {
    const uint32_t w = kw[j];
    f16x2 s2;
    if constexpr (D == 128) {
      const f16x2 s = fp8x2<false>(ks);  // (scale of block 2g, scale of block 2g+1)
      const _Float16 sv = (j < 2) ? s[0] : s[1];
      s2 = f16x2{sv, sv};
    } else {
      const f16x2 s = fp8x2<false>(ks);
      s2 = f16x2{s[0], s[0]};
    }
    return cat4(fp4x2<0>(w) * s2, fp4x2<1>(w) * s2, fp4x2<2>(w) * s2, fp4x2<3>(w) * s2);
  } else {
    const uint32_t w0 = kw[2 * j], w1 = kw[2 * j + 1];
    return cat4(fp8x2<false>(w0), fp8x2<true>(w0), fp8x2<false>(w1), fp8x2<true>(w1));
  }
}

// V elements of one token for this lane as f16 pairs (d0,d1),(d2,d3),...
template <int KVF, int D>
__device__ inline void v_pairs(uint32_t vw0, uint32_t vw1, uint32_t vs, f16x2* out) {
  using Gm = Geo<KVF, D>;
  if constexpr (KVF == KVQ_NVFP4) {
    const f16x2 s = fp8x2<false>(vs);
    const f16x2 s2 = f16x2{s[0], s[0]};
    out[0] = fp4x2<0>(vw0) * s2;
    out[1] = fp4x2<1>(vw0) * s2;
    if constexpr (Gm::kPvElems == 8) {
      out[2] = fp4x2<2>(vw0) * s2;
      out[3] = fp4x2<3>(vw0) * s2;
    }
  } else {
    out[0] = fp8x2<false>(vw0);
    out[1] = fp8x2<true>(vw0);
    if constexpr (Gm::kPvElems == 8) {
      out[2] = fp8x2<false>(vw1);
      out[3] = fp8x2<true>(vw1);
    }
  }
}

// Rows of one head.  Lane column c of a 16-lane row is MFMA row c = sub * G
// + h; the rows of head h are the 16 / G columns with c mod G = h.  The max /
// sum over the head's rows is an all-reduce by DPP rotations of 8, 4, .. G
// lanes inside the row (every lane of the head receives the same value:
// each step adds or maxes a pair symmetrically).
template <int G, bool SUM>
__device__ inline float head_rows_reduce(float x) {
  auto op = [](float u, float v) { return SUM ? u + v : fmaxf(u, v); };
  if constexpr (G <= 8) x = op(x, lanes::row_ror<8>(x));
  if constexpr (G <= 4) x = op(x, lanes::row_ror<4>(x));
  if constexpr (G <= 2) x = op(x, lanes::row_ror<2>(x));
  if constexpr (G <= 1) x = op(x, lanes::row_ror<1>(x));
  return x;
}

// ------------------------------------------------------------------ tiles
// Registers holding one tile's packed K (codes + block scales) and V, as
// loaded from HBM.  K and V are separate so that the next tile's K can be in
// flight during this tile's Q.K^T and its V during this tile's P.V.
template <int KVF, int D, int NT>
struct KTile {
  using Gm = Geo<KVF, D>;
  uint32_t k[NT][Gm::kKWords];
  uint32_t ks[NT];
};
template <int KVF, int D, int NT>
struct VTile {
  using Gm = Geo<KVF, D>;
  static constexpr int kVW = (Gm::kVBytes + 3) / 4;  // V code dwords per token
  uint32_t v[NT][4][kVW];   // row layout: [sub-tile][token][dword]
  uint32_t vs[NT][4];
  uint32_t t4[NT][8];       // TOKEN4 layout: [sub-tile][dword of the lane's 16 / 32 bytes]
};

// Output of the fused path (split + combine in one launch).
struct FusedOut {
  void* out;              // [B][Hq][Dv], out_dtype
  int out_dtype;
  const float* out_scale; // FP8 output scale
  float* lse_out;         // [B][Hq] or null
  int* counters;          // [B][Hkv], zero on entry, left zero
};

// ------------------------------------------------------------------ kernel
// Template: KVF cache format, G query heads per kv head, D head_dim,
// QT query type (kQBf16; kQF32: fp32 queries, hi/lo split; kQFp8: E4M3
// codes with a scale), PSPLIT 2 = P carried as f16 hi + lo,
// FUSED: the last work-group of each (request, kv head) merges the partials
// and writes the final output (one launch per decode step).
// Work-groups per CU the register allocation is sized for: 8 waves per CU
// (2 per SIMD, up to 256 VGPRs each).
constexpr int kQBf16 = 0, kQF32 = 1, kQFp8 = 2;
// The fp32-query accuracy path (Q and P split into f16 hi + lo parts) is
// sized for one work-group per CU, so that its larger register set never
// spills to scratch memory.
template <int KVF, int G, int QT, int VL>
constexpr int decode_min_blocks() {
  return QT == 1 ? 1 : 8 / kWaves;
}

// element i of a new K / V row ([B][Hkv][D], dt BF16 / F16 / F32)
__device__ inline float load_new(const void* p, int dt, int64_t i) {
  if (dt == KVQ_F32) return static_cast<const float*>(p)[i];
  const uint16_t u = static_cast<const uint16_t*>(p)[i];
  if (dt == KVQ_BF16) return __uint_as_float(static_cast<uint32_t>(u) << 16);
  return static_cast<float>(__builtin_bit_cast(_Float16, u));
}

// Quantize-on-append, run by the extra work-group (split index num_splits)
// of a (request, kv head): packs the new token's K and V rows with the
// planes' own scales into row pos = min(kv_lens[b], max_kv_len) - 1 of the
// planes (the bytes the pack kernels write: same encoders), then writes the
// token's contribution as partial s_idx of each of the G heads: with one
// token the softmax weight is 1, so the partial output is the dequantized V
// row and its log-sum-exp the token's score.  The other work-groups stream
// [0, pos) and never read row pos, so nothing in this launch waits for the
// write.  (TOKEN4 V: the token's nibbles / bytes of its 4-token group are
// replaced, the other tokens' kept.)
template <int KVF, int G, int D, int QT, int VL, bool PAGED, bool FUSED>
__device__ void append_token(const kvq_decode_args& a, int b, int kvh, int np, int s_idx, float (*lds_new)[128]) {
  using Gm = Geo<KVF, D>;
  constexpr int RB = Gm::kRowBytes;
  constexpr int SB = Gm::kScaleBytes;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int Lr = a.kv_lens[b];
  Lr = Lr < a.max_kv_len ? Lr : a.max_kv_len;
  const int pos = (Lr > 0 ? Lr : 0) - 1;   // the new token (none below 0)
  const int sh = a.kv_scale_per_head ? kvh : 0;
  const float kscale = a.k_scale[sh];
  const float vscale = a.v_scale[sh];
  // the query elements this lane needs for the scores, requested up front
  constexpr int kHw = (G + kWaves - 1) / kWaves;   // heads per wave
  constexpr int kDl = (D + 63) / 64;              // elements per lane and head
  float qv[kHw][kDl];
#pragma unroll
  for (int k = 0; k < kHw; ++k) {
    const int h = wave + k * kWaves;
    const int64_t qb = static_cast<int64_t>(b) * a.q_sb + static_cast<int64_t>(kvh * G + (h < G ? h : 0)) * a.q_sh;
#pragma unroll
    for (int e = 0; e < kDl; ++e) {
      const int d = lane + 64 * e;
      float x = 0.0f;
      if (h < G && d < D) {
        if constexpr (QT == kQF32) x = static_cast<const float*>(a.q)[qb + d];
        else if constexpr (QT == kQFp8) x = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(static_cast<const uint8_t*>(a.q)[qb + d]), 0);
        else x = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.q)[qb + d]) << 16);
      }
      qv[k][e] = x;
    }
  }
  if (pos >= 0 && t < 128) {
    int64_t base;   // plane row of token 0 of pos's block (paged) or of the request
    int tin;        // pos inside it
    if constexpr (PAGED) {
      const int bsh = __builtin_ctz(static_cast<unsigned>(a.block_size));
      const int blk = a.block_table[static_cast<int64_t>(b) * a.bt_stride + (pos >> bsh)];
      base = static_cast<int64_t>(blk) * a.kv_sblk + static_cast<int64_t>(kvh) * a.kv_sh;
      tin = pos & (a.block_size - 1);
    } else {
      base = static_cast<int64_t>(b) * a.kv_sb + static_cast<int64_t>(kvh) * a.kv_sh;
      tin = pos;
    }
    const int64_t st = (VL == KVQ_PLANE_TOKEN4) ? 1 : a.kv_st;
    const int64_t row = base + tin * st;       // K row, V row (row layout)
    const int64_t grow = base + (tin & ~3);    // first row of the TOKEN4 group
    const int j = tin & 3;                     // the token's slot in the group
    const bool isv = t >= 64;                  // wave 0: K, wave 1: V
    const bool t4 = isv && VL == KVQ_PLANE_TOKEN4;
    const void* src = isv ? a.new_v : a.new_k;
    const int64_t off = (static_cast<int64_t>(b) * a.Hkv + kvh) * D;
    uint8_t* codes = const_cast<uint8_t*>(isv ? a.v_codes : a.k_codes);
    const float scl = isv ? vscale : kscale;   // s_t (NVFP4) or the FP8 scale
    if constexpr (KVF == KVQ_NVFP4) {
      uint8_t* scales = const_cast<uint8_t*>(isv ? a.v_scales : a.k_scales);
      if (lane < D / 16) {   // block `lane` of the row
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = load_new(src, a.new_dtype, off + 16 * lane + i);
        uint32_t c[16];
        const uint32_t sc = codec::encode_nvfp4_block(v, scl, c);
        const float sv = static_cast<float>(codec::e4m3_value(sc));
#pragma unroll
        for (int i = 0; i < 16; ++i) lds_new[isv][16 * lane + i] = codec::e2m1_value(c[i]) * sv;   // exact
        if (!t4) {
          uint32_t lo = 0, hi = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            lo |= c[i] << (4 * i);
            hi |= c[8 + i] << (4 * i);
          }
          *reinterpret_cast<uint2*>(codes + row * RB + 8 * lane) = make_uint2(lo, hi);
          scales[row * SB + lane] = static_cast<uint8_t>(sc);
        } else {
          // element x of token j: nibble (j & 1) of byte 2x + (j >> 1) of the
          // group, so block `lane` lives in the group's bytes [32 lane, 32 lane
          // + 32): one read of that span, the token's 16 nibbles replaced in
          // registers, one write (the other tokens' nibbles written back as read)
          uint4* span = reinterpret_cast<uint4*>(codes + grow * RB + 32 * lane);
          uint4 w0 = span[0], w1 = span[1];
          uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
          const int sh = 4 * (j & 1) + 8 * (j >> 1);   // bit offset of the token's nibble in a 2-byte pair
#pragma unroll
          for (int i = 0; i < 16; ++i) {   // element 16 lane + i: byte pair i of the span
            const int bit = 16 * (i & 1) + sh;
            wd[i >> 1] = (wd[i >> 1] & ~(0xFu << bit)) | (c[i] << bit);
          }
          span[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
          span[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
          scales[grow * SB + 4 * lane + j] = static_cast<uint8_t>(sc);   // block `lane` of token j
        }
      }
    } else {
      const double dscale = static_cast<double>(scl);
      const float inv = 1.0f / scl;
      for (int x = lane; x < D; x += 64) {
        const uint32_t cde = codec::encode_fp8(load_new(src, a.new_dtype, off + x), inv, dscale);
        lds_new[isv][x] = static_cast<float>(codec::e4m3_value(cde));
        if (!t4) codes[row * RB + x] = static_cast<uint8_t>(cde);
        else codes[grow * RB + 4 * x + j] = static_cast<uint8_t>(cde);   // element x of token j
      }
    }
  }
  __syncthreads();
  // the token's score per head (fp32) and the partial
#pragma unroll
  for (int k = 0; k < kHw; ++k) {
    const int h = wave + k * kWaves;
    if (h >= G) break;
    const int hq = kvh * G + h;
    const int64_t bh = static_cast<int64_t>(b) * a.Hq + hq;
    float lse = -INFINITY;
    if (pos >= 0) {
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < kDl; ++e) {
        const int d = lane + 64 * e;
        if (d < D) dot += qv[k][e] * lds_new[0][d];
      }
      dot = lanes::wave_all<lanes::Sum>(dot);
      float qk_scale = a.softmax_scale * kscale * kLog2e;
      if constexpr (QT == kQFp8) qk_scale *= a.q_scale[a.q_scale_per_head ? hq : 0];
      lse = dot * qk_scale * kLn2;
    }
    const int64_t po = bh * np + s_idx;
    for (int d = lane; d < D; d += 64) {
      const float o = pos >= 0 ? lds_new[1][d] * vscale : 0.0f;
      if constexpr (FUSED) __hip_atomic_store(a.part_o + po * D + d, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else a.part_o[po * D + d] = o;
    }
    if (lane == 0) {
      if constexpr (FUSED) __hip_atomic_store(a.part_lse + po, lse, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else a.part_lse[po] = lse;
    }
  }
}

// Block-table entries a work-group of a paged cache keeps in LDS (the
// blocks its chunk touches).
constexpr int kMaxChunkBlocks = kPagedMaxChunkBlocks;

// PM: 0 attention, 1 FP8-P pass 1 (scores), 2 FP8-P pass 2 (quantized P . V).
// PAGED: the planes are paged (block table; block size a multiple of the
// tile, so every tile lies in one block).
template <int KVF, int G, int D, int QT, int PSPLIT, bool FUSED, int VL, int PM, bool PAGED, bool APP>
__global__ void __launch_bounds__(kThreads, (decode_min_blocks<KVF, G, QT, VL>())) k_decode_gqa(kvq_decode_args a, int num_splits, FusedOut fo) {
  static_assert(!APP || (PM == 0 && QT == kQBf16), "the fused append: exact probabilities, bf16 queries");
  constexpr bool QF32 = QT == kQF32;
  constexpr bool q8 = QT == kQFp8;   // FP8 query codes: 8 bytes per query word instead of 16
  static_assert(PM == 0 || (!FUSED && PSPLIT == 1), "the FP8-P passes write partials only");
  using Gm = Geo<KVF, D>;
  constexpr int kCPK = k_load_policy<KVF, PM>();   // cache policies of the K and V plane loads
  constexpr int kCPV = v_load_policy<KVF>();
  constexpr int NSUB = 16 / G;                  // row groups in the 16 MFMA columns
  constexpr int NT = NSUB < 2 ? 2 : NSUB;       // sub-tiles (16 tokens) per tile
  constexpr int NACC = NT / NSUB;               // score accumulators per tile
  constexpr int NG = NT <= 4 ? 4 : 1;           // tiles per softmax group
  constexpr int TT = 16 * NT;                   // tokens per tile
  constexpr int NQ = QF32 ? 2 : 1;
  using KT = KTile<KVF, D, NT>;
  using VT = VTile<KVF, D, NT>;

  __shared__ float lds_o[kWaves][16][D];
  __shared__ float lds_m[kWaves][16];   // per wave and head: running max (log2 units)
  __shared__ float lds_l[kWaves][16];   //                    denominator
  __shared__ float lds_lse[16];         // FP8-P pass 2: output factor per head
  __shared__ int lds_last;
  __shared__ int lds_bt[PAGED ? kMaxChunkBlocks : 1];   // paged: block-table entries of the chunk

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int c = lane & 15;   // MFMA column / row-within-16 of this lane
  const int g = lane >> 4;   // lane group (k-slice of the MFMA operands)
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int hq0 = kvh * G;
  const int my_h = c % G;
  const int my_sub = c / G;
  // fused append of the new token: one more work-group per (request, kv
  // head) writes it and its partial (index num_splits).  Those work-groups
  // form extra z planes after the B request planes (request (z - B) *
  // num_splits + x), so that they are dispatched after the streaming
  // work-groups and share a compute unit with one only briefly.
  constexpr bool app = APP;
  const int np = num_splits + (app ? 1 : 0);   // partials per head

  // ---------------- fused combine: the last work-group of (b, kv head) to
  // finish merges the np partials of its G heads.
  // Publication.  Every partial is written with an agent-scope atomic store
  // and read back with an agent-scope atomic load: on gfx950 these are
  // issued with the cache-coherence bits that write through and read past
  // the per-XCD L2, so each access is coherent across the device on its
  // own.  What must be ordered is the stores before the counter increment:
  // each thread waits for its stores to be acknowledged (s_waitcnt 0: the
  // write has reached the device coherence point), the barrier then orders
  // all four waves before thread 0's increment, and the merging work-group
  // issues its loads only after its increment returned the last count.
  // This is the hardware's ordering, not a release/acquire pair of the HIP
  // memory model: agent-scope release / acquire fences give the same
  // results here but write back and invalidate the whole L2 of the XCD on
  // every call, which measured 27.6 us instead of 19.5 us per decode step
  // at the GQA 32K shape (and 4x slower at MHA 32K, 512 work-groups).  The
  // GPU tests require the fused output to be bit-identical to the
  // two-launch path, which reads the partials after a kernel boundary.
  auto fused_tail = [&](int b) {
    __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores are acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
      int* ctr = fo.counters + static_cast<int64_t>(b) * a.Hkv + kvh;
      const int prev = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = (prev == np - 1);
      if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // ready for the next call
      lds_last = last;
    }
    __syncthreads();
    if (!lds_last) return;
    const float osc = (fo.out_dtype == KVQ_FP8E4M3) ? *fo.out_scale : 1.0f;
    // one head per wave (the routine of the standalone combine kernel)
    for (int h = wave; h < G; h += kWaves) {
      const int64_t bh = static_cast<int64_t>(b) * a.Hq + hq0 + h;
      combine_head<true>(a.part_lse + bh * np, a.part_o + bh * np * D, np, D, 0, D, fo.out, fo.out_dtype, bh * D,
                         osc, fo.lse_out != nullptr ? fo.lse_out + bh : nullptr);
    }
  };
  if constexpr (APP) {
    if (b >= a.B) {
      const int ba = (b - a.B) * num_splits + split;   // the request of this append work-group
      if (ba >= a.B) return;
      __shared__ float lds_new[2][128];
      append_token<KVF, G, D, QT, VL, PAGED, FUSED>(a, ba, kvh, np, num_splits, lds_new);
      if constexpr (FUSED) fused_tail(ba);
      return;
    }
  }

  // ---- chunking: c = ceil(max_kv_len / s) rounded up to the tile; split j
  // covers [j c, min((j+1) c, L)).  It depends on kernel arguments only, so
  // the tile addresses are known before the request length is read.
  int chunk = (a.max_kv_len + num_splits - 1) / num_splits;
  chunk = (chunk + TT - 1) / TT * TT;
  const int cs = split * chunk;
  int ce_ld = (cs + chunk < a.max_kv_len) ? cs + chunk : a.max_kv_len;   // load bound (rows present)

  // ---- prologue loads, issued together so that they cost one memory round
  // trip: the query words of this lane (vector), the first K tile, the
  // request's length and the two tensor scales (scalar).
  constexpr int kQRaw = QF32 ? 2 * Gm::kQkJ : Gm::kQkJ;   // 16-byte query words per lane
  uint4 qraw[kQRaw];
  if constexpr (PM != 2) {
    // lane (g, c) holds Q[h = c % G][g*QKE + 8j + e] (q rows and strides are 16-byte aligned,
    // 8-byte aligned for FP8 codes)
    const int64_t qb = static_cast<int64_t>(b) * a.q_sb + static_cast<int64_t>(hq0 + my_h) * a.q_sh +
                       g * Gm::kQkElems;
    if constexpr (q8) {
      const uint2* qp = reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(a.q) + qb);
#pragma unroll
      for (int j = 0; j < kQRaw; ++j) {
        const uint2 w = qp[j];
        qraw[j] = make_uint4(w.x, w.y, 0u, 0u);
      }
    } else {
      const uint4* qp = QF32 ? reinterpret_cast<const uint4*>(static_cast<const float*>(a.q) + qb)
                             : reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qb);
#pragma unroll
      for (int j = 0; j < kQRaw; ++j) qraw[j] = qp[j];
    }
  }
  // per-(request, kv head) plane bases (paged: the kv head's offset inside
  // a block; the block comes from the table per tile)
  const int64_t head_row = (PAGED ? 0 : static_cast<int64_t>(b) * a.kv_sb) + static_cast<int64_t>(kvh) * a.kv_sh;
  const uint8_t* kc = a.k_codes + head_row * Gm::kRowBytes;
  const uint8_t* vc = a.v_codes + head_row * Gm::kRowBytes;
  const uint8_t* ksc = (KVF == KVQ_NVFP4) ? a.k_scales + head_row * Gm::kScaleBytes : kc;
  const uint8_t* vsc = (KVF == KVQ_NVFP4) ? a.v_scales + head_row * Gm::kScaleBytes : vc;
  // token stride in rows (always 1 with a TOKEN4 V plane, K and V share it)
  const int st = (VL == KVQ_PLANE_TOKEN4) ? 1 : static_cast<int>(a.kv_st);
  constexpr int RB = Gm::kRowBytes;
  constexpr int SB = Gm::kScaleBytes;

  // Paged cache: the block-table entries of the chunk's blocks go to LDS
  // once; tile tb then lies in block tb / bs (the block size is a multiple
  // of the tile) at row (tb mod bs) of that block.  The request length and
  // the entry of this wave's first tile are read beside them (scalar
  // loads), so that the first K tile can be requested before the barrier
  // that publishes the LDS copy.  An entry is used only for tokens below
  // the request length; every entry read lies inside the table row
  // (ce_ld <= max_kv_len <= bt_stride * bs).
  // The block size is a power of two: block tb >> bsh, row tb & (bs - 1).
  const int bs = PAGED ? a.block_size : 1;
  const int bsh = PAGED ? __builtin_ctz(static_cast<unsigned>(bs)) : 0;
  const int blk0 = cs >> bsh;
  int len_pg = 0;     // paged: the request length
  int first_blk = 0;  //        the table entry of this wave's first tile
  if constexpr (PAGED) {
    const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.bt_stride + blk0;
    len_pg = a.kv_lens[b];
    const int ft = cs + wave * TT;
    first_blk = ft < ce_ld ? bt[(ft >> bsh) - blk0] : 0;
    const int nblk = ce_ld > cs ? ((ce_ld - 1) >> bsh) - blk0 + 1 : 0;   // blocks holding rows [cs, ce_ld)
    for (int i = threadIdx.x; i < nblk; i += kThreads) lds_bt[i] = bt[i];
  }
  // Paged: the plane rows of a wave's tiles sit in registers, lane j of a
  // window holding the row of the wave's tile 64 w + j (tokens at or past
  // ce_ld get 0); a window is refilled from the LDS table when a load
  // reaches the next 64 tiles.  K and V loads keep one window each (the V
  // loads trail the K loads).
  struct RowWin {
    int w;          // window index (wave-uniform)
    uint32_t lo, hi;
  };
  RowWin win_k{-1, 0u, 0u}, win_v{-1, 0u, 0u};
  auto refill = [&](RowWin& rw, int w) {
    const int tb = cs + (wave + (64 * w + lane) * kWaves) * TT;
    int64_t row = 0;
    if (tb < ce_ld)
      row = static_cast<int64_t>(lds_bt[(tb >> bsh) - blk0]) * a.kv_sblk + static_cast<int64_t>(tb & (bs - 1)) * st;
    rw.w = w;
    rw.lo = static_cast<uint32_t>(row);
    rw.hi = static_cast<uint32_t>(static_cast<uint64_t>(row) >> 32);
  };
  // plane row (relative to the kv head's base) of token tb's tile (a tile
  // of this wave), and the rows available from there (a paged tile ends at
  // its block's end)
  auto tile_row = [&](RowWin& rw, int tb) -> int64_t {
    if constexpr (PAGED) {
      const int k = ((tb - cs) / TT - wave) / kWaves;   // the wave's k-th tile
      if ((k >> 6) != rw.w) refill(rw, k >> 6);
      const uint32_t lo = __builtin_amdgcn_readlane(rw.lo, k & 63);
      const uint32_t hi = __builtin_amdgcn_readlane(rw.hi, k & 63);
      return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    } else {
      (void)rw;
      return static_cast<int64_t>(tb) * st;
    }
  };
  auto tile_rows = [&](int nv) { return PAGED ? (nv < TT ? nv : TT) : nv; };

  // Every load goes through a buffer resource whose base is the tile's
  // first token and whose size ends at the chunk end ce (for the first K
  // tile, issued before the request length is known, at the end of the
  // chunk's rows in the plane): lanes whose token is at or past that end
  // read zeros (hardware range check, nothing is fetched), and the
  // prefetch past a wave's last tile touches no memory.
  // Lane offsets are fixed for the whole chunk, so the loop does no
  // address arithmetic.  (All byte offsets stay below 2^31.)
  const int lk = c * st * RB + g * (Gm::kKWords * 4);          // K codes: token c, quarter g
  const int lks = c * st * SB + (D == 128 ? 2 * g : g);          // K scales of that quarter
  const int lv = 4 * g * st * RB + c * Gm::kVBytes;              // V codes (row layout)
  const int lvs = 4 * g * st * SB + (c * Gm::kPvElems) / 16;     // V scales (row layout)
  constexpr int GB = 4 * RB;                // TOKEN4: bytes per 4-token group (codes)
  constexpr int GS = 4 * SB;                //         bytes per 4-token group (scales)
  constexpr int CB = 4 * Gm::kVBytes;       //         this lane's run inside a group
  const int lvt = g * GB + c * CB;
  const int lvts = g * GS + (c / 2) * 4;

  // (the lane offsets are re-materialized per call, so that the constant
  // parts fold into the loads' immediate offsets instead of occupying
  // loop-invariant registers)
  auto opaque = [](int x) { asm volatile("" : "+v"(x)); return x; };
  // (first_base >= 0: the tile's plane row, given by the caller)
  auto load_ktile = [&](KT& R, int tile, int64_t first_base = -1) {
    const int tb = cs + tile * TT;
    const int lk_ = opaque(lk), lks_ = opaque(lks);
    const int nv = tile_rows(ce_ld - tb);
    const int64_t base = first_base >= 0 ? first_base : tile_row(win_k, tb);
    const Rsrc rk = make_rsrc(kc + base * RB, nv * st * RB);
    const Rsrc rks = make_rsrc(ksc + base * SB, nv * st * SB);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int o = lk_ + u * 16 * st * RB;
      if constexpr (Gm::kKWords == 8) {
        const u32x4 x0 = ld128_p<kCPK>(rk, o), x1 = ld128_p<kCPK>(rk, o + 16);
#pragma unroll
        for (int w = 0; w < 4; ++w) { R.k[u][w] = x0[w]; R.k[u][4 + w] = x1[w]; }
      } else if constexpr (Gm::kKWords == 4) {
        const u32x4 x0 = ld128_p<kCPK>(rk, o);
#pragma unroll
        for (int w = 0; w < 4; ++w) R.k[u][w] = x0[w];
      } else {
        const u32x2 x0 = ld64_p<kCPK>(rk, o);
        R.k[u][0] = x0[0]; R.k[u][1] = x0[1];
      }
      if constexpr (KVF == KVQ_NVFP4) {
        const int os = lks_ + u * 16 * st * SB;
        R.ks[u] = (D == 128) ? ld16_p<kCPK>(rks, os) : ld8_p<kCPK>(rks, os);
      }
    }
  };
  // the first K tile of this wave, loaded before the request length arrives
  // (scores of tokens at or past the request's end are masked to -inf)
  KT KA, KB;
  // (paged: after the request length, so that only the table entries of
  // tokens below it are used)
  if constexpr (PM != 2 && NG > 1 && !PAGED) load_ktile(KA, wave);

  // per-tensor scales, or one per kv head (FP8 with the attn_head strategy)
  const int sh = a.kv_scale_per_head ? kvh : 0;
  const float kscale = a.k_scale[sh];
  const float vscale = a.v_scale[sh];
  int L = PAGED ? len_pg : a.kv_lens[b];
  L = L < a.max_kv_len ? L : a.max_kv_len;
  L = L > 0 ? L : 0;
  if constexpr (APP) L = L > 0 ? L - 1 : 0;   // the new token is the append work-group's
  const int ce = (cs + chunk < L) ? cs + chunk : L;
  ce_ld = ce;   // every later load stops at the request's end
  if constexpr (PAGED) {
    if constexpr (PM != 2 && NG > 1) {   // (pass 2 reads no K)
      const int ft = cs + wave * TT;
      load_ktile(KA, wave, ft < ce ? static_cast<int64_t>(first_blk) * a.kv_sblk + static_cast<int64_t>(ft % bs) * st
                                   : 0);
    }
    __syncthreads();   // the chunk's table entries are in LDS
    refill(win_k, 0);
    win_v = win_k;
  }

  float qk_scale = a.softmax_scale * kscale * kLog2e;
  // FP8 query: its scale (per tensor, or this lane's query head) joins the score factor
  if constexpr (q8) qk_scale *= a.q_scale[a.q_scale_per_head ? hq0 + my_h : 0];

  float m_run = -INFINITY;  // running max of row c's head (log2 domain; the same for all its rows)
  float l_run = 0.0f;       // this lane's share of row c's denominator
  f32x4 acc_o[Gm::kPvJ];
#pragma unroll
  for (int j = 0; j < Gm::kPvJ; ++j) acc_o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = cs < ce ? (ce - cs + TT - 1) / TT : 0;

  {   // (waves without a tile run through with empty loads and no loop iterations)
    // ---- query operand: lane (g, c) holds Q[h = c % G][g*QKE + 8j + e]
    f16x8 qop[NQ][Gm::kQkJ];
    if constexpr (PM != 2) {
#pragma unroll
      for (int j = 0; j < Gm::kQkJ; ++j) {
        if constexpr (q8) {   // E4M3 codes -> f16, exact
          const uint4 w = qraw[j];
          qop[0][j] = cat4(fp8x2<false>(w.x), fp8x2<true>(w.x), fp8x2<false>(w.y), fp8x2<true>(w.y));
          continue;
        }
        float x[8];
        if constexpr (QF32) {
          const uint4 w0 = qraw[2 * j], w1 = qraw[2 * j + 1];
          x[0] = __uint_as_float(w0.x); x[1] = __uint_as_float(w0.y);
          x[2] = __uint_as_float(w0.z); x[3] = __uint_as_float(w0.w);
          x[4] = __uint_as_float(w1.x); x[5] = __uint_as_float(w1.y);
          x[6] = __uint_as_float(w1.z); x[7] = __uint_as_float(w1.w);
        } else {
          const uint4 w = qraw[j];
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {   // bf16 pair -> two fp32 (exact)
            x[2 * k] = __uint_as_float(ws[k] << 16);
            x[2 * k + 1] = __uint_as_float(ws[k] & 0xFFFF0000u);
          }
        }
        f16x2 hi[4], lo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          hi[k] = f16x2{static_cast<_Float16>(x[2 * k]), static_cast<_Float16>(x[2 * k + 1])};
          if constexpr (QF32)
            lo[k] = f16x2{static_cast<_Float16>(x[2 * k] - static_cast<float>(hi[k][0])),
                          static_cast<_Float16>(x[2 * k + 1] - static_cast<float>(hi[k][1]))};
        }
        qop[0][j] = cat4(hi[0], hi[1], hi[2], hi[3]);
        if constexpr (QF32) qop[1][j] = cat4(lo[0], lo[1], lo[2], lo[3]);
      }
    }

    auto load_vtile = [&](VT& R, int tile) {
      const int tb = cs + tile * TT;
      const int lvt_ = opaque(lvt), lvts_ = opaque(lvts), lv_ = opaque(lv), lvs_ = opaque(lvs);
      const int nv = tile_rows(ce - tb);
      const int64_t vbase = tile_row(win_v, tb);   // TOKEN4: st = 1
      if constexpr (VL == KVQ_PLANE_TOKEN4) {
        // Group 4u+g of the tile (lane group g): for this lane's elements
        // [8c, 8c+8) the 4 tokens' codes are one contiguous run (16 bytes
        // NVFP4, 32 bytes FP8) and block c/2's 4 scale bytes one dword.  A
        // group that straddles ce is read whole; pv_tile clears its tokens
        // past ce.
        const int ng = nv > 0 ? (nv + 3) / 4 : 0;
        const Rsrc rv = make_rsrc(vc + vbase * RB, ng * GB);
        const Rsrc rvs = make_rsrc(vsc + vbase * SB, ng * GS);
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          const int o = lvt_ + u * 4 * GB;
          const u32x4 x0 = ld128_p<kCPV>(rv, o);
#pragma unroll
          for (int w = 0; w < 4; ++w) R.t4[u][w] = x0[w];
          if constexpr (CB == 32) {
            const u32x4 x1 = ld128_p<kCPV>(rv, o + 16);
#pragma unroll
            for (int w = 0; w < 4; ++w) R.t4[u][4 + w] = x1[w];
          }
          if constexpr (KVF == KVQ_NVFP4) R.vs[u][0] = ld32_p<kCPV>(rvs, lvts_ + u * 4 * GS);
        }
      } else {
        const Rsrc rv = make_rsrc(vc + vbase * RB, nv * st * RB);
        const Rsrc rvs = make_rsrc(vsc + vbase * SB, nv * st * SB);
#pragma unroll
        for (int u = 0; u < NT; ++u) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int o = lv_ + (16 * u + i) * st * RB;
            if constexpr (Gm::kVBytes == 8) {
              const u32x2 x = ld64_p<kCPV>(rv, o);
              R.v[u][i][0] = x[0]; R.v[u][i][1] = x[1];
            } else if constexpr (Gm::kVBytes == 4) {
              R.v[u][i][0] = ld32_p<kCPV>(rv, o);
            } else {
              R.v[u][i][0] = ld16_p<kCPV>(rv, o);
            }
            if constexpr (KVF == KVQ_NVFP4) R.vs[u][i] = ld8_p<kCPV>(rvs, lvs_ + (16 * u + i) * st * SB);
          }
        }
      }
    };
    // TOKEN4: clear the codes and scales of tokens at or past ce inside the
    // group that straddles it (their probabilities are zero, and zero must
    // never meet bytes that were never written)
    auto mask_vtile = [&](VT& R, int tile) {
      if constexpr (VL == KVQ_PLANE_TOKEN4) {
        const int tb = cs + tile * TT;
        if (tb + TT > ce) {
#pragma unroll
          for (int u = 0; u < NT; ++u) {
            const int nvalid = ce - (tb + 16 * u + 4 * g);
            uint32_t keep = 0xFFFFFFFFu, keep_s = 0xFFFFFFFFu;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (j >= nvalid) {
                keep_s &= ~(0xFFu << (8 * j));
                keep &= (KVF == KVQ_NVFP4) ? ~(0x000F000Fu << (4 * j)) : ~(0xFFu << (8 * j));
              }
            }
#pragma unroll
            for (int w = 0; w < CB / 4; ++w) R.t4[u][w] &= keep;
            R.vs[u][0] &= keep_s;
          }
        }
      }
    };

    // Scores of one tile for this lane's row c (log2 domain; tokens past ce
    // are -inf).  Every sub-tile u is multiplied by the full (unmasked)
    // query operand into its own accumulator; lane column c then keeps the
    // sub-tile of its row group (u % NSUB == c / G): the block-diagonal
    // selection costs one select per score instead of a masked operand per
    // MFMA.
    auto qk_scores = [&](const KT& R, int tile, float (&sc)[NACC][4]) {
      const int tb = cs + tile * TT;
      f32x4 acc_u[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        acc_u[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < Gm::kQkJ; ++j) {
          const f16x8 kop = k_operand<KVF, D>(R.k[u], R.ks[u], j);
#pragma unroll
          for (int qq = 0; qq < NQ; ++qq) acc_u[u] = mfma(kop, qop[qq][j], acc_u[u]);
        }
      }
#pragma unroll
      for (int x = 0; x < NACC; ++x) {
        f32x4 acc_s = acc_u[x * NSUB];
#pragma unroll
        for (int r = 1; r < NSUB; ++r) {
          const bool pick = (my_sub == r);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc_s[i] = pick ? acc_u[x * NSUB + r][i] : acc_s[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[x][i] = acc_s[i] * qk_scale;
      }
      if (tb + TT > ce) {   // the chunk's last, partial tile (uniform branch)
#pragma unroll
        for (int x = 0; x < NACC; ++x)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tb + 16 * (x * NSUB + my_sub) + 4 * g + i >= ce) sc[x][i] = -INFINITY;
      }
    };

    // Online softmax over a group of n tiles at once: one row maximum, at
    // most one rescale of the accumulators per group, then the
    // probabilities of every tile of the group (f16, hi + lo parts when
    // PSPLIT == 2).  The reference is the running maximum itself, so the
    // dominant probability of a peaked row is exactly 1 in f16.
    auto softmax_group = [&](const float (&sc)[NG][NACC][4], int n, f16x2 (&ph)[NG][NACC][2],
                             f16x2 (&pl)[NG][NACC][2]) {
      float tmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < NG; ++t)
        if (t < n)
#pragma unroll
          for (int x = 0; x < NACC; ++x)
#pragma unroll
            for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sc[t][x][i]);
      tmax = lanes::across_rows<lanes::Max>(tmax);   // the row's max over its four lane groups
      tmax = head_rows_reduce<G, false>(tmax);        // one maximum per head: its rows add up unweighted
      const bool bump = tmax > m_run;
      if (__any(bump)) {
        const float m_new = bump ? tmax : m_run;
        const float fac = bump ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;   // 0 when m_run = -inf
        l_run *= fac;
        float fr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fr[i] = __shfl(fac, 4 * g + i);
#pragma unroll
        for (int j = 0; j < Gm::kPvJ; ++j) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc_o[j][i] *= fr[i];
        }
        m_run = m_new;
      }
      const float m_ref = (m_run == -INFINITY) ? 0.0f : m_run;  // rows with no valid token yet
#pragma unroll
      for (int t = 0; t < NG; ++t) {
        if (t < n) {
#pragma unroll
          for (int x = 0; x < NACC; ++x) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              p[i] = __builtin_amdgcn_exp2f(sc[t][x][i] - m_ref);   // masked scores: exp2(-inf) = 0
              l_run += p[i];
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              const _Float16 h0 = static_cast<_Float16>(p[2 * k]);
              const _Float16 h1 = static_cast<_Float16>(p[2 * k + 1]);
              ph[t][x][k] = f16x2{h0, h1};
              if constexpr (PSPLIT == 2)
                pl[t][x][k] = f16x2{static_cast<_Float16>(p[2 * k] - static_cast<float>(h0)),
                                    static_cast<_Float16>(p[2 * k + 1] - static_cast<float>(h1))};
            }
          }
        }
      }
    };

    auto pv_tile = [&](const VT& R, const f16x2 (&p_hi)[NACC][2], const f16x2 (&p_lo)[NACC][2]) {
      // ---------------- P.V over sub-tile pairs (u0, u1) = (2q, 2q+1)
#pragma unroll
      for (int q = 0; q < NT / 2; ++q) {
        const int u0 = 2 * q, u1 = 2 * q + 1;
        // A operand: k = 8g + e; e < 4 -> sub-tile u0 token 4g+e; e >= 4 -> u1
        const bool own0 = (my_sub == (u0 % NSUB));
        const bool own1 = (my_sub == (u1 % NSUB));
        const f16x2 z2 = {0, 0};
        f16x8 pa[PSPLIT];
        {
          const f16x2 a0 = own0 ? p_hi[u0 / NSUB][0] : z2, a1 = own0 ? p_hi[u0 / NSUB][1] : z2;
          const f16x2 b0 = own1 ? p_hi[u1 / NSUB][0] : z2, b1 = own1 ? p_hi[u1 / NSUB][1] : z2;
          pa[0] = cat4(a0, a1, b0, b1);
          if constexpr (PSPLIT == 2) {
            const f16x2 c0 = own0 ? p_lo[u0 / NSUB][0] : z2, c1 = own0 ? p_lo[u0 / NSUB][1] : z2;
            const f16x2 d0 = own1 ? p_lo[u1 / NSUB][0] : z2, d1 = own1 ? p_lo[u1 / NSUB][1] : z2;
            pa[1] = cat4(c0, c1, d0, d1);
          }
        }
        if constexpr (VL == KVQ_PLANE_TOKEN4) {
          // element-major groups: one convert yields element j of two tokens
          // (already the token-contiguous operand); block scales per token pair
          f16x2 s2[4];
          if constexpr (KVF == KVQ_NVFP4) {
            s2[0] = fp8x2<false>(R.vs[u0][0]);  // (token 0, token 1) of u0
            s2[1] = fp8x2<true>(R.vs[u0][0]);   // (token 2, token 3)
            s2[2] = fp8x2<false>(R.vs[u1][0]);
            s2[3] = fp8x2<true>(R.vs[u1][0]);
          }
#pragma unroll
          for (int j = 0; j < Gm::kPvElems; ++j) {
            f16x2 x0, x1, x2, x3;
            if constexpr (KVF == KVQ_NVFP4) {
              const uint32_t w0 = R.t4[u0][j >> 1], w1 = R.t4[u1][j >> 1];
              const int sel = 2 * (j & 1);
              x0 = fp4x2_sel(w0, sel) * s2[0];
              x1 = fp4x2_sel(w0, sel + 1) * s2[1];
              x2 = fp4x2_sel(w1, sel) * s2[2];
              x3 = fp4x2_sel(w1, sel + 1) * s2[3];
            } else {
              x0 = fp8x2<false>(R.t4[u0][j]);
              x1 = fp8x2<true>(R.t4[u0][j]);
              x2 = fp8x2<false>(R.t4[u1][j]);
              x3 = fp8x2<true>(R.t4[u1][j]);
            }
            const f16x8 bv = cat4(x0, x1, x2, x3);
#pragma unroll
            for (int ps = 0; ps < PSPLIT; ++ps) acc_o[j] = mfma(pa[ps], bv, acc_o[j]);
          }
        } else {
          // V: tokens 4g..4g+3 of u0 and u1, head_dim run [c*PVE, (c+1)*PVE).
          // For each pair of head_dim elements k: convert the pair of every
          // token, then transpose 2x2 blocks (tokens x elements) so that each
          // register holds two tokens of one element, then scale by the two
          // tokens' block scales.
          uint32_t w[8];
          f16x2 s2[4];
  #pragma unroll
          for (int tt = 0; tt < 8; ++tt) w[tt] = R.v[tt < 4 ? u0 : u1][tt & 3][0];
          if constexpr (KVF == KVQ_NVFP4) {
  #pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
              const int ua = pr < 2 ? u0 : u1;
              if constexpr (VL == KVQ_PLANE_TOKEN4) {
                // the 4 tokens' scale bytes arrive in one dword
                s2[pr] = (pr & 1) ? fp8x2<true>(R.vs[ua][0]) : fp8x2<false>(R.vs[ua][0]);
              } else {
                const uint32_t sb =
                    __builtin_amdgcn_perm(R.vs[ua][2 * (pr & 1) + 1], R.vs[ua][2 * (pr & 1)], 0x0c0c0400u);
                s2[pr] = fp8x2<false>(sb);  // (scale of token 2pr, scale of token 2pr+1)
              }
            }
          }
  #pragma unroll
          for (int k = 0; k < Gm::kPvElems / 2; ++k) {
            f16x2 x[8];
  #pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
              if constexpr (KVF == KVQ_NVFP4) {
                switch (k) {
                  case 0: x[tt] = fp4x2<0>(w[tt]); break;
                  case 1: x[tt] = fp4x2<1>(w[tt]); break;
                  case 2: x[tt] = fp4x2<2>(w[tt]); break;
                  default: x[tt] = fp4x2<3>(w[tt]); break;
                }
              } else {
                const uint32_t ww = (k < 2) ? w[tt] : R.v[tt < 4 ? u0 : u1][tt & 3][VT::kVW - 1];
                x[tt] = (k & 1) ? fp8x2<true>(ww) : fp8x2<false>(ww);
              }
            }
            // output columns j = 2k (low halves) and 2k+1 (high halves)
            uint32_t lo[4], hi[4];
  #pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
              const uint32_t x0 = as_u32(x[2 * pr]), x1 = as_u32(x[2 * pr + 1]);
              lo[pr] = __builtin_amdgcn_perm(x1, x0, 0x05040100u);
              hi[pr] = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
            }
            f16x2 lo2[4], hi2[4];
  #pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
              lo2[pr] = as_h2(lo[pr]);
              hi2[pr] = as_h2(hi[pr]);
              if constexpr (KVF == KVQ_NVFP4) {
                lo2[pr] = lo2[pr] * s2[pr];
                hi2[pr] = hi2[pr] * s2[pr];
              }
            }
            const f16x8 blo = cat4(lo2[0], lo2[1], lo2[2], lo2[3]);
            const f16x8 bhi = cat4(hi2[0], hi2[1], hi2[2], hi2[3]);
  #pragma unroll
            for (int ps = 0; ps < PSPLIT; ++ps) {
              acc_o[2 * k] = mfma(pa[ps], blo, acc_o[2 * k]);
              acc_o[2 * k + 1] = mfma(pa[ps], bhi, acc_o[2 * k + 1]);
            }
          }
        }
      }
    };

    // software pipeline: the next tile's K is loaded while this tile's
    // scores are computed, and its V while this tile's P.V runs, so every
    // load has a full tile of compute to hide behind.  (Narrow query groups
    // have 8-16 sub-tiles per tile and use one register set.)
    // Tile loop.  The wave's tiles (wave, wave + 4, ...) are taken in groups
    // of NG: phase 1 computes the scores of every tile of the group, one
    // softmax step handles the whole group, phase 2 runs P.V.  Operands
    // stream through two register sets per kind (K in phase 1, V in phase
    // 2): the load of the next operand is issued before the current one is
    // used, so every load has one tile of compute to hide behind, and the
    // K and V sets are never live at the same time except at the phase
    // boundaries.  Loads past the wave's last tile are empty.
    const int nw = (ntiles - wave + kWaves - 1) / kWaves;   // this wave's tiles
    auto tile_of = [&](int k) { return wave + k * kWaves; };
    VT VA, VB;
    // (the tile count n of a group is a compile-time constant: a runtime
    // count made the compiler keep the register sets in a scratch array)
    auto group = [&](int k0, auto nn) {
      constexpr int n = decltype(nn)::value;
      float sc[NG][NACC][4];
      f16x2 ph[NG][NACC][2], pl[NG][NACC][2];
#pragma unroll
      for (int i = 0; i < n; ++i) {
        {
          if (i + 1 < n) load_ktile((i & 1) ? KA : KB, tile_of(k0 + i + 1));
          else load_vtile(VA, tile_of(k0));
          __builtin_amdgcn_sched_barrier(0);
          qk_scores((i & 1) ? KB : KA, tile_of(k0 + i), sc[i]);
        }
      }
      softmax_group(sc, n, ph, pl);
#pragma unroll
      for (int i = 0; i < n; ++i) {
        {
          if (i + 1 < n) load_vtile((i & 1) ? VA : VB, tile_of(k0 + i + 1));
          else load_ktile(KA, tile_of(k0 + NG));   // first tile of the next group
          __builtin_amdgcn_sched_barrier(0);
          mask_vtile((i & 1) ? VB : VA, tile_of(k0 + i));
          pv_tile((i & 1) ? VB : VA, ph[i], pl[i]);
        }
      }
    };
    // FP8-P scratch: spilled scores [B][Hq][sp_stride] (fp32, log2 units)
    const int64_t sp_stride = (static_cast<int64_t>(a.max_kv_len) + 3) / 4 * 4;
    const int64_t bh_row = static_cast<int64_t>(b) * a.Hq + hq0 + my_h;   // this lane's head
    if constexpr (PM == 1) {
      // ---- FP8-P pass 1: the scores of every tile, spilled to the scratch
      // (tokens < ce only), and the running max / denominator of each row
      float* const sp_row = a.p_scratch + bh_row * sp_stride;
      auto spill_and_stats = [&](int tile, const float (&sc)[NACC][4]) {
        const int tb = cs + tile * TT;
#pragma unroll
        for (int x = 0; x < NACC; ++x) {
          const int t0 = tb + 16 * (x * NSUB + my_sub) + 4 * g;
          if (t0 + 4 <= ce) {
            *reinterpret_cast<float4*>(sp_row + t0) = make_float4(sc[x][0], sc[x][1], sc[x][2], sc[x][3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (t0 + i < ce) sp_row[t0 + i] = sc[x][i];
          }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int x = 0; x < NACC; ++x)
#pragma unroll
          for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sc[x][i]);
        tmax = lanes::across_rows<lanes::Max>(tmax);   // the row's max over its four lane groups
        tmax = head_rows_reduce<G, false>(tmax);        // and over the head's rows
        if (tmax > m_run) {
          l_run *= __builtin_amdgcn_exp2f(m_run - tmax);   // 0 when m_run = -inf
          m_run = tmax;
        }
        const float m_ref = (m_run == -INFINITY) ? 0.0f : m_run;
#pragma unroll
        for (int x = 0; x < NACC; ++x)
#pragma unroll
          for (int i = 0; i < 4; ++i) l_run += __builtin_amdgcn_exp2f(sc[x][i] - m_ref);
      };
      float sc[NACC][4];
      if constexpr (NG > 1) {   // two K register sets: the next tile loads during this one (KA: tile 0, loaded above)
        for (int k = 0; k < nw; k += 2) {
          load_ktile(KB, tile_of(k + 1));
          __builtin_amdgcn_sched_barrier(0);
          qk_scores(KA, tile_of(k), sc);
          spill_and_stats(tile_of(k), sc);
          if (k + 1 < nw) {
            load_ktile(KA, tile_of(k + 2));
            __builtin_amdgcn_sched_barrier(0);
            qk_scores(KB, tile_of(k + 1), sc);
            spill_and_stats(tile_of(k + 1), sc);
          }
        }
      } else {
        for (int k = 0; k < nw; ++k) {
          load_ktile(KA, tile_of(k));
          qk_scores(KA, tile_of(k), sc);
          spill_and_stats(tile_of(k), sc);
        }
      }
    } else if constexpr (PM == 2) {
      // ---- FP8-P pass 2: P_t = exp2(sigma_t - LSE2) with LSE2 the head's
      // log-sum-exp over all splits (log2 units), P~ = E4M3(P / prob_scale)
      // (round to nearest even, saturating at 448); the codes' values are
      // exact in f16 and prob_scale is applied with the output.
      float M2 = -INFINITY;
      for (int j = 0; j < num_splits; ++j) M2 = fmaxf(M2, a.part_lse[bh_row * num_splits + j] * kLog2e);
      float S2 = 0.0f;
      for (int j = 0; j < num_splits; ++j) {
        const float l2 = a.part_lse[bh_row * num_splits + j] * kLog2e;
        S2 += (l2 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(l2 - M2);
      }
      const float lse2 = M2 + log2f(S2);   // this chunk has tokens, so S2 > 0
      const float ps = a.prob_scale;
      const float* const sp_row = a.p_scratch + bh_row * sp_stride;
      auto probs = [&](int tile, f16x2 (&ph)[NACC][2]) {
        const int tb = cs + tile * TT;
#pragma unroll
        for (int x = 0; x < NACC; ++x) {
          const int t0 = tb + 16 * (x * NSUB + my_sub) + 4 * g;
          float sg[4];
          if (t0 + 4 <= ce) {
            const float4 v4 = *reinterpret_cast<const float4*>(sp_row + t0);
            sg[0] = v4.x; sg[1] = v4.y; sg[2] = v4.z; sg[3] = v4.w;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) sg[i] = (t0 + i < ce) ? sp_row[t0 + i] : -INFINITY;
          }
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const float r0 = fminf(__builtin_amdgcn_exp2f(sg[2 * k] - lse2) / ps, 448.0f);
            const float r1 = fminf(__builtin_amdgcn_exp2f(sg[2 * k + 1] - lse2) / ps, 448.0f);
            ph[x][k] = fp8x2<false>(static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false)));
          }
        }
      };
      f16x2 ph[NACC][2], pl[NACC][2];
      if constexpr (NG > 1) {   // two V register sets
        load_vtile(VA, tile_of(0));
        for (int k = 0; k < nw; k += 2) {
          load_vtile(VB, tile_of(k + 1));
          __builtin_amdgcn_sched_barrier(0);
          probs(tile_of(k), ph);
          mask_vtile(VA, tile_of(k));
          pv_tile(VA, ph, pl);
          if (k + 1 < nw) {
            load_vtile(VA, tile_of(k + 2));
            __builtin_amdgcn_sched_barrier(0);
            probs(tile_of(k + 1), ph);
            mask_vtile(VB, tile_of(k + 1));
            pv_tile(VB, ph, pl);
          }
        }
      } else {
        for (int k = 0; k < nw; ++k) {
          load_vtile(VA, tile_of(k));
          probs(tile_of(k), ph);
          mask_vtile(VA, tile_of(k));
          pv_tile(VA, ph, pl);
        }
      }
    } else if constexpr (NG > 1) {   // (KA holds tile 0, loaded above)
      static_assert(NG == 4, "grouped tiles come in fours");
      int k0 = 0;
      for (; k0 + NG <= nw; k0 += NG) group(k0, std::integral_constant<int, NG>{});
      if constexpr (NG == 4) {
        switch (nw - k0) {
          case 1: group(k0, std::integral_constant<int, 1>{}); break;
          case 2: group(k0, std::integral_constant<int, 2>{}); break;
          case 3: group(k0, std::integral_constant<int, 3>{}); break;
          default: break;
        }
      }
    } else {
      // wide tiles (8-16 sub-tiles): one register set, no cross-tile
      // prefetch.  FP8 tiles of 16 sub-tiles (256 tokens, 64 KB per wave)
      // load V after the scores, into the registers K leaves free.
      constexpr bool kLateV = (KVF == KVQ_FP8E4M3) && NT >= 16;
      for (int k = 0; k < nw; ++k) {
        float sc[1][NACC][4];
        f16x2 ph[1][NACC][2], pl[1][NACC][2];
        load_ktile(KA, tile_of(k));
        if constexpr (!kLateV) load_vtile(VA, tile_of(k));
        qk_scores(KA, tile_of(k), sc[0]);
        if constexpr (kLateV) {
          __builtin_amdgcn_sched_barrier(0);
          load_vtile(VA, tile_of(k));
        }
        softmax_group(sc, 1, ph, pl);
        mask_vtile(VA, tile_of(k));
        pv_tile(VA, ph[0], pl[0]);
      }
    }
  }

  // ---------------- per-wave state -> LDS.  The rows of one head share
  // the running maximum, so within a wave they add up unweighted; each wave
  // leaves one maximum and one denominator per head.
  float l_tot = lanes::across_rows<lanes::Sum>(l_run);
  l_tot = head_rows_reduce<G, true>(l_tot);
  if (lane < G) {   // lane c = h of lane group 0
    lds_m[wave][lane] = m_run;
    lds_l[wave][lane] = l_tot;
  }
  if constexpr (PM != 1) {
#pragma unroll
    for (int j = 0; j < Gm::kPvJ; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_o[wave][4 * g + i][c * Gm::kPvElems + j] = acc_o[j][i];
    }
  }
  if (PM == 2 && wave == 0 && lane < G) {
    // FP8-P pass 2: rows hold plain sums of P~ . V (no running max), merged
    // with weight 1; the output factor of head h is prob_scale / w_j with
    // w_j = exp(lse_j - LSE) this split's share of the head's softmax mass
    // (0 for an empty split, whose sum is 0 too).
    const int64_t bh = static_cast<int64_t>(b) * a.Hq + hq0 + lane;
    float M2 = -INFINITY;
    for (int j = 0; j < num_splits; ++j) M2 = fmaxf(M2, a.part_lse[bh * num_splits + j] * kLog2e);
    float S2 = 0.0f;
    for (int j = 0; j < num_splits; ++j) {
      const float l2 = a.part_lse[bh * num_splits + j] * kLog2e;
      S2 += (l2 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(l2 - M2);
    }
    const float own = a.part_lse[bh * num_splits + split] * kLog2e;
    const float wj = (own == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(own - (M2 + log2f(S2)));
    lds_lse[lane] = wj > 0.0f ? a.prob_scale / wj : 0.0f;
  }
  __syncthreads();

  // ---------------- merge of the waves, head h: M = max_w m_w, weights
  // f_w = exp2(m_w - M) / sum_w f_w l_w (every thread computes those of its
  // own head from the LDS state: no second barrier), lse = (M + log2 den) ln 2
  auto wave_weights = [&](int h, float (&wt)[kWaves]) -> float {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds_m[w][h]);
    float den = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mv = lds_m[w][h];
      wt[w] = (mv == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mv - M);
      den += wt[w] * lds_l[w][h];
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) wt[w] *= inv;
    return den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
  };
  if constexpr (PM == 1) {   // pass 1 writes the split's lse only
    if (threadIdx.x < G) {
      float wt[kWaves];
      const int64_t bh = static_cast<int64_t>(b) * a.Hq + hq0 + threadIdx.x;
      a.part_lse[bh * num_splits + split] = wave_weights(threadIdx.x, wt);
    }
    return;
  }
  const bool direct = FUSED && np == 1;   // no partials needed
  // items (head h, 64-column block kb) spread over the waves; columns
  // d = 64 kb + lane; the LDS reads do not wait for the weights
  constexpr int kBlk = (D + 63) / 64;
  // blocks per item: as many as spread the G * kBlk blocks over the waves, within one head
  constexpr int kPer = (G * kBlk / kWaves >= kBlk) ? kBlk : ((G * kBlk >= kWaves) ? G * kBlk / kWaves : 1);
  for (int it = wave; it * kPer < G * kBlk; it += kWaves) {
    const int h = (it * kPer) / kBlk;
    const int kb0 = (it * kPer) % kBlk;
    float wt[kWaves];
    float lse = 0.0f;
    if constexpr (PM == 2) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) wt[w] = 1.0f;
    } else {
      lse = wave_weights(h, wt);
    }
    const int64_t bh = static_cast<int64_t>(b) * a.Hq + hq0 + h;
    constexpr int kCols = kPer;
    float sw[kCols][kWaves];
#pragma unroll
    for (int k = 0; k < kCols; ++k) {
      const int d = lane + 64 * (kb0 + k);
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        float x = 0.0f;
#pragma unroll
        for (int s = 0; s < NSUB; ++s) x += (d < D) ? lds_o[w][s * G + h][d] : 0.0f;
        sw[k][w] = x;
      }
    }
#pragma unroll
    for (int k = 0; k < kCols; ++k) {
      const int d = lane + 64 * (kb0 + k);
      if (d >= D) continue;
      float num = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) num += wt[w] * sw[k][w];
      const float o = (PM == 2) ? num * vscale * lds_lse[h] : num * vscale;
      if (direct) {
        store_out(fo.out, fo.out_dtype, bh * D + d, o, fo.out_dtype == KVQ_FP8E4M3 ? *fo.out_scale : 1.0f);
        if (d == 0 && fo.lse_out != nullptr) fo.lse_out[bh] = lse;
      } else {
        const int64_t po = bh * np + split;
        if constexpr (FUSED) {   // device-scope stores: read back by another work-group
          __hip_atomic_store(a.part_o + po * D + d, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (d == 0) __hip_atomic_store(a.part_lse + po, lse, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          a.part_o[po * D + d] = o;
          if (PM == 0 && d == 0) a.part_lse[po] = lse;   // pass 2 keeps pass 1's lse
        }
      }
    }
  }
  if constexpr (!FUSED) return;
  if (direct) return;
  fused_tail(b);
}

// ------------------------------------------------------------------ dispatch
// The instantiated combinations (everything else is refused by the API's
// argument checks before a launch):
//   D = 128: V planes in the TOKEN4 layout; bf16 queries (contiguous or
//            paged planes, with or without the fused append, split or fused
//            combine, exact or FP8 probabilities), FP8 queries (contiguous
//            or paged, split or fused, exact or FP8 probabilities), fp32 queries
//            (contiguous planes, split or fused, exact or FP8 probabilities);
//   D = 64:  V planes in the row layout; bf16 and fp32 queries over
//            contiguous planes (split or fused, exact or FP8 probabilities).
//   G in {1, 2, 4, 8, 16}, NVFP4 and FP8 caches.
template <int KVF, int G, int D, int QT, int PSPLIT, int PM, bool PAGED, bool APP>
hipError_t launch_p(const kvq_decode_args& a, const DecodePlan& p, const FusedOut* fo, hipStream_t st) {
  constexpr int VL = (D == 128) ? KVQ_PLANE_TOKEN4 : KVQ_PLANE_ROWS;
  // (a fused append adds ceil(B / s) z planes: one work-group per (request, kv head))
  const int zapp = APP ? (a.B + p.s - 1) / p.s : 0;
  dim3 grid(p.s, a.Hkv, a.B + zapp);
  if constexpr (PM == 0) {
    if (fo != nullptr) {
      hipLaunchKernelGGL((k_decode_gqa<KVF, G, D, QT, PSPLIT, true, VL, 0, PAGED, APP>), grid, dim3(kThreads), 0, st,
                         a, p.s, *fo);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_decode_gqa<KVF, G, D, QT, PSPLIT, false, VL, PM, PAGED, APP>), grid, dim3(kThreads), 0, st, a,
                     p.s, FusedOut{});
  return hipGetLastError();
}

// contiguous or paged planes (D = 128 only), then the fused append (bf16
// queries, exact probabilities, D = 128 only)
template <int KVF, int G, int D, int QT, int PSPLIT, int PM>
hipError_t launch_layout(const kvq_decode_args& a, const DecodePlan& p, const FusedOut* fo, hipStream_t st) {
  constexpr bool kPagedOk = (D == 128) && QT != kQF32;
  constexpr bool kAppOk = (D == 128) && PM == 0 && QT == kQBf16;
  if (a.block_table != nullptr) {
    if constexpr (kPagedOk) {
      if constexpr (kAppOk) {
        if (a.new_k != nullptr) return launch_p<KVF, G, D, QT, PSPLIT, PM, true, true>(a, p, fo, st);
      }
      return launch_p<KVF, G, D, QT, PSPLIT, PM, true, false>(a, p, fo, st);
    }
    return hipErrorInvalidValue;
  }
  if constexpr (kAppOk) {
    if (a.new_k != nullptr) return launch_p<KVF, G, D, QT, PSPLIT, PM, false, true>(a, p, fo, st);
  }
  if (a.new_k != nullptr) return hipErrorInvalidValue;
  return launch_p<KVF, G, D, QT, PSPLIT, PM, false, false>(a, p, fo, st);
}

template <int KVF, int G, int D, int PM>
hipError_t launch_q(const kvq_decode_args& a, const DecodePlan& p, const FusedOut* fo, hipStream_t st) {
  if constexpr (PM == 2) return launch_layout<KVF, G, D, kQBf16, 1, 2>(a, p, fo, st);   // reads no Q
  // fp32 queries select the fp32-accuracy path (hi/lo split of Q, and of P
  // when P is not quantized)
  if (a.q_dtype == KVQ_F32) return launch_layout<KVF, G, D, kQF32, (PM == 0 ? 2 : 1), PM>(a, p, fo, st);
  if (a.q_dtype == KVQ_FP8E4M3) {   // D = 128; exact probabilities or FP8-P pass 1
    if constexpr ((PM == 0 || PM == 1) && D == 128) return launch_layout<KVF, G, D, kQFp8, 1, PM>(a, p, fo, st);
    return hipErrorInvalidValue;
  }
  return launch_layout<KVF, G, D, kQBf16, 1, PM>(a, p, fo, st);
}

template <int KVF, int D, int PM>
hipError_t launch_g(const kvq_decode_args& a, const DecodePlan& p, const FusedOut* fo, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_q<KVF, 1, D, PM>(a, p, fo, st);
    case 2: return launch_q<KVF, 2, D, PM>(a, p, fo, st);
    case 4: return launch_q<KVF, 4, D, PM>(a, p, fo, st);
    case 8: return launch_q<KVF, 8, D, PM>(a, p, fo, st);
    case 16: return launch_q<KVF, 16, D, PM>(a, p, fo, st);
    default: return hipErrorInvalidValue;
  }
}

// One (format, head_dim) pair: pm 0 attention, 1 / 2 the FP8-P passes.
template <int KVF, int D>
hipError_t dispatch_fmt(int pm, const kvq_decode_args& a, const DecodePlan& p, const FusedOut* fo, hipStream_t st) {
  if (pm == 1) return launch_g<KVF, D, 1>(a, p, fo, st);
  if (pm == 2) return launch_g<KVF, D, 2>(a, p, fo, st);
  return launch_g<KVF, D, 0>(a, p, fo, st);
}

}  // namespace gqa

// Defined by decode_gqa_<format>_d<head_dim>.hip, one instantiation set each.
hipError_t gqa_dispatch_nvfp4_d128(int pm, const kvq_decode_args& a, const DecodePlan& p, const gqa::FusedOut* fo,
                                   hipStream_t st);
hipError_t gqa_dispatch_nvfp4_d64(int pm, const kvq_decode_args& a, const DecodePlan& p, const gqa::FusedOut* fo,
                                  hipStream_t st);
hipError_t gqa_dispatch_fp8_d128(int pm, const kvq_decode_args& a, const DecodePlan& p, const gqa::FusedOut* fo,
                                 hipStream_t st);
hipError_t gqa_dispatch_fp8_d64(int pm, const kvq_decode_args& a, const DecodePlan& p, const gqa::FusedOut* fo,
                                hipStream_t st);

}  // namespace kvq
