// Chunked prefill over an NVFP4 or FP8 E4M3 KV cache, GQA / MHA layout, for
// gfx950 (wave64, MFMA 16x16x32 f16).
//
// What it computes: the prefill path the pages time beside their split-KV
// decode (Model-Optimizer PR #1832 "Add quant+sparse attention for vLLM
// serving", Testing section: the "prefill" column of both decode-latency
// tables, and triton_fa.py in the coverage report): attention of a chunk of
// Sq new query tokens per request over the quantized cache, which already
// holds the chunk's own K/V rows.  Query i of request b sits at position
// p_i = kv_len[b] - Sq + i and attends causally to the cached tokens
// t <= p_i; a query with p_i < 0 sees nothing (output 0, lse -inf).  Cache
// formats as the decode kernels (Model-Optimizer PR #714 Testing section:
// NVFP4 = E2M1 codes, E4M3 scale per 16 elements, fp32 tensor scale;
// compressed-tensors PR #436 kv_cache_scheme: per-tensor FP8 E4M3).
//
// Design for CDNA4.  The chunk gives many query rows per kv head, so both
// contractions are dense and run on MFMA (the decode kernels fill the MFMA
// columns with tokens because there one query row meets each kv head):
//  * a work-group of 8 waves owns 256 query rows of one (request, kv head):
//    256 / G consecutive query tokens x the G heads of the group (row r ->
//    token r / G, head r % G); each wave owns 32 rows as two 16-row blocks.
//  * the waves form two groups of 4 (A: waves 0-3, B: waves 4-7; waves w
//    and w + 4 share a SIMD) that run the same tile half a step apart
//    (ping-pong): each tile takes four phases separated by barriers, and in
//    every phase one group is in its matrix-core work while the other is in
//    vector work, so the SIMD issues both at once:
//        phase      1           2           3           4
//        A          Q.K^T       softmax     P.V         stage K(n+1)
//        B          stage V(n+1) Q.K^T      softmax     P.V
//  * per 64-token KV tile K and V are dequantized once into LDS as f16
//    (E2M1 or E4M3 -> f16 with the hardware convert, exact; times the E4M3
//    block scale, an exact f16 product) for all 256 rows: group A stages K
//    and group B stages V, each from raw bytes it loaded one tile ahead, into
//    two stages of LDS.
//  * S^T = K . Q^T: the K tile is the A operand (16 tokens x 32 dims from
//    LDS), the query rows the B operand (registers, loaded once).  A lane
//    then holds 4 tokens of one query row, so the row maximum is a local
//    max and two lane swaps (no LDS), and the same registers, converted to
//    f16, are the B operand of O^T = V^T . P^T: the order in which the
//    contraction meets the tokens is free, and V^T is stored in LDS with
//    its token slots permuted to match.  A lane's output column is again
//    its query row, so the softmax rescale is a per-lane scalar.
//  * LDS: K rows of 256 B with a 16-byte-chunk XOR swizzle (chunk j of row
//    r at j ^ (r mod 16)), staged token-major (a 16-lane row of a wave
//    writes 16 tokens); V^T rows of 64 token slots padded to 160 B.  Both
//    measured free of bank conflicts on gfx950 for the MFMA reads and the
//    staging writes (SQ_LDS_BANK_CONFLICT of a probe of each access
//    pattern; a 144-byte V^T pitch, or four consecutive lanes per K token,
//    is not).  2 x 36 KB per work-group, two work-groups per CU.
//  * the per-tensor scales are applied in fp32: s_t,K inside the score
//    scale, s_t,V at the end.  P enters the second MFMA as f16.
//  * query blocks are dispatched longest first (the last block of the chunk
//    sees the most tokens).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "decode_common.h"
#include "kvq_internal.h"
#include "wave_reduce.h"

namespace kvq {
namespace pf {

using namespace dec;

constexpr int kThreads = 512;                 // two groups of 4 waves
constexpr int kRows = 256;                    // query rows per work-group
constexpr int kTile = 64;                     // KV tokens per tile
constexpr int kD = 128;                       // head_dim
constexpr int kKRow = kD * 2;                 // f16 K row in LDS (bytes)
constexpr int kKBytes = kTile * kKRow;        // 16 KB
constexpr int kVtRow = kTile * 2 + 32;        // f16 V^T row of 64 token slots + 32 B of padding
constexpr int kVtBytes = kD * kVtRow;         // 20 KB
constexpr int kStage = kKBytes + kVtBytes;
constexpr int kLdsBytes = 2 * kStage;         // 73,728 B

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// token slot of tile token t in a V^T row: tokens 16u + 4g + e (u = 0..3,
// g = 0..3, e = 0..3) go to 32 (u / 2) + 8 g + 4 (u % 2) + e, so that the 8
// tokens a lane of group g holds for 32-token chunk kc (sub-tiles 2kc and
// 2kc + 1) are the contiguous slots 32 kc + 8 g .. + 7
__device__ inline int vt_slot(int t) {
  const int u = t >> 4, g = (t >> 2) & 3, e = t & 3;
  return 32 * (u >> 1) + 8 * g + 4 * (u & 1) + e;
}

__device__ inline uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Work-group barrier that orders LDS only: the fences cover the local
// address space, so global loads still in flight (the next tile's raw
// bytes) are not waited for, as they would be at __syncthreads().
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <class T>
__device__ inline T lds_ld(const uint8_t* p) {
  return *reinterpret_cast<const T*>(p);
}
template <class T>
__device__ inline void lds_st(uint8_t* p, T v) {
  *reinterpret_cast<T*>(p) = v;
}

// One tile's raw bytes in registers (the thread's share).
template <int KVF>
struct Raw {
  static constexpr bool kFp4 = KVF == KVQ_NVFP4;
  u32x4 k[kFp4 ? 1 : 2];   // K: 32 elements of one token
  u32x4 v[kFp4 ? 1 : 2];   // V: 8 elements of a 4-token group
  uint32_t ks;             // NVFP4: the 2 block scales of the K elements
  uint32_t vs;             // NVFP4: block scale of the V elements, 4 tokens
};

// Q8: the queries are FP8 E4M3 codes with a scale (the QKV-FP8 schemes).
// Over an FP8 cache (K8) both operands of Q.K^T are E4M3 codes and the
// contraction runs on the FP8 matrix cores, K staged in LDS as its raw bytes
// (no conversion); over an NVFP4 cache the codes are converted to f16
// (exact) and the f16 path runs.
typedef long i64x1;
__device__ inline f32x4 mfma_fp8(i64x1 a, i64x1 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

template <int KVF, int G, bool PAGED, bool Q8>
__global__ void __launch_bounds__(kThreads, 1) k_prefill_gqa(PrefillParams P) {
  constexpr bool kFp4 = KVF == KVQ_NVFP4;
  constexpr bool K8 = Q8 && KVF == KVQ_FP8E4M3;   // Q.K^T on FP8 MFMA
  constexpr int RB = kFp4 ? kD / 2 : kD;   // code bytes per row
  constexpr int SB = kD / 16;              // NVFP4 scale bytes per row
  constexpr int QB = kRows / G;            // query tokens per work-group

  __shared__ __align__(16) uint8_t lds[kLdsBytes];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  // XCD-aware order: work-groups are handed to the 8 XCDs in turn (slot L
  // to XCD L mod 8), and slot L takes work item (L mod 8) * (N / 8) + L / 8,
  // so each XCD holds whole (request, kv head) groups, whose query blocks all
  // read the same K and V through that XCD's L2 (a bijection of the N items:
  // the results do not depend on the dispatch order; 1024-token chunk over
  // the 32K cache: 1039-1054 -> 1010-1033 us side by side).  Within an XCD
  // the query blocks still start longest first.
  int item = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  if (const int n_items = gridDim.x * gridDim.y * gridDim.z; n_items % 8 == 0) item = (item % 8) * (n_items / 8) + item / 8;
  const int qb = static_cast<int>(gridDim.x) - 1 - item % static_cast<int>(gridDim.x);   // longest first
  const int hk = (item / gridDim.x) % gridDim.y, b = item / (gridDim.x * gridDim.y);
  const int i0 = qb * QB;

  int L = P.kv_lens[b];
  L = L < 0 ? 0 : (L > P.max_kv_len ? P.max_kv_len : L);
  const int pos0 = L - P.Sq;                                  // position of query token 0
  const int i_last = (i0 + QB < P.Sq ? i0 + QB : P.Sq) - 1;   // last query token of the block
  int n_end = pos0 + i_last + 1;                              // keys [0, n_end) are seen by some row
  n_end = n_end < 0 ? 0 : (n_end > L ? L : n_end);
  const int p_min = pos0 + i0;                                // position of the block's first row
  const int ntiles = (n_end + kTile - 1) / kTile;

  const float ksc = P.k_scale[P.per_head ? hk : 0];
  const float vsc = P.v_scale[P.per_head ? hk : 0];
  // raw score -> log2 units, per row block (an FP8 query's scale may be per head)
  float c2r[2];

  // ---- this lane's query rows: B operand of S^T = K . Q^T, lane (g, c)
  // holds row c of each block, elements 32 kk + 8 g .. + 7
  f16x8 qop[2][4];
  i64x1 qop8[2][4];   // K8: the E4M3 codes themselves
  int prow[2];   // key positions <= prow are visible to the lane's row
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = 32 * w + 16 * rb + c;
    const int qi = i0 + r / G, h = hk * G + r % G;
    prow[rb] = pos0 + qi;
    const bool valid = qi < P.Sq;
    const float qs = Q8 ? P.q_scale[P.q_scale_per_head ? h : 0] : 1.0f;
    c2r[rb] = P.softmax_scale * ksc * qs * kLog2e;
    if constexpr (Q8) {
      const uint8_t* qp8 = reinterpret_cast<const uint8_t*>(P.q) + b * P.q_sb + static_cast<int64_t>(qi) * P.q_st +
                           h * P.q_sh + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint2 wv = valid ? *reinterpret_cast<const uint2*>(qp8 + 32 * kk) : uint2{0, 0};
        if constexpr (K8) {
          qop8[rb][kk] = static_cast<i64x1>((static_cast<uint64_t>(wv.y) << 32) | wv.x);
        } else {   // E4M3 -> f16, exact
          qop[rb][kk] = cat4(fp8x2<false>(wv.x), fp8x2<true>(wv.x), fp8x2<false>(wv.y), fp8x2<true>(wv.y));
        }
      }
      continue;
    }
    const uint16_t* qp = P.q + b * P.q_sb + static_cast<int64_t>(qi) * P.q_st + h * P.q_sh + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 wv = valid ? *reinterpret_cast<const uint4*>(qp + 32 * kk) : uint4{0, 0, 0, 0};
      const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
      f16x8 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) {   // bf16 pair -> f16 pair through fp32 (RNE)
        o[2 * k] = static_cast<_Float16>(__uint_as_float(ws[k] << 16));
        o[2 * k + 1] = static_cast<_Float16>(__uint_as_float(ws[k] & 0xFFFF0000u));
      }
      qop[rb][kk] = o;
    }
  }

  // ---- staging roles: K token kt, elements 32 kq .. + 31; V group vq (tokens
  // 4 vq .. + 3), elements 8 vr .. + 7
  // (f16 K: token-major, lane (g, c) of wave w stages token 16 w + c, quarter
  // g, so that a 16-lane row of the wave writes 16 tokens: conflict-free
  // under the 256-byte K rows' swizzle; FP8 K: four consecutive lanes per
  // token, conflict-free under its 128-byte rows' swizzle.  Both read the
  // tile's bytes with fully used 64-byte runs per token.)
  // (group A's threads stage K, group B's stage V: t8 is the thread's index
  // in its group)
  const int t8 = tid & 255;
  const bool grp_a = tid < 256;   // wave-uniform
  const int kt = K8 ? t8 >> 2 : 16 * (t8 >> 6) + (t8 & 15);
  const int kq = K8 ? t8 & 3 : (t8 >> 4) & 3;
  const int vr = t8 >> 4, vq = t8 & 15;
  const int kst_off = kt * kKRow;
  const int vst_off = (8 * vr) * kVtRow + 2 * vt_slot(4 * vq);

  auto tile_row = [&](int t0) -> int64_t {   // plane row of tile token 0
    if constexpr (PAGED) {
      // tiles past the seen keys are loaded with empty ranges: their table
      // entry is never used, so read the entry of the last seen key instead
      const int tc = t0 < n_end ? t0 : (n_end > 0 ? n_end - 1 : 0);
      const int blk = P.block_table[b * P.bt_stride + (tc >> P.log2_bs)];
      return static_cast<int64_t>(blk) * P.kv_sblk + hk * P.kv_sh + (t0 & ((1 << P.log2_bs) - 1));
    } else {
      return b * P.kv_sb + hk * P.kv_sh + t0;
    }
  };
  // keys of tile n that some row sees (<= 0 past the last tile: the range-
  // checked loads of such a tile read nothing and return zeros)
  auto tile_keys = [&](int n) { return n_end - n * kTile < kTile ? n_end - n * kTile : kTile; };

  Raw<KVF> raw;
  auto load_k = [&](int n) {
    const int nv = tile_keys(n);
    const int64_t row = tile_row(n * kTile);
    const Rsrc rk = make_rsrc(P.k_codes + row * RB, nv * RB);
    if constexpr (kFp4) {
      raw.k[0] = ld128(rk, kt * RB + 16 * kq);
      const Rsrc rks = make_rsrc(P.k_scales + row * SB, nv * SB);
      raw.ks = ld16(rks, kt * SB + 2 * kq);
    } else {
      raw.k[0] = ld128(rk, kt * RB + 32 * kq);
      raw.k[1] = ld128(rk, kt * RB + 32 * kq + 16);
    }
  };
  auto load_v = [&](int n) {
    const int nv = tile_keys(n);
    const int ng = nv > 0 ? (nv + 3) >> 2 : 0;
    const int64_t row = tile_row(n * kTile);
    const Rsrc rv = make_rsrc(P.v_codes + row * RB, ng * 4 * RB);
    if constexpr (kFp4) {
      raw.v[0] = ld128(rv, vq * 4 * RB + 16 * vr);
      const Rsrc rvs = make_rsrc(P.v_scales + row * SB, ng * 4 * SB);
      raw.vs = ld32(rvs, vq * 4 * SB + 4 * (vr >> 1));
    } else {
      raw.v[0] = ld128(rv, vq * 4 * RB + 32 * vr);
      raw.v[1] = ld128(rv, vq * 4 * RB + 32 * vr + 16);
    }
  };

  // K: 4 chunks of 8 elements, chunk j of row kt at 16 (j ^ (kt & 15))
  int kst[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kst[j] = kst_off + 16 * ((4 * kq + j) ^ (kt & 15));
  auto stage_k = [&](uint8_t* kb) {
    if constexpr (K8) {
      // the token's 32 code bytes as 4 chunks of 8 (elements 32 kq + 8 j ..),
      // chunk j of row kt at 8 ((4 kq + j) ^ (kt & 15)) of a 128-byte row
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 x = {raw.k[j >> 1][2 * (j & 1)], raw.k[j >> 1][2 * (j & 1) + 1]};
        lds_st<u32x2>(kb + kt * kD + 8 * ((4 * kq + j) ^ (kt & 15)), x);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x8 x;
      if constexpr (kFp4) {
        const uint32_t wd = raw.k[0][j];
        x = cat4(fp4x2<0>(wd), fp4x2<1>(wd), fp4x2<2>(wd), fp4x2<3>(wd));
        const f16x2 s2 = fp8x2<false>(raw.ks);
        const _Float16 sc = j < 2 ? s2[0] : s2[1];
        x = x * sc;
      } else {
        const uint32_t w0 = raw.k[j >> 1][2 * (j & 1)], w1 = raw.k[j >> 1][2 * (j & 1) + 1];
        x = cat4(fp8x2<false>(w0), fp8x2<true>(w0), fp8x2<false>(w1), fp8x2<true>(w1));
      }
      lds_st<f16x8>(kb + kst[j], x);
    }
  };
  // V: for each of the 8 elements, the 4 tokens' values (8 bytes) at their
  // slots in row 8 vr + x; tokens at or past the tile's seen keys are
  // cleared (a group that straddles them may hold stale or NaN bytes there)
  auto stage_v = [&](auto partial_tag, uint8_t* vb, int nv) {
    constexpr bool PARTIAL = decltype(partial_tag)::value;   // the tile holds fewer than kTile seen keys
    uint32_t m01 = 0xFFFFFFFFu, m23 = 0xFFFFFFFFu;
    const bool straddle = PARTIAL && 4 * vq + 4 > nv;
    if (straddle) {
      const int t = 4 * vq;
      m01 = (t + 0 < nv ? 0x0000FFFFu : 0u) | (t + 1 < nv ? 0xFFFF0000u : 0u);
      m23 = (t + 2 < nv ? 0x0000FFFFu : 0u) | (t + 3 < nv ? 0xFFFF0000u : 0u);
    }
    f16x2 lo[8], hi[8];   // tokens (0, 1) and (2, 3) of element 8 vr + x
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      if constexpr (kFp4) {
        const uint32_t wd = raw.v[0][x >> 1];
        const f16x2 s01 = fp8x2<false>(raw.vs), s23 = fp8x2<true>(raw.vs);
        if (x & 1) {
          lo[x] = fp4x2<2>(wd) * s01;
          hi[x] = fp4x2<3>(wd) * s23;
        } else {
          lo[x] = fp4x2<0>(wd) * s01;
          hi[x] = fp4x2<1>(wd) * s23;
        }
      } else {
        const uint32_t wd = raw.v[x >> 2][x & 3];
        lo[x] = fp8x2<false>(wd);
        hi[x] = fp8x2<true>(wd);
      }
    }
    if constexpr (PARTIAL) {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        lo[x] = as_h2(as_u32(lo[x]) & m01);
        hi[x] = as_h2(as_u32(hi[x]) & m23);
      }
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) lds_st<u32x2>(vb + vst_off + x * kVtRow, u32x2{as_u32(lo[x]), as_u32(hi[x])});
  };

  // ---- MFMA operand addresses (bytes inside a stage)
  int kld[4];   // K row 16 u + c, chunk 4 kk + g (swizzled); + 16 u rows per sub-tile
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) kld[kk] = c * kKRow + 16 * ((4 * kk + g) ^ c);
  const int vld = c * kVtRow + 16 * g;   // V^T row 16 db + c, slots 32 kc + 8 g

  // S^T = K . Q^T: s[rb][u][e] = score of tile token 16 u + 4 g + e, row c.
  // The K operands of sub-tile u + 1 are read from LDS while the MFMAs of
  // sub-tile u run (the scheduling fences keep that order).
  auto qk = [&](const uint8_t* kb, f32x4 (&sc)[2][4]) {
    if constexpr (K8) {
      // A = K codes (16 tokens x 32 elements, 8 bytes a lane), B = Q^T codes
      int kl8[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kl8[kk] = c * kD + 8 * ((4 * kk + g) ^ c);
      i64x1 ka8[2][4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) ka8[0][kk] = lds_ld<i64x1>(kb + kl8[kk]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (u < 3) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) ka8[(u + 1) & 1][kk] = lds_ld<i64x1>(kb + kl8[kk] + (u + 1) * 16 * kD);
        }
        __builtin_amdgcn_sched_barrier(0);
        sc[0][u] = f32x4{0.f, 0.f, 0.f, 0.f};
        sc[1][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          sc[0][u] = mfma_fp8(ka8[u & 1][kk], qop8[0][kk], sc[0][u]);
          sc[1][u] = mfma_fp8(ka8[u & 1][kk], qop8[1][kk], sc[1][u]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
    f16x8 ka[2][4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) ka[0][kk] = lds_ld<f16x8>(kb + kld[kk]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u < 3) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) ka[(u + 1) & 1][kk] = lds_ld<f16x8>(kb + kld[kk] + (u + 1) * 16 * kKRow);
      }
      __builtin_amdgcn_sched_barrier(0);
      sc[0][u] = f32x4{0.f, 0.f, 0.f, 0.f};
      sc[1][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        sc[0][u] = mfma(ka[u & 1][kk], qop[0][kk], sc[0][u]);
        sc[1][u] = mfma(ka[u & 1][kk], qop[1][kk], sc[1][u]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- running state per row block: reference maximum (log2 units),
  // denominator, O^T accumulators (lane (g, c): row c, elements 16 db + 4 g
  // .. + 3).  The denominator is one more MFMA accumulator: an all-ones A
  // operand times the P^T operand sums the f16 probabilities of row c that
  // P.V uses (every element of lane (g, c) holds row c's sum), so the
  // softmax phase forms no sums and the epilogue no cross-lane reduction;
  // numerator and denominator then carry the same rounded probabilities.
  // The reference is raised only when a tile's maximum exceeds it by more
  // than kLazy (then the accumulators are rescaled); otherwise probabilities
  // up to 2^kLazy are formed against the old reference, which is exact in
  // real arithmetic and keeps f16's relative precision for P.
  constexpr float kLazy = 8.f;
  float m[2] = {-INFINITY, -INFINITY};
  f32x4 lsum[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const f16x8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
  f32x4 acc[2][8];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The softmax of tile n in two parts.  tile_max: (MASK: clear the scores
  // of keys past each row's position,) take the tile's row maxima and move
  // the reference maxima, giving the factors alpha by which the
  // accumulators and the denominator are rescaled (any != 1 in the wave:
  // `rescale`).  probs: P = exp2(score * c2 - m) as the f16 P^T operands.
  float alpha[2] = {1.f, 1.f};
  bool rescale = false;
  auto tile_max = [&](auto mask_tag, f32x4 (&sc)[2][4], int n) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int t0 = n * kTile;
    rescale = false;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      if constexpr (MASK) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (t0 + 16 * u + 4 * g + e > prow[rb]) sc[rb][u][e] = -INFINITY;
      }
      float mx = sc[rb][0][0];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sc[rb][u][e]);
      mx = lanes::across_rows<lanes::Max>(mx) * c2r[rb];
      const bool up = mx > m[rb] + kLazy;   // false when mx = -inf
      alpha[rb] = up ? __builtin_amdgcn_exp2f(m[rb] - mx) : 1.f;   // 0 when m = -inf
      m[rb] = up ? mx : m[rb];
      rescale |= up;
    }
  };
  auto probs = [&](const f32x4 (&sc)[2][4], f16x8 (&pb)[2][2]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float m_use = m[rb] == -INFINITY ? 0.f : m[rb];
      float p[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[u][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[rb][u][e], c2r[rb], -m_use));
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = static_cast<_Float16>(p[2 * kc][e]);
          v[4 + e] = static_cast<_Float16>(p[2 * kc + 1][e]);
        }
        pb[rb][kc] = v;
      }
    }
  };
  auto rescale_acc = [&]() {
    if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[rb][db] *= alpha[rb];
        lsum[rb] *= alpha[rb];
      }
    }
  };

  // O^T += V^T . P^T: A = V^T (16 elements x 32 token slots), B = P^T;
  // element block db + 1's operands are read while block db's MFMAs run;
  // then the denominator: all-ones A times the same P^T
  auto pv = [&](const uint8_t* vb, const f16x8 (&pb)[2][2]) {
    f16x8 va[2][2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) va[0][kc] = lds_ld<f16x8>(vb + vld + kc * 64);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      if (db < 7) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) va[(db + 1) & 1][kc] = lds_ld<f16x8>(vb + vld + (db + 1) * 16 * kVtRow + kc * 64);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        acc[0][db] = mfma(va[db & 1][kc], pb[0][kc], acc[0][db]);
        acc[1][db] = mfma(va[db & 1][kc], pb[1][kc], acc[1][db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      lsum[0] = mfma(ones, pb[0][kc], lsum[0]);
      lsum[1] = mfma(ones, pb[1][kc], lsum[1]);
    }
  };

  // ---- the tile loop.  Two LDS stages (K and V^T of one tile each): tile n
  // is read from stage n % 2 while tile n + 1 is staged into the other one,
  // in the phase order of the header (K(n + 1) is staged after B's Q.K^T of
  // tile n, V(n + 1) before A's P.V of tile n + 1; every stage is written
  // only after both groups' last read of its previous tile).  The raw bytes
  // of tile n + 2 are loaded right after tile n + 1 is staged.
  uint8_t* const kbuf = lds;
  uint8_t* const vbuf = lds + 2 * kKBytes;
  // tiles whose keys every row sees (no causal mask needed)
  int n_open = p_min >= kTile - 1 ? (p_min - (kTile - 1)) / kTile + 1 : 0;
  n_open = n_open < ntiles ? n_open : ntiles;
  auto stage_v_tile = [&](uint8_t* vb, int n) {
    if (tile_keys(n) < kTile)
      stage_v(std::true_type{}, vb, tile_keys(n));
    else
      stage_v(std::false_type{}, vb, kTile);
  };
  if (ntiles > 0) {
    if (grp_a) {
      load_k(0);
      stage_k(kbuf);
      load_k(1);
    } else {
      load_v(0);
      stage_v_tile(vbuf, 0);
      load_v(1);
    }
  }
  lds_barrier();
  auto step = [&](auto mask_tag, int n) {
    f32x4 sc[2][4];
    f16x8 pb[2][2];
    uint8_t* const kb = kbuf + (n & 1) * kKBytes;
    uint8_t* const vb = vbuf + (n & 1) * kVtBytes;
    uint8_t* const kb1 = kbuf + ((n + 1) & 1) * kKBytes;
    uint8_t* const vb1 = vbuf + ((n + 1) & 1) * kVtBytes;
    auto softmax = [&]() {
      tile_max(mask_tag, sc, n);
      rescale_acc();
      probs(sc, pb);
    };
    if (grp_a) {   // phase 1
      qk(kb, sc);
    } else {
      stage_v_tile(vb1, n + 1);
      load_v(n + 2);
    }
    lds_barrier();
    if (grp_a)     // phase 2
      softmax();
    else
      qk(kb, sc);
    lds_barrier();
    if (grp_a)     // phase 3
      pv(vb, pb);
    else
      softmax();
    lds_barrier();
    if (grp_a) {   // phase 4
      stage_k(kb1);
      load_k(n + 2);
    } else {
      pv(vb, pb);
    }
    lds_barrier();
  };
  int n = 0;
  for (; n < n_open; ++n) step(std::false_type{}, n);
  for (; n < ntiles; ++n) step(std::true_type{}, n);

  // ---- epilogue: o = acc / l * s_t,V, lse = ln 2 (m + log2 l), l = the
  // denominator (every element of lsum holds it)
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float lt = lsum[rb][0];
    const int r = 32 * w + 16 * rb + c;
    const int qi = i0 + r / G, h = hk * G + r % G;
    if (qi >= P.Sq) continue;
    const float inv = lt > 0.f ? vsc / lt : 0.f;
    const int64_t ob = b * P.o_sb + static_cast<int64_t>(qi) * P.o_st + h * P.o_sh + 4 * g;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const f32x4 o = acc[rb][db] * inv;
      if (P.out_dtype == KVQ_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(P.out) + ob + 16 * db) = o;
      } else {
        const u32x2 pk = {static_cast<uint32_t>(bf16_rne(o[0])) | (static_cast<uint32_t>(bf16_rne(o[1])) << 16),
                          static_cast<uint32_t>(bf16_rne(o[2])) | (static_cast<uint32_t>(bf16_rne(o[3])) << 16)};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(P.out) + ob + 16 * db) = pk;
      }
    }
    if (P.lse != nullptr && g == 0)
      P.lse[(static_cast<int64_t>(b) * P.Sq + qi) * P.Hq + h] = lt > 0.f ? kLn2 * (m[rb] + __log2f(lt)) : -INFINITY;
  }
}

template <int KVF, int G>
hipError_t launch_g(const PrefillParams& p, hipStream_t st) {
  const dim3 grid((p.Sq * G + kRows - 1) / kRows, p.Hkv, p.B);
  const bool q8 = p.q_dtype == KVQ_FP8E4M3;
  if (p.block_table != nullptr) {
    if (q8)
      hipLaunchKernelGGL((k_prefill_gqa<KVF, G, true, true>), grid, dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL((k_prefill_gqa<KVF, G, true, false>), grid, dim3(kThreads), 0, st, p);
  } else {
    if (q8)
      hipLaunchKernelGGL((k_prefill_gqa<KVF, G, false, true>), grid, dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL((k_prefill_gqa<KVF, G, false, false>), grid, dim3(kThreads), 0, st, p);
  }
  return hipGetLastError();
}

template <int KVF>
hipError_t launch_fmt(const PrefillParams& p, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_g<KVF, 1>(p, st);
    case 2: return launch_g<KVF, 2>(p, st);
    case 4: return launch_g<KVF, 4>(p, st);
    default: return launch_g<KVF, 8>(p, st);
  }
}

}  // namespace pf

hipError_t launch_prefill_gqa(const PrefillParams& p, int kv_format, int G, hipStream_t st) {
  return kv_format == KVQ_NVFP4 ? pf::launch_fmt<KVQ_NVFP4>(p, G, st) : pf::launch_fmt<KVQ_FP8E4M3>(p, G, st);
}

}  // namespace kvq
