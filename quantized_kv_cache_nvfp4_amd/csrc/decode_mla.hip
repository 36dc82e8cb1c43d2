// Split-KV flash decode over a DeepSeek-style MLA latent cache (NVFP4
// latent c + bf16 rope key) for gfx950.
//
// Method: Model-Optimizer PR #714 (KV-cache quantization for MLAAttention in
// vLLM fake-quant), "What does this PR do?" and "Testing": MLA attention
// caches one latent row c per token (kv_lora_rank 512) plus a rope key; only
// the latent is quantized (NVFP4, blocks of 16); the absorbed query gives
// score = softmax_scale * (q_c . c_hat + q_r . k_r) and output = P . c_hat.
// The split-KV scheme is that of Model-Optimizer PR #1832 "Add quant+sparse
// attention for vLLM serving", Testing section.
//
// Design for CDNA4:
//  * one work-group = 4 waves = one chunk of one request; all 16 query
//    heads share every latent row, so they are the 16 MFMA rows and no
//    query-group packing is needed.
//  * tiles of 64 tokens (4 sub-tiles of 16).  Scores: wave w covers the
//    sub-tiles u = (w & 1) + 2q of the tile over latent half (w >> 1) (256
//    dims) and rope half (32 dims): per sub-tile 8 MFMA 16x16x32 f16 steps
//    over the dequantized latent plus one bf16 step over the rope; the two
//    latent halves' partial scores meet in LDS.  The dequantized latent rows
//    (f16) are staged in LDS.  Two barriers per tile.
//  * P.V: wave w owns output columns 128w .. 128w+127 for all 64 tokens (two
//    32-token steps); its A operand (latent, token-contiguous per column)
//    comes from the staged rows through the LDS transpose read
//    ds_read_b64_tr_b16, so the latent is dequantized once and used by both
//    contractions, and its B operand (P) is already in the right lanes (the
//    token order of the P.V contraction is chosen to match the score
//    layout).
//  * every wave computes the softmax of the whole tile (8 scores per lane),
//    so the four waves share one reference maximum and one denominator.
//  * loads use buffer resources sized to the chunk (tokens past its end read
//    zeros), as in the GQA kernel.
//  * paged caches (vLLM-style block tables): the block size is a power of
//    two and a multiple of the tile, so every 64-token tile lies in one
//    block; a work-group copies its chunk's table entries into LDS once and
//    addresses each tile through them (the first tile through an entry read
//    directly, so that its loads need not wait for the copy).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_common.h"
#include "kvq_internal.h"
#include "wave_reduce.h"

#ifndef KVQ_MLA_AHEAD
#define KVQ_MLA_AHEAD 1
#endif
#ifndef KVQ_MLA_TILE
#define KVQ_MLA_TILE 64
#endif

namespace kvq {
namespace {

using namespace dec;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kW = 4;                      // waves per work-group
constexpr int kThreads = 64 * kW;
constexpr int kT = KVQ_MLA_TILE;           // tokens per tile (32 or 64)
constexpr int kQ = kT / 32;                // 16-token sub-tiles per wave: u = th + 2 q, q < kQ
constexpr int kH = 16;                     // query heads (MFMA rows)
constexpr int kD = 512;                    // latent rank
constexpr int kDr = 64;                    // rope dims
constexpr int kRow = kD / 2;               // latent code bytes per token
constexpr int kSRow = kD / 16;             // latent scale bytes per token
constexpr int kPitch = kD * 2 + 32;        // staged f16 row pitch in LDS (bytes; +32 spreads banks)
constexpr int kAhead = KVQ_MLA_AHEAD;      // tiles loaded ahead of the one being computed

__device__ inline f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// QNV: the latent query q_c arrives as NVFP4 codes + block scales + tensor
// scale (dequantized exactly to f16 in the prologue) instead of bf16
template <bool PAGED, bool QNV>
__global__ void __launch_bounds__(kThreads, 2) k_decode_mla(kvq_decode_args a, int num_splits) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_c[kT * kPitch];   // staged latent rows (f16)
  __shared__ __attribute__((aligned(16))) f32x4 lds_s[kW][kQ][64];      // partial scores per wave, sub-tile, lane
  __shared__ int lds_bt[PAGED ? kMlaPagedMaxChunkBlocks : 1];          // paged: the chunk's block-table entries

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;   // MFMA row / column index of this lane
  const int g = lane >> 4;   // lane group (k-slice of the MFMA operands)
  const int th = wave & 1;   // token half of the tile this wave scores
  const int dh = wave >> 1;  // latent / rope half this wave scores
  // LDS bank spreading of the staged rows: chunk k (16 bytes) of row r sits at
  // k ^ swz(r), swz(r) = bit 2 of r xor bit 3 of r, which makes both the
  // row-wise 16-byte stores and the transposed 8-byte reads conflict-free.
  const int swz_w = ((c >> 2) ^ (c >> 3)) & 1;   // rows 16 th + c (stores)
  const int swz_r = (g ^ (g >> 1)) & 1;          // rows 4 g + m/4 and 16 + 4 g + m/4 (transposed reads)
  const int split = blockIdx.x;
  const int b = blockIdx.y;

  // chunking from kernel arguments only: c = ceil(max_kv_len / s) rounded
  // up to the tile, split j covers [j c, min((j+1) c, L)); the first tiles'
  // addresses are known before the request length is read
  int chunk = (a.max_kv_len + num_splits - 1) / num_splits;
  chunk = (chunk + kT - 1) / kT * kT;
  const int cs = split * chunk;
  int ce_ld = (cs + chunk < a.max_kv_len) ? cs + chunk : a.max_kv_len;   // load bound (rows present)

  // per-request plane bases (rows of the latent, scale and rope planes);
  // paged planes are addressed from the plane start through the table
  const int64_t row0 = PAGED ? 0 : static_cast<int64_t>(b) * a.kv_sb;
  const int st = static_cast<int>(a.kv_st);
  const uint8_t* cc = a.k_codes + row0 * kRow;
  const uint8_t* csc = a.k_scales + row0 * kSRow;
  const uint8_t* cr = static_cast<const uint8_t*>(a.k_rope) + row0 * (kDr * 2);

  // paged: block tb >> bsh holds token tb at row tb & (bs - 1); entries are
  // kept for the blocks of rows [cs, ce) only, so the request length is
  // read before the first loads (an entry past the request's end need not
  // be a valid block)
  const int bs = PAGED ? a.block_size : 1;
  const int bsh = PAGED ? __builtin_ctz(static_cast<unsigned>(bs)) : 0;
  const int blk0 = cs >> bsh;
  int L = 0, ce = 0;
  int64_t first_row = 0;   // paged: plane row of the chunk's first token
  if constexpr (PAGED) {
    L = a.kv_lens[b];
    L = L < a.max_kv_len ? L : a.max_kv_len;
    L = L > 0 ? L : 0;
    ce = (cs + chunk < L) ? cs + chunk : L;
    ce_ld = ce;
    const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.bt_stride + blk0;
    if (cs < ce) first_row = static_cast<int64_t>(bt[0]) * a.kv_sblk + static_cast<int64_t>(cs & (bs - 1)) * st;
    const int nblk = ce > cs ? ((ce - 1) >> bsh) - blk0 + 1 : 0;
    for (int i = threadIdx.x; i < nblk; i += kThreads) lds_bt[i] = bt[i];
  }
  // plane row of tile's first token (relative to the request's base when
  // the cache is contiguous); tiles past the chunk's end get 0 (they load
  // nothing).  Paged tiles after the first read the LDS copy of the table.
  auto tile_row = [&](int tile) -> int64_t {
    const int tb = cs + tile * kT;
    if constexpr (PAGED) {
      if (tile == 0) return first_row;
      if (tb >= ce_ld) return 0;
      return static_cast<int64_t>(lds_bt[(tb >> bsh) - blk0]) * a.kv_sblk + static_cast<int64_t>(tb & (bs - 1)) * st;
    } else {
      return static_cast<int64_t>(tb) * st;
    }
  };

  // loads of one tile: for each of the wave's sub-tiles u = th + 2 q, token
  // 16 u + c; latent bytes [128 dh + 32 g, +32), scale bytes [16 dh + 4 g,
  // +4), rope bytes [64 dh + 16 g, +16).  Tokens at or past the load bound
  // ce_ld read zeros; a tile past it reads nothing.
  struct Raw {
    u32x4 cw0[kQ], cw1[kQ], rw[kQ];
    uint32_t sw[kQ];
  };
  auto load_tile = [&](Raw& R, int tile) {
    const int64_t trow = tile_row(tile);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int t0 = cs + tile * kT + 16 * (th + 2 * q);
      const int nv = ce_ld - t0;
      const int64_t r0 = trow + static_cast<int64_t>(16 * (th + 2 * q)) * st;
      const Rsrc rc_ = make_rsrc(cc + r0 * kRow, nv * st * kRow);
      const Rsrc rs_ = make_rsrc(csc + r0 * kSRow, nv * st * kSRow);
      const Rsrc rr_ = make_rsrc(cr + r0 * (kDr * 2), nv * st * (kDr * 2));
      R.cw0[q] = ld128(rc_, c * st * kRow + 128 * dh + 32 * g);
      R.cw1[q] = ld128(rc_, c * st * kRow + 128 * dh + 32 * g + 16);
      R.sw[q] = ld32(rs_, c * st * kSRow + 16 * dh + 4 * g);
      R.rw[q] = ld128(rr_, c * st * (kDr * 2) + 64 * dh + 16 * g);
    }
  };
  // ---- query words, lane (g, c) = head c:
  //   latent MFMA j (0..7): dims 256 dh + 64 g + 8 j + e; rope: 32 dh + 8 g + e
  //   (NVFP4 latent query: the same 64 elements are code bytes [128 dh +
  //   32 g, +32) and scale bytes [16 dh + 4 g, +4) of head c's row)
  uint4 qraw[8], qrraw;
  uint32_t qsw = 0;
  {
    if constexpr (QNV) {
      const int64_t qrow = static_cast<int64_t>(b) * a.q_sb + static_cast<int64_t>(c) * a.q_sh;
      const uint8_t* qc = static_cast<const uint8_t*>(a.q) + qrow * (kD / 2) + 128 * dh + 32 * g;
      qraw[0] = *reinterpret_cast<const uint4*>(qc);
      qraw[1] = *reinterpret_cast<const uint4*>(qc + 16);
      qsw = *reinterpret_cast<const uint32_t*>(a.q_block_scales + qrow * (kD / 16) + 16 * dh + 4 * g);
    } else {
      const uint16_t* qc = static_cast<const uint16_t*>(a.q) + static_cast<int64_t>(b) * a.q_sb +
                           static_cast<int64_t>(c) * a.q_sh + 256 * dh + 64 * g;
#pragma unroll
      for (int j = 0; j < 8; ++j) qraw[j] = *reinterpret_cast<const uint4*>(qc + 8 * j);
    }
    const uint16_t* qrp = static_cast<const uint16_t*>(a.q_rope) + static_cast<int64_t>(b) * a.qr_sb +
                          static_cast<int64_t>(c) * a.qr_sh + 32 * dh + 8 * g;
    qrraw = *reinterpret_cast<const uint4*>(qrp);
  }

  // the first kAhead tiles, requested with the query and the request length
  // (one memory round trip); kAhead tiles are in flight while one computes:
  // buffer (tile mod kAhead+1) holds tile's data.  Tiles past the chunk load
  // nothing.
  Raw buf[kAhead + 1];
#pragma unroll
  for (int k = 0; k < kAhead; ++k) {
    load_tile(buf[k], k);
    __builtin_amdgcn_sched_barrier(0);   // issue order = tile order, so a wait for one tile spares the later ones
  }

  if constexpr (PAGED) {
    __syncthreads();   // the LDS table copy is visible to the later tiles' loads
  } else {
    L = a.kv_lens[b];
    L = L < a.max_kv_len ? L : a.max_kv_len;
    L = L > 0 ? L : 0;
    ce = (cs + chunk < L) ? cs + chunk : L;
    ce_ld = ce;   // later loads stop at the request's end
  }
  const int ntiles = cs < ce ? (ce - cs + kT - 1) / kT : 0;

  const float s_t = *a.k_scale;
  // latent scores carry the tensor scale of the latent (and of an NVFP4 query)
  const float sc_lat = a.softmax_scale * s_t * (QNV ? *a.q_scale : 1.0f) * kLog2e;
  const float sc_rope = a.softmax_scale * kLog2e;

  f16x8 qop[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (QNV) {
      // elements 8j..8j+7 of the lane's 64: code dword j, block j / 2
      // (E2M1 x E4M3 is exact in f16)
      const uint4& qw = j < 4 ? qraw[0] : qraw[1];
      const uint32_t w = (j & 3) == 0 ? qw.x : ((j & 3) == 1 ? qw.y : ((j & 3) == 2 ? qw.z : qw.w));
      const f16x2 s2 = fp8x2<false>(qsw >> (16 * ((j >> 1) >> 1)));
      const _Float16 sv = ((j >> 1) & 1) ? s2[1] : s2[0];
      const f16x2 sp = f16x2{sv, sv};
      qop[j] = cat4(fp4x2<0>(w) * sp, fp4x2<1>(w) * sp, fp4x2<2>(w) * sp, fp4x2<3>(w) * sp);
      continue;
    }
    const uint32_t ws[4] = {qraw[j].x, qraw[j].y, qraw[j].z, qraw[j].w};
    f16x2 h[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)   // bf16 pair -> fp32 (exact) -> f16 (exact in f16's normal range)
      h[k] = f16x2{static_cast<_Float16>(__uint_as_float(ws[k] << 16)),
                   static_cast<_Float16>(__uint_as_float(ws[k] & 0xFFFF0000u))};
    qop[j] = cat4(h[0], h[1], h[2], h[3]);
  }
  const bf16x8 qr = __builtin_bit_cast(bf16x8, qrraw);

  float m_run = -INFINITY;   // running max of head c (log2 domain), the same in every wave
  float l_run = 0.0f;        // this lane's share of head c's denominator (its 8 tokens per tile)
  f32x4 acc_o[8];            // O^T rows d = 128*wave + 16*jj + 4g + i, column head c
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc_o[jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](Raw& cur, int tile) {
    const int tb = cs + tile * kT;
    // the chunk's last tile: rows of tokens at or past the request's end
    // (read before the length was known) become zeros, so that the staged
    // latent of masked tokens is 0 (their probability is 0).  (The empty asm
    // keeps this a branch taken once per chunk instead of selects on every
    // tile.)
    if (tb + kT > ce) {
      asm volatile("");
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        if (tb + 16 * (th + 2 * q) + c >= ce) {
          cur.cw0[q] = u32x4{0u, 0u, 0u, 0u};
          cur.cw1[q] = cur.cw0[q];
          cur.rw[q] = cur.cw0[q];
          cur.sw[q] = 0u;
        }
      }
    }

    // ---- partial scores S^T[token][head] of the wave's sub-tiles over its
    // latent / rope halves; stage the f16 rows.  (Two latent accumulators,
    // even and odd steps: half the dependent MFMA chain.)
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const u32x4 cw0 = cur.cw0[q], cw1 = cur.cw1[q], rw = cur.rw[q];
      const uint32_t sw = cur.sw[q];
      f32x4 acc_l[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, acc_r = {0.f, 0.f, 0.f, 0.f};
      // token row 16 u + c (u = th + 2 q), dims 256 dh + 64 g ..; 16-byte
      // chunk k of the row is stored at k ^ swz(row) (swz uses row bits 2
      // and 3, those of c)
      uint8_t* stage = lds_c + (16 * (th + 2 * q) + c) * kPitch + 512 * dh + 128 * g;
      uint8_t* const stage_even = stage + 16 * swz_w;   // chunks with even k move by +16 bytes when swz = 1
      uint8_t* const stage_odd = stage - 16 * swz_w;    // odd k by -16
      const f16x2 sp0 = fp8x2<false>(sw), sp1 = fp8x2<true>(sw);             // scales of the lane's 4 blocks
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w = (j < 4) ? cw0[j] : cw1[j - 4];
        const _Float16 sv = (j < 4) ? ((j < 2) ? sp0[0] : sp0[1]) : ((j < 6) ? sp1[0] : sp1[1]);   // block j/2
        const f16x2 s2 = {sv, sv};
        const f16x8 kop = cat4(fp4x2<0>(w) * s2, fp4x2<1>(w) * s2, fp4x2<2>(w) * s2, fp4x2<3>(w) * s2);
        acc_l[j & 1] = mfma(kop, qop[j], acc_l[j & 1]);
        *reinterpret_cast<f16x8*>(((j & 1) ? stage_odd : stage_even) + 16 * j) = kop;
      }
      acc_r = mfma_bf16(__builtin_bit_cast(bf16x8, rw), qr, acc_r);
      f32x4 ps;
#pragma unroll
      for (int i = 0; i < 4; ++i) ps[i] = (acc_l[0][i] + acc_l[1][i]) * sc_lat + acc_r[i] * sc_rope;
      lds_s[wave][q][lane] = ps;
    }
    __syncthreads();   // staged rows and partial scores visible

    // ---- the whole tile's scores for this lane: tokens 16 u + 4 g + i of
    // every sub-tile u (latent halves: waves (u & 1) and 2 + (u & 1))
    float sc[2 * kQ][4];
#pragma unroll
    for (int u = 0; u < 2 * kQ; ++u) {
      const f32x4 p0 = lds_s[u & 1][u >> 1][lane], p1 = lds_s[2 + (u & 1)][u >> 1][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[u][i] = p0[i] + p1[i];
    }
    if (tb + kT > ce) {   // the chunk's last tile (uniform branch)
      asm volatile("");
#pragma unroll
      for (int u = 0; u < 2 * kQ; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tb + 16 * u + 4 * g + i >= ce) sc[u][i] = -INFINITY;
    }
    float tm = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2 * kQ; ++u)
      tm = fmaxf(tm, fmaxf(fmaxf(sc[u][0], sc[u][1]), fmaxf(sc[u][2], sc[u][3])));
    tm = lanes::across_rows<lanes::Max>(tm);   // head c's max over the four lane groups
    if (__any(tm > m_run)) {   // the same decision for column c in every wave
      const bool bump = tm > m_run;
      const float fac = bump ? __builtin_amdgcn_exp2f(m_run - tm) : 1.0f;   // 0 when m_run = -inf
      l_run *= fac;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_o[jj][i] *= fac;
      m_run = bump ? tm : m_run;
    }
    const float m_ref = (m_run == -INFINITY) ? 0.0f : m_run;
    // B operand of P.V step ks (k = 8g + e): e < 4 -> token 4g+e of sub-tile
    // 2 ks, e >= 4 -> token 4g+e-4 of sub-tile 2 ks + 1
    f16x8 pb[kQ];
#pragma unroll
    for (int ks = 0; ks < kQ; ++ks) {
      f16x2 ph[4];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float p0 = __builtin_amdgcn_exp2f(sc[2 * ks + x][2 * k] - m_ref);   // masked: exp2(-inf) = 0
          const float p1 = __builtin_amdgcn_exp2f(sc[2 * ks + x][2 * k + 1] - m_ref);
          l_run += p0 + p1;
          ph[2 * x + k] = f16x2{static_cast<_Float16>(p0), static_cast<_Float16>(p1)};
        }
      pb[ks] = cat4(ph[0], ph[1], ph[2], ph[3]);
    }

    // ---- P.V for this wave's 128 output columns over the tile's tokens,
    // 32 per step.  A = latent^T rows d, k = the tokens above: two
    // transposed reads of 4 token rows; lane m of the 16-lane group points
    // at row r + m/4, columns d0 + 4(m%4) .. +3, and receives column d0 + m
    // of the 4 rows.
#pragma unroll
    for (int ks = 0; ks < kQ; ++ks) {
      const int rlo = 32 * ks + 4 * g + (c >> 2), rhi = 32 * ks + 16 + 4 * g + (c >> 2);   // both have swz = swz_r
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int col = 256 * wave + 32 * jj + 16 * (((c >> 1) & 1) ^ swz_r) + 8 * (c & 1);
        const f16x4 lo = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(lds_c + rlo * kPitch + col)));
        const f16x4 hi = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(lds_c + rhi * kPitch + col)));
        const f16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc_o[jj] = mfma(av, pb[ks], acc_o[jj]);
      }
    }
    __syncthreads();   // the tile's LDS may be overwritten
  };

  // the loop is unrolled over the buffers so that each has fixed registers
  for (int t0 = 0; t0 < ntiles; t0 += kAhead + 1) {
#pragma unroll
    for (int u = 0; u <= kAhead; ++u) {
      if (t0 + u >= ntiles) break;
      load_tile(buf[(u + kAhead) % (kAhead + 1)], t0 + u + kAhead);
      __builtin_amdgcn_sched_barrier(0);
      process(buf[u], t0 + u);
    }
  }

  // ---- partials: o = acc * s_t / l, lse = (m + log2 l) ln 2 (l is the same in every wave)
  const float lt = lanes::across_rows<lanes::Sum>(l_run);
  const float f = lt > 0.0f ? s_t / lt : 0.0f;
  const int64_t po = (static_cast<int64_t>(b) * a.Hq + c) * num_splits + split;
  float* op = a.part_o + po * kD + 128 * wave + 4 * g;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj)
    *reinterpret_cast<float4*>(op + 16 * jj) =
        make_float4(acc_o[jj][0] * f, acc_o[jj][1] * f, acc_o[jj][2] * f, acc_o[jj][3] * f);
  if (wave == 0 && g == 0) a.part_lse[po] = lt > 0.0f ? (m_run + log2f(lt)) * kLn2 : -INFINITY;
}

}  // namespace

int mla_tile_tokens() { return kT; }

bool mla_supported(const kvq_decode_args& a) {
  return a.kv_format == KVQ_NVFP4 && a.Hq == kH && a.Hkv == 1 && a.D == kD && a.Dv == kD && a.Drope == kDr &&
         (a.q_dtype == KVQ_BF16 || a.q_dtype == KVQ_NVFP4);
}

hipError_t launch_decode_mla(const kvq_decode_args& a, const DecodePlan& p, hipStream_t st) {
  const dim3 grid(p.s, a.B);
  const bool qnv = a.q_dtype == KVQ_NVFP4;
  if (a.block_table != nullptr) {
    if (qnv)
      hipLaunchKernelGGL((k_decode_mla<true, true>), grid, dim3(kThreads), 0, st, a, p.s);
    else
      hipLaunchKernelGGL((k_decode_mla<true, false>), grid, dim3(kThreads), 0, st, a, p.s);
  } else {
    if (qnv)
      hipLaunchKernelGGL((k_decode_mla<false, true>), grid, dim3(kThreads), 0, st, a, p.s);
    else
      hipLaunchKernelGGL((k_decode_mla<false, false>), grid, dim3(kThreads), 0, st, a, p.s);
  }
  return hipGetLastError();
}

}  // namespace kvq
