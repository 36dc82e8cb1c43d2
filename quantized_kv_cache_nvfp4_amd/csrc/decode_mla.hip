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
//  * one work-group = 8 waves = one chunk of one request, as two groups of
//    4 waves that take alternate tiles of the chunk and merge their states
//    at the end (half the partials of two 4-wave work-groups per compute
//    unit, at the same two waves per SIMD); all 16 query heads share every
//    latent row, so they are the 16 MFMA columns and no query-group packing
//    is needed.
//  * tiles of 64 tokens; wave w owns sub-tile w (16 tokens) whole: its
//    scores over the full latent (16 MFMA 16x16x32 f16 steps over the
//    dequantized rows) plus the rope (2 bf16 steps), its softmax, and the
//    staging of its 16 dequantized rows (f16) into LDS.  Nothing of the
//    scores crosses waves; the probabilities do, through LDS (fp32), with
//    the reference each wave used.
//  * one reference maximum per head, shared by the four waves and raised
//    lazily: a wave whose tile maximum exceeds it by more than 2^8 (in P)
//    uses its own and says so; after the barrier every wave takes the
//    largest reference of the tile, rescales its accumulators when that
//    moved, and scales the probabilities of waves that used a smaller one
//    (exact fp32 products, then one rounding to f16).  Most tiles need no
//    rescale and no correction (wave-uniform branches).
//  * P.V: wave w owns output columns 128w .. 128w+127 for all 64 tokens (two
//    32-token steps); its A operand (latent, token-contiguous per column)
//    comes from the staged rows through the LDS transpose read
//    ds_read_b64_tr_b16, so the latent is dequantized once and used by both
//    contractions, and its B operand (P) is read from LDS in the token order
//    of that contraction.  Two barriers per tile; the two groups run half
//    a tile apart (one scores while the other runs P.V).
//  * the head_dim order of Q.K^T is free: lane group g of load instruction
//    k reads bytes [64 k + 16 g, +16) of its token's latent codes (each
//    instruction covers 64 contiguous bytes of every row), i.e. latent dims
//    128 k + 32 g .. + 31, and the query operand follows the same order.
//  * loads use buffer resources sized to the chunk (tokens past its end read
//    zeros), as in the GQA kernel.
//  * paged caches (vLLM-style block tables): the block size is a power of
//    two and a multiple of the tile, so every 64-token tile lies in one
//    block; a work-group copies its chunk's table entries into LDS once and
//    addresses each tile through them (each group's first tile through an
//    entry read directly, so that its loads need not wait for the copy).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_common.h"
#include "kvq_internal.h"
#include "wave_reduce.h"

namespace kvq {
namespace {

using namespace dec;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kW = 4;                      // waves per group
constexpr int kGrp = 2;                    // groups per work-group (alternate tiles)
constexpr int kThreads = 64 * kW * kGrp;
constexpr int kT = 16 * kW;                // tokens per tile: wave w owns tokens 16 w .. 16 w + 15
constexpr int kH = 16;                     // query heads (MFMA columns)
constexpr int kD = 512;                    // latent rank
constexpr int kDr = 64;                    // rope dims
constexpr int kRow = kD / 2;               // latent code bytes per token
constexpr int kSRow = kD / 16;             // latent scale bytes per token
constexpr int kPitch = kD * 2 + 32;        // staged f16 row pitch in LDS (bytes; +32 spreads banks)
constexpr int kPPitch = kT;                // P^T row pitch in LDS (floats, one row per head; 16-byte
                                           // chunk k of row c at k ^ c: conflict-free writes and reads)
constexpr float kLazy = 8.0f;              // a wave's own reference only past P = 2^8

__device__ inline f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// QNV: the latent query q_c arrives as NVFP4 codes + block scales + tensor
// scale (dequantized exactly to f16 in the prologue) instead of bf16
template <bool PAGED, bool QNV>
__global__ void __launch_bounds__(kThreads, 1) k_decode_mla(kvq_decode_args a, int num_splits) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_c_[kGrp][kT * kPitch];   // staged latent rows (f16)
  __shared__ __attribute__((aligned(16))) float lds_p_[kGrp][kH * kPPitch];    // the tile's P^T (fp32), head rows
  __shared__ __attribute__((aligned(16))) float lds_r_[kGrp][kH][kW];          // each wave's reference per head
  __shared__ int lds_bt[PAGED ? kMlaPagedMaxChunkBlocks : 1];                  // paged: the chunk's block-table entries

  const int lane = threadIdx.x & 63;
  const int w8 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = w8 >> 2;   // this wave's group: tiles grp, grp + 2, grp + 4, ...
  const int wave = w8 & 3;   // its role in the group: sub-tile, output columns
  uint8_t* const lds_c = lds_c_[grp];
  float* const lds_p = lds_p_[grp];
  float (*const lds_r)[kW] = lds_r_[grp];
  const int c = lane & 15;   // MFMA row (token) / column (head) index of this lane
  const int g = lane >> 4;   // lane group (k-slice of the MFMA operands)
  // LDS bank spreading of the staged rows: chunk k (16 bytes) of row r sits at
  // k ^ swz(r), swz(r) = bit 2 of r xor bit 3 of r, which makes both the
  // row-wise 16-byte stores and the transposed 8-byte reads conflict-free.
  const int swz_w = ((c >> 2) ^ (c >> 3)) & 1;   // rows 16 w + c (stores)
  const int swz_r = (g ^ (g >> 1)) & 1;          // rows 4 g + m/4 and 16 + 4 g + m/4 (transposed reads)
  // the two scale bytes of this lane's blocks 8 k + 2 g, + 1 out of a pair of scale dwords
  const uint32_t ssel = static_cast<uint32_t>(2 * g) | (static_cast<uint32_t>(2 * g + 1) << 8);
  // XCD-aware order: work-groups are handed to the 8 XCDs in turn, so
  // dispatch slot L goes to XCD L mod 8; slot L takes work item
  // (L mod 8) * (N / 8) + L / 8, which gives each XCD a contiguous range of
  // (request, split) items (whole requests at the bench shape).  A bijection
  // of the N items, so the results do not depend on the dispatch order
  // (B = 32, 8 splits: decode step 34.4 -> 33.6 us side by side).
  int item = blockIdx.x + gridDim.x * blockIdx.y;
  if (const int n_items = gridDim.x * gridDim.y; n_items % 8 == 0) item = (item % 8) * (n_items / 8) + item / 8;
  const int split = item % gridDim.x;
  const int b = item / gridDim.x;

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
  int64_t first_row = 0;   // paged: plane row of the group's first tile (tile grp)
  if constexpr (PAGED) {
    L = a.kv_lens[b];
    L = L < a.max_kv_len ? L : a.max_kv_len;
    L = L > 0 ? L : 0;
    ce = (cs + chunk < L) ? cs + chunk : L;
    ce_ld = ce;
    const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.bt_stride + blk0;
    const int ft = cs + grp * kT;
    if (ft < ce)
      first_row = static_cast<int64_t>(bt[(ft >> bsh) - blk0]) * a.kv_sblk + static_cast<int64_t>(ft & (bs - 1)) * st;
    const int nblk = ce > cs ? ((ce - 1) >> bsh) - blk0 + 1 : 0;
    for (int i = threadIdx.x; i < nblk; i += kThreads) lds_bt[i] = bt[i];
  }
  // plane row of tile's first token (relative to the request's base when
  // the cache is contiguous); tiles past the chunk's end get 0 (they load
  // nothing).  Paged tiles after the group's first read the LDS copy of the
  // table.
  auto tile_row = [&](int tile) -> int64_t {
    const int tb = cs + tile * kT;
    if constexpr (PAGED) {
      if (tile == grp) return first_row;
      if (tb >= ce_ld) return 0;
      return static_cast<int64_t>(lds_bt[(tb >> bsh) - blk0]) * a.kv_sblk + static_cast<int64_t>(tb & (bs - 1)) * st;
    } else {
      return static_cast<int64_t>(tb) * st;
    }
  };

  // loads of one tile for this wave's sub-tile: token 16 w + c; latent code
  // bytes [64 k + 16 g, +16) for k < 4, the token's 32 scale bytes, rope
  // bytes [64 k + 16 g, +16) for k < 2.  Tokens at or past the load bound
  // ce_ld read zeros; a tile past it reads nothing.
  struct Raw {
    u32x4 cw[4], sw[2], rw[2];
  };
  auto load_tile = [&](Raw& R, int tile) {
    const int64_t trow = tile_row(tile);
    const int nv = ce_ld - (cs + tile * kT + 16 * wave);
    const int64_t r0 = trow + static_cast<int64_t>(16 * wave) * st;
    const Rsrc rc_ = make_rsrc(cc + r0 * kRow, nv * st * kRow);
    const Rsrc rs_ = make_rsrc(csc + r0 * kSRow, nv * st * kSRow);
    const Rsrc rr_ = make_rsrc(cr + r0 * (kDr * 2), nv * st * (kDr * 2));
#pragma unroll
    for (int k = 0; k < 4; ++k) R.cw[k] = ld128(rc_, c * st * kRow + 64 * k + 16 * g);
    R.sw[0] = ld128(rs_, c * st * kSRow);
    R.sw[1] = ld128(rs_, c * st * kSRow + 16);
#pragma unroll
    for (int k = 0; k < 2; ++k) R.rw[k] = ld128(rr_, c * st * (kDr * 2) + 64 * k + 16 * g);
  };
  // scale dwords 2 k, 2 k + 1 of a 32-byte scale row -> f16 scales of blocks 8 k + 2 g, + 1
  auto block_scales = [&](const u32x4 (&sw)[2], int k) -> f16x2 {
    const u32x4 v = sw[k >> 1];
    const uint32_t lo = (k & 1) ? v[2] : v[0], hi = (k & 1) ? v[3] : v[1];
    return fp8x2<false>(__builtin_amdgcn_perm(hi, lo, ssel));
  };

  // ---- the request's query, read once per work-group with coalesced
  // 16-byte loads (thread t: chunks t, t + 512) and staged in the second
  // group's row area, which is free until its first tile: latent rows of
  // kQRow bytes per head, then rope rows of kRRow bytes (each padded by 16
  // bytes, so that the operand reads below are conflict-free).
  constexpr int kQRow = (QNV ? kD / 2 : kD * 2) + 16;   // latent query row pitch (bytes)
  constexpr int kQsOff = kH * kQRow;                     // NVFP4: the scale rows (32 bytes + 16)
  constexpr int kQrOff = kQsOff + (QNV ? kH * 48 : 0);   // the rope rows (128 bytes + 16)
  constexpr int kQLat = kH * (QNV ? kD / 32 : kD / 8);   // 16-byte chunks of the latent query
  constexpr int kQSc = QNV ? kH * 2 : 0;                 //   of its scales
  constexpr int kQChunks = kQLat + kQSc + kH * 8;        //   in all
  uint8_t* const lds_q = lds_c_[1];
  uint4 qstage[(kQChunks + kThreads - 1) / kThreads];
#pragma unroll
  for (int r = 0; r < (kQChunks + kThreads - 1) / kThreads; ++r) {
    const int i = static_cast<int>(threadIdx.x) + r * kThreads;
    if (i < kQLat) {
      constexpr int per = QNV ? kD / 32 : kD / 8;   // chunks per head row
      const int h = i / per, k = i % per;
      const int64_t qrow = static_cast<int64_t>(b) * a.q_sb + static_cast<int64_t>(h) * a.q_sh;
      qstage[r] = QNV ? *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.q) + qrow * (kD / 2) + 16 * k)
                      : *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qrow + 8 * k);
    } else if (i < kQLat + kQSc) {
      const int u = i - kQLat, h = u >> 1;
      const int64_t qrow = static_cast<int64_t>(b) * a.q_sb + static_cast<int64_t>(h) * a.q_sh;
      qstage[r] = *reinterpret_cast<const uint4*>(a.q_block_scales + qrow * (kD / 16) + 16 * (u & 1));
    } else if (i < kQChunks) {
      const int u = i - kQLat - kQSc, h = u >> 3;
      qstage[r] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q_rope) +
                                                  static_cast<int64_t>(b) * a.qr_sb +
                                                  static_cast<int64_t>(h) * a.qr_sh + 8 * (u & 7));
    }
  }

  // the group's first tile, requested with the query and the request length
  // (one memory round trip); one tile is in flight while one computes
  Raw buf[2];
  load_tile(buf[0], grp);
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int r = 0; r < (kQChunks + kThreads - 1) / kThreads; ++r) {
    const int i = static_cast<int>(threadIdx.x) + r * kThreads;
    int off = -1;
    if (i < kQLat) {
      constexpr int per = QNV ? kD / 32 : kD / 8;
      off = (i / per) * kQRow + 16 * (i % per);
    } else if (i < kQLat + kQSc) {
      const int u = i - kQLat;
      off = kQsOff + (u >> 1) * 48 + 16 * (u & 1);
    } else if (i < kQChunks) {
      const int u = i - kQLat - kQSc;
      off = kQrOff + (u >> 3) * 144 + 16 * (u & 7);
    }
    if (off < 0) continue;
    if (!QNV && i < kQLat) {   // bf16 pair -> fp32 (exact) -> f16 (exact in f16's normal range)
      const uint4 w = qstage[r];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      f16x2 h[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        h[k] = f16x2{static_cast<_Float16>(__uint_as_float(ws[k] << 16)),
                     static_cast<_Float16>(__uint_as_float(ws[k] & 0xFFFF0000u))};
      *reinterpret_cast<f16x8*>(lds_q + off) = cat4(h[0], h[1], h[2], h[3]);
    } else {
      *reinterpret_cast<uint4*>(lds_q + off) = qstage[r];
    }
  }

  __syncthreads();   // the staged query (and, paged, the LDS table copy) are visible


  if constexpr (!PAGED) {
    L = a.kv_lens[b];
    L = L < a.max_kv_len ? L : a.max_kv_len;
    L = L > 0 ? L : 0;
    ce = (cs + chunk < L) ? cs + chunk : L;
    ce_ld = ce;   // later loads stop at the request's end
  }
  const int ntiles = cs < ce ? (ce - cs + kT - 1) / kT : 0;
  // both groups run the same number of steps (their barriers are the
  // work-group's): with an odd tile count the second group's last step is
  // a tile past the chunk, which loads nothing and has every token masked
  const int nsteps = (ntiles + 1) / 2;

  const float s_t = *a.k_scale;
  // latent scores carry the tensor scale of the latent (and of an NVFP4 query)
  const float sc_lat = a.softmax_scale * s_t * (QNV ? *a.q_scale : 1.0f) * kLog2e;
  const float sc_rope = a.softmax_scale * kLog2e;

  // ---- query operand, lane (g, c) = head c: latent MFMA J = 4 k + jj
  //   (0..15) takes dims 128 k + 32 g + 8 jj .. + 7 (f16: the bf16 query
  //   converted by the staging; NVFP4: code bytes [64 k + 16 g, +16) and
  //   the scales of head c's row, dequantized here, E2M1 x E4M3 exact in
  //   f16); rope MFMA k (0, 1) dims 32 k + 8 g .. + 7 (bf16)
  f16x8 qop[16];
  if constexpr (QNV) {
    u32x4 qsw[2];
    qsw[0] = *reinterpret_cast<const u32x4*>(lds_q + kQsOff + c * 48);
    qsw[1] = *reinterpret_cast<const u32x4*>(lds_q + kQsOff + c * 48 + 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4 qw = *reinterpret_cast<const u32x4*>(lds_q + c * kQRow + 64 * k + 16 * g);
      const f16x2 s2 = block_scales(qsw, k);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const _Float16 sv = jj < 2 ? s2[0] : s2[1];
        const f16x2 sp = f16x2{sv, sv};
        const uint32_t w = qw[jj];
        qop[4 * k + jj] = cat4(fp4x2<0>(w) * sp, fp4x2<1>(w) * sp, fp4x2<2>(w) * sp, fp4x2<3>(w) * sp);
      }
    }
  } else {
#pragma unroll
    for (int J = 0; J < 16; ++J)
      qop[J] = *reinterpret_cast<const f16x8*>(lds_q + c * kQRow + 256 * (J >> 2) + 64 * g + 16 * (J & 3));
  }
  const bf16x8 qr[2] = {*reinterpret_cast<const bf16x8*>(lds_q + kQrOff + c * 144 + 16 * g),
                        *reinterpret_cast<const bf16x8*>(lds_q + kQrOff + c * 144 + 64 + 16 * g)};
  __syncthreads();   // every wave holds its query operand: the staging area is free

  float m_ref = -INFINITY;   // reference maximum of head c (log2 domain), the same in every wave
  float l_run = 0.0f;        // this lane's share of head c's denominator (its tokens, against m_ref)
  f32x4 acc_o[8];            // O^T rows d = 128*wave + 16*jj + 4g + i, column head c
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc_o[jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint8_t* const stage = lds_c + (16 * wave + c) * kPitch;   // this lane's staged row (token 16 w + c)

  auto process = [&](Raw& cur, int tile) {
    const int tb = cs + tile * kT;
    // the chunk's last tile: the row of a token at or past the request's end
    // (read before the length was known) becomes zeros, so that its staged
    // latent is 0 (its probability is 0).  (The empty asm keeps this a
    // branch taken once per chunk instead of selects on every tile.)
    if (tb + kT > ce) {
      asm volatile("");
      if (tb + 16 * wave + c >= ce) {
#pragma unroll
        for (int k = 0; k < 4; ++k) cur.cw[k] = u32x4{0u, 0u, 0u, 0u};
        cur.sw[0] = cur.sw[1] = cur.rw[0] = cur.rw[1] = u32x4{0u, 0u, 0u, 0u};
      }
    }

    // ---- scores S^T[token 16 w + 4 g + i][head c] over the whole latent and
    // rope; stage the f16 rows (chunk 16 k + 4 g + jj of the row, swizzled).
    // Four latent accumulators: dependent MFMA chains of 4.
    f32x4 acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    f32x4 acc_r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f16x2 sp = block_scales(cur.sw, k);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t w = cur.cw[k][jj];
        const _Float16 sv = jj < 2 ? sp[0] : sp[1];
        const f16x2 s2 = {sv, sv};
        const f16x8 kop = cat4(fp4x2<0>(w) * s2, fp4x2<1>(w) * s2, fp4x2<2>(w) * s2, fp4x2<3>(w) * s2);
        acc[jj] = mfma(kop, qop[4 * k + jj], acc[jj]);
        *reinterpret_cast<f16x8*>(stage + 16 * ((16 * k + 4 * g + jj) ^ swz_w)) = kop;
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) acc_r = mfma_bf16(__builtin_bit_cast(bf16x8, cur.rw[k]), qr[k], acc_r);
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = ((acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i])) * sc_lat + acc_r[i] * sc_rope;
    if (tb + kT > ce) {   // the chunk's last tile (uniform branch)
      asm volatile("");
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tb + 16 * wave + 4 * g + i >= ce) sc[i] = -INFINITY;
    }

    // ---- softmax of the wave's 16 tokens against the shared reference,
    // or against the wave's own maximum when that exceeds it by more than 2^8
    float tm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    tm = lanes::across_rows<lanes::Max>(tm);   // head c's max over the four lane groups
    const float r = tm > m_ref + kLazy ? tm : m_ref;
    const float ru = r == -INFINITY ? 0.0f : r;
    f32x4 p;
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - ru);   // masked: exp2(-inf) = 0
    const float l_tile = (p[0] + p[1]) + (p[2] + p[3]);
    *reinterpret_cast<f32x4*>(lds_p + c * kPPitch + 4 * ((4 * wave + g) ^ c)) = p;
    if (g == 0) lds_r[c][wave] = r;
    __syncthreads();   // staged rows, P and the references visible

    // ---- the tile's reference: the largest any wave used (>= m_ref)
    const f32x4 rr = *reinterpret_cast<const f32x4*>(&lds_r[c][0]);
    const float R = fmaxf(fmaxf(rr[0], rr[1]), fmaxf(rr[2], rr[3]));
    if (__any(R > m_ref)) {   // the same decision for column c in every wave
      const float fac = R > m_ref ? __builtin_amdgcn_exp2f(m_ref - R) : 1.0f;   // 0 when m_ref = -inf
      l_run *= fac;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_o[jj][i] *= fac;
      m_ref = fmaxf(m_ref, R);
    }
    l_run += r == R ? l_tile : l_tile * __builtin_amdgcn_exp2f(r - R);

    // ---- B operand of P.V step ks (k = 8 g + e): e < 4 -> token 32 ks + 4 g
    // + e (wave 2 ks), e >= 4 -> token 32 ks + 16 + 4 g + e - 4 (wave 2 ks + 1);
    // a wave that used a smaller reference has its P scaled down to R first
    const bool fix = __any(rr[0] != R || rr[1] != R || rr[2] != R || rr[3] != R);
    f16x8 pb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f32x4 p0 = *reinterpret_cast<const f32x4*>(lds_p + c * kPPitch + 4 * ((8 * ks + g) ^ c));
      f32x4 p1 = *reinterpret_cast<const f32x4*>(lds_p + c * kPPitch + 4 * ((8 * ks + 4 + g) ^ c));
      if (fix) {
        const float r0 = rr[2 * ks], r1 = rr[2 * ks + 1];
        const float f0 = r0 == R ? 1.0f : __builtin_amdgcn_exp2f(r0 - R);
        const float f1 = r1 == R ? 1.0f : __builtin_amdgcn_exp2f(r1 - R);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p0[i] *= f0;
          p1[i] *= f1;
        }
      }
      pb[ks] = f16x8{static_cast<_Float16>(p0[0]), static_cast<_Float16>(p0[1]), static_cast<_Float16>(p0[2]),
                     static_cast<_Float16>(p0[3]), static_cast<_Float16>(p1[0]), static_cast<_Float16>(p1[1]),
                     static_cast<_Float16>(p1[2]), static_cast<_Float16>(p1[3])};
    }

    // ---- P.V for this wave's 128 output columns over the tile's tokens,
    // 32 per step.  A = latent^T rows d, k = the tokens above: two
    // transposed reads of 4 token rows; lane m of the 16-lane group points
    // at row r + m/4, columns d0 + 4(m%4) .. +3, and receives column d0 + m
    // of the 4 rows.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
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

  // the loop is unrolled over the two buffers so that each has fixed
  // registers; step n processes tile 2 n + grp.  The second group starts
  // one barrier later and the first ends with one more, so the groups run
  // half a tile apart: while one dequantizes and scores, the other runs
  // P.V (the two waves of a SIMD are one of each), and their loads go out
  // in alternate halves.  Each group's LDS is its own, and between any two
  // of its halves lies one work-group barrier.  The two extra barriers sit
  // in branches that are uniform per wave (grp is the wave's), so this is
  // the hardware's barrier rather than the HIP model's: s_barrier releases
  // once every wave of the work-group has reached an s_barrier, whichever
  // instruction it is, and every wave reaches 2 nsteps + 1 of them (then
  // the epilogue's), so the k-th barrier of one group pairs with the k-th
  // of the other.  The GPU tests check this path bit for bit across the
  // paged and contiguous forms and against the oracle.
  if (grp == 1) __syncthreads();
  for (int n = 0; n < nsteps; n += 2) {
    load_tile(buf[1], 2 * (n + 1) + grp);
    __builtin_amdgcn_sched_barrier(0);
    process(buf[0], 2 * n + grp);
    if (n + 1 >= nsteps) break;
    load_tile(buf[0], 2 * (n + 2) + grp);
    __builtin_amdgcn_sched_barrier(0);
    process(buf[1], 2 * (n + 1) + grp);
  }
  if (grp == 0) __syncthreads();

  // ---- each group's denominator: l summed over the lanes of its waves
  // (each holds its own tokens' share)
  const float lw = lanes::across_rows<lanes::Sum>(l_run);
  if (g == 0) lds_r[c][wave] = lw;
  __syncthreads();
  const f32x4 lv = *reinterpret_cast<const f32x4*>(&lds_r[c][0]);
  float lt = (lv[0] + lv[1]) + (lv[2] + lv[3]);
  __syncthreads();   // (the LDS below is reused)
  // ---- the second group hands its state to the first: accumulators (the
  // same lane layout), reference maximum and denominator per head
  // (accumulator jj of every lane of the group contiguous: conflict-free)
  f32x4* const xacc = reinterpret_cast<f32x4*>(lds_c_[0]) + wave * 64 + lane;
  if (grp == 1) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) xacc[jj * kW * 64] = acc_o[jj];
    if (wave == 0 && g == 0) {
      lds_r_[1][c][0] = m_ref;
      lds_r_[1][c][1] = lt;
    }
  }
  __syncthreads();
  if (grp == 1) return;
  {
    const float m1 = lds_r_[1][c][0], l1 = lds_r_[1][c][1];
    const float M = fmaxf(m_ref, m1);
    const float f0 = m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_ref - M);
    const float f1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - M);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const f32x4 x = xacc[jj * kW * 64];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_o[jj][i] = acc_o[jj][i] * f0 + x[i] * f1;
    }
    lt = lt * f0 + l1 * f1;
    m_ref = M;
  }

  // ---- partials: o = acc * s_t / l, lse = (m + log2 l) ln 2 (non-temporal
  // stores: the partials are read once, by the merge; the end-of-kernel
  // burst of 8.4 MB at B = 32 measured 0.9 us shorter than with cached stores)
  const float f = lt > 0.0f ? s_t / lt : 0.0f;
  const int64_t po = (static_cast<int64_t>(b) * a.Hq + c) * num_splits + split;
  float* op = a.part_o + po * kD + 128 * wave + 4 * g;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const f32x4 ov = {acc_o[jj][0] * f, acc_o[jj][1] * f, acc_o[jj][2] * f, acc_o[jj][3] * f};
    __builtin_nontemporal_store(ov, reinterpret_cast<f32x4*>(op + 16 * jj));
  }
  if (wave == 0 && g == 0) a.part_lse[po] = lt > 0.0f ? (m_ref + log2f(lt)) * kLn2 : -INFINITY;
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
