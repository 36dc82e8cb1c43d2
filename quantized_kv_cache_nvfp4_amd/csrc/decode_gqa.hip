// Split-KV flash decode over an NVFP4 or FP8 E4M3 KV cache, GQA / MHA layout,
// for gfx950 (wave64, MFMA 16x16x32 f16).
//
// Method: Model-Optimizer PR #1832 "Add quant+sparse attention for vLLM
// serving", Testing section: the KV sequence of one (request, head) is cut
// into s contiguous chunks; each program keeps a running max and denominator
// of the softmax over its chunk and accumulates the probability-weighted V,
// and a combine step merges the s partials.  Cache formats: Model-Optimizer
// PR #714 Testing section (NVFP4: E2M1 codes, E4M3 scale per 16 elements
// along head_dim, per-tensor fp32 scale) and compressed-tensors PR #436
// kv_cache_scheme (per-tensor FP8 E4M3).
//
// Design for CDNA4 (not a translation of the pages' Triton kernel):
//  * one work-group = 4 waves = one chunk of one (request, kv head); the
//    waves take interleaved tiles of the chunk and are merged through LDS.
//  * dequantization happens in registers: E2M1 -> f16 with the hardware
//    convert (exact), times the E4M3 block scale (an exact f16 product:
//    at most 5 significant bits, inside f16's normal range); the per-tensor
//    scale is applied in fp32 after the contraction.
//  * Q.K^T and P.V run on MFMA 16x16x32 f16.  The query group is narrow
//    (G = Hq/Hkv query heads share a kv head), so the 16 MFMA columns are
//    filled with (sub-tile, head) pairs: sub-tile u of 16 tokens only
//    meets the Q columns of its own row group (block-diagonal B operand), so
//    one 16x16 score tile holds 16*16/G tokens x G heads with no padding.
//    Each of the 16 rows keeps its own online-softmax state; rows of the same
//    head are merged at the end of the chunk.
//  * Q.K^T contracts over head_dim, and the order of that contraction is
//    free: lane group g owns a contiguous quarter of head_dim, so each lane
//    reads its K codes with one 128-bit load per token.  P.V contracts over
//    tokens, and V is stored token-major, so each lane loads a short run of
//    head_dim for 4 tokens and transposes 2x2 blocks of f16 in registers
//    (v_perm_b32) into the token-contiguous MFMA operand; the output
//    columns are permuted the same way and un-permuted on the final store.
//  * fp32 queries are split into f16 hi + lo parts and, when asked, P is
//    split the same way (two MFMAs each) for the fp32-accuracy path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "combine_impl.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ inline f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// E2M1 pair (byte SEL of w) -> f16x2, exact (scale argument 1.0)
template <int SEL>
__device__ inline f16x2 fp4x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}
// E4M3 pair (16-bit half HI of w) -> f16x2, exact
template <bool HI>
__device__ inline f16x2 fp8x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// fp4x2 with a byte select that is a constant after unrolling
__device__ inline f16x2 fp4x2_sel(uint32_t w, int sel) {
  switch (sel) {
    case 0: return fp4x2<0>(w);
    case 1: return fp4x2<1>(w);
    case 2: return fp4x2<2>(w);
    default: return fp4x2<3>(w);
  }
}

__device__ inline f16x8 cat4(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  f16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ inline f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ loads
// Raw buffer loads: base and size live in a (uniform) buffer resource, the
// lane supplies a byte offset; offsets at or past the size read as zero.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcFlags = 0x00020000;   // gfx9 raw buffer: 32-bit data format, no swizzle

__device__ inline Rsrc make_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes > 0 ? bytes : 0, kRsrcFlags);
}
__device__ inline u32x4 ld128(Rsrc r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline u32x2 ld64(Rsrc r, int off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ inline uint32_t ld32(Rsrc r, int off) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline uint32_t ld16(Rsrc r, int off) {
  return static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}
__device__ inline uint32_t ld8(Rsrc r, int off) {
  return static_cast<uint8_t>(__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0));
}

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
// QF32 fp32 queries (hi/lo split), PSPLIT 2 = P carried as f16 hi + lo,
// FUSED: the last work-group of each (request, kv head) merges the partials
// and writes the final output (one launch per decode step).
template <int KVF, int G, int D, bool QF32, int PSPLIT, bool FUSED, int VL>
__global__ void __launch_bounds__(kThreads, 2) k_decode_gqa(kvq_decode_args a, int num_splits, FusedOut fo) {
  using Gm = Geo<KVF, D>;
  constexpr int NSUB = 16 / G;                  // row groups in the 16 MFMA columns
  constexpr int NT = NSUB < 2 ? 2 : NSUB;       // sub-tiles (16 tokens) per tile
  constexpr int NACC = NT / NSUB;               // score accumulators per tile
  constexpr int TT = 16 * NT;                   // tokens per tile
  constexpr int NQ = QF32 ? 2 : 1;
  using KT = KTile<KVF, D, NT>;
  using VT = VTile<KVF, D, NT>;

  __shared__ float lds_o[kWaves][16][D];
  __shared__ float lds_m[kWaves][16];
  __shared__ float lds_l[kWaves][16];
  __shared__ int lds_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int c = lane & 15;   // MFMA column / row-within-16 of this lane
  const int g = lane >> 4;   // lane group (k-slice of the MFMA operands)
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;

  int L = a.kv_lens[b];
  L = L < a.max_kv_len ? L : a.max_kv_len;
  L = L > 0 ? L : 0;
  int chunk = (L + num_splits - 1) / num_splits;
  chunk = (chunk + TT - 1) / TT * TT;
  const int cs = split * chunk;
  const int ce = (cs + chunk < L) ? cs + chunk : L;

  const int hq0 = kvh * G;
  const int my_h = c % G;
  const int my_sub = c / G;

  const float kscale = *a.k_scale;
  const float vscale = *a.v_scale;
  const float qk_scale = a.softmax_scale * kscale * kLog2e;

  float m_run = -INFINITY;  // running max of row c (log2 domain)
  float l_run = 0.0f;       // this lane's share of row c's denominator
  f32x4 acc_o[Gm::kPvJ];
#pragma unroll
  for (int j = 0; j < Gm::kPvJ; ++j) acc_o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = cs < ce ? (ce - cs + TT - 1) / TT : 0;

  if (wave < ntiles) {
    // ---- query operand: lane (g, c) holds Q[h = c % G][g*QKE + 8j + e]
    f16x8 qop[NQ][Gm::kQkJ];
    {
      const int64_t qb = static_cast<int64_t>(b) * a.q_sb + static_cast<int64_t>(hq0 + my_h) * a.q_sh;
#pragma unroll
      for (int j = 0; j < Gm::kQkJ; ++j) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = g * Gm::kQkElems + 8 * j + e;
          float x;
          if constexpr (QF32) x = static_cast<const float*>(a.q)[qb + d];
          else x = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.q)[qb + d]) << 16);
          const _Float16 hi = static_cast<_Float16>(x);
          qop[0][j][e] = hi;
          if constexpr (QF32) qop[1][j][e] = static_cast<_Float16>(x - static_cast<float>(hi));
        }
      }
    }

    // per-(request, kv head) plane bases
    const int64_t head_row = static_cast<int64_t>(b) * a.kv_sb + static_cast<int64_t>(kvh) * a.kv_sh;
    const uint8_t* kc = a.k_codes + head_row * Gm::kRowBytes;
    const uint8_t* vc = a.v_codes + head_row * Gm::kRowBytes;
    const uint8_t* ksc = (KVF == KVQ_NVFP4) ? a.k_scales + head_row * Gm::kScaleBytes : kc;
    const uint8_t* vsc = (KVF == KVQ_NVFP4) ? a.v_scales + head_row * Gm::kScaleBytes : vc;
    // token stride in rows (always 1 with a TOKEN4 V plane, K and V share it)
    const int st = (VL == KVQ_PLANE_TOKEN4) ? 1 : static_cast<int>(a.kv_st);
    constexpr int RB = Gm::kRowBytes;
    constexpr int SB = Gm::kScaleBytes;

    // Every load goes through a buffer resource whose base is the tile's
    // first token and whose size ends at the chunk end ce: lanes whose token
    // is at or past ce read zeros (hardware range check, nothing is
    // fetched), and the prefetch past a wave's last tile touches no memory.
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

    auto load_ktile = [&](KT& R, int tile) {
      const int tb = cs + tile * TT;
      const int nv = ce - tb;
      const int64_t base = static_cast<int64_t>(tb) * st;
      const Rsrc rk = make_rsrc(kc + base * RB, nv * st * RB);
      const Rsrc rks = make_rsrc(ksc + base * SB, nv * st * SB);
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int o = lk + u * 16 * st * RB;
        if constexpr (Gm::kKWords == 8) {
          const u32x4 x0 = ld128(rk, o), x1 = ld128(rk, o + 16);
#pragma unroll
          for (int w = 0; w < 4; ++w) { R.k[u][w] = x0[w]; R.k[u][4 + w] = x1[w]; }
        } else if constexpr (Gm::kKWords == 4) {
          const u32x4 x0 = ld128(rk, o);
#pragma unroll
          for (int w = 0; w < 4; ++w) R.k[u][w] = x0[w];
        } else {
          const u32x2 x0 = ld64(rk, o);
          R.k[u][0] = x0[0]; R.k[u][1] = x0[1];
        }
        if constexpr (KVF == KVQ_NVFP4) {
          const int os = lks + u * 16 * st * SB;
          R.ks[u] = (D == 128) ? ld16(rks, os) : ld8(rks, os);
        }
      }
    };
    auto load_vtile = [&](VT& R, int tile) {
      const int tb = cs + tile * TT;
      const int nv = ce - tb;
      if constexpr (VL == KVQ_PLANE_TOKEN4) {
        // Group 4u+g of the tile (lane group g): for this lane's elements
        // [8c, 8c+8) the 4 tokens' codes are one contiguous run (16 bytes
        // NVFP4, 32 bytes FP8) and block c/2's 4 scale bytes one dword.  A
        // group that straddles ce is read whole; pv_tile clears its tokens
        // past ce.
        const int ng = nv > 0 ? (nv + 3) / 4 : 0;
        const Rsrc rv = make_rsrc(vc + static_cast<int64_t>(tb) * RB, ng * GB);
        const Rsrc rvs = make_rsrc(vsc + static_cast<int64_t>(tb) * SB, ng * GS);
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          const int o = lvt + u * 4 * GB;
          const u32x4 x0 = ld128(rv, o);
#pragma unroll
          for (int w = 0; w < 4; ++w) R.t4[u][w] = x0[w];
          if constexpr (CB == 32) {
            const u32x4 x1 = ld128(rv, o + 16);
#pragma unroll
            for (int w = 0; w < 4; ++w) R.t4[u][4 + w] = x1[w];
          }
          if constexpr (KVF == KVQ_NVFP4) R.vs[u][0] = ld32(rvs, lvts + u * 4 * GS);
        }
      } else {
        const int64_t base = static_cast<int64_t>(tb) * st;
        const Rsrc rv = make_rsrc(vc + base * RB, nv * st * RB);
        const Rsrc rvs = make_rsrc(vsc + base * SB, nv * st * SB);
#pragma unroll
        for (int u = 0; u < NT; ++u) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int o = lv + (16 * u + i) * st * RB;
            if constexpr (Gm::kVBytes == 8) {
              const u32x2 x = ld64(rv, o);
              R.v[u][i][0] = x[0]; R.v[u][i][1] = x[1];
            } else if constexpr (Gm::kVBytes == 4) {
              R.v[u][i][0] = ld32(rv, o);
            } else {
              R.v[u][i][0] = ld16(rv, o);
            }
            if constexpr (KVF == KVQ_NVFP4) R.vs[u][i] = ld8(rvs, lvs + (16 * u + i) * st * SB);
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

    auto qk_tile = [&](const KT& R, int tile, f16x2 (&p_hi)[NACC][2], f16x2 (&p_lo)[NACC][2]) {
      const int tb = cs + tile * TT;
      // ---------------- scores.  Every sub-tile u is multiplied by the full
      // (unmasked) query operand into its own accumulator; lane column c
      // then keeps the sub-tile of its row group (u % NSUB == c / G): the
      // block-diagonal selection costs one select per score instead of a
      // masked operand per MFMA.
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
      f32x4 acc_s[NACC];
#pragma unroll
      for (int x = 0; x < NACC; ++x) {
        acc_s[x] = acc_u[x * NSUB];
#pragma unroll
        for (int r = 1; r < NSUB; ++r) {
          const bool pick = (my_sub == r);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc_s[x][i] = pick ? acc_u[x * NSUB + r][i] : acc_s[x][i];
        }
      }
      // ---------------- online softmax per row c (this lane: 4*NACC tokens)
      const bool full_tile = (tb + TT <= ce);
      float sc[NACC][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int x = 0; x < NACC; ++x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tb + 16 * (x * NSUB + my_sub) + 4 * g + i;
          const float v = (full_tile || t < ce) ? acc_s[x][i] * qk_scale : -INFINITY;
          sc[x][i] = v;
          tmax = fmaxf(tmax, v);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      if (__any(m_new > m_run)) {
        const float fac = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
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
#pragma unroll
      for (int x = 0; x < NACC; ++x) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = (sc[x][i] == -INFINITY) ? 0.0f : exp2f(sc[x][i] - m_run);
          l_run += p[i];
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const _Float16 h0 = static_cast<_Float16>(p[2 * k]);
          const _Float16 h1 = static_cast<_Float16>(p[2 * k + 1]);
          p_hi[x][k] = f16x2{h0, h1};
          if constexpr (PSPLIT == 2)
            p_lo[x][k] = f16x2{static_cast<_Float16>(p[2 * k] - static_cast<float>(h0)),
                               static_cast<_Float16>(p[2 * k + 1] - static_cast<float>(h1))};
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
    f16x2 p_hi[NACC][2], p_lo[NACC][2];
    if constexpr (NT <= 4) {
      // loads past the wave's last tile are empty (size-0 resources)
      KT KA, KB;
      VT VA, VB;
      // (scheduling barriers keep each prefetch ahead of the compute that
      // follows it, so a full tile of work hides every load)
      int tile = wave;
      load_ktile(KA, tile);
      load_vtile(VA, tile);
      while (true) {
        load_ktile(KB, tile + kWaves);
        __builtin_amdgcn_sched_barrier(0);
        qk_tile(KA, tile, p_hi, p_lo);
        load_vtile(VB, tile + kWaves);
        __builtin_amdgcn_sched_barrier(0);
        mask_vtile(VA, tile);
        pv_tile(VA, p_hi, p_lo);
        tile += kWaves;
        if (tile >= ntiles) break;
        load_ktile(KA, tile + kWaves);
        __builtin_amdgcn_sched_barrier(0);
        qk_tile(KB, tile, p_hi, p_lo);
        load_vtile(VA, tile + kWaves);
        __builtin_amdgcn_sched_barrier(0);
        mask_vtile(VB, tile);
        pv_tile(VB, p_hi, p_lo);
        tile += kWaves;
        if (tile >= ntiles) break;
      }
    } else {
      KT KA;
      VT VA;
      for (int tile = wave; tile < ntiles; tile += kWaves) {
        load_ktile(KA, tile);
        load_vtile(VA, tile);
        qk_tile(KA, tile, p_hi, p_lo);
        mask_vtile(VA, tile);
        pv_tile(VA, p_hi, p_lo);
      }
    }
  }

  // ---------------- per-wave state -> LDS
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (g == 0) {
    lds_m[wave][c] = m_run;
    lds_l[wave][c] = l_tot;
  }
#pragma unroll
  for (int j = 0; j < Gm::kPvJ; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_o[wave][4 * g + i][c * Gm::kPvElems + j] = acc_o[j][i];
  }
  __syncthreads();

  // ---------------- merge rows (wave, sub) of each head
  const bool direct = FUSED && num_splits == 1;   // no partials needed
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int s = 0; s < NSUB; ++s) M = fmaxf(M, lds_m[w][s * G + h]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          const float mv = lds_m[w][s * G + h];
          const float f = (mv == -INFINITY) ? 0.0f : exp2f(mv - M);
          num += f * lds_o[w][s * G + h][d];
          den += f * lds_l[w][s * G + h];
        }
    }
    const float o = den > 0.0f ? (num / den) * vscale : 0.0f;
    const float lse = den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
    const int64_t bh = static_cast<int64_t>(b) * a.Hq + hq0 + h;
    if (direct) {
      store_out(fo.out, fo.out_dtype, bh * D + d, o, fo.out_dtype == KVQ_FP8E4M3 ? *fo.out_scale : 1.0f);
      if (d == 0 && fo.lse_out != nullptr) fo.lse_out[bh] = lse;
    } else {
      const int64_t po = bh * num_splits + split;
      a.part_o[po * D + d] = o;
      if (d == 0) a.part_lse[po] = lse;
    }
  }
  if constexpr (!FUSED) return;
  if (direct) return;

  // ---------------- fused combine: the last work-group of (b, kv head) to
  // finish merges the num_splits partials of its G heads
  __threadfence();   // partials visible device-wide before the count
  __syncthreads();
  if (threadIdx.x == 0) {
    int* ctr = fo.counters + static_cast<int64_t>(b) * a.Hkv + kvh;
    const int prev = atomicAdd(ctr, 1);
    const int last = (prev == num_splits - 1);
    if (last) *ctr = 0;   // reset for the next call
    lds_last = last;
  }
  __syncthreads();
  if (!lds_last) return;
  __threadfence();   // acquire: see every other work-group's partials
  const float osc = (fo.out_dtype == KVQ_FP8E4M3) ? *fo.out_scale : 1.0f;
  // lds_o is free now: stage the split weights there
  float* w_s = &lds_o[0][0][0];            // [G][num_splits] weights
  float* inv_s = &lds_o[1][0][0];          // [G] 1/sum, [G] merged lse
  for (int idx = threadIdx.x; idx < G; idx += kThreads) {
    const int64_t bh = static_cast<int64_t>(b) * a.Hq + hq0 + idx;
    split_weights(a.part_lse + bh * num_splits, num_splits, w_s + idx * num_splits, inv_s[idx], inv_s[G + idx]);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    const int64_t bh = static_cast<int64_t>(b) * a.Hq + hq0 + h;
    const float o = combine_column(a.part_o + bh * num_splits * D + d, D, w_s + h * num_splits, num_splits, inv_s[h]);
    store_out(fo.out, fo.out_dtype, bh * D + d, o, osc);
    if (d == 0 && fo.lse_out != nullptr) fo.lse_out[bh] = inv_s[G + h];
  }
}

template <int KVF, int G, int D, bool QF32, int PSPLIT, int VL>
hipError_t launch_v(const kvq_decode_args& a, const DecodePlan& p, const FusedOut* fo, hipStream_t st) {
  dim3 grid(p.s, a.Hkv, a.B);
  if (fo != nullptr)
    hipLaunchKernelGGL((k_decode_gqa<KVF, G, D, QF32, PSPLIT, true, VL>), grid, dim3(kThreads), 0, st, a, p.s, *fo);
  else
    hipLaunchKernelGGL((k_decode_gqa<KVF, G, D, QF32, PSPLIT, false, VL>), grid, dim3(kThreads), 0, st, a, p.s,
                       FusedOut{});
  return hipGetLastError();
}

template <int KVF, int G, int D, bool QF32, int PSPLIT>
hipError_t launch_t(const kvq_decode_args& a, const DecodePlan& p, const FusedOut* fo, hipStream_t st) {
  if constexpr (D == 128) {
    if (a.v_layout == KVQ_PLANE_TOKEN4) return launch_v<KVF, G, D, QF32, PSPLIT, KVQ_PLANE_TOKEN4>(a, p, fo, st);
  }
  return launch_v<KVF, G, D, QF32, PSPLIT, KVQ_PLANE_ROWS>(a, p, fo, st);
}

template <int KVF, int G, int D>
hipError_t launch_q(const kvq_decode_args& a, const DecodePlan& p, const FusedOut* fo, hipStream_t st) {
  // fp32 queries select the fp32-accuracy path (hi/lo split of Q and P)
  if (a.q_dtype == KVQ_F32) return launch_t<KVF, G, D, true, 2>(a, p, fo, st);
  return launch_t<KVF, G, D, false, 1>(a, p, fo, st);
}

template <int KVF, int D>
hipError_t launch_g(const kvq_decode_args& a, const DecodePlan& p, const FusedOut* fo, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_q<KVF, 1, D>(a, p, fo, st);
    case 2: return launch_q<KVF, 2, D>(a, p, fo, st);
    case 4: return launch_q<KVF, 4, D>(a, p, fo, st);
    case 8: return launch_q<KVF, 8, D>(a, p, fo, st);
    case 16: return launch_q<KVF, 16, D>(a, p, fo, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t dispatch(const kvq_decode_args& a, const DecodePlan& p, const FusedOut* fo, hipStream_t st) {
  if (a.kv_format == KVQ_NVFP4)
    return a.D == 128 ? launch_g<KVQ_NVFP4, 128>(a, p, fo, st) : launch_g<KVQ_NVFP4, 64>(a, p, fo, st);
  return a.D == 128 ? launch_g<KVQ_FP8E4M3, 128>(a, p, fo, st) : launch_g<KVQ_FP8E4M3, 64>(a, p, fo, st);
}

}  // namespace

int gqa_tile_tokens(int G) {
  const int nsub = 16 / G;
  return 16 * (nsub < 2 ? 2 : nsub);
}

bool gqa_supported(int kv_format, int G, int D, int q_dtype) {
  if (kv_format != KVQ_NVFP4 && kv_format != KVQ_FP8E4M3) return false;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return false;
  if (D != 64 && D != 128) return false;
  return q_dtype == KVQ_BF16 || q_dtype == KVQ_F32;
}

hipError_t launch_decode_gqa(const kvq_decode_args& a, const DecodePlan& p, hipStream_t st) {
  return dispatch(a, p, nullptr, st);
}

hipError_t launch_decode_gqa_fused(const kvq_decode_args& a, const DecodePlan& p, void* out, int out_dtype,
                                   const float* out_scale, float* lse_out, int* counters, hipStream_t st) {
  FusedOut fo{out, out_dtype, out_scale, lse_out, counters};
  return dispatch(a, p, &fo, st);
}

}  // namespace kvq
