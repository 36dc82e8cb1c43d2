// Max calibration, NVFP4 / FP8 E4M3 packing and unpacking for gfx950.
//
// Formats: Model-Optimizer PR #714 "KV cache quantization for MLAAttention in
// vLLM fakequant", Testing section (E2M1 elements in blocks of 16 along the
// last dim, dynamic E4M3 block scale, per-tensor amax from a max
// calibrator); compressed-tensors PR #436 kv_cache_scheme (per-tensor
// symmetric static FP8 E4M3 from a min-max observer).
//
// Every rounding decision is the exact real-number decision.  The inputs have
// at most 24 significant bits and every decision threshold (an E2M1 midpoint
// times s_hat * s_t, or an E4M3 midpoint times 6 * s_t or times the FP8
// scale) at most 32, so two that differ do so by at least 2^-32 relative;
// a correctly rounded float64 quotient (error 2^-53) therefore lands on the
// same side of every threshold as the real quotient, and exactly on it when
// the real quotient is a tie.  Rounding is then done by power-of-two scaling
// and rint (round half to even) on that float64 quotient.  A float32
// quotient would not be exact here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"
#include "pack_codec.h"
#include "wave_reduce.h"

namespace kvq {
namespace {

using namespace codec;

constexpr int kThreads = 256;

// unravel a flat row index into the (i0, i1, i2) of `r`
__device__ inline void unravel(int64_t row, const Rows& r, int64_t& i0, int64_t& i1, int64_t& i2) {
  i2 = row % r.n2;
  int64_t t = row / r.n2;
  i1 = t % r.n1;
  i0 = t / r.n1;
}

__device__ inline int64_t row_off(const Rows& r, int64_t i0, int64_t i1, int64_t i2) {
  return i0 * r.s0 + i1 * r.s1 + i2 * r.s2;
}

// TOKEN4 plane layout: four consecutive tokens (4q .. 4q+3) share the 4R
// bytes that start at the group's first row; inside, elements are stored in
// order and, for each element, the codes of the four tokens in token order:
// NVFP4 element x of token j is nibble (j & 1) of byte 2x + (j >> 1), FP8
// element x of token j is byte 4x + j, NVFP4 block b's scale of token j is
// byte 4b + j.  (Requires token stride 1 and 4-aligned groups.)
__device__ inline int64_t group_row(const Rows& r, int64_t i0, int64_t i1, int64_t t0) {
  return i0 * r.s0 + i1 * r.s1 + t0;  // row index of the group's first token
}


// ---------------------------------------------------------------- loads
// 16-byte load with the non-temporal hint, for the calibration's single
// pass over a tensor (28.4 -> 27.2 us over 134 MB of bf16; the packs
// measured 15-20 % slower with it and keep plain loads)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline uint4 load_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// n (<= N) consecutive elements starting at element offset off of x, as
// fp32 (0 past n); 16-byte vector loads when the run is whole and aligned.
template <int N>
__device__ inline void load_run(const void* x, int dt, int64_t off, int n, float (&v)[N]) {
  if (dt == KVQ_F32) {
    const float* p = static_cast<const float*>(x) + off;
    if (n == N && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
#pragma unroll
      for (int q = 0; q < N / 4; ++q) {
        const float4 w = reinterpret_cast<const float4*>(p)[q];
        v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = i < n ? p[i] : 0.0f;
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(x) + off;
    if (N % 8 == 0 && n == N && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
#pragma unroll
      for (int q = 0; q < N / 8; ++q) {
        const uint4 w = reinterpret_cast<const uint4*>(p)[q];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {   // bf16 pair -> two fp32 (exact)
          v[8 * q + 2 * k] = __uint_as_float(ws[k] << 16);
          v[8 * q + 2 * k + 1] = __uint_as_float(ws[k] & 0xFFFF0000u);
        }
      }
      return;
    }
    if (N == 4 && n == 4 && (reinterpret_cast<uintptr_t>(p) & 7u) == 0) {
      const uint2 w = *reinterpret_cast<const uint2*>(p);
      v[0] = __uint_as_float(w.x << 16);
      v[1] = __uint_as_float(w.x & 0xFFFF0000u);
      v[2] = __uint_as_float(w.y << 16);
      v[3] = __uint_as_float(w.y & 0xFFFF0000u);
      return;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = i < n ? __uint_as_float(static_cast<uint32_t>(p[i]) << 16) : 0.0f;
  }
}

// Work layout of the row kernels: blockIdx.y walks the (i0, i1) heads of a
// Rows set, blockIdx.x with the threads the items (row, run) of one head, so
// no per-item 64-bit index arithmetic on the flat row index is needed.
__device__ inline int64_t head_items_stride() { return static_cast<int64_t>(gridDim.x) * kThreads; }
__device__ inline int64_t head_items_start() { return blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; }

// ---------------------------------------------------------------- amax
__global__ void k_zero_n(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0.0f;
}

// max |x| over the rows (tokens at or past kv_lens[i0] excluded); runs of 8
// elements per item, a wave and then a work-group reduction, one atomic per
// work-group (non-negative floats order as their bit patterns, so an
// unsigned max on the bits is a float max).  The grid is kept to about four
// work-groups per compute unit: atomics on one address serialize.
// Work-group max of m, merged into *dst with one atomic (non-negative
// floats order as their bit patterns).  Called by the whole work-group.
__device__ inline void wg_max_atomic(float m, float* dst) {
  __shared__ float wmax[kThreads / 64];
  m = lanes::wave_all<lanes::Max>(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = wmax[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) b = fmaxf(b, wmax[w]);
    atomicMax(reinterpret_cast<unsigned int*>(dst), __float_as_uint(b));
  }
  __syncthreads();   // wmax may be reused
}

// per_head: out[i1] receives the max over the rows of head i1 (one atomic
// per work-group and head), else out[0] the max over everything
__global__ void __launch_bounds__(kThreads) k_amax(const void* __restrict__ x, int dt, Rows r, int d,
                                                   const int32_t* __restrict__ kv_lens, float* __restrict__ out,
                                                   int per_head) {
  const uint32_t nrun = static_cast<uint32_t>((d + 7) / 8);
  float m = 0.0f;
  const int64_t nh = r.n0 * r.n1;
  for (int64_t h = blockIdx.y; h < nh; h += gridDim.y) {
    const int64_t i0 = h / r.n1, i1 = h - i0 * r.n1;
    if (per_head) m = 0.0f;
    int64_t n2 = r.n2;
    if (kv_lens != nullptr) {
      const int64_t len = kv_lens[i0];
      n2 = len < n2 ? (len > 0 ? len : 0) : n2;
    }
    const int64_t items = n2 * nrun;
    const int64_t base = i0 * r.s0 + i1 * r.s1;
    const size_t esz = (dt == KVQ_F32) ? 4 : 2;
    if (r.s2 == d && d % 8 == 0 && (reinterpret_cast<uintptr_t>(static_cast<const uint8_t*>(x) + base * esz) & 15u) == 0) {
      // contiguous rows: the head is one flat run of n2 * d elements, read
      // as 16-byte vectors with no per-load branches, eight loads in flight
      // per thread (the grid is kept small so that the per-work-group
      // atomics stay few)
      constexpr int U = 8;
      const int64_t stride = head_items_stride();
      const int64_t start = head_items_start();
      if (dt == KVQ_F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + base);
        int64_t it = start;
        for (; it + (U - 1) * stride < items; it += U * stride) {
          float4 w[U][2];
#pragma unroll
          for (int u = 0; u < U; ++u) { w[u][0] = p[2 * (it + u * stride)]; w[u][1] = p[2 * (it + u * stride) + 1]; }
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < 2; ++k)
              m = fmaxf(m, fmaxf(fmaxf(fabsf(w[u][k].x), fabsf(w[u][k].y)), fmaxf(fabsf(w[u][k].z), fabsf(w[u][k].w))));
        }
        for (; it < items; it += stride) {
          const float4 a = p[2 * it], b2 = p[2 * it + 1];
          m = fmaxf(m, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
          m = fmaxf(m, fmaxf(fmaxf(fabsf(b2.x), fabsf(b2.y)), fmaxf(fabsf(b2.z), fabsf(b2.w))));
        }
      } else {
        // bf16: |x| of a pair = the two halves with the sign bits cleared
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + base);
        auto fold = [&](const uint4 w) {
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int k = 0; k < 4; ++k)
            m = fmaxf(m, fmaxf(__uint_as_float((ws[k] << 16) & 0x7FFF0000u), __uint_as_float(ws[k] & 0x7FFF0000u)));
        };
        int64_t it = start;
        for (; it + (U - 1) * stride < items; it += U * stride) {
          uint4 w[U];
#pragma unroll
          for (int u = 0; u < U; ++u) w[u] = load_nt(p + it + u * stride);
#pragma unroll
          for (int u = 0; u < U; ++u) fold(w[u]);
        }
        for (; it < items; it += stride) fold(load_nt(p + it));
      }
    } else {
      for (int64_t it = head_items_start(); it < items; it += head_items_stride()) {
        const int64_t t = it / nrun;
        const int run = static_cast<int>(it - t * nrun);
        float v[8];
        load_run<8>(x, dt, base + t * r.s2 + 8 * run, d - 8 * run < 8 ? d - 8 * run : 8, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
      }
    }
    if (per_head) wg_max_atomic(m, out + i1);   // (the head loop is uniform over the work-group)
  }
  if (!per_head) wg_max_atomic(m, out);
}

// ---------------------------------------------------------------- NVFP4 pack
// The pack kernels encode whole blocks with the hardware converters and take
// encode_nvfp4_block's float64 decisions only where a converter's input lies
// near a rounding boundary, so the bytes are the same as that routine's.
//  * Block scale: the E4M3 code of the real quotient bamax / (6 s_t) is the
//    hardware conversion (round to nearest even) of the float32 quotient
//    bamax * inv6 (inv6 = 1 / (6 s_t) in float32: relative error below
//    2^-22 for the product) unless that lies within 2^-20 (relative) of one
//    of the two midpoints around the candidate; then e4m3_rne_code decides.
//  * Elements: with D = value(scale code) * s_t, the float32 products
//    x * ih and x * il, ih and il = rcp(D) (1 +- 2^-19), lie on either side
//    of the real x / D (their errors are below 2^-21), strictly; the
//    hardware E2M1 conversion (round to nearest even, saturating at 6, sign
//    kept) is monotone, so where it gives both the same code, that is the
//    code of x / D (a tie, exactly at a midpoint, always splits them).
//    Where they differ (adjacent codes: one midpoint between them), the
//    element is decided exactly: the sign of (midpoint * s_hat) * s_t - |x|
//    from one fused multiply-add, ties to the even code (e2m1_resolve).  With
//    bf16 inputs and calibrated scales such elements are not rare (a few in
//    a thousand at the synthetic GQA cache), so they are resolved one by
//    one.  Blocks with a non-finite element, a zero scale code or D outside
//    [2^-100, 2^100] take encode_nvfp4_block whole.
constexpr float kSide = 0x1p-19f;

__device__ inline uint32_t nvfp4_scale_code(float bamax, float s_t, float inv6) {
  const float qa = fminf(bamax * inv6, 448.0f);
  uint32_t c = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(qa, 0.0f, 0, false)) & 0x7Fu;
  const uint32_t trio = (c > 0u ? c - 1u : 0u) | (c << 8) | ((c < 0x7Eu ? c + 1u : c) << 16);
  const float vp = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(trio), 0);
  const float vc = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(trio), 1);
  const float vn = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(trio), 2);
  const float mh = 0.5f * (vc + vn), ml = 0.5f * (vc + vp);   // exact in float32
  const bool near = (c < 0x7Eu && fabsf(qa - mh) <= mh * 0x1p-20f) || (c > 0u && fabsf(qa - ml) <= ml * 0x1p-20f);
  if (near) c = e4m3_rne_code(static_cast<double>(bamax) / (6.0 * static_cast<double>(s_t)));
  return c;
}

// A block's scale code and the two multipliers; ok false: the block takes
// encode_nvfp4_block (the element test comes on top)
struct Nvfp4Prep {
  uint32_t sc;
  float ih, il;
  bool ok;
};
__device__ inline Nvfp4Prep nvfp4_prep(const float (&v)[16], float s_t, float inv6) {
  uint32_t mb = 0;   // the largest |x| as bits: equal to the float maximum when all are finite
#pragma unroll
  for (int i = 0; i < 16; ++i) mb = max(mb, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  const bool fin = mb < 0x7F800000u;
  Nvfp4Prep p;
  p.sc = fin ? nvfp4_scale_code(__uint_as_float(mb), s_t, inv6) : 0u;
  const float D = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(p.sc), 0) * s_t;
  const float inv = __builtin_amdgcn_rcpf(D);
  p.ih = inv * (1.0f + kSide);
  p.il = inv * (1.0f - kSide);
  p.ok = fin && p.sc != 0u && D >= 0x1p-100f && D <= 0x1p100f;
  return p;
}

// E2M1 code of x / D for an element whose two side codes ca, cb differ:
// their magnitudes are adjacent, and x is decided against the midpoint m
// between them: m * s_hat has at most 9 significant bits (exact in float32),
// so (m s_hat) * s_t - |x| is formed exactly inside one fused multiply-add and
// its rounded result has the exact sign (0 only for a tie; D >= 2^-100 keeps
// nonzero results clear of underflow); ties to the even code; the sign is
// x's (as in ca)
__device__ inline uint32_t e2m1_resolve(float x, uint32_t ca, uint32_t cb, float shat, float s_t) {
  constexpr uint32_t kTwice = 0xC8643210u;   // nibble m: twice the E2M1 magnitude of code m
  const uint32_t ma = ca & 7u, mb = cb & 7u;
  const uint32_t hi_m = ma > mb ? ma : mb, lo_m = ma > mb ? mb : ma;
  const uint32_t s4 = ((kTwice >> (4 * ma)) & 15u) + ((kTwice >> (4 * mb)) & 15u);   // 4 x the midpoint
  const float dd = __builtin_fmaf(static_cast<float>(s4) * 0.25f * shat, s_t, -fabsf(x));
  const uint32_t m = dd < 0.0f ? hi_m : (dd > 0.0f ? lo_m : ((hi_m & 1u) == 0u ? hi_m : lo_m));
  return m | (ca & 8u);
}

// the nibble at bit sh of w (its other side's nibble differs where d has
// bits) decided by e2m1_resolve
__device__ inline void resolve_nibble(uint32_t& w, uint32_t d, int sh, float x, float shat, float s_t) {
  const uint32_t dn = (d >> sh) & 15u;
  if (dn != 0u) {
    const uint32_t ca = (w >> sh) & 15u;
    w = (w & ~(15u << sh)) | (e2m1_resolve(x, ca, ca ^ dn, shat, s_t) << sh);
  }
}

// v[i] for a per-lane index i: a tree of bit selects on the index bits (no
// indexed access, which would put v in scratch memory)
__device__ inline float pick16(const float (&v)[16], int i) {
  const uint32_t m0 = 0u - static_cast<uint32_t>(i & 1), m1 = 0u - static_cast<uint32_t>((i >> 1) & 1);
  const uint32_t m2 = 0u - static_cast<uint32_t>((i >> 2) & 1), m3 = 0u - static_cast<uint32_t>((i >> 3) & 1);
  uint32_t a[8], b[4];
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = (__float_as_uint(v[2 * k + 1]) & m0) | (__float_as_uint(v[2 * k]) & ~m0);
#pragma unroll
  for (int k = 0; k < 4; ++k) b[k] = (a[2 * k + 1] & m1) | (a[2 * k] & ~m1);
  const uint32_t c0 = (b[1] & m2) | (b[0] & ~m2), c1 = (b[3] & m2) | (b[2] & ~m2);
  return __uint_as_float((c1 & m3) | (c0 & ~m3));
}

__device__ inline float e4m3_val(uint32_t sc) { return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(sc), 0); }

// 8 E2M1 codes of x[o .. o + 7] * m (element o + i in nibble i)
__device__ inline uint32_t e2m1_word(const float (&x)[16], int o, float m) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[o] * m, x[o + 1] * m, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[o + 2] * m, x[o + 3] * m, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[o + 4] * m, x[o + 5] * m, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[o + 6] * m, x[o + 7] * m, 1.0f, 3);
  return w;
}

// TOKEN4: codes of tokens (2H, 2H + 1) of a group (element i: byte 2i + H of
// the 32, dword i / 2, byte 2 (i & 1) + H), with the multipliers of the side m
template <int H>
__device__ inline void t4_pair(const float (&v0)[16], const float (&v1)[16], float m0, float m1, uint32_t (&w)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    w[k] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[k], v0[2 * k] * m0, v1[2 * k] * m1, 1.0f, H);
    w[k] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[k], v0[2 * k + 1] * m0, v1[2 * k + 1] * m1, 1.0f, 2 + H);
  }
}

// TOKEN4: the codes of tokens (2H, 2H + 1) in w (the ih side) where the il
// side (wl, this pair's bytes only) differs, decided exactly
template <int H>
__device__ inline void t4_pair_resolve(const float (&v0)[16], const float (&v1)[16], float sh0, float sh1, float s_t,
                                       const uint32_t (&wl)[8], uint32_t (&w)[8]) {
  constexpr uint32_t kMask = 0x00FF00FFu << (8 * H);
  uint32_t any = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) any |= (w[k] ^ wl[k]) & kMask;
  if (any == 0u) return;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t d = (w[k] ^ wl[k]) & kMask;
    resolve_nibble(w[k], d, 8 * H, v0[2 * k], sh0, s_t);
    resolve_nibble(w[k], d, 8 * H + 4, v1[2 * k], sh1, s_t);
    resolve_nibble(w[k], d, 16 + 8 * H, v0[2 * k + 1], sh0, s_t);
    resolve_nibble(w[k], d, 16 + 8 * H + 4, v1[2 * k + 1], sh1, s_t);
  }
}

// item it of a head -> (row or group, block); nb a power of two takes a shift
__device__ inline void split_item(int64_t it, uint32_t nb, int nbsh, int64_t& t, int& blk) {
  if (nbsh >= 0) {
    t = it >> nbsh;
    blk = static_cast<int>(it & (nb - 1u));
  } else {
    t = it / nb;
    blk = static_cast<int>(it - t * nb);
  }
}

// ROWS layout: one item per (row, 16-element block) -> 8 code bytes (one
// 64-bit store), 1 scale byte
__device__ inline void pack_nvfp4_rows(const PackJob& J, float s_t, float inv6) {
  const int d = J.d;
  const uint32_t nb = static_cast<uint32_t>(d / 16);
  const int nbsh = (nb & (nb - 1u)) == 0u ? __builtin_ctz(nb) : -1;
  const Rows xr = J.xr, dr = J.dr;
  const int64_t nh = xr.n0 * xr.n1;
  for (int64_t h = blockIdx.y; h < nh; h += gridDim.y) {
    const int64_t i0 = h / xr.n1, i1 = h - i0 * xr.n1;
    const int64_t pos = J.dst_pos != nullptr ? J.dst_pos[i0] : 0;
    const int64_t xbase = i0 * xr.s0 + i1 * xr.s1, dbase = i0 * dr.s0 + i1 * dr.s1;
    const int64_t items = xr.n2 * nb;
    for (int64_t it = head_items_start(); it < items; it += head_items_stride()) {
      int64_t t;
      int blk;
      split_item(it, nb, nbsh, t, blk);
      const int64_t dt_ = t + pos;
      if (dt_ < 0 || dt_ >= dr.n2) continue;  // outside the destination plane
      float v[16];
      load_run<16>(J.x, J.dt, xbase + t * xr.s2 + blk * 16, 16, v);
      const Nvfp4Prep p = nvfp4_prep(v, s_t, inv6);
      uint32_t sc = p.sc;
      uint32_t lo = e2m1_word(v, 0, p.ih), hi = e2m1_word(v, 8, p.ih);
      const uint32_t dlo = lo ^ e2m1_word(v, 0, p.il), dhi = hi ^ e2m1_word(v, 8, p.il);
      if (p.ok) {
        // elements next to a midpoint: exact decisions, one differing nibble
        // per lane and pass (usually one pass)
        uint64_t dd = (static_cast<uint64_t>(dhi) << 32) | dlo;
        uint64_t code = (static_cast<uint64_t>(hi) << 32) | lo;
        const float shat = e4m3_val(sc);
        while (__any(dd != 0u)) {
          if (dd != 0u) {
            const int sh = __builtin_ctzll(dd) & ~3;
            const uint32_t ca = static_cast<uint32_t>(code >> sh) & 15u;
            const uint32_t cb = ca ^ (static_cast<uint32_t>(dd >> sh) & 15u);
            code = (code & ~(15ull << sh)) | (static_cast<uint64_t>(e2m1_resolve(pick16(v, sh >> 2), ca, cb, shat, s_t)) << sh);
            dd &= ~(15ull << sh);
          }
        }
        lo = static_cast<uint32_t>(code);
        hi = static_cast<uint32_t>(code >> 32);
      } else {
        uint32_t c[16];
        sc = encode_nvfp4_block(v, s_t, c);
        lo = 0;
        hi = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          lo |= c[i] << (4 * i);
          hi |= c[8 + i] << (4 * i);
        }
      }
      const int64_t drow = dbase + dt_ * dr.s2;
      *reinterpret_cast<uint2*>(J.codes + drow * (d / 2) + blk * 8) = make_uint2(lo, hi);
      J.scales[drow * nb + blk] = static_cast<uint8_t>(sc);
    }
  }
}

// Group slots per (i0, i1) that a pack into a TOKEN4 plane visits: rows
// [pos, pos + n2) touch at most n2/4 + 2 groups.
__device__ inline int64_t t4_slots(int64_t n2) { return n2 / 4 + 2; }

// For group slot gl of (i0, i1): first destination token t0 and, per token
// j, the source row (or -1).  Returns false if the slot has no source row.
__device__ inline bool t4_group(const Rows& xr, const Rows& dr, const int32_t* dst_pos, int64_t i0, int64_t gl,
                                int64_t& t0, int64_t (&src)[4]) {
  const int64_t pos = dst_pos != nullptr ? dst_pos[i0] : 0;
  const int64_t q = (pos >= 0 ? pos / 4 : -((-pos + 3) / 4)) + gl;  // floor(pos / 4) + gl
  t0 = 4 * q;
  bool any = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t = t0 + j;
    const int64_t r = t - pos;
    const bool ok = t >= 0 && t < dr.n2 && r >= 0 && r < xr.n2;
    src[j] = ok ? r : -1;
    any |= ok;
  }
  return any;
}

// TOKEN4 layout: one item per (4-token group slot, 16-element block): 32
// code bytes (two 16-byte stores) and one 4-byte scale word; tokens of the
// group that this call does not write keep their bytes.
__device__ inline void pack_nvfp4_t4(const PackJob& J, float s_t, float inv6) {
  const int d = J.d;
  const uint32_t nb = static_cast<uint32_t>(d / 16);
  const int nbsh = (nb & (nb - 1u)) == 0u ? __builtin_ctz(nb) : -1;
  const Rows xr = J.xr, dr = J.dr;
  const int64_t slots = t4_slots(xr.n2);
  const int64_t nh = xr.n0 * xr.n1;
  for (int64_t h = blockIdx.y; h < nh; h += gridDim.y) {
    const int64_t i0 = h / xr.n1, i1 = h - i0 * xr.n1;
    const int64_t xbase = i0 * xr.s0 + i1 * xr.s1;
    const int64_t items = slots * nb;
    for (int64_t it = head_items_start(); it < items; it += head_items_stride()) {
      int64_t gl;
      int blk;
      split_item(it, nb, nbsh, gl, blk);
      int64_t t0, src[4];
      if (!t4_group(xr, dr, J.dst_pos, i0, gl, t0, src)) continue;
      const int64_t grow = group_row(dr, i0, i1, t0);
      uint4* cp = reinterpret_cast<uint4*>(J.codes + grow * (d / 2) + blk * 32);
      uint32_t* sp = reinterpret_cast<uint32_t*>(J.scales + grow * nb + blk * 4);
      const bool partial = src[0] < 0 || src[1] < 0 || src[2] < 0 || src[3] < 0;
      if (!partial) {   // a whole group: tokens (0, 1), then (2, 3), two at a time
        uint32_t wh[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        uint32_t scw = 0;
        bool ok = true;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float v0[16], v1[16];
          load_run<16>(J.x, J.dt, xbase + src[2 * h] * xr.s2 + blk * 16, 16, v0);
          load_run<16>(J.x, J.dt, xbase + src[2 * h + 1] * xr.s2 + blk * 16, 16, v1);
          const Nvfp4Prep p0 = nvfp4_prep(v0, s_t, inv6), p1 = nvfp4_prep(v1, s_t, inv6);
          ok = ok && p0.ok && p1.ok;
          scw |= (p0.sc | (p1.sc << 8)) << (16 * h);
          uint32_t wl[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
          if (h == 0) {
            t4_pair<0>(v0, v1, p0.ih, p1.ih, wh);
            t4_pair<0>(v0, v1, p0.il, p1.il, wl);
            if (p0.ok && p1.ok) t4_pair_resolve<0>(v0, v1, e4m3_val(p0.sc), e4m3_val(p1.sc), s_t, wl, wh);
          } else {
            t4_pair<1>(v0, v1, p0.ih, p1.ih, wh);
            t4_pair<1>(v0, v1, p0.il, p1.il, wl);
            if (p0.ok && p1.ok) t4_pair_resolve<1>(v0, v1, e4m3_val(p0.sc), e4m3_val(p1.sc), s_t, wl, wh);
          }
        }
        if (ok) {
          cp[0] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
          cp[1] = make_uint4(wh[4], wh[5], wh[6], wh[7]);
          *sp = scw;
          continue;
        }
      }
      uint4 w0 = partial ? cp[0] : make_uint4(0, 0, 0, 0);
      uint4 w1 = partial ? cp[1] : make_uint4(0, 0, 0, 0);
      uint32_t sw = partial ? *sp : 0u;
      uint32_t* wd[8] = {&w0.x, &w0.y, &w0.z, &w0.w, &w1.x, &w1.y, &w1.z, &w1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (src[j] < 0) continue;
        float v[16];
        load_run<16>(J.x, J.dt, xbase + src[j] * xr.s2 + blk * 16, 16, v);
        uint32_t c[16];
        const uint32_t sc = encode_nvfp4_block(v, s_t, c);
        sw = (sw & ~(0xFFu << (8 * j))) | (sc << (8 * j));
        // element i: byte 2i + (j >> 1), nibble j & 1 -> dword i / 2, bit 16 (i & 1) + 8 (j >> 1) + 4 (j & 1)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int sh = 16 * (i & 1) + 8 * (j >> 1) + 4 * (j & 1);
          *wd[i >> 1] = (*wd[i >> 1] & ~(0xFu << sh)) | (c[i] << sh);
        }
      }
      cp[0] = w0;
      cp[1] = w1;
      *sp = sw;
    }
  }
}

// grid: (items of one head, heads, jobs)
__global__ void __launch_bounds__(kThreads) k_pack_nvfp4(PackJobs P) {
  const PackJob& J = P.j[blockIdx.z];
  const float s_t = nvfp4_tensor_scale(*J.amax);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && J.sout != nullptr) *J.sout = s_t;
  const float inv6 = 1.0f / (6.0f * s_t);
  if (J.layout == KVQ_PLANE_TOKEN4) pack_nvfp4_t4(J, s_t, inv6);
  else pack_nvfp4_rows(J, s_t, inv6);
}

// ---------------------------------------------------------------- FP8 pack
// As for NVFP4, the bulk pack converts every element twice with the
// hardware (x * ih and x * il, ih and il = (1 / scale) (1 +- 2^-19), both
// clamped to +-448, converted two at a time into the code word): the two
// products lie strictly on either side of x / scale (errors below 2^-21), so
// equal codes are the code of encode_fp8, and where they differ (adjacent
// codes) one fused multiply-add decides exactly (e4m3_resolve).  Runs with a
// non-finite element, partial runs and scales below 2^-100 take encode_fp8.

// E4M3 code of x / scale where the side codes ca, cb (bytes, with x's sign)
// differ: |x| against the midpoint between them times scale; the midpoint
// has at most 5 significant bits, so m * scale - |x| is formed exactly
// inside the fused multiply-add and its rounded result has the exact sign
// (and is 0 only for a tie), ties to the even code
__device__ inline uint32_t e4m3_resolve(float x, uint32_t ca, uint32_t cb, float scale) {
  const uint32_t ma = ca & 0x7Fu, mb = cb & 0x7Fu;
  const uint32_t hi_m = ma > mb ? ma : mb, lo_m = ma > mb ? mb : ma;
  const float vh = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(hi_m), 0);
  const float vl = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(lo_m), 0);
  const float dd = __builtin_fmaf(0.5f * (vh + vl), scale, -fabsf(x));
  const uint32_t m = dd < 0.0f ? hi_m : (dd > 0.0f ? lo_m : ((hi_m & 1u) == 0u ? hi_m : lo_m));
  return m | (ca & 0x80u);
}

// the byte at bit sh of w (its other side's byte differs where d has bits)
// decided by e4m3_resolve
__device__ inline void resolve_byte(uint32_t& w, uint32_t d, int sh, float x, float scale) {
  if (((d >> sh) & 0xFFu) != 0u) {
    const uint32_t ca = (w >> sh) & 0xFFu, cb = ca ^ ((d >> sh) & 0xFFu);
    w = (w & ~(0xFFu << sh)) | (e4m3_resolve(x, ca, cb, scale) << sh);
  }
}

// codes of x0 .. x3 (byte i) on the side m
__device__ inline uint32_t e4m3_word(float x0, float x1, float x2, float x3, float m) {
  const float a0 = __builtin_amdgcn_fmed3f(x0 * m, -448.0f, 448.0f), a1 = __builtin_amdgcn_fmed3f(x1 * m, -448.0f, 448.0f);
  const float a2 = __builtin_amdgcn_fmed3f(x2 * m, -448.0f, 448.0f), a3 = __builtin_amdgcn_fmed3f(x3 * m, -448.0f, 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, w, true);
  return static_cast<uint32_t>(w);
}

// the exact codes of x0 .. x3 (all finite; scale >= 2^-100)
__device__ inline uint32_t fp8_word_fast(float x0, float x1, float x2, float x3, float ih, float il, float scale) {
  uint32_t w = e4m3_word(x0, x1, x2, x3, ih);
  const uint32_t d = w ^ e4m3_word(x0, x1, x2, x3, il);
  if (d != 0u) {
    resolve_byte(w, d, 0, x0, scale);
    resolve_byte(w, d, 8, x1, scale);
    resolve_byte(w, d, 16, x2, scale);
    resolve_byte(w, d, 24, x3, scale);
  }
  return w;
}

template <int N>
__device__ inline bool all_finite(const float (&v)[N]) {
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) mb = max(mb, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  return mb < 0x7F800000u;
}

// ROWS layout: one item per (row, 16-element run): 16 code bytes (one
// 16-byte store; d % 16 != 0 leaves a shorter last run, stored per word)
// The scale of head i1: one per tensor, or amax[i1] / 448 with one scale
// per kv head (written to sout[i1] by one work-group).
__device__ inline void fp8_head_scale(const PackJob& J, int64_t i0, int64_t i1, double& dscale, float& inv) {
  if (!J.per_head) return;
  const float scale = fp8_tensor_scale(J.amax[i1]);
  if (i0 == 0 && blockIdx.x == 0 && threadIdx.x == 0 && J.sout != nullptr) J.sout[i1] = scale;
  dscale = static_cast<double>(scale);
  inv = 1.0f / scale;
}

__device__ inline void pack_fp8_rows(const PackJob& J, double dscale0, float inv0) {
  const int d = J.d;
  const uint32_t nr = static_cast<uint32_t>((d + 15) / 16);
  const Rows xr = J.xr, dr = J.dr;
  const int64_t nh = xr.n0 * xr.n1;
  for (int64_t h = blockIdx.y; h < nh; h += gridDim.y) {
    const int64_t i0 = h / xr.n1, i1 = h - i0 * xr.n1;
    double dscale = dscale0;
    float inv = inv0;
    fp8_head_scale(J, i0, i1, dscale, inv);
    const float fsc = static_cast<float>(dscale), ih = inv * (1.0f + 0x1p-19f), il = inv * (1.0f - 0x1p-19f);
    const bool fast = fsc >= 0x1p-100f;
    const int64_t pos = J.dst_pos != nullptr ? J.dst_pos[i0] : 0;
    const int64_t xbase = i0 * xr.s0 + i1 * xr.s1, dbase = i0 * dr.s0 + i1 * dr.s1;
    const int64_t items = xr.n2 * nr;
    for (int64_t it = head_items_start(); it < items; it += head_items_stride()) {
      const int64_t t = it / nr;
      const int run = static_cast<int>(it - t * nr);
      const int64_t dt_ = t + pos;
      if (dt_ < 0 || dt_ >= dr.n2) continue;  // outside the destination plane
      const int n = d - 16 * run < 16 ? d - 16 * run : 16;   // a multiple of 4
      float v[16];
      load_run<16>(J.x, J.dt, xbase + t * xr.s2 + 16 * run, n, v);
      uint32_t w[4];
      if (fast && n == 16 && all_finite(v)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = fp8_word_fast(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], ih, il, fsc);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          w[q] = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[q] |= encode_fp8(v[4 * q + i], inv, dscale) << (8 * i);
        }
      }
      uint8_t* dst = J.codes + (dbase + dt_ * dr.s2) * d + 16 * run;
      if (n == 16 && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (4 * q < n) reinterpret_cast<uint32_t*>(dst)[q] = w[q];
      }
    }
  }
}

// TOKEN4 layout: one item per (4-token group slot, 16 elements): 64 code
// bytes (4 elements and 16 bytes when d is not a multiple of 16)
__device__ inline void pack_fp8_t4(const PackJob& J, double dscale0, float inv0) {
  const int d = J.d;
  const int per = d % 16 == 0 ? 4 : 1;   // 16-byte code words per item
  const uint32_t nw = static_cast<uint32_t>(d / (4 * per));
  const int nwsh = (nw & (nw - 1u)) == 0u ? __builtin_ctz(nw) : -1;
  const Rows xr = J.xr, dr = J.dr;
  const int64_t slots = t4_slots(xr.n2);
  const int64_t nh = xr.n0 * xr.n1;
  for (int64_t h = blockIdx.y; h < nh; h += gridDim.y) {
    const int64_t i0 = h / xr.n1, i1 = h - i0 * xr.n1;
    double dscale = dscale0;
    float inv = inv0;
    fp8_head_scale(J, i0, i1, dscale, inv);
    const float fsc = static_cast<float>(dscale), ih = inv * (1.0f + 0x1p-19f), il = inv * (1.0f - 0x1p-19f);
    const bool fast = fsc >= 0x1p-100f;
    const int64_t xbase = i0 * xr.s0 + i1 * xr.s1;
    const int64_t items = slots * nw;
    for (int64_t it = head_items_start(); it < items; it += head_items_stride()) {
      int64_t gl;
      int r;
      split_item(it, nw, nwsh, gl, r);
      int64_t t0, src[4];
      if (!t4_group(xr, dr, J.dst_pos, i0, gl, t0, src)) continue;
      uint4* cp = reinterpret_cast<uint4*>(J.codes + group_row(dr, i0, i1, t0) * d + r * 16 * per);
      const bool partial = src[0] < 0 || src[1] < 0 || src[2] < 0 || src[3] < 0;
      if (fast && !partial && per == 4) {   // a whole group, 16 elements: dword e = element 16 r + e of tokens 0 .. 3
        float x[4][16];
#pragma unroll
        for (int j = 0; j < 4; ++j) load_run<16>(J.x, J.dt, xbase + src[j] * xr.s2 + r * 16, 16, x[j]);
        if (all_finite(x[0]) && all_finite(x[1]) && all_finite(x[2]) && all_finite(x[3])) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              o[i] = fp8_word_fast(x[0][4 * q + i], x[1][4 * q + i], x[2][4 * q + i], x[3][4 * q + i], ih, il, fsc);
            cp[q] = make_uint4(o[0], o[1], o[2], o[3]);
          }
          continue;
        }
      }
      for (int q = 0; q < per; ++q) {   // 4 elements at a time: w = the word of the row
        const int w = r * per + q;
        if (fast && !partial) {   // a whole group: dword i = element 4w + i of tokens 0 .. 3
          float x[4][4];
#pragma unroll
          for (int j = 0; j < 4; ++j) load_run<4>(J.x, J.dt, xbase + src[j] * xr.s2 + w * 4, 4, x[j]);
          if (all_finite(x[0]) && all_finite(x[1]) && all_finite(x[2]) && all_finite(x[3])) {
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = fp8_word_fast(x[0][i], x[1][i], x[2][i], x[3][i], ih, il, fsc);
            cp[q] = make_uint4(o[0], o[1], o[2], o[3]);
            continue;
          }
        }
        uint4 wv = partial ? cp[q] : make_uint4(0, 0, 0, 0);
        uint32_t* wd[4] = {&wv.x, &wv.y, &wv.z, &wv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (src[j] < 0) continue;
          float v[4];
          load_run<4>(J.x, J.dt, xbase + src[j] * xr.s2 + w * 4, 4, v);
#pragma unroll
          for (int i = 0; i < 4; ++i)  // element 4w + i of token j: byte 4 (4w + i) + j
            *wd[i] = (*wd[i] & ~(0xFFu << (8 * j))) | (encode_fp8(v[i], inv, dscale) << (8 * j));
        }
        cp[q] = wv;
      }
    }
  }
}

__global__ void __launch_bounds__(kThreads) k_pack_fp8(PackJobs P) {
  const PackJob& J = P.j[blockIdx.z];
  const float scale = fp8_tensor_scale(*J.amax);   // (per head: replaced per head)
  if (!J.per_head && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && J.sout != nullptr) *J.sout = scale;
  const float inv = 1.0f / scale;   // candidate quotients only; decisions are exact
  if (J.layout == KVQ_PLANE_TOKEN4) pack_fp8_t4(J, static_cast<double>(scale), inv);
  else pack_fp8_rows(J, static_cast<double>(scale), inv);
}

// ---------------------------------------------------------------- unpack
__global__ void __launch_bounds__(kThreads) k_unpack_nvfp4(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales, Rows sr, int layout, int d,
                                                           const float* __restrict__ ts, float* __restrict__ out,
                                                           Rows orow) {
  const float s_t = *ts;
  const int nb = d / 16;
  const int64_t total = sr.n0 * sr.n1 * sr.n2 * nb;
  for (int64_t gid = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; gid < total;
       gid += static_cast<int64_t>(gridDim.x) * kThreads) {
    int64_t row = gid / nb;
    int blk = static_cast<int>(gid - row * nb);
    int64_t i0, i1, i2;
    unravel(row, sr, i0, i1, i2);
    uint32_t c[16];
    uint32_t sc;
    if (layout == KVQ_PLANE_TOKEN4) {
      const int64_t grow = group_row(sr, i0, i1, i2 & ~int64_t(3));
      const int j = static_cast<int>(i2 & 3);
      const uint8_t* cb = codes + grow * (d / 2) + blk * 32;
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = (cb[2 * i + (j >> 1)] >> (4 * (j & 1))) & 15u;
      sc = scales[grow * nb + blk * 4 + j];
    } else {
      const int64_t r = row_off(sr, i0, i1, i2);
      const uint2 cw = *reinterpret_cast<const uint2*>(codes + r * (d / 2) + blk * 8);
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = ((i < 8 ? cw.x : cw.y) >> (4 * (i & 7))) & 15u;
      sc = scales[r * nb + blk];
    }
    const float s_hat = static_cast<float>(e4m3_value(sc));
    float* o = out + row_off(orow, i0, i1, i2) + blk * 16;
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = (e2m1_value(c[i]) * s_hat) * s_t;  // e * s_hat exact in fp32, one rounding
  }
}

__global__ void __launch_bounds__(kThreads) k_unpack_fp8(const uint8_t* __restrict__ codes, Rows sr, int layout, int d,
                                                         const float* __restrict__ scale, float* __restrict__ out,
                                                         Rows orow) {
  const float sc = *scale;
  const int64_t total = sr.n0 * sr.n1 * sr.n2 * d;
  for (int64_t gid = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; gid < total;
       gid += static_cast<int64_t>(gridDim.x) * kThreads) {
    int64_t row = gid / d;
    int col = static_cast<int>(gid - row * d);
    int64_t i0, i1, i2;
    unravel(row, sr, i0, i1, i2);
    uint32_t c;
    if (layout == KVQ_PLANE_TOKEN4)
      c = codes[group_row(sr, i0, i1, i2 & ~int64_t(3)) * d + 4 * col + (i2 & 3)];
    else
      c = codes[row_off(sr, i0, i1, i2) * d + col];
    out[row_off(orow, i0, i1, i2) + col] = static_cast<float>(e4m3_value(c)) * sc;
  }
}

int grid_for(int64_t items) {
  int64_t g = (items + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;  // grid-stride loops cover the rest
  return static_cast<int>(g);
}

}  // namespace

// grid of the row kernels: y = heads (at most 65535, the kernels stride over
// the rest), x = enough blocks for the items of one head, about 8192 blocks
// in all
static dim3 head_grid(int64_t heads, int64_t items_per_head, int z, int64_t budget = 8192) {
  int64_t y = heads < 1 ? 1 : (heads > 65535 ? 65535 : heads);
  int64_t x = (items_per_head + kThreads - 1) / kThreads;
  const int64_t xmax = budget / y > 1 ? budget / y : 1;
  x = x < 1 ? 1 : (x > xmax ? xmax : x);
  return dim3(static_cast<unsigned>(x), static_cast<unsigned>(y), static_cast<unsigned>(z));
}

hipError_t launch_amax(const void* x, int x_dtype, Rows rows, int d, const int32_t* kv_lens, float* amax_out,
                       bool accumulate, bool per_head, hipStream_t st) {
  const int64_t nout = per_head ? rows.n1 : 1;
  if (!accumulate && nout > 0)
    hipLaunchKernelGGL(k_zero_n, dim3(static_cast<unsigned>((nout + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                       amax_out, nout);
  const int64_t heads = rows.n0 * rows.n1;
  if (heads > 0 && rows.n2 > 0)
    hipLaunchKernelGGL(k_amax, head_grid(heads, rows.n2 * ((d + 7) / 8), 1, 1024), dim3(kThreads), 0, st, x, x_dtype,
                       rows, d, kv_lens, amax_out, per_head ? 1 : 0);
  return hipGetLastError();
}

// items of one head of one job: (row, 16-block) / (row, 16-element run), or
// (4-token group slot, 16-block / 16 elements, or 4 when d is not a multiple
// of 16) for TOKEN4 destinations
static int64_t pack_items_per_head(const PackJob& J, bool fp4) {
  const bool t4 = J.layout == KVQ_PLANE_TOKEN4;
  const int64_t per = fp4 ? J.d / 16 : (t4 ? (J.d % 16 == 0 ? J.d / 16 : J.d / 4) : (J.d + 15) / 16);
  return (t4 ? J.xr.n2 / 4 + 2 : J.xr.n2) * per;
}

static hipError_t launch_pack(const PackJobs& P, bool fp4, hipStream_t st) {
  int64_t items = 0, heads = 0;
  for (int i = 0; i < P.n; ++i) {
    const int64_t n = pack_items_per_head(P.j[i], fp4), h = P.j[i].xr.n0 * P.j[i].xr.n1;
    items = n > items ? n : items;
    heads = h > heads ? h : heads;
  }
  const dim3 grid = head_grid(heads, items, P.n);
  if (fp4) hipLaunchKernelGGL(k_pack_nvfp4, grid, dim3(kThreads), 0, st, P);
  else hipLaunchKernelGGL(k_pack_fp8, grid, dim3(kThreads), 0, st, P);
  return hipGetLastError();
}

hipError_t launch_pack_nvfp4(const PackJobs& P, hipStream_t st) { return launch_pack(P, true, st); }
hipError_t launch_pack_fp8(const PackJobs& P, hipStream_t st) { return launch_pack(P, false, st); }

hipError_t launch_unpack_nvfp4(const uint8_t* codes, const uint8_t* scales, Rows sr, int layout, int d, const float* ts,
                               float* out, Rows orow, hipStream_t st) {
  const int64_t items = sr.n0 * sr.n1 * sr.n2 * (d / 16);
  hipLaunchKernelGGL(k_unpack_nvfp4, dim3(grid_for(items)), dim3(kThreads), 0, st, codes, scales, sr, layout, d, ts, out,
                     orow);
  return hipGetLastError();
}

hipError_t launch_unpack_fp8(const uint8_t* codes, Rows sr, int layout, int d, const float* scale, float* out, Rows orow,
                             hipStream_t st) {
  const int64_t items = sr.n0 * sr.n1 * sr.n2 * d;
  hipLaunchKernelGGL(k_unpack_fp8, dim3(grid_for(items)), dim3(kThreads), 0, st, codes, sr, layout, d, scale, out, orow);
  return hipGetLastError();
}

}  // namespace kvq
