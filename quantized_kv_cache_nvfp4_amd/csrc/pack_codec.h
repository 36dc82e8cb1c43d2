// Exact E2M1 / E4M3 encoders shared by the pack kernels and the decode
// kernel's fused append of the new token (so that both write the same
// bytes).  Every rounding decision is the exact real-number decision: the
// inputs have at most 24 significant bits and every threshold at most 32,
// so a correctly rounded float64 quotient or product lands on the same side
// of every threshold as the real one (and exactly on it for a tie); ties go
// to the even code.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {
namespace codec {

// E4M3 (FN) code of the round-to-nearest-even of a non-negative double q,
// saturating at 448.
__device__ inline uint32_t e4m3_rne_code(double q) {
  if (!(q < 448.0)) return 0x7E;
  int ex;
  (void)frexp(q, &ex);             // q = f * 2^ex, f in [0.5, 1)
  int e = ex - 1;                  // floor(log2 q)
  if (e < -6) e = -6;              // subnormal binade shares 2^-6's quantum
  double n = rint(ldexp(q, 3 - e));  // exact scaling, round half to even
  int ni = static_cast<int>(n);
  if (ni == 0) return 0;
  if (ni == 16) { e += 1; ni = 8; }
  if (ni < 8) return static_cast<uint32_t>(ni);  // subnormal (e == -6)
  return static_cast<uint32_t>(((e + 7) << 3) | (ni - 8));
}

// E2M1 code (0..7) of the round-to-nearest-even of a non-negative double r,
// saturating at 6.
__device__ inline uint32_t e2m1_rne_code(double r) {
  if (!(r < 6.0)) return 7;
  int ex;
  (void)frexp(r, &ex);
  int e = ex - 1;
  if (e < 0) e = 0;
  int ni = static_cast<int>(rint(ldexp(r, 1 - e)));
  if (ni == 4) { e += 1; ni = 2; }
  if (ni < 2) return static_cast<uint32_t>(ni);  // 0 or 0.5
  return static_cast<uint32_t>(((e + 1) << 1) | (ni - 2));
}

__device__ inline double e4m3_value(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  double mag = (e == 0) ? ldexp(static_cast<double>(m), -9) : ldexp(static_cast<double>(8 + m), static_cast<int>(e) - 10);
  return (c & 0x80u) ? -mag : mag;
}

__device__ inline float e2m1_value(uint32_t c) {
  uint32_t e = (c >> 1) & 3u, m = c & 1u;
  float mag = (e == 0) ? 0.5f * static_cast<float>(m) : ldexpf(1.0f + 0.5f * static_cast<float>(m), static_cast<int>(e) - 1);
  return (c & 8u) ? -mag : mag;
}

__device__ inline float nvfp4_tensor_scale(float amax) {
  return amax > 0.0f ? static_cast<float>(static_cast<double>(amax) / 2688.0) : 1.0f;
}

__device__ inline float fp8_tensor_scale(float amax) {
  return amax > 0.0f ? static_cast<float>(static_cast<double>(amax) / 448.0) : 1.0f;
}

// NVFP4 encoding of one 16-element block with tensor scale s_t: returns the
// E4M3 scale code and writes the 16 E2M1 codes (sign in bit 3); a block whose
// scale rounds to 0 gets all-zero codes.  The E2M1 decision for |x| / D
// (D = s_hat * s_t) is taken by comparing |x| with the seven midpoints of the
// E2M1 magnitudes times D: each product has at most 31 significant bits, so
// it is exact in float64 and every comparison is the exact real one.  Ties
// go to the even code: strictly above 0.25, 1.25, 2.5 and 5, at or above
// 0.75, 1.75 and 3.5.  (The same decisions as rounding the quotient.)
// float32 neighbours of a positive double t: round down / round up
__device__ inline float f32_rd(double t) {
  const float f = static_cast<float>(t);
  return static_cast<double>(f) > t ? __uint_as_float(__float_as_uint(f) - 1u) : f;
}
__device__ inline float f32_ru(double t) {
  const float f = static_cast<float>(t);
  return static_cast<double>(f) < t ? __uint_as_float(__float_as_uint(f) + 1u) : f;
}

__device__ inline uint32_t encode_nvfp4_block(const float* v, float s_t, uint32_t* c) {
  float bamax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) bamax = fmaxf(bamax, fabsf(v[i]));
  const uint32_t sc = e4m3_rne_code(static_cast<double>(bamax) / (6.0 * static_cast<double>(s_t)));
  if (sc == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = 0;
    return 0;
  }
  // The seven thresholds t_k = midpoint_k * D (exact in float64), compared
  // with the float32 |x| through float32 neighbours: for a float32 a,
  // a > t <=> a > RD(t) and a >= t <=> a >= RU(t) (no float32 lies between
  // RD(t) and RU(t)), so every comparison below is the exact real one.  The
  // code is the number of thresholds passed, found by a three-level binary
  // search (levels 1 and 2 use the "at or above" thresholds 1.75, 0.75 /
  // 3.5, level 3 the "above" ones 0.25 / 1.25 / 2.5 / 5).
  const double den = e4m3_value(sc) * static_cast<double>(s_t);  // exact
  const float t0 = f32_rd(0.25 * den), t1 = f32_ru(0.75 * den), t2 = f32_rd(1.25 * den), t3 = f32_ru(1.75 * den);
  const float t4 = f32_rd(2.5 * den), t5 = f32_ru(3.5 * den), t6 = f32_rd(5.0 * den);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float ax = fabsf(v[i]);
    const bool b1 = ax >= t3;
    const bool b2 = ax >= (b1 ? t5 : t1);
    const bool b3 = ax > (b1 ? (b2 ? t6 : t4) : (b2 ? t2 : t0));
    uint32_t q = (b1 ? 4u : 0u) | (b2 ? 2u : 0u) | (b3 ? 1u : 0u);
    q = (ax != ax) ? 7u : q;   // NaN: as the quotient path (not below 6 -> saturate)
    c[i] = q | ((__float_as_uint(v[i]) >> 28) & 8u);
  }
  return sc;
}

// 2^k as a double (k in the normal range)
__device__ inline double pow2d(int k) { return __hiloint2double((k + 1023) << 20, 0); }

// Exact check of an E4M3 candidate code c for the real quotient ax / scale
// (c the exact code or a neighbour): compare ax with the two midpoints
// around value(c), scaled exactly in float64 (5 x 24 significant bits), ties
// to the even code.
__device__ inline uint32_t e4m3_fixup(uint32_t c, float ax, double dscale) {
  const int e = static_cast<int>(c >> 3), m = static_cast<int>(c & 7u);
  const int ue = (e == 0) ? -9 : e - 10;                       // value = mant * 2^ue
  const double val = static_cast<double>(e == 0 ? m : 8 + m) * pow2d(ue);
  const double half = pow2d(ue - 1);
  const double mid_hi = (val + half) * dscale;                           // between c and c + 1
  const double mid_lo = (val - ((m == 0 && e >= 2) ? 0.5 * half : half)) * dscale;   // between c - 1 and c
  const double axd = static_cast<double>(ax);
  const bool up = c < 0x7Eu && (axd > mid_hi || (axd == mid_hi && ((c + 1u) & 1u) == 0u));
  const bool dn = c > 0u && (axd < mid_lo || (axd == mid_lo && ((c - 1u) & 1u) == 0u));
  return c + (up ? 1u : 0u) - (dn ? 1u : 0u);
}

// FP8 code of v / scale: the round-to-nearest-even E4M3 code of |v| / scale
// (exact decision, saturating at 448), sign of v.  The candidate is the
// hardware conversion of the float32 quotient |v| * (1 / scale), whose
// relative error is below 2^-22: it is the exact code unless that quotient
// lies within 2^-20 (relative) of one of the two midpoints around the
// candidate's value.  Only then is it checked exactly: m * scale - |v| is
// formed by one fused multiply-add, rounded once, so its sign (and whether
// it is zero) is that of the exact difference (a midpoint has at most 5
// significant bits; a nonzero exact difference is at least the smallest
// float32 subnormal); ties go to the even code.  Scales below 2^-100, where
// m * scale could underflow, take the float64 check of e4m3_fixup.
__device__ inline uint32_t encode_fp8(float v, float inv, double dscale) {
  const float ax = fabsf(v);
  const float qa = fminf(ax * inv, 448.0f);   // NaN and inf -> 448
  uint32_t c = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(qa, 0.0f, 0, false)) & 0x7Fu;
  // values of c - 1, c, c + 1 (the neighbours only where they exist)
  const uint32_t trio = ((c > 0u ? c - 1u : 0u)) | (c << 8) | ((c < 0x7Eu ? c + 1u : c) << 16);
  const float vp = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(trio), 0);
  const float vc = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(trio), 1);
  const float vn = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(trio), 2);
  const float mh = 0.5f * (vc + vn), ml = 0.5f * (vc + vp);   // exact in float32
  const bool near = (c < 0x7Eu && fabsf(qa - mh) <= mh * 0x1p-20f) || (c > 0u && fabsf(qa - ml) <= ml * 0x1p-20f);
  if (near) {
    const float scale = static_cast<float>(dscale);
    if (scale >= 0x1p-100f) {
      const float dh = __builtin_fmaf(mh, scale, -ax);   // sign of mh * scale - |v|
      const float dl = __builtin_fmaf(ml, scale, -ax);
      const bool up = c < 0x7Eu && (dh < 0.0f || (dh == 0.0f && ((c + 1u) & 1u) == 0u));
      const bool dn = c > 0u && (dl > 0.0f || (dl == 0.0f && ((c - 1u) & 1u) == 0u));
      c = c + (up ? 1u : 0u) - (dn ? 1u : 0u);
    } else {
      c = e4m3_fixup(c, ax, dscale);
    }
  }
  return c | ((__float_as_uint(v) >> 24) & 0x80u);
}

}  // namespace codec
}  // namespace kvq
