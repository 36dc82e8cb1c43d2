// Device helpers shared by the decode kernels (GQA and MLA): f16 / f32
// vector types, the exact FP4 / FP8 -> f16 hardware converts, the MFMA
// wrappers and raw buffer loads with hardware range checking.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {
namespace dec {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

}  // namespace dec
}  // namespace kvq
