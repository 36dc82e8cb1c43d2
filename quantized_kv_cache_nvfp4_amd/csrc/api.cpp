// C-ABI entry points: argument validation, split planning and dispatch to the
// HIP kernels.  Every check runs on the host before anything is launched, so
// a rejected call leaves the stream untouched.  No allocation, no host sync.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "kvq_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return KVQ_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_rows(const kvq_rows& r, const char* name) {
  if (r.n0 < 0 || r.n1 < 0 || r.n2 < 0) return fail(KVQ_ERR_ARG, "%s: negative extent", name);
  if (r.n0 > (1LL << 31) || r.n1 > (1LL << 31) || r.n2 > (1LL << 31))
    return fail(KVQ_ERR_ARG, "%s: extent too large", name);
  return KVQ_OK;
}

bool same_extents(const kvq_rows& a, const kvq_rows& b) { return a.n0 == b.n0 && a.n1 == b.n1 && a.n2 == b.n2; }

// destination plane of a pack: same n0, n1 as the source, at least as long along i2
bool fits_dst(const kvq_rows& x, const kvq_rows& d) { return x.n0 == d.n0 && x.n1 == d.n1 && d.n2 >= x.n2; }

int64_t n_rows(const kvq_rows& r) { return r.n0 * r.n1 * r.n2; }

int check_float_input(const void* x, int32_t dt, const char* name) {
  if (x == nullptr) return fail(KVQ_ERR_ARG, "%s is null", name);
  if (dt != KVQ_F32 && dt != KVQ_BF16) return fail(KVQ_ERR_UNSUPPORTED, "%s: dtype %d not supported (F32, BF16)", name, dt);
  if (!aligned(x, dt == KVQ_F32 ? 4 : 2)) return fail(KVQ_ERR_ALIGN, "%s is not element-aligned", name);
  return KVQ_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// TOKEN4 planes: groups of four consecutive tokens (s2 == 1, s0, s1 and the
// plane length along i2 multiples of 4)
int check_layout(int32_t layout, const kvq_rows& r, const char* name) {
  if (layout == KVQ_PLANE_ROWS) return KVQ_OK;
  if (layout != KVQ_PLANE_TOKEN4) return fail(KVQ_ERR_ARG, "%s: unknown plane layout %d", name, layout);
  if (r.n2 > 1 && r.s2 != 1) return fail(KVQ_ERR_ALIGN, "%s: TOKEN4 layout needs token stride 1", name);
  if ((r.n0 > 1 && r.s0 % 4 != 0) || (r.n1 > 1 && r.s1 % 4 != 0) || r.n2 % 4 != 0)
    return fail(KVQ_ERR_ALIGN, "%s: TOKEN4 layout needs s0, s1 and the plane length to be multiples of 4", name);
  return KVQ_OK;
}

// Validation of one pack job (the rules of kvq_pack_nvfp4 / kvq_pack_fp8).
int check_pack_job(const kvq_pack_job& j, bool fp4) {
  int rc;
  if ((rc = check_float_input(j.x, j.x_dtype, "x")) != KVQ_OK) return rc;
  if ((rc = check_rows(j.x_rows, "x_rows")) != KVQ_OK) return rc;
  if ((rc = check_rows(j.dst_rows, "dst_rows")) != KVQ_OK) return rc;
  if (fp4) {
    if (j.d <= 0 || j.d % 16 != 0 || j.d > 1024)
      return fail(KVQ_ERR_ARG, "d must be a positive multiple of 16, <= 1024 (got %d)", j.d);
    if (j.amax == nullptr || j.codes == nullptr || j.scales == nullptr)
      return fail(KVQ_ERR_ARG, "amax, codes and scales must be non-null");
  } else {
    if (j.d <= 0 || j.d % 4 != 0 || j.d > 4096)
      return fail(KVQ_ERR_ARG, "d must be a positive multiple of 4, <= 4096 (got %d)", j.d);
    if (j.amax == nullptr || j.codes == nullptr) return fail(KVQ_ERR_ARG, "amax and codes must be non-null");
  }
  if (j.scale_per_head != 0 && (fp4 || j.scale_per_head != 1))
    return fail(KVQ_ERR_ARG, "scale_per_head must be 0 or 1, and 1 only for FP8");
  if (!fits_dst(j.x_rows, j.dst_rows))
    return fail(KVQ_ERR_ARG, "dst_rows must match x_rows in n0, n1 and be at least as long in n2");
  if (!aligned(j.codes, fp4 ? 8 : 4)) return fail(KVQ_ERR_ALIGN, "codes plane must be %d-byte aligned", fp4 ? 8 : 4);
  return check_layout(j.dst_layout, j.dst_rows, "dst_rows");
}

int pack_batch(const kvq_pack_job* jobs, int32_t n_jobs, bool fp4, const char* what, void* stream) {
  if (jobs == nullptr || n_jobs < 1 || n_jobs > KVQ_MAX_PACK_JOBS)
    return fail(KVQ_ERR_ARG, "%s: n_jobs must be in [1, %d] with a non-null jobs array", what, KVQ_MAX_PACK_JOBS);
  kvq::PackJobs P{};
  P.n = 0;
  for (int i = 0; i < n_jobs; ++i) {
    const kvq_pack_job& j = jobs[i];
    int rc = check_pack_job(j, fp4);
    if (rc != KVQ_OK) return rc;
    if (n_rows(j.x_rows) == 0) continue;
    P.j[P.n++] = kvq::PackJob{j.x, j.x_dtype, kvq::to_rows(j.x_rows), j.d, j.amax, j.codes, j.scales,
                              kvq::to_rows(j.dst_rows), j.dst_layout, j.dst_pos, j.scale_out, j.scale_per_head};
  }
  if (P.n == 0) return ok();
  const hipError_t e = fp4 ? kvq::launch_pack_nvfp4(P, as_stream(stream)) : kvq::launch_pack_fp8(P, as_stream(stream));
  return hip_status(e, what);
}

}  // namespace

extern "C" {

const char* kvq_last_error(void) { return g_err.c_str(); }

int32_t kvq_version(void) { return 100; }  // 0.1.0

size_t kvq_decode_args_size(void) { return sizeof(kvq_decode_args); }

namespace {
int amax_call(const void* x, int32_t x_dtype, kvq_rows x_rows, int32_t d, const int32_t* kv_lens, float* amax_out,
              int32_t accumulate, bool per_head, void* stream) {
  int rc;
  if ((rc = check_float_input(x, x_dtype, "x")) != KVQ_OK) return rc;
  if ((rc = check_rows(x_rows, "x_rows")) != KVQ_OK) return rc;
  if (d <= 0) return fail(KVQ_ERR_ARG, "d must be > 0 (got %d)", d);
  if (amax_out == nullptr) return fail(KVQ_ERR_ARG, "amax_out is null");
  if (!aligned(amax_out, 4)) return fail(KVQ_ERR_ALIGN, "amax_out is not 4-byte aligned");
  if (per_head && x_rows.n1 > (1 << 16)) return fail(KVQ_ERR_ARG, "at most 65536 heads (got %lld)", (long long)x_rows.n1);
  return hip_status(kvq::launch_amax(x, x_dtype, kvq::to_rows(x_rows), d, kv_lens, amax_out, accumulate != 0, per_head,
                                     as_stream(stream)),
                    per_head ? "kvq_amax_heads launch" : "kvq_amax launch");
}
}  // namespace

int kvq_amax(const void* x, int32_t x_dtype, kvq_rows x_rows, int32_t d, const int32_t* kv_lens, float* amax_out,
             int32_t accumulate, void* stream) {
  return amax_call(x, x_dtype, x_rows, d, kv_lens, amax_out, accumulate, false, stream);
}

int kvq_amax_heads(const void* x, int32_t x_dtype, kvq_rows x_rows, int32_t d, const int32_t* kv_lens,
                   float* amax_out, int32_t accumulate, void* stream) {
  return amax_call(x, x_dtype, x_rows, d, kv_lens, amax_out, accumulate, true, stream);
}

int kvq_pack_nvfp4(const void* x, int32_t x_dtype, kvq_rows x_rows, int32_t d, const float* amax, uint8_t* codes,
                   uint8_t* scales, kvq_rows dst_rows, int32_t dst_layout, const int32_t* dst_pos,
                   float* tensor_scale_out, void* stream) {
  const kvq_pack_job j{x, x_dtype, x_rows, d, amax, codes, scales, dst_rows, dst_layout, dst_pos, tensor_scale_out, 0};
  return pack_batch(&j, 1, true, "kvq_pack_nvfp4", stream);
}

int kvq_pack_fp8(const void* x, int32_t x_dtype, kvq_rows x_rows, int32_t d, const float* amax, uint8_t* codes,
                 kvq_rows dst_rows, int32_t dst_layout, const int32_t* dst_pos, float* scale_out, void* stream) {
  const kvq_pack_job j{x, x_dtype, x_rows, d, amax, codes, nullptr, dst_rows, dst_layout, dst_pos, scale_out, 0};
  return pack_batch(&j, 1, false, "kvq_pack_fp8", stream);
}

int kvq_pack_fp8_heads(const void* x, int32_t x_dtype, kvq_rows x_rows, int32_t d, const float* amax, uint8_t* codes,
                       kvq_rows dst_rows, int32_t dst_layout, const int32_t* dst_pos, float* scale_out, void* stream) {
  const kvq_pack_job j{x, x_dtype, x_rows, d, amax, codes, nullptr, dst_rows, dst_layout, dst_pos, scale_out, 1};
  return pack_batch(&j, 1, false, "kvq_pack_fp8_heads", stream);
}

int kvq_pack_nvfp4_batch(const kvq_pack_job* jobs, int32_t n_jobs, void* stream) {
  return pack_batch(jobs, n_jobs, true, "kvq_pack_nvfp4_batch", stream);
}

int kvq_pack_fp8_batch(const kvq_pack_job* jobs, int32_t n_jobs, void* stream) {
  return pack_batch(jobs, n_jobs, false, "kvq_pack_fp8_batch", stream);
}

int kvq_unpack_nvfp4(const uint8_t* codes, const uint8_t* scales, kvq_rows src_rows, int32_t src_layout, int32_t d,
                     const float* tensor_scale, float* out, kvq_rows out_rows, void* stream) {
  int rc;
  if ((rc = check_rows(src_rows, "src_rows")) != KVQ_OK) return rc;
  if ((rc = check_rows(out_rows, "out_rows")) != KVQ_OK) return rc;
  if (d <= 0 || d % 16 != 0 || d > 1024) return fail(KVQ_ERR_ARG, "d must be a positive multiple of 16, <= 1024 (got %d)", d);
  if (codes == nullptr || scales == nullptr || tensor_scale == nullptr || out == nullptr)
    return fail(KVQ_ERR_ARG, "codes, scales, tensor_scale and out must be non-null");
  if (!same_extents(src_rows, out_rows)) return fail(KVQ_ERR_ARG, "out_rows extents differ from src_rows extents");
  if (!aligned(codes, 8) || !aligned(out, 4)) return fail(KVQ_ERR_ALIGN, "codes must be 8-byte, out 4-byte aligned");
  if ((rc = check_layout(src_layout, src_rows, "src_rows")) != KVQ_OK) return rc;
  if (n_rows(src_rows) == 0) return ok();
  return hip_status(kvq::launch_unpack_nvfp4(codes, scales, kvq::to_rows(src_rows), src_layout, d, tensor_scale, out,
                                             kvq::to_rows(out_rows), as_stream(stream)),
                    "kvq_unpack_nvfp4 launch");
}

int kvq_unpack_fp8(const uint8_t* codes, kvq_rows src_rows, int32_t src_layout, int32_t d, const float* scale,
                   float* out, kvq_rows out_rows, void* stream) {
  int rc;
  if ((rc = check_rows(src_rows, "src_rows")) != KVQ_OK) return rc;
  if ((rc = check_rows(out_rows, "out_rows")) != KVQ_OK) return rc;
  if (d <= 0 || d > 4096) return fail(KVQ_ERR_ARG, "d must be in [1, 4096] (got %d)", d);
  if (codes == nullptr || scale == nullptr || out == nullptr)
    return fail(KVQ_ERR_ARG, "codes, scale and out must be non-null");
  if (!same_extents(src_rows, out_rows)) return fail(KVQ_ERR_ARG, "out_rows extents differ from src_rows extents");
  if (!aligned(out, 4)) return fail(KVQ_ERR_ALIGN, "out must be 4-byte aligned");
  if ((rc = check_layout(src_layout, src_rows, "src_rows")) != KVQ_OK) return rc;
  if (src_layout == KVQ_PLANE_TOKEN4 && d % 4 != 0) return fail(KVQ_ERR_ARG, "TOKEN4 FP8 planes need d % 4 == 0");
  if (n_rows(src_rows) == 0) return ok();
  return hip_status(kvq::launch_unpack_fp8(codes, kvq::to_rows(src_rows), src_layout, d, scale, out, kvq::to_rows(out_rows),
                                           as_stream(stream)),
                    "kvq_unpack_fp8 launch");
}

// ------------------------------------------------------------ split planning
int kvq_auto_num_splits(int32_t num_cus, int32_t B, int32_t programs_per_req, int32_t max_kv_len, int32_t Dv,
                        int32_t Hq, int32_t* s_out) {
  if (s_out == nullptr) return fail(KVQ_ERR_ARG, "s_out is null");
  if (num_cus <= 0 || B <= 0 || programs_per_req <= 0 || Dv <= 0 || Hq <= 0 || max_kv_len < 0)
    return fail(KVQ_ERR_ARG, "kvq_auto_num_splits: non-positive argument");
  // 1) enough work-groups for every compute unit: one each where the query
  //    group has 4 or more heads (the GQA kernel then runs its grouped
  //    tiles, which keep two tiles of loads in flight per wave, and the MLA
  //    kernel's work-groups are 8 waves, two per SIMD; fewer partials make
  //    the combine cheaper), two each otherwise (the single-register-set
  //    tiles of query groups of 1 or 2 need a second work-group per CU to
  //    cover their load latency) as long as their chunks stay 1024 tokens or
  //    longer, else one.  Measured on MI355X: GQA 4:1 B=2 at 8K and 32K
  //    fastest at 16 splits; MHA B=1/2 at 32K at 2 work-groups per CU (2048-
  //    token chunks), MHA B=2 at 8K at one (2 per CU: 512-token chunks, 9 %
  //    slower).
  const int64_t base = static_cast<int64_t>(B) * programs_per_req;
  int64_t per_cu = static_cast<int64_t>(Hq) >= 4LL * programs_per_req ? 1 : 2;
  if (per_cu == 2) {
    const int64_t s2 = (2LL * num_cus + base - 1) / base;
    if (static_cast<int64_t>(max_kv_len) < 1024LL * s2) per_cu = 1;
  }
  int64_t s = (per_cu * num_cus + base - 1) / base;
  // 2) no split shorter than 256 tokens
  const int64_t by_len = (static_cast<int64_t>(max_kv_len) + 255) / 256;
  if (s > by_len) s = by_len;
  // 3) the partials (written and read once: 8 bytes per element) stay under
  //    a third of the packed KV bytes (about 9/8 * Dv bytes per token and
  //    program for NVFP4 K and V).  Only the wide-head single-program case
  //    (the MLA latent, 16 heads x 512 per request) comes near this bound;
  //    on MI355X its decode step measured fastest at two work-groups per
  //    compute unit, where the partials are about a third of the KV bytes.
  const double kv_bytes = static_cast<double>(base) * max_kv_len * (9.0 * Dv / 8.0);
  const double per_split = static_cast<double>(B) * Hq * (Dv + 1) * 8.0;
  const int64_t by_traffic = static_cast<int64_t>(kv_bytes / (3.0 * per_split));
  if (s > by_traffic) s = by_traffic;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  *s_out = static_cast<int32_t>(s);
  return ok();
}

int32_t attn_decode_tile_tokens(int32_t Hq, int32_t Hkv) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return 0;
  return kvq::gqa_tile_tokens(Hq / Hkv);
}

int kvq_device_cu_count(int32_t* num_cus_out) {
  if (num_cus_out == nullptr) return fail(KVQ_ERR_ARG, "num_cus_out is null");
  int dev = 0, n = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "kvq_device_cu_count: %s", hipGetErrorString(e));
  *num_cus_out = n;
  return ok();
}

size_t kvq_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Dv, int32_t s) {
  if (B <= 0 || Hq <= 0 || Dv <= 0 || s <= 0) return 0;
  // part_o [B][Hq][s][Dv] and part_lse [B][Hq][s], float32
  return static_cast<size_t>(B) * Hq * s * (static_cast<size_t>(Dv) + 1) * sizeof(float);
}

size_t kvq_fp8p_scratch_floats(int32_t B, int32_t Hq, int32_t s, int32_t max_kv_len) {
  if (B <= 0 || Hq <= 0 || s <= 0 || max_kv_len < 0) return 0;
  // the spilled scores: one row of roundup(max_kv_len, 4) floats per (request, head)
  return static_cast<size_t>(B) * Hq * ((static_cast<size_t>(max_kv_len) + 3) / 4 * 4);
}

}  // extern "C"

namespace {

// Validates decode arguments and resolves the split count.  need_partials:
// whether part_o / part_lse are written (false only for the fused path with
// s == 1).
int validate_decode(const kvq_decode_args* a, int32_t* s_out, bool fused) {
  if (a == nullptr) return fail(KVQ_ERR_ARG, "args is null");
  if (a->kv_format != KVQ_NVFP4 && a->kv_format != KVQ_FP8E4M3)
    return fail(KVQ_ERR_UNSUPPORTED, "kv_format %d not supported (NVFP4, FP8E4M3)", a->kv_format);
  if (a->layout != KVQ_LAYOUT_GQA && a->layout != KVQ_LAYOUT_MLA)
    return fail(KVQ_ERR_ARG, "layout %d unknown", a->layout);
  if (a->B <= 0 || a->Hq <= 0 || a->Hkv <= 0) return fail(KVQ_ERR_ARG, "B, Hq and Hkv must be positive");
  if (a->B > 65535 || a->Hkv > 65535) return fail(KVQ_ERR_ARG, "B and Hkv must be <= 65535");
  if (a->Hq % a->Hkv != 0) return fail(KVQ_ERR_ARG, "Hq (%d) must be a multiple of Hkv (%d)", a->Hq, a->Hkv);
  if (a->max_kv_len < 0) return fail(KVQ_ERR_ARG, "max_kv_len must be >= 0");
  if (a->q == nullptr || a->k_codes == nullptr || a->k_scale == nullptr || a->kv_lens == nullptr)
    return fail(KVQ_ERR_ARG, "q, k_codes, k_scale and kv_lens must be non-null");
  if (a->kv_format == KVQ_NVFP4 && a->k_scales == nullptr) return fail(KVQ_ERR_ARG, "NVFP4 needs k_scales");
  if (a->kv_scale_per_head != 0 &&
      (a->kv_scale_per_head != 1 || a->kv_format != KVQ_FP8E4M3 || a->layout != KVQ_LAYOUT_GQA))
    return fail(KVQ_ERR_UNSUPPORTED, "kv_scale_per_head must be 0 or 1, and 1 only for FP8 with the GQA layout");
  if (a->q_dtype == KVQ_FP8E4M3) {   // FP8 query codes with their scale
    if (a->layout != KVQ_LAYOUT_GQA) return fail(KVQ_ERR_UNSUPPORTED, "FP8 queries are decoded for the GQA layout only");
    if (a->q_scale == nullptr) return fail(KVQ_ERR_ARG, "an FP8 query needs q_scale");
    if (a->q_scale_per_head != 0 && a->q_scale_per_head != 1) return fail(KVQ_ERR_ARG, "q_scale_per_head must be 0 or 1");
    if (!aligned(a->q_scale, 4)) return fail(KVQ_ERR_ALIGN, "q_scale must be 4-byte aligned");
    if (!aligned(a->q, 8) || a->q_sb % 8 != 0 || a->q_sh % 8 != 0)
      return fail(KVQ_ERR_ALIGN, "FP8 query rows must be 8-byte aligned (q, q_sb, q_sh)");
  } else if (a->q_dtype == KVQ_NVFP4) {   // NVFP4 latent query (MLA)
    if (a->layout != KVQ_LAYOUT_MLA) return fail(KVQ_ERR_UNSUPPORTED, "NVFP4 queries are decoded for the MLA layout only");
    if (a->q_block_scales == nullptr || a->q_scale == nullptr)
      return fail(KVQ_ERR_ARG, "an NVFP4 query needs q_block_scales and q_scale");
    if (!aligned(a->q, 16) || !aligned(a->q_block_scales, 4) || !aligned(a->q_scale, 4))
      return fail(KVQ_ERR_ALIGN, "NVFP4 query codes must be 16-byte, its scales 4-byte aligned");
    if (a->q_sb < 0 || a->q_sh < 0) return fail(KVQ_ERR_ARG, "query row strides must be >= 0");
  } else if (a->q_dtype != KVQ_BF16 && a->q_dtype != KVQ_F32) {
    return fail(KVQ_ERR_UNSUPPORTED, "q_dtype must be BF16, F32, (GQA) FP8E4M3 or (MLA) NVFP4");
  }
  if (!(a->softmax_scale > 0.0f) || a->softmax_scale != a->softmax_scale || a->softmax_scale > 3.0e38f)
    return fail(KVQ_ERR_ARG, "softmax_scale must be a positive finite number");
  if (!aligned(a->k_codes, 16)) return fail(KVQ_ERR_ALIGN, "k_codes must be 16-byte aligned");
  if (a->k_scales != nullptr && !aligned(a->k_scales, 4)) return fail(KVQ_ERR_ALIGN, "k_scales must be 4-byte aligned");
  if (a->q_dtype == KVQ_F32 || a->q_dtype == KVQ_BF16) {
    // query rows are read with 16-byte loads: the base 16-byte aligned and
    // the strides whole 16-byte units (8 bf16 or 4 fp32 elements)
    const int64_t unit = a->q_dtype == KVQ_F32 ? 4 : 8;
    if (!aligned(a->q, 16) || a->q_sb % unit != 0 || a->q_sh % unit != 0)
      return fail(KVQ_ERR_ALIGN, "q must be 16-byte aligned with q_sb and q_sh multiples of %d elements",
                  static_cast<int>(unit));
  }
  if (a->kv_st < 0 || a->kv_sb < 0 || a->kv_sh < 0) return fail(KVQ_ERR_ARG, "cache strides must be >= 0");
  // token offsets inside one (request, kv head) are computed in 32 bits
  const int64_t row_bytes = a->kv_format == KVQ_NVFP4 ? a->D / 2 : a->D;
  if (static_cast<int64_t>(a->max_kv_len) * a->kv_st * row_bytes >= (int64_t(1) << 31))
    return fail(KVQ_ERR_ARG, "max_kv_len * kv_st * row bytes must stay below 2^31");

  int32_t s = a->num_splits;
  if (s <= 0) {
    int32_t cus = 0;
    int rc = kvq_device_cu_count(&cus);
    if (rc != KVQ_OK) return rc;
    const int ppr = a->layout == KVQ_LAYOUT_MLA ? 1 : a->Hkv;
    rc = kvq_auto_num_splits(cus, a->B, ppr, a->max_kv_len, a->Dv, a->Hq, &s);
    if (rc != KVQ_OK) return rc;
  }
  if (s > 64) return fail(KVQ_ERR_ARG, "num_splits %d exceeds 64", s);
  // fused append of the new token: one more partial per head
  const bool append = a->new_k != nullptr || a->new_v != nullptr;
  if (append) {
    if (a->new_k == nullptr || a->new_v == nullptr) return fail(KVQ_ERR_ARG, "new_k and new_v must both be given");
    if (a->layout != KVQ_LAYOUT_GQA) return fail(KVQ_ERR_UNSUPPORTED, "the fused append is implemented for the GQA layout only");
    if (a->quantize_p) return fail(KVQ_ERR_UNSUPPORTED, "the fused append decodes with exact probabilities only");
    if (a->q_dtype != KVQ_BF16) return fail(KVQ_ERR_UNSUPPORTED, "the fused append is implemented for bf16 queries");
    if (a->new_dtype != KVQ_BF16 && a->new_dtype != KVQ_F16 && a->new_dtype != KVQ_F32)
      return fail(KVQ_ERR_UNSUPPORTED, "new_dtype must be BF16, F16 or F32");
    if (!aligned(a->new_k, a->new_dtype == KVQ_F32 ? 4 : 2) || !aligned(a->new_v, a->new_dtype == KVQ_F32 ? 4 : 2))
      return fail(KVQ_ERR_ALIGN, "new_k / new_v misaligned");
    if (a->D > 128) return fail(KVQ_ERR_UNSUPPORTED, "the fused append supports D <= 128");
    if (s == 64) {
      if (a->num_splits > 0) return fail(KVQ_ERR_ARG, "with a fused append num_splits must be <= 63");
      s = 63;
    }
    if (a->B + (a->B + s - 1) / s > 65535) return fail(KVQ_ERR_ARG, "B too large for the fused append's grid");
  }
  const int np = s + (append ? 1 : 0);   // partials per head
  // the FP8-probability passes and the MLA kernel always go through the
  // partials (the latter followed by the combine launch)
  const bool need_partials = a->quantize_p || a->layout == KVQ_LAYOUT_MLA || !(fused && np == 1);
  if (need_partials) {
    if (a->part_o == nullptr || a->part_lse == nullptr) return fail(KVQ_ERR_ARG, "part_o and part_lse must be non-null");
    if (!aligned(a->part_o, 4) || !aligned(a->part_lse, 4)) return fail(KVQ_ERR_ALIGN, "partials must be 4-byte aligned");
    if (np > a->part_capacity)
      return fail(KVQ_ERR_WORKSPACE, "%d partials per head exceed part_capacity %d", np, a->part_capacity);
  }
  if (a->quantize_p) {
    if (a->layout != KVQ_LAYOUT_GQA) return fail(KVQ_ERR_UNSUPPORTED, "quantize_p is implemented for the GQA layout only");
    if (!(a->prob_scale > 0.0f) || a->prob_scale > 3.0e38f)
      return fail(KVQ_ERR_ARG, "prob_scale must be a positive finite number");
    if (a->p_scratch == nullptr) return fail(KVQ_ERR_ARG, "quantize_p needs p_scratch (kvq_fp8p_scratch_floats)");
    if (!aligned(a->p_scratch, 16)) return fail(KVQ_ERR_ALIGN, "p_scratch must be 16-byte aligned");
  }
  if (a->layout == KVQ_LAYOUT_GQA) {
    if (a->v_codes == nullptr || a->v_scale == nullptr) return fail(KVQ_ERR_ARG, "GQA needs v_codes and v_scale");
    if (a->kv_format == KVQ_NVFP4 && a->v_scales == nullptr) return fail(KVQ_ERR_ARG, "NVFP4 needs v_scales");
    if (!aligned(a->v_codes, 16)) return fail(KVQ_ERR_ALIGN, "v_codes must be 16-byte aligned");
    if (a->v_scales != nullptr && !aligned(a->v_scales, 4)) return fail(KVQ_ERR_ALIGN, "v_scales must be 4-byte aligned");
    if (a->Dv != a->D) return fail(KVQ_ERR_ARG, "GQA layout needs Dv == D");
    if (a->v_layout != KVQ_PLANE_ROWS && a->v_layout != KVQ_PLANE_TOKEN4)
      return fail(KVQ_ERR_ARG, "v_layout %d unknown", a->v_layout);
    if (a->v_layout == KVQ_PLANE_TOKEN4) {
      if (a->D != 128) return fail(KVQ_ERR_UNSUPPORTED, "TOKEN4 V planes are decoded for D == 128 only");
      if (a->kv_st != 1 || a->kv_sb % 4 != 0 || a->kv_sh % 4 != 0)
        return fail(KVQ_ERR_ALIGN, "TOKEN4 V planes need kv_st == 1 and kv_sb, kv_sh multiples of 4");
    }
    const int G = a->Hq / a->Hkv;
    if (const char* why = kvq::gqa_unsupported(*a))
      return fail(KVQ_ERR_UNSUPPORTED, "GQA decode (G=%d, D=%d): %s", G, a->D, why);
    if (a->block_table != nullptr) {   // paged cache
      const int tile = kvq::gqa_tile_tokens(G);
      if (a->block_size <= 0 || a->block_size % tile != 0 || (a->block_size & (a->block_size - 1)) != 0)
        return fail(KVQ_ERR_ARG, "block_size must be a power of two and a multiple of the decode tile (%d tokens for G=%d)",
                    tile, G);
      const int64_t need = (static_cast<int64_t>(a->max_kv_len) + a->block_size - 1) / a->block_size;
      if (a->bt_stride < need) return fail(KVQ_ERR_ARG, "bt_stride must cover ceil(max_kv_len / block_size) blocks");
      if (a->kv_sblk < 0) return fail(KVQ_ERR_ARG, "kv_sblk must be >= 0");
      if (!aligned(a->block_table, 4)) return fail(KVQ_ERR_ALIGN, "block_table must be 4-byte aligned");
      if (a->v_layout == KVQ_PLANE_TOKEN4 && (a->kv_sblk % 4 != 0 || a->block_size % 4 != 0))
        return fail(KVQ_ERR_ALIGN, "TOKEN4 V planes need kv_sblk and block_size multiples of 4");
      int64_t chunk = (static_cast<int64_t>(a->max_kv_len) + s - 1) / s;
      chunk = (chunk + tile - 1) / tile * tile;
      if (chunk / a->block_size + 2 > kvq::kPagedMaxChunkBlocks)
        return fail(KVQ_ERR_ARG, "a split spans more than %d blocks: use more splits or larger blocks",
                    kvq::kPagedMaxChunkBlocks - 2);
    }
  } else {
    if (a->kv_format != KVQ_NVFP4) return fail(KVQ_ERR_UNSUPPORTED, "MLA layout supports NVFP4 only");
    if (a->block_table != nullptr) {   // paged latent cache
      const int tile = kvq::mla_tile_tokens();
      if (a->block_size <= 0 || a->block_size % tile != 0 || (a->block_size & (a->block_size - 1)) != 0)
        return fail(KVQ_ERR_ARG, "block_size must be a power of two and a multiple of the MLA decode tile (%d tokens)",
                    tile);
      const int64_t need = (static_cast<int64_t>(a->max_kv_len) + a->block_size - 1) / a->block_size;
      if (a->bt_stride < need) return fail(KVQ_ERR_ARG, "bt_stride must cover ceil(max_kv_len / block_size) blocks");
      if (a->kv_sblk < 0) return fail(KVQ_ERR_ARG, "kv_sblk must be >= 0");
      if (!aligned(a->block_table, 4)) return fail(KVQ_ERR_ALIGN, "block_table must be 4-byte aligned");
      int64_t chunk = (static_cast<int64_t>(a->max_kv_len) + s - 1) / s;
      chunk = (chunk + tile - 1) / tile * tile;
      if (chunk / a->block_size + 2 > kvq::kMlaPagedMaxChunkBlocks)
        return fail(KVQ_ERR_ARG, "a split spans more than %d blocks: use more splits or larger blocks",
                    kvq::kMlaPagedMaxChunkBlocks - 2);
    }
    if (a->Hkv != 1) return fail(KVQ_ERR_ARG, "MLA layout needs Hkv == 1");
    if (a->k_scales == nullptr || a->q_rope == nullptr || a->k_rope == nullptr)
      return fail(KVQ_ERR_ARG, "MLA needs k_scales, q_rope and k_rope");
    if (!kvq::mla_supported(*a))
      return fail(KVQ_ERR_UNSUPPORTED,
                  "MLA decode: implemented for Hq = 16, D = Dv = 512, Drope = 64, bf16 or NVFP4 latent queries (got "
                  "Hq=%d D=%d Dv=%d Drope=%d)", a->Hq, a->D, a->Dv, a->Drope);
    if (!aligned(a->q, 16) || (a->q_dtype == KVQ_BF16 && (a->q_sh % 8 != 0 || a->q_sb % 8 != 0)) ||
        !aligned(a->q_rope, 16) || a->qr_sh % 8 != 0 || a->qr_sb % 8 != 0)
      return fail(KVQ_ERR_ALIGN, "MLA queries must be 16-byte aligned with strides multiple of 8 elements");
    if (!aligned(a->k_scales, 8) || !aligned(a->k_rope, 16))
      return fail(KVQ_ERR_ALIGN, "MLA k_scales must be 8-byte and k_rope 16-byte aligned");
    if (a->kv_st < 1) return fail(KVQ_ERR_ARG, "MLA cache token stride must be >= 1");
  }
  *s_out = s;
  return KVQ_OK;
}

int check_out(void* out, int32_t out_dtype, const float* out_scale) {
  if (out == nullptr) return fail(KVQ_ERR_ARG, "out must be non-null");
  if (out_dtype != KVQ_F32 && out_dtype != KVQ_BF16 && out_dtype != KVQ_FP8E4M3)
    return fail(KVQ_ERR_UNSUPPORTED, "out_dtype %d not supported (F32, BF16, FP8E4M3)", out_dtype);
  if (out_dtype == KVQ_FP8E4M3 && out_scale == nullptr) return fail(KVQ_ERR_ARG, "FP8 output needs out_scale");
  if (!aligned(out, out_dtype == KVQ_F32 ? 4 : (out_dtype == KVQ_BF16 ? 2 : 1)))
    return fail(KVQ_ERR_ALIGN, "out misaligned");
  return KVQ_OK;
}

}  // namespace

extern "C" {

int attn_decode_splitkv(const kvq_decode_args* a, int32_t* splits_used, void* stream) {
  int32_t s = 0;
  int rc = validate_decode(a, &s, false);
  if (rc != KVQ_OK) return rc;
  if (splits_used) *splits_used = s + (a->new_k != nullptr ? 1 : 0);   // partials written per head
  kvq::DecodePlan plan{s, 0};
  if (a->layout == KVQ_LAYOUT_MLA)
    return hip_status(kvq::launch_decode_mla(*a, plan, as_stream(stream)), "attn_decode_splitkv launch");
  if (a->quantize_p)
    return hip_status(kvq::launch_decode_fp8p(*a, plan, as_stream(stream)), "attn_decode_splitkv launch");
  return hip_status(kvq::launch_decode_gqa(*a, plan, as_stream(stream)), "attn_decode_splitkv launch");
}

int attn_decode(const kvq_decode_args* a, void* out, int32_t out_dtype, const float* out_scale, float* lse_out,
                int32_t* counters, int32_t* splits_used, void* stream) {
  int32_t s = 0;
  int rc = validate_decode(a, &s, true);
  if (rc != KVQ_OK) return rc;
  if ((rc = check_out(out, out_dtype, out_scale)) != KVQ_OK) return rc;
  if (a->layout == KVQ_LAYOUT_MLA || a->quantize_p) {
    // MLA and FP8 probabilities: split kernel(s) + combine kernel on the stream
    if (a->part_o == nullptr || a->part_lse == nullptr) return fail(KVQ_ERR_ARG, "part_o and part_lse must be non-null");
    if (splits_used) *splits_used = s;
    kvq::DecodePlan plan{s, 0};
    hipError_t e = a->quantize_p ? kvq::launch_decode_fp8p(*a, plan, as_stream(stream))
                                 : kvq::launch_decode_mla(*a, plan, as_stream(stream));
    if (e == hipSuccess)
      e = kvq::launch_combine(a->part_o, a->part_lse, a->B, a->Hq, a->Dv, s, out, out_dtype, out_scale, lse_out,
                              as_stream(stream));
    return hip_status(e, "attn_decode launch");
  }
  const int np = s + (a->new_k != nullptr ? 1 : 0);
  if (np > 1 && counters == nullptr) return fail(KVQ_ERR_ARG, "counters must be non-null when more than one partial is merged");
  if (splits_used) *splits_used = np;
  kvq::DecodePlan plan{s, 0};
  return hip_status(kvq::launch_decode_gqa_fused(*a, plan, out, out_dtype, out_scale, lse_out, counters,
                                                 as_stream(stream)),
                    "attn_decode launch");
}

int attn_decode_combine(const float* part_o, const float* part_lse, int32_t B, int32_t Hq, int32_t Dv,
                        int32_t num_splits, void* out, int32_t out_dtype, const float* out_scale, float* lse_out,
                        void* stream) {
  if (part_o == nullptr || part_lse == nullptr || out == nullptr)
    return fail(KVQ_ERR_ARG, "part_o, part_lse and out must be non-null");
  if (B <= 0 || Hq <= 0 || Dv <= 0) return fail(KVQ_ERR_ARG, "B, Hq and Dv must be positive");
  if (num_splits <= 0 || num_splits > 64) return fail(KVQ_ERR_ARG, "num_splits must be in [1, 64] (got %d)", num_splits);
  int rc = check_out(out, out_dtype, out_scale);
  if (rc != KVQ_OK) return rc;
  return hip_status(kvq::launch_combine(part_o, part_lse, B, Hq, Dv, num_splits, out, out_dtype, out_scale, lse_out,
                                        as_stream(stream)),
                    "attn_decode_combine launch");
}

size_t kvq_prefill_args_size(void) { return sizeof(kvq_prefill_args); }

int attn_prefill(const kvq_prefill_args* a, void* stream) {
  if (a == nullptr) return fail(KVQ_ERR_ARG, "args is null");
  if (a->kv_format != KVQ_NVFP4 && a->kv_format != KVQ_FP8E4M3)
    return fail(KVQ_ERR_UNSUPPORTED, "kv_format %d not supported (NVFP4, FP8E4M3)", a->kv_format);
  if (a->B <= 0 || a->Hq <= 0 || a->Hkv <= 0) return fail(KVQ_ERR_ARG, "B, Hq and Hkv must be positive");
  if (a->B > 65535 || a->Hkv > 65535) return fail(KVQ_ERR_ARG, "B and Hkv must be <= 65535");
  if (a->Hq % a->Hkv != 0) return fail(KVQ_ERR_ARG, "Hq (%d) must be a multiple of Hkv (%d)", a->Hq, a->Hkv);
  const int G = a->Hq / a->Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(KVQ_ERR_UNSUPPORTED, "query groups of %d heads are not implemented (1, 2, 4, 8)", G);
  if (a->D != 128) return fail(KVQ_ERR_UNSUPPORTED, "head_dim %d not implemented (128)", a->D);
  if (a->Sq < 0 || a->Sq > (1 << 24)) return fail(KVQ_ERR_ARG, "Sq must be in [0, 2^24]");
  if (a->max_kv_len < 0) return fail(KVQ_ERR_ARG, "max_kv_len must be >= 0");
  if (a->k_codes == nullptr || a->v_codes == nullptr || a->k_scale == nullptr || a->v_scale == nullptr ||
      a->kv_lens == nullptr || (a->Sq > 0 && (a->q == nullptr || a->out == nullptr)))
    return fail(KVQ_ERR_ARG, "q, k_codes, v_codes, k_scale, v_scale, kv_lens and out must be non-null");
  if (a->kv_format == KVQ_NVFP4 && (a->k_scales == nullptr || a->v_scales == nullptr))
    return fail(KVQ_ERR_ARG, "NVFP4 needs k_scales and v_scales");
  if (a->q_dtype != KVQ_BF16 && a->q_dtype != KVQ_FP8E4M3)
    return fail(KVQ_ERR_UNSUPPORTED, "q_dtype must be BF16 or FP8E4M3");
  const bool q8 = a->q_dtype == KVQ_FP8E4M3;
  if (q8 && a->q_scale == nullptr) return fail(KVQ_ERR_ARG, "FP8 queries need q_scale");
  if (q8 && a->q_scale_per_head != 0 && a->q_scale_per_head != 1)
    return fail(KVQ_ERR_ARG, "q_scale_per_head must be 0 or 1");
  if (a->v_layout != KVQ_PLANE_TOKEN4) return fail(KVQ_ERR_UNSUPPORTED, "V planes must be in the TOKEN4 layout");
  if (a->kv_scale_per_head != 0 && (a->kv_scale_per_head != 1 || a->kv_format != KVQ_FP8E4M3))
    return fail(KVQ_ERR_UNSUPPORTED, "kv_scale_per_head must be 0 or 1, and 1 only for FP8");
  if (!(a->softmax_scale > 0.0f) || a->softmax_scale != a->softmax_scale || a->softmax_scale > 3.0e38f)
    return fail(KVQ_ERR_ARG, "softmax_scale must be a positive finite number");
  if (a->out_dtype != KVQ_F32 && a->out_dtype != KVQ_BF16)
    return fail(KVQ_ERR_UNSUPPORTED, "out_dtype must be F32 or BF16");
  if (!aligned(a->q, q8 ? 8 : 16) || a->q_sb % 8 != 0 || a->q_st % 8 != 0 || a->q_sh % 8 != 0)
    return fail(KVQ_ERR_ALIGN, "q must be %d-byte aligned with q_sb, q_st and q_sh multiples of 8 elements",
                q8 ? 8 : 16);
  if (q8 && !aligned(a->q_scale, 4)) return fail(KVQ_ERR_ALIGN, "q_scale must be 4-byte aligned");
  if (!aligned(a->k_codes, 16) || !aligned(a->v_codes, 16))
    return fail(KVQ_ERR_ALIGN, "k_codes and v_codes must be 16-byte aligned");
  if ((a->k_scales != nullptr && !aligned(a->k_scales, 4)) || (a->v_scales != nullptr && !aligned(a->v_scales, 4)))
    return fail(KVQ_ERR_ALIGN, "k_scales and v_scales must be 4-byte aligned");
  if (!aligned(a->k_scale, 4) || !aligned(a->v_scale, 4) || !aligned(a->kv_lens, 4))
    return fail(KVQ_ERR_ALIGN, "k_scale, v_scale and kv_lens must be 4-byte aligned");
  if (!aligned(a->out, a->out_dtype == KVQ_F32 ? 16 : 8) || a->o_sb % 4 != 0 || a->o_st % 4 != 0 || a->o_sh % 4 != 0)
    return fail(KVQ_ERR_ALIGN, "out must be %d-byte aligned with o_sb, o_st and o_sh multiples of 4 elements",
                a->out_dtype == KVQ_F32 ? 16 : 8);
  if (a->lse_out != nullptr && !aligned(a->lse_out, 4)) return fail(KVQ_ERR_ALIGN, "lse_out must be 4-byte aligned");
  if (a->kv_sb < 0 || a->kv_sh < 0) return fail(KVQ_ERR_ARG, "cache strides must be >= 0");
  if (a->kv_sh % 4 != 0 || (a->block_table == nullptr && a->kv_sb % 4 != 0))
    return fail(KVQ_ERR_ALIGN, "TOKEN4 V planes need kv_sb and kv_sh multiples of 4");
  int log2_bs = 0;
  if (a->block_table != nullptr) {
    if (a->block_size < 64 || (a->block_size & (a->block_size - 1)) != 0)
      return fail(KVQ_ERR_ARG, "block_size must be a power of two >= 64 (the prefill tile)");
    const int64_t need = (static_cast<int64_t>(a->max_kv_len) + a->block_size - 1) / a->block_size;
    if (a->bt_stride < need) return fail(KVQ_ERR_ARG, "bt_stride must cover ceil(max_kv_len / block_size) blocks");
    if (a->kv_sblk < 0) return fail(KVQ_ERR_ARG, "kv_sblk must be >= 0");
    if (a->kv_sblk % 4 != 0) return fail(KVQ_ERR_ALIGN, "TOKEN4 V planes need kv_sblk to be a multiple of 4");
    while ((1 << log2_bs) < a->block_size) ++log2_bs;
  }
  if (a->Sq == 0) return ok();

  kvq::PrefillParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.q_dtype = a->q_dtype; p.q_scale = a->q_scale; p.q_scale_per_head = q8 ? a->q_scale_per_head : 0;
  p.q_sb = a->q_sb; p.q_st = a->q_st; p.q_sh = a->q_sh;
  p.k_codes = a->k_codes; p.k_scales = a->k_scales; p.v_codes = a->v_codes; p.v_scales = a->v_scales;
  p.k_scale = a->k_scale; p.v_scale = a->v_scale; p.per_head = a->kv_scale_per_head;
  p.kv_lens = a->kv_lens; p.max_kv_len = a->max_kv_len;
  p.kv_sb = a->kv_sb; p.kv_sh = a->kv_sh;
  p.block_table = a->block_table; p.log2_bs = log2_bs; p.bt_stride = a->bt_stride; p.kv_sblk = a->kv_sblk;
  p.B = a->B; p.Hq = a->Hq; p.Hkv = a->Hkv; p.Sq = a->Sq;
  p.softmax_scale = a->softmax_scale;
  p.out = a->out; p.out_dtype = a->out_dtype;
  p.o_sb = a->o_sb; p.o_st = a->o_st; p.o_sh = a->o_sh;
  p.lse = a->lse_out;
  return hip_status(kvq::launch_prefill_gqa(p, a->kv_format, G, as_stream(stream)), "attn_prefill launch");
}

}  // extern "C"

// ------------------------------------------------------------ no-allocation entry
// For callers that cannot allocate or pass a workspace: the partials and the
// merge counters of attn_decode live in a static device array of this file,
// one copy per GPU (each device gets its own instance of the code object's
// globals), looked up once per device with hipGetSymbolAddress.  Layout:
// [0, 64 KiB) counters of the fused merge (zero at load, cleared once more by
// a kernel at the first call on a device, and left zero by every completed
// call), then part_o and part_lse.
namespace {

constexpr size_t kScratchBytes = KVQ_NOALLOC_SCRATCH_BYTES;
constexpr size_t kCounterBytes = 64 * 1024;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void k_zero_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the device address of this GPU's scratch array (set up on first use)
int scratch_of_current_device(void** out, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "attn_decode_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_ERR_UNSUPPORTED, "attn_decode_noalloc: device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(KVQ_ERR_HIP, "attn_decode_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    constexpr int n = static_cast<int>(kCounterBytes / 4);
    hipLaunchKernelGGL(k_zero_words, dim3((n + 255) / 256), dim3(256), 0, st, static_cast<uint32_t*>(ptr), n);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "attn_decode_noalloc: counter clear: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KVQ_OK;
}

}  // namespace

extern "C" int attn_decode_noalloc(const kvq_decode_args* args, void* out, int32_t out_dtype, const float* out_scale,
                                   float* lse_out, int32_t* splits_used, void* stream) {
  if (args == nullptr) return fail(KVQ_ERR_ARG, "args is null");
  if (args->quantize_p)
    return fail(KVQ_ERR_UNSUPPORTED,
                "attn_decode_noalloc: FP8 probabilities need a score scratch of B*Hq*max_kv_len floats; use attn_decode");
  void* base = nullptr;
  int rc = scratch_of_current_device(&base, as_stream(stream));
  if (rc != KVQ_OK) return rc;
  uint8_t* const part_base = static_cast<uint8_t*>(base) + kCounterBytes;
  kvq_decode_args a = *args;
  a.part_o = reinterpret_cast<float*>(part_base);   // provisional, to resolve the split count
  a.part_lse = a.part_o;
  a.part_capacity = 64;
  a.p_scratch = nullptr;
  int32_t s = 0;
  if ((rc = validate_decode(&a, &s, true)) != KVQ_OK) return rc;
  const size_t np = static_cast<size_t>(s) + (a.new_k != nullptr ? 1 : 0);
  const size_t n_o = static_cast<size_t>(a.B) * a.Hq * np * a.Dv;
  const size_t lse_off = (n_o * sizeof(float) + 255) / 256 * 256;
  const size_t need = lse_off + static_cast<size_t>(a.B) * a.Hq * np * sizeof(float);
  if (need > kScratchBytes - kCounterBytes)
    return fail(KVQ_ERR_WORKSPACE,
                "attn_decode_noalloc: %zu partials per head need %zu bytes, the scratch holds %zu; use fewer splits or "
                "attn_decode with a workspace", np, need, kScratchBytes - kCounterBytes);
  if (static_cast<size_t>(a.B) * a.Hkv * sizeof(int32_t) > kCounterBytes)
    return fail(KVQ_ERR_WORKSPACE, "attn_decode_noalloc: B * Hkv must be <= %zu", kCounterBytes / sizeof(int32_t));
  a.part_o = reinterpret_cast<float*>(part_base);
  a.part_lse = reinterpret_cast<float*>(part_base + lse_off);
  a.part_capacity = static_cast<int32_t>(np);
  return attn_decode(&a, out, out_dtype, out_scale, lse_out, static_cast<int32_t*>(base), splits_used, stream);
}
