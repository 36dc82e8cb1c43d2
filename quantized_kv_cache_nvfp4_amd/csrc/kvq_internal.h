// Internal declarations shared by the C-ABI layer (api.cpp) and the HIP
// kernel files.  Not part of the public interface (that is include/kvq.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

struct Rows {
  int64_t n0, n1, n2;
  int64_t s0, s1, s2;
};

inline Rows to_rows(const kvq_rows& r) { return Rows{r.n0, r.n1, r.n2, r.s0, r.s1, r.s2}; }

// One plane pack: source rows x (dt, xr, d) quantized with the calibrated
// amax into the destination plane (codes, NVFP4 scales, dr, layout) at
// rows + dst_pos[i0]; sout receives the tensor scale (or is null).
struct PackJob {
  const void* x;
  int dt;
  Rows xr;
  int d;
  const float* amax;
  uint8_t* codes;
  uint8_t* scales;
  Rows dr;
  int layout;
  const int32_t* dst_pos;
  float* sout;
  int per_head;   // FP8: amax / sout hold one value per i1
};
constexpr int kMaxPackJobs = KVQ_MAX_PACK_JOBS;
struct PackJobs {
  PackJob j[kMaxPackJobs];
  int n;
};

// ---- quantization kernels (quant_kernels.hip) ----
hipError_t launch_amax(const void* x, int x_dtype, Rows rows, int d, const int32_t* kv_lens, float* amax_out,
                       bool accumulate, bool per_head, hipStream_t st);
// every job of one call in one launch (blockIdx.y = job)
hipError_t launch_pack_nvfp4(const PackJobs& jobs, hipStream_t st);
hipError_t launch_pack_fp8(const PackJobs& jobs, hipStream_t st);
hipError_t launch_unpack_nvfp4(const uint8_t* codes, const uint8_t* scales, Rows sr, int layout, int d, const float* ts,
                               float* out, Rows orow, hipStream_t st);
hipError_t launch_unpack_fp8(const uint8_t* codes, Rows sr, int layout, int d, const float* scale, float* out, Rows orow,
                             hipStream_t st);

// ---- decode (decode_gqa.hip, decode_mla.hip, combine.hip) ----
struct DecodePlan {
  int s;           // number of splits
  int chunk;       // tokens per split (multiple of the kernel tile)
};

hipError_t launch_decode_gqa(const kvq_decode_args& a, const DecodePlan& p, hipStream_t st);
hipError_t launch_decode_gqa_fused(const kvq_decode_args& a, const DecodePlan& p, void* out, int out_dtype,
                                   const float* out_scale, float* lse_out, int* counters, hipStream_t st);
hipError_t launch_decode_mla(const kvq_decode_args& a, const DecodePlan& p, hipStream_t st);
hipError_t launch_decode_fp8p(const kvq_decode_args& a, const DecodePlan& p, hipStream_t st);
hipError_t launch_combine(const float* part_o, const float* part_lse, int B, int Hq, int Dv, int s, void* out,
                          int out_dtype, const float* out_scale, float* lse_out, hipStream_t st);

// tile (tokens) of the GQA kernel for a query-group width G and of the MLA kernel
int gqa_tile_tokens(int G);
int mla_tile_tokens();
constexpr int kPagedMaxChunkBlocks = 2048;   // block-table entries one work-group keeps (LDS)
constexpr int kMlaPagedMaxChunkBlocks = 512;  // the same for the MLA kernel (two work-groups per CU share the LDS)
// null if the GQA kernel implements this combination of format, query
// group, head_dim, query type, V layout, paging and fused append; otherwise
// the reason it does not
const char* gqa_unsupported(const kvq_decode_args& a);
// is the MLA configuration implemented (NVFP4 latent 512 + rope 64, 16 heads, bf16 queries)
bool mla_supported(const kvq_decode_args& a);


// ---- chunked prefill (prefill_gqa.hip) ----
// Kernel parameters, from a validated kvq_prefill_args (contiguous or paged
// planes, K rows, V TOKEN4, head_dim 128, bf16 queries).
struct PrefillParams {
  const uint16_t* q;              // bf16 elements, or (q_dtype FP8) E4M3 code bytes
  int q_dtype;
  const float* q_scale;           // FP8 queries: float[1] or float[Hq]
  int q_scale_per_head;
  int64_t q_sb, q_st, q_sh;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  const float* k_scale;
  const float* v_scale;
  int per_head;
  const int32_t* kv_lens;
  int max_kv_len;
  int64_t kv_sb, kv_sh;
  const int32_t* block_table;   // null: contiguous planes
  int log2_bs;
  int64_t bt_stride, kv_sblk;
  int B, Hq, Hkv, Sq;
  float softmax_scale;
  void* out;
  int out_dtype;
  int64_t o_sb, o_st, o_sh;
  float* lse;
};
hipError_t launch_prefill_gqa(const PrefillParams& p, int kv_format, int G, hipStream_t st);

}  // namespace kvq
