/*
 * kvq.h - quantized KV-cache attention decode for AMD MI355X (gfx950).
 *
 * A plain C ABI: pointers (host or device, as stated per argument), sizes,
 * and a HIP stream passed as `void*` (a hipStream_t; NULL = the default
 * stream).  No allocation happens inside the library: every buffer is owned
 * by the caller.  Work is enqueued on the given stream and the call returns
 * without synchronizing.  Arguments are validated before anything is
 * launched; a rejected call launches nothing and returns a nonzero status
 * with a message retrievable by kvq_last_error() (thread-local).  Faults in
 * device memory named by the caller surface at the caller's next
 * synchronization, not here.
 *
 * Method sources (cited by page title and section):
 *  - NVFP4 KV cache: Model-Optimizer PR #714 "KV cache quantization for
 *    MLAAttention in vLLM fakequant", Testing section (quantizer dump:
 *    E2M1 "(2, 1) bit" elements, blocks of 16 along the last dim, dynamic
 *    E4M3 "scale_bits (4, 3)" block scales, per-tensor amax from a
 *    MaxCalibrator; only the latent kv_c quantizer of QuantMLAAttention is
 *    enabled, the query quantizer is disabled).
 *  - FP8 KV cache: compressed-tensors PR #436 (llm-compressor attention /
 *    KV-cache quantization), kv_cache_scheme JSON: 8-bit float, tensor
 *    strategy, symmetric, min-max observer, static.
 *  - Split-KV decode and combine: Model-Optimizer PR #1832 "Add quant+sparse
 *    attention for vLLM serving", Testing section (split-KV description and
 *    the auto split count chosen from the compute-unit count and
 *    batch x heads).
 *  - FP8 probabilities and FP8 output: vLLM PR #15734 "[Quantization][FP8]
 *    Add support for FP8 models with input_scale for output projection and QK
 *    quantization", items 1 and 2.
 *  - A missing KV scale served as 1: Model-Optimizer PR #673 "Fix KV cache
 *    quantization bugs", comments.
 *
 * Numeric conventions (readings where the pages are silent):
 *  - NVFP4: s_t = fp32(amax / 2688) (1 if amax == 0); block scale
 *    s_hat = E4M3(bamax / (6 s_t)); code = E2M1(x / (s_hat s_t)).  Every
 *    rounding decision is the exact real-number one (round to nearest, ties
 *    to the even code, saturating, sign of zero kept); a block whose scale
 *    rounds to 0 stores scale byte 0 and code bytes 0.
 *  - FP8: scale = fp32(amax / 448) (1 if amax == 0); code = E4M3(x / scale),
 *    same rounding rules.  E4M3 is the FN variant (max 448, NaN = 0x7F/0xFF).
 *  - Packed NVFP4 rows: element 2j in the low nibble of byte j; scale byte k
 *    is the E4M3 bits of block k (elements 16k..16k+15).
 *  - GQA head mapping: query head h reads kv head h / (Hq / Hkv).
 *  - Partials: part_o[b][h][j][0..Dv) = normalized output of split j,
 *    part_lse[b][h][j] = natural-log log-sum-exp of the scaled scores of
 *    split j (-inf for an empty split).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define KVQ_OK 0
#define KVQ_ERR_ARG 1         /* null pointer, bad size, inconsistent shape   */
#define KVQ_ERR_UNSUPPORTED 2 /* valid but not implemented (dtype, D, G ...)  */
#define KVQ_ERR_ALIGN 3       /* a plane base or stride breaks the alignment  */
#define KVQ_ERR_WORKSPACE 4   /* workspace too small                          */
#define KVQ_ERR_HIP 5         /* a HIP runtime call or launch failed          */

/* ---- element types ------------------------------------------------------ */
#define KVQ_F32 0
#define KVQ_BF16 1
#define KVQ_F16 2
#define KVQ_FP8E4M3 3
#define KVQ_NVFP4 4

/* ---- packed plane layouts ----------------------------------------------- */
/*
 * KVQ_PLANE_ROWS: row r of a plane occupies bytes [r*R, (r+1)*R), R = the
 *   plane's row bytes.
 * KVQ_PLANE_TOKEN4: rows are taken in groups of four consecutive tokens
 *   (i2 = 4q .. 4q+3), which share the 4*R bytes starting at the address
 *   the group's first row has in KVQ_PLANE_ROWS.  Inside a group the
 *   elements are stored in order and, for each element, the codes of the
 *   four tokens in token order: NVFP4 element x of token 4q+j is nibble
 *   (j & 1) (low nibble first) of byte 2x + (j >> 1); FP8 element x of token
 *   4q+j is byte 4x + j; the NVFP4 scale of block b of token 4q+j is byte
 *   4b + j.  One byte then holds one element of two consecutive tokens, so
 *   the hardware FP4 -> f16 convert yields the token-contiguous pair a
 *   wave64 lane feeds to the P.V matrix multiply, and one 16-byte load gives
 *   a lane 8 elements of 4 tokens.  Requires the token stride s2 == 1 and s0,
 *   s1 and the plane length along i2 to be multiples of 4.
 */
#define KVQ_PLANE_ROWS 0
#define KVQ_PLANE_TOKEN4 1

/* ---- cache layouts ------------------------------------------------------ */
#define KVQ_LAYOUT_GQA 0 /* K and V planes per (request, kv head, token)      */
#define KVQ_LAYOUT_MLA 1 /* one latent plane per (request, token) + bf16 rope */

/*
 * Row addressing.  A tensor of rows of `d` contiguous elements is addressed
 * by three indices (i0, i1, i2) with extents n0, n1, n2: row (i0, i1, i2)
 * starts at base + i0*s0 + i1*s1 + i2*s2.  For unquantized tensors (x, out)
 * the strides count elements of the tensor's dtype; for packed planes they
 * count rows of the plane (a plane row is d/2 code bytes or d/16 scale
 * bytes for NVFP4, d bytes for FP8), so one kvq_rows describes the code and
 * the scale plane together.
 */
typedef struct {
  int64_t n0, n1, n2;
  int64_t s0, s1, s2;
} kvq_rows;

/* Message of the last failed call on this thread ("" if none). */
const char* kvq_last_error(void);

/* Library version as 10000*major + 100*minor + patch. */
int32_t kvq_version(void);

/* sizeof(kvq_decode_args) as compiled into the library (binding check). */
size_t kvq_decode_args_size(void);

/*
 * kvq_amax - per-tensor max |x| (max calibration; Model-Optimizer PR #714,
 * Testing section, MaxCalibrator; compressed-tensors PR #436 min-max
 * observer).
 *   x        device, dtype x_dtype (KVQ_F32 or KVQ_BF16), rows per x_rows.
 *   d        elements per row (> 0).
 *   kv_lens  device int32[n0] or NULL: rows with i2 >= kv_lens[i0] are
 *            skipped (padding of a ragged cache).
 *   amax_out device float[1].  If accumulate == 0 it is overwritten with the
 *            result; if accumulate != 0 the result is max-merged into the
 *            value already there (which must be >= 0).
 * The result is exact (an element of x).  NaN inputs are not supported.
 */
int kvq_amax(const void* x, int32_t x_dtype, kvq_rows x_rows, int32_t d, const int32_t* kv_lens,
             float* amax_out, int32_t accumulate, void* stream);

/*
 * kvq_amax_heads - one max |x| per kv head (the attn_head strategy:
 * compressed-tensors PR #436, Changes, "attn_head" in _flatten_attention;
 * Testing, strategy="attn_head" with the static_minmax observer): amax_out[h]
 * is the max over the rows with i1 == h (all i0, i2 < kv_lens[i0]).
 * Arguments as kvq_amax; amax_out is device float[x_rows.n1].
 */
int kvq_amax_heads(const void* x, int32_t x_dtype, kvq_rows x_rows, int32_t d, const int32_t* kv_lens,
                   float* amax_out, int32_t accumulate, void* stream);

/*
 * kvq_pack_nvfp4 - quantize rows to NVFP4 (Model-Optimizer PR #714, Testing
 * section quantizer dump).
 *   x            device, KVQ_F32 or KVQ_BF16, rows per x_rows, d elements each.
 *   d            multiple of 16, <= 1024.
 *   amax         device float[1]: the calibrated per-tensor amax (>= 0).
 *   codes        device uint8 plane, rows of d/2 bytes.
 *   scales       device uint8 plane, rows of d/16 bytes.
 *   dst_rows     the destination plane: n0, n1 equal to x_rows', n2 (the
 *                plane's length along i2) >= x_rows.n2; strides in plane rows.
 *   dst_layout   KVQ_PLANE_ROWS or KVQ_PLANE_TOKEN4 (both planes).
 *   dst_pos      device int32[n0] or NULL: row (i0, i1, i2) of x is stored at
 *                plane row (i0, i1, i2 + dst_pos[i0]) (append of new tokens);
 *                rows that would land outside [0, dst_rows.n2) are skipped.
 *   tensor_scale_out  device float[1] or NULL: receives s_t.
 * Deterministic and bit-exact with the exact-real definition above.
 */
int kvq_pack_nvfp4(const void* x, int32_t x_dtype, kvq_rows x_rows, int32_t d, const float* amax,
                   uint8_t* codes, uint8_t* scales, kvq_rows dst_rows, int32_t dst_layout,
                   const int32_t* dst_pos, float* tensor_scale_out, void* stream);

/*
 * kvq_pack_fp8 - quantize rows to per-tensor FP8 E4M3 (compressed-tensors
 * PR #436 kv_cache_scheme).  Arguments as kvq_pack_nvfp4; codes rows are d
 * bytes (d > 0, d % 4 == 0, <= 4096); scale_out (device float[1] or NULL)
 * receives the scale amax/448 (1 if amax == 0).
 */
int kvq_pack_fp8(const void* x, int32_t x_dtype, kvq_rows x_rows, int32_t d, const float* amax,
                 uint8_t* codes, kvq_rows dst_rows, int32_t dst_layout, const int32_t* dst_pos,
                 float* scale_out, void* stream);

/*
 * kvq_pack_fp8_heads - FP8 E4M3 with one scale per kv head (the attn_head
 * strategy, compressed-tensors PR #436): the rows with i1 == h are quantized
 * with scale_h = amax[h] / 448 (1 if amax[h] == 0), exactly as kvq_pack_fp8
 * quantizes a whole tensor.  Arguments as kvq_pack_fp8, except amax (device
 * float[x_rows.n1]) and scale_out (device float[x_rows.n1] or NULL).
 */
int kvq_pack_fp8_heads(const void* x, int32_t x_dtype, kvq_rows x_rows, int32_t d, const float* amax,
                       uint8_t* codes, kvq_rows dst_rows, int32_t dst_layout, const int32_t* dst_pos,
                       float* scale_out, void* stream);

/*
 * Batched packing: several planes (for instance the K and the V rows of the
 * new tokens of one decode step) quantized in ONE launch.  Each job carries
 * exactly the arguments of one kvq_pack_nvfp4 / kvq_pack_fp8 call (scales
 * is ignored for FP8; scale_out receives the tensor scale or is NULL) and is
 * validated as that call would be; the destinations of different jobs must
 * not overlap.  jobs is a host array of 1..KVQ_MAX_PACK_JOBS entries, read
 * before the call returns.  Errors: as the single-plane calls, plus
 * KVQ_ERR_ARG for n_jobs outside [1, KVQ_MAX_PACK_JOBS].
 */
#define KVQ_MAX_PACK_JOBS 8
typedef struct {
  const void* x;
  int32_t x_dtype;
  kvq_rows x_rows;
  int32_t d;
  const float* amax;
  uint8_t* codes;
  uint8_t* scales;
  kvq_rows dst_rows;
  int32_t dst_layout;
  const int32_t* dst_pos;
  float* scale_out;
  int32_t scale_per_head;   /* FP8 only: 1 = amax and scale_out hold one
                               value per i1 (kvq_pack_fp8_heads), 0 = one */
} kvq_pack_job;

int kvq_pack_nvfp4_batch(const kvq_pack_job* jobs, int32_t n_jobs, void* stream);
int kvq_pack_fp8_batch(const kvq_pack_job* jobs, int32_t n_jobs, void* stream);

/*
 * kvq_unpack_nvfp4 - dequantize NVFP4 rows to float32: out = fp32(E2M1(c) *
 * s_hat * s_t) (one rounding; e * s_hat is exact).  This is the fake-quant
 * value of Model-Optimizer PR #714, Testing section (the quantizer dump's
 * "fake" mode returns the dequantized tensor): the value the decode kernels
 * reconstruct in registers.  Test / inspection path.
 *   codes, scales  device planes per src_rows and src_layout (KVQ_PLANE_*);
 *                  tensor_scale device float[1];
 *   out            device float32 rows per out_rows (extents == src_rows').
 */
int kvq_unpack_nvfp4(const uint8_t* codes, const uint8_t* scales, kvq_rows src_rows, int32_t src_layout,
                     int32_t d, const float* tensor_scale, float* out, kvq_rows out_rows, void* stream);

/*
 * kvq_unpack_fp8 - out = fp32(E4M3(c) * scale): the dequantized value of the
 * per-tensor FP8 kv_cache_scheme (compressed-tensors PR #436, Changes;
 * symmetric, so no zero point).  Arguments and errors as kvq_unpack_nvfp4;
 * scale is device float[1].
 */
int kvq_unpack_fp8(const uint8_t* codes, kvq_rows src_rows, int32_t src_layout, int32_t d, const float* scale,
                   float* out, kvq_rows out_rows, void* stream);

/*
 * Decode arguments (one query token per request).
 *
 * GQA / MHA (layout KVQ_LAYOUT_GQA): q [B][Hq][D]; K and V planes indexed by
 * (request b, kv head, token t) with row strides kv_sb, kv_sh, kv_st (in
 * plane rows, shared by the code and scale planes of K and V); D == Dv;
 * Hq % Hkv == 0.
 *
 * MLA (layout KVQ_LAYOUT_MLA): q = absorbed latent query q_c [B][Hq][D]
 * (D = Dv = latent rank), q_rope = q_r [B][Hq][Drope] (bf16); k_codes /
 * k_scales = the NVFP4 latent plane c, used as keys and as values (v_* are
 * ignored); k_rope = bf16 rope keys [.. Drope] addressed with the same row
 * strides (in rows of Drope elements); Hkv must be 1; kv_sh is ignored.
 *
 * Scores are softmax_scale * (q . K_t) with K_t dequantized (and, for MLA,
 * + q_r . k_rope_t); tokens t >= min(kv_lens[b], max_kv_len) are masked.
 */
typedef struct {
  int32_t kv_format;   /* KVQ_NVFP4 or KVQ_FP8E4M3 (MLA: KVQ_NVFP4)       */
  int32_t layout;      /* KVQ_LAYOUT_GQA or KVQ_LAYOUT_MLA                 */
  int32_t B, Hq, Hkv;  /* batch, query heads, kv heads                     */
  int32_t D, Dv, Drope;
  int32_t max_kv_len;  /* upper bound on kv_lens and rows allocated per request */
  const void* q;       /* device, q_dtype, [B][Hq][D] with element strides: */
  int32_t q_dtype;     /* KVQ_BF16, KVQ_F32, or (GQA layout) KVQ_FP8E4M3:  */
  int64_t q_sb, q_sh;  /*   q + b*q_sb + h*q_sh                            */
  const void* q_rope;  /* MLA: device bf16 [B][Hq][Drope], element strides */
  int64_t qr_sb, qr_sh;
  const uint8_t* k_codes;   /* device plane (NVFP4: d/2 B rows; FP8: d B rows) */
  const uint8_t* k_scales;  /* device NVFP4 scale plane (d/16 B rows); NULL for FP8 */
  const float* k_scale;     /* device float[1]: s_t (NVFP4) or scale (FP8);
                               float[Hkv] with kv_scale_per_head            */
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  const float* v_scale;
  int32_t v_layout;         /* GQA: KVQ_PLANE_TOKEN4 at D = 128 (kv_st = 1,
                               kv_sb and kv_sh multiples of 4, the V planes
                               at least roundup(max_kv_len, 4) tokens
                               long), KVQ_PLANE_ROWS at D = 64; other
                               pairings: KVQ_ERR_UNSUPPORTED.  K planes are
                               always ROWS.  At D = 64 the planes are
                               contiguous (no block table), there is no
                               fused append and queries are bf16 or fp32;
                               fp32 queries need contiguous planes.       */
  const void* k_rope;       /* MLA: device bf16 rope-key rows              */
  int64_t kv_sb, kv_sh, kv_st;
  const int32_t* kv_lens;   /* device int32[B]                             */
  float softmax_scale;
  int32_t num_splits;       /* >= 1 explicit; <= 0: kvq_auto_num_splits    */
  int32_t quantize_p;       /* 1: FP8 probabilities (vLLM PR #15734 item 2) */
  float prob_scale;         /* P~ = E4M3(P / prob_scale) * prob_scale      */
  float* part_o;            /* device float32 [B][Hq][s][Dv] (split stride s) */
  float* part_lse;          /* device float32 [B][Hq][s]                   */
  int32_t part_capacity;    /* the partial buffers hold at least this many
                               splits; s must not exceed it                */
  float* p_scratch;         /* quantize_p only: device float32 buffer of
                               kvq_fp8p_scratch_floats(...) floats; else NULL */
  int32_t kv_scale_per_head;  /* FP8, GQA layout: 1 = k_scale and v_scale are
                               device float[Hkv], kv head h dequantized with
                               its own scale (kvq_pack_fp8_heads); 0 = one
                               per-tensor scale each */
  /* Paged cache (GQA and MLA layouts; vLLM's block tables, the serving
     setting of Model-Optimizer PR #1832 "Purpose" and "Testing").  GQA
     paged caches are decoded with exact or FP8-quantized probabilities.
     NULL block_table: the planes are addressed by kv_sb / kv_sh / kv_st as
     above.  Otherwise token t of request b, kv head h is plane row
       block_table[b * bt_stride + t / block_size] * kv_sblk
         + h * kv_sh + (t % block_size) * kv_st
     (kv_sb unused; for planes [num_blocks][Hkv][block_size][row]:
     kv_sblk = Hkv * block_size, kv_sh = block_size, kv_st = 1).
     GQA: entries are read for t < max_kv_len; only those of tokens
     t < kv_lens[b] are used as block indices (they must be valid there);
     block_size is a power of two and a multiple of the decode tile
     (attn_decode_tile_tokens).
     MLA (latent, scale and rope planes [num_blocks][block_size][row], one
     table for all three; h = 0): only entries of tokens t < kv_lens[b] are
     read; block_size is a power of two and a multiple of 64 (the MLA
     kernel's tile), and one split may span at most 510 blocks.
     Errors: KVQ_ERR_ARG for a block size, bt_stride or kv_sblk out of
     these bounds. */
  const int32_t* block_table;
  int32_t block_size;
  int64_t bt_stride;
  int64_t kv_sblk;
  /* FP8 query (GQA layout; the QKV-FP8 schemes of compressed-tensors PR #436,
     "Changes" and "Testing": the attention's input activations quantized to
     FP8 E4M3 per tensor or per head).  With q_dtype = KVQ_FP8E4M3, q holds
     E4M3 codes (q 8-byte aligned, q_sb and q_sh multiples of 8) — e.g. from
     kvq_pack_fp8 / kvq_pack_fp8_heads of the query viewed as [B][Hq][1][D] —
     and q_scale their scale: device float[1], or float[Hq] with
     q_scale_per_head = 1 (query head h dequantized with q_scale[h]).  The
     codes enter the score contraction exactly; the scale multiplies the
     score (beside the K tensor scale and softmax_scale).  Exact or
     FP8 probabilities (quantize_p: pass 1 forms the scores from the
     codes).  Unused otherwise. */
  const float* q_scale;
  int32_t q_scale_per_head;
  /* Quantize-on-append fused into the decode step (GQA layout, bf16
     queries, exact probabilities; the cache grows by one token per step as the model
     serves, Model-Optimizer PR #714 "Usage").  new_k, new_v: device rows
     [B][Hkv][D] (contiguous, new_dtype KVQ_BF16, KVQ_F16 or KVQ_F32) of the
     step's new token, or NULL for none.  The token is request b's last, at
     position kv_lens[b] - 1 (kv_lens counts it; clamped to max_kv_len).  It
     is packed with the planes' own scales (k_scale, v_scale; per kv head
     with kv_scale_per_head) into that row of the K and V planes — the bytes
     kvq_pack_*_batch writes with the amax those scales came from — and is
     attended from its fresh codes: the splits cover [0, kv_lens[b] - 1) and
     one more work-group per (request, kv head) writes the token's
     contribution as partial number s, so splits_used reports s + 1
     (s <= 63) and part_capacity must be at least s + 1.  The planes are
     written although declared const. */
  const void* new_k;
  const void* new_v;
  int32_t new_dtype;
  /* NVFP4 latent query (MLA layout; the q_bmm_quantizer of Model-Optimizer
     PR #714 "Testing" — present in QuantMLAAttention beside the latent's
     kv_c_bmm_quantizer and shown disabled there — read as the same NVFP4
     quantizer applied to the absorbed query q_c): with q_dtype =
     KVQ_NVFP4, q holds the E2M1 codes of q_c (rows of D/2 bytes, element
     2j in the low nibble), q_block_scales the E4M3 block scales (rows of
     D/16 bytes) and q_scale its fp32 tensor scale (device float[1]); q_sb
     and q_sh then count query rows (a row = D/2 code bytes and D/16 scale
     bytes).  The dequantized query enters the latent contraction exactly;
     the tensor scale multiplies the latent score.  The rope query q_r stays
     bf16.  q 16-byte and q_block_scales 4-byte aligned.  NULL otherwise. */
  const uint8_t* q_block_scales;
} kvq_decode_args;

/*
 * attn_decode_tile_tokens - tokens per tile of the GQA decode kernel for
 * query groups of G = Hq / Hkv heads (32 to 256): paged caches need a block
 * size that is a multiple of it.  0 if G is unsupported.
 */
int32_t attn_decode_tile_tokens(int32_t Hq, int32_t Hkv);

/*
 * attn_decode_splitkv - split-KV flash decode over the packed cache
 * (Model-Optimizer PR #1832, Testing section): each work-group takes one
 * contiguous chunk of one (request, kv head), dequantizes in registers,
 * computes the scores, keeps an online softmax (running max and
 * denominator) and accumulates P.V; it writes per-split partials.
 * Chunking: c = ceil(max_kv_len / s) rounded up to the kernel tile; split j
 * covers [j c, min((j+1) c, L_b)) (empty when j c >= L_b).  The chunk
 * depends on kernel arguments only, so the first tile is requested together
 * with L_b; rows of the planes up to max_kv_len may be read, and tokens at
 * or past L_b never contribute.
 * With quantize_p = 1 (GQA only; vLLM PR #15734 "[Quantization][FP8] Add
 * support for FP8 models with input_scale for output projection and QK
 * quantization", item 2) the probabilities are the normalized softmax over
 * the whole sequence, P_t = exp(sigma_t - LSE), quantized as
 * P~_t = E4M3(P_t / prob_scale) * prob_scale (round to nearest even,
 * saturating), and attn_decode_combine then returns sum_t P~_t V_t (not
 * renormalized) and the exact LSE.  Two launches: pass 1 reads K, spills
 * the scores to p_scratch and writes each split's lse to part_lse; pass 2
 * reads V and the spilled scores and writes part_o as
 * sum_{t in j} P~_t V_t / exp(lse_j - LSE).  p_scratch: device float32,
 * kvq_fp8p_scratch_floats(...) elements, 16-byte aligned; prob_scale > 0.
 * The scratch and the partials must not be shared by overlapping calls.
 *   splits_used  host int32* or NULL: receives the split count s used.
 */
int attn_decode_splitkv(const kvq_decode_args* args, int32_t* splits_used, void* stream);

/*
 * attn_decode_combine - merge the s split partials into one output per
 * (request, head) (Model-Optimizer PR #1832, Testing section: the split-KV
 * description ends with a small separate kernel that merges the per-split
 * results):
 * LSE = log sum_j exp(lse_j), o = sum_j exp(lse_j - LSE) o_j; empty splits
 * (lse_j = -inf) are skipped; a request with no tokens gives o = 0, lse =
 * -inf.
 *   out        device [B][Hq][Dv], out_dtype KVQ_F32, KVQ_BF16 (RNE) or
 *              KVQ_FP8E4M3 (code = E4M3(o / out_scale), saturating; vLLM
 *              PR #15734 item 1).
 *   out_scale  device float[1], required for KVQ_FP8E4M3, else ignored.
 *   lse_out    device float[B][Hq] or NULL.
 */
int attn_decode_combine(const float* part_o, const float* part_lse, int32_t B, int32_t Hq, int32_t Dv,
                        int32_t num_splits, void* out, int32_t out_dtype, const float* out_scale,
                        float* lse_out, void* stream);

/*
 * attn_decode - attn_decode_splitkv and attn_decode_combine in one launch:
 * the last work-group to finish a (request, kv head) merges its s partials
 * and writes the output (with s == 1 the output is written directly and no
 * partials or counters are touched).  Same results as the two-call path.
 * MLA and quantize_p = 1 run as the split launch(es) followed by the
 * combine launch (counters unused).
 *   out, out_dtype, out_scale, lse_out  as attn_decode_combine.
 *   counters  device int32[B * Hkv]: all zero before the first call; every
 *             completed call leaves them zero.  Calls sharing a counters
 *             buffer or partial buffers must not overlap (same stream is
 *             fine).  Unused (may be NULL) when s == 1.
 *   splits_used  host int32* or NULL: receives s.
 */
int attn_decode(const kvq_decode_args* args, void* out, int32_t out_dtype, const float* out_scale, float* lse_out,
                int32_t* counters, int32_t* splits_used, void* stream);

/*
 * attn_decode_noalloc - attn_decode for callers that cannot allocate memory
 * or pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the split partials and the merge
 * counters live in a static device array of the library, one per GPU, of
 * KVQ_NOALLOC_SCRATCH_BYTES (held until the process ends).  The call
 * allocates nothing.  Arguments and results as attn_decode (same kernels,
 * same bits); args->part_o, part_lse, part_capacity and p_scratch are
 * ignored.  Limits: the partials, B * Hq * s' * (Dv + 1) * 4 bytes with s'
 * = s (s + 1 with a fused append), must fit in KVQ_NOALLOC_SCRATCH_BYTES -
 * 64 KiB, and B * Hkv <= 16384: otherwise KVQ_ERR_WORKSPACE, nothing
 * launched.  FP8 probabilities (quantize_p) need a score scratch of the
 * sequence's size and are refused (KVQ_ERR_UNSUPPORTED).  The first call on
 * a device looks the array up (hipGetSymbolAddress) and clears its counters
 * with a kernel on `stream`; every completed call leaves them zero.  All
 * calls on one GPU share its array, which keeps the last call's partials:
 * calls that overlap on a GPU (other streams or threads) race; calls on one
 * stream are ordered and safe.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES (24u << 20)
int attn_decode_noalloc(const kvq_decode_args* args, void* out, int32_t out_dtype, const float* out_scale,
                        float* lse_out, int32_t* splits_used, void* stream);

/*
 * kvq_auto_num_splits - split count when the caller passes num_splits <= 0
 * (Model-Optimizer PR #1832, Testing section: the built-in heuristic picks s
 * from the compute-unit count and batch x heads).  Host-only, no device
 * access.  Rule: s = ceil(w num_cus / (B programs_per_req)), w = 1
 * work-group per compute unit when Hq >= 4 programs_per_req and Dv <= 256
 * (query groups of 4+ heads: the grouped-tile GQA kernel) and w = 2
 * otherwise (query groups of 1-2 heads, the MLA latent), capped at
 * ceil(max_kv_len / 256), at
 * floor(KV bytes / (3 x partial bytes)) with KV bytes = B programs_per_req
 * max_kv_len (9/8) Dv and partial bytes = B Hq (Dv + 1) 8 per split, and at
 * 64; at least 1.
 *   num_cus           compute units of the device (256 on MI355X).
 *   programs_per_req  kv heads per request (1 for MLA).
 *   max_kv_len        longest kv length in the batch.
 *   Dv, Hq            value width and query heads (partial-traffic bound).
 *   s_out             host int32*: receives s in [1, 64].
 */
int kvq_auto_num_splits(int32_t num_cus, int32_t B, int32_t programs_per_req, int32_t max_kv_len,
                        int32_t Dv, int32_t Hq, int32_t* s_out);

/*
 * kvq_device_cu_count - compute units of the current HIP device, the first
 * input of the automatic split count (Model-Optimizer PR #1832, Testing
 * section: the heuristic sizes num_kv_splits from the GPU's compute-unit
 * count and batch x heads).  Host call; needs a GPU.  num_cus_out: host
 * int32*.  Errors: KVQ_ERR_ARG (null), KVQ_ERR_HIP (no device).
 */
int kvq_device_cu_count(int32_t* num_cus_out);

/*
 * kvq_decode_workspace_bytes - bytes of the split partials for s splits:
 * part_o [B][Hq][s][Dv] plus part_lse [B][Hq][s], float32, i.e.
 * B * Hq * s * (Dv + 1) * 4 (Model-Optimizer PR #1832, Testing section: each
 * split writes its partial output and log-sum-exp for the combine).  A
 * caller that passes num_splits <= 0 sizes for kvq_auto_num_splits' result
 * (or for 64, its maximum); with a fused append pass s + 1.  Host-only;
 * returns 0 for a non-positive argument.  The caller allocates: the library
 * never does.
 */
size_t kvq_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Dv, int32_t s);

/*
 * kvq_fp8p_scratch_floats - float32 elements of p_scratch needed by the
 * FP8-probability path (quantize_p = 1; vLLM PR #15734 "[Quantization][FP8]
 * Add support for FP8 models with input_scale for output projection and QK
 * quantization", item 2: the softmax probabilities quantized to FP8, which
 * with normalized probabilities needs the scores of the whole sequence
 * before P is formed): the spilled scores, one row of
 * roundup(max_kv_len, 4) floats per (request, query head); s is accepted for
 * interface stability and does not change the size.  Host-only.
 */
size_t kvq_fp8p_scratch_floats(int32_t B, int32_t Hq, int32_t s, int32_t max_kv_len);

/*
 * Chunked prefill over the packed cache (Model-Optimizer PR #1832 "Add
 * quant+sparse attention for vLLM serving", Testing section: the prefill
 * path timed in the "prefill" column of both decode-latency tables, the
 * triton_fa.py entry of the coverage report).  A chunk of Sq new query
 * tokens per request attends to the quantized cache, which already holds
 * the chunk's own K/V rows (they were packed with kvq_pack_* first): query
 * i of request b sits at position p_i = kv_lens[b] - Sq + i and sees the
 * cached tokens t <= p_i (causal); a query with p_i < 0 sees nothing and
 * gets output 0 and lse -inf.  Scores and dequantization as in decode
 * (scores softmax_scale * (q . K_t), K_t and V_t dequantized; the tensor
 * scales in fp32), GQA head mapping h -> h / (Hq / Hkv).
 *
 * Layout: q [B][Sq][Hq][D] bf16 with element strides q_sb, q_st, q_sh
 * (or FP8 codes, below);
 * out [B][Sq][Hq][D] with element strides o_sb, o_st, o_sh; lse_out
 * contiguous [B][Sq][Hq] float32 or NULL.  K planes in the row layout, V
 * planes in KVQ_PLANE_TOKEN4 (the decode layout at D = 128), plane rows
 * indexed (request, kv head, token) with strides kv_sb, kv_sh and token
 * stride 1, at least roundup(max_kv_len, 4) rows per (request, kv head);
 * or paged (block_table non-NULL; same addressing as kvq_decode_args,
 * block_size a power of two >= 64; entries are read for the tokens a query
 * sees, t < kv_lens[b], and must be valid there).  The caller owns every
 * buffer; the call allocates nothing and keeps no state.
 */
typedef struct {
  int32_t kv_format;         /* KVQ_NVFP4 or KVQ_FP8E4M3                     */
  int32_t B, Hq, Hkv, D;     /* D = 128; Hq / Hkv in {1, 2, 4, 8}            */
  int32_t Sq;                /* query tokens per request (>= 0)             */
  int32_t max_kv_len;        /* upper bound on kv_lens; rows per request    */
  const void* q;             /* device bf16 16-byte aligned, or FP8 codes   */
  int32_t q_dtype;           /* KVQ_BF16 or KVQ_FP8E4M3                     */
  int64_t q_sb, q_st, q_sh;  /* element strides, multiples of 8             */
  const uint8_t* k_codes;
  const uint8_t* k_scales;   /* NVFP4 only                                  */
  const float* k_scale;      /* device float[1] (float[Hkv] with kv_scale_per_head) */
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  const float* v_scale;
  int32_t v_layout;          /* KVQ_PLANE_TOKEN4                            */
  int32_t kv_scale_per_head; /* FP8: 1 = one scale per kv head              */
  int64_t kv_sb, kv_sh;      /* plane-row strides (multiples of 4)          */
  const int32_t* kv_lens;    /* device int32[B], cache length incl. the chunk */
  float softmax_scale;       /* > 0                                         */
  const int32_t* block_table;/* NULL: contiguous planes                     */
  int32_t block_size;
  int64_t bt_stride, kv_sblk;
  void* out;                 /* device, out_dtype                           */
  int32_t out_dtype;         /* KVQ_F32 (16-byte aligned) or KVQ_BF16 (8-byte) */
  int64_t o_sb, o_st, o_sh;  /* element strides, multiples of 4             */
  float* lse_out;            /* device float[B][Sq][Hq] or NULL             */
  /* FP8 queries (the QKV-FP8 schemes of compressed-tensors PR #436,
     "Changes" and "Testing": the attention's query activations quantized
     to FP8 E4M3 per tensor or per head).  With q_dtype = KVQ_FP8E4M3, q
     holds E4M3 codes, one byte an element (q 8-byte aligned, strides as
     above) — e.g. kvq_pack_fp8 / kvq_pack_fp8_heads of the chunk viewed as
     [B * Sq][Hq][1][D] — and q_scale their scale: device float[1], or
     float[Hq] with q_scale_per_head = 1.  The codes enter the score
     contraction exactly (over an FP8 cache both operands are E4M3 codes
     on the FP8 matrix cores, products exact, sums in fp32); the scale
     multiplies the score beside the K tensor scale and softmax_scale.
     Unused for bf16 queries. */
  const float* q_scale;
  int32_t q_scale_per_head;
} kvq_prefill_args;

/* sizeof(kvq_prefill_args) as compiled into the library (binding check). */
size_t kvq_prefill_args_size(void);

/*
 * attn_prefill - the chunked prefill above, one launch, no workspace.
 * Both contractions (Q.K^T over head_dim, P.V over tokens) run on the
 * matrix cores; the softmax is online over 64-token tiles; each query row
 * sees its keys in one pass (no split, no partials).  Every row of the
 * planes that a query sees is read; rows at or past kv_lens[b] (at most
 * max_kv_len) are never used.
 * Errors (nothing launched): KVQ_ERR_ARG (null pointers, negative sizes,
 * softmax_scale <= 0, kv_lens bound, block-table geometry),
 * KVQ_ERR_UNSUPPORTED (D != 128, group width outside {1, 2, 4, 8}, query
 * dtype, V layout, output dtype), KVQ_ERR_ALIGN (bases or strides off the
 * alignment above), KVQ_ERR_HIP (launch).
 */
int attn_prefill(const kvq_prefill_args* args, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
