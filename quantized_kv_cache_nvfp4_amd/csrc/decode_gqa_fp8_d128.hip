// Instantiations of the GQA / MHA split-KV decode kernel (decode_gqa_kernel.h)
// for fp8 caches with head_dim 128; one source per (format, head_dim) so the
// instantiation sets compile in parallel.
#include "decode_gqa_kernel.h"

namespace kvq {

hipError_t gqa_dispatch_fp8_d128(int pm, const kvq_decode_args& a, const DecodePlan& p, const gqa::FusedOut* fo,
                                 hipStream_t st) {
  return gqa::dispatch_fmt<KVQ_FP8E4M3, 128>(pm, a, p, fo, st);
}

}  // namespace kvq
