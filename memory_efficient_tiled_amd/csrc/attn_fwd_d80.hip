// attn_fwd_d80.hip -- the attention forward kernels for head dimension 80
// (one translation unit per head dimension, so they compile in parallel).

#include "attn_fwd_kernel.h"

namespace attn_fwd_detail {

template <>
hipError_t launch_fwd_d<80, 80>(const Params& p, int cfg, bool causal, bool split, bool strided,
                           bool masked, bool bf16, hipStream_t st) {
  return bf16 ? dispatch_d<80, 80, TagBF16>(p, cfg, causal, split, strided, masked, st)
              : dispatch_d<80, 80, TagF16>(p, cfg, causal, split, strided, masked, st);
}

template <>
hipError_t launch_combine_d<80>(const Params& p, bool strided, bool bf16, hipStream_t st) {
  return bf16 ? launch_combine<80, TagBF16>(p, strided, st)
              : launch_combine<80, TagF16>(p, strided, st);
}

}  // namespace attn_fwd_detail
