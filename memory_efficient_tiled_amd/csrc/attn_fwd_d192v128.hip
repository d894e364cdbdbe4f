// attn_fwd_d192v128.hip -- the attention forward kernels for 192-element
// query and key rows with 128-element value and output rows (the head
// dimensions of multi-head latent attention at prefill, where each head's
// query and key carry an extra positional part).  The merge of split
// partials is the DV = 128 one, in attn_fwd_d128.hip.

#include "attn_fwd_kernel.h"

namespace attn_fwd_detail {

template <>
hipError_t launch_fwd_d<192, 128>(const Params& p, int cfg, bool causal, bool split,
                                  bool strided, bool masked, bool bf16, hipStream_t st) {
  return bf16 ? dispatch_d<192, 128, TagBF16>(p, cfg, causal, split, strided, masked, st)
              : dispatch_d<192, 128, TagF16>(p, cfg, causal, split, strided, masked, st);
}

}  // namespace attn_fwd_detail
