// Forward instantiations for the MaskCausal mask_mod (every score_mod, D = 64 and 128).
#include "fwd_kernel.hpp"

namespace fa {
fa_status launch_forward_causal(int D, int score_kind, const FwdParams& p, hipStream_t stream) {
  return launch_forward_mask<MaskCausal>(D, score_kind, p, stream);
}
}  // namespace fa
