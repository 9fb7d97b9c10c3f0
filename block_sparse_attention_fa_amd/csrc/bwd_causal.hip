// Backward instantiations for the MaskCausal mask_mod (every score_mod, D = 64 and 128).
#include "bwd_kernel.hpp"

namespace fa {
fa_status launch_backward_causal(int D, int score_kind, const BwdParams& p, hipStream_t stream) {
  return launch_backward_mask<MaskCausal>(D, score_kind, p, stream);
}
}  // namespace fa
