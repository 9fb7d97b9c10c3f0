// Backward instantiations for the MaskPrefixLM mask_mod (every score_mod, D = 64 and 128).
#include "bwd_kernel.hpp"

namespace fa {
fa_status launch_backward_prefix_lm(int D, int score_kind, const BwdParams& p, hipStream_t stream) {
  return launch_backward_mask<MaskPrefixLM>(D, score_kind, p, stream);
}
}  // namespace fa
