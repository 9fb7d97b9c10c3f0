// Backward instantiations for the MaskWindow mask_mod (every score_mod, D = 64 and 128).
#include "bwd_kernel.hpp"

namespace fa {
fa_status launch_backward_window(int D, int score_kind, const BwdParams& p, hipStream_t stream) {
  return launch_backward_mask<MaskWindow>(D, score_kind, p, stream);
}
}  // namespace fa
