// Forward instantiations for the MaskDocument mask_mod (every score_mod, D = 64 and 128).
#include "fwd_kernel.hpp"

namespace fa {
fa_status launch_forward_document(int D, int score_kind, const FwdParams& p, hipStream_t stream) {
  return launch_forward_mask<MaskDocument>(D, score_kind, p, stream);
}
}  // namespace fa
