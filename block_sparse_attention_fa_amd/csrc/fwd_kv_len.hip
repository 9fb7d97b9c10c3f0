// Forward instantiations for the MaskKvLen mask_mod (every score_mod, D = 64 and 128).
#include "fwd_kernel.hpp"

namespace fa {
fa_status launch_forward_kv_len(int D, int score_kind, const FwdParams& p, hipStream_t stream) {
  return launch_forward_mask<MaskKvLen>(D, score_kind, p, stream);
}
}  // namespace fa
