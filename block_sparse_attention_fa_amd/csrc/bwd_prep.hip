// Backward preprocessing: Delta = rowsum(dO * O) and the base-2 LSE per query row.
#include "bwd_kernel.hpp"

namespace fa {
fa_status launch_backward_prep(int D, const BwdParams& p, hipStream_t stream) {
  const long long rows = (long long)p.f.B * p.f.Hq * p.sq_pad;
  const unsigned grid = (unsigned)((rows + kBwdThreads / 64 - 1) / (kBwdThreads / 64));
  if (D == 128)
    hipLaunchKernelGGL(bwd_prep_kernel<128>, dim3(grid), dim3(kBwdThreads), 0, stream, p);
  else if (D == 64)
    hipLaunchKernelGGL(bwd_prep_kernel<64>, dim3(grid), dim3(kBwdThreads), 0, stream, p);
  else
    return FA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
}  // namespace fa
