// Backward preprocessing: Delta = rowsum(dO * O) and the base-2 LSE per query row.
#include "bwd_kernel.hpp"

namespace fa {
fa_status launch_backward_prep(int D, const BwdParams& p, hipStream_t stream) {
  const long long rows = (long long)p.f.B * p.f.Hq * p.sq_pad;
  auto grid = [&](int rows_per_wave) {
    const long long per_block = (long long)rows_per_wave * (kBwdThreads / 64);
    return (unsigned)((rows + per_block - 1) / per_block);
  };
  if (D == 128)
    hipLaunchKernelGGL(bwd_prep_kernel<128>, dim3(grid(kPrepRowsPerWave<128>)), dim3(kBwdThreads), 0, stream, p);
  else if (D == 64)
    hipLaunchKernelGGL(bwd_prep_kernel<64>, dim3(grid(kPrepRowsPerWave<64>)), dim3(kBwdThreads), 0, stream, p);
  else
    return FA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}
}  // namespace fa
