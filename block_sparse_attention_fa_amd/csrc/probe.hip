// Measurement probes: what the chip reaches in practice for the two resources
// the attention kernels are bound by, so their throughput can be reported as a
// fraction of a measured peak as well as of the published one.
//
// mfma_probe_kernel: every wave runs 8 independent accumulation chains of
// v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic in the
// loop), 2 waves per SIMD, the matrix pipe's issue rate being the only limit.
// copy_probe_kernel: a grid-stride 16-byte load/store copy with four loads in
// flight per lane before their stores, so HBM read and write bandwidth is the
// only limit.
#include <hip/hip_runtime.h>

#include "fa_internal.hpp"

namespace fa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kChains = 8;

__global__ __launch_bounds__(kProbeThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_probe_kernel(int iterations, float* sink) {
  const int tid = threadIdx.x;
  // operands that depend on the lane, so nothing folds at compile time
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f / (float)(1 + ((tid + i) & 7)));
    b[i] = (__bf16)(0.5f / (float)(1 + ((tid * 3 + i) & 7)));
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16_t{};
  for (int it = 0; it < iterations; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[(long long)blockIdx.x * kProbeThreads + tid] = s;
}

__global__ __launch_bounds__(kProbeThreads) void copy_probe_kernel(const u32x4_t* __restrict__ src,
                                                                   u32x4_t* __restrict__ dst, long long n) {
  constexpr int U = 4;
  const long long stride = (long long)gridDim.x * kProbeThreads;
  long long i = (long long)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(x[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

fa_status launch_probe_mfma(int workgroups, int iterations, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream, iterations, sink);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

double probe_mfma_flops(int workgroups, int iterations) {
  const double waves = (double)workgroups * (kProbeThreads / 64);
  return waves * iterations * kChains * (2.0 * 32 * 32 * 16);
}

fa_status launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const long long n = (long long)(bytes / 16);
  const long long want = (n + kProbeThreads * 4 - 1) / (kProbeThreads * 4);
  const unsigned grid = (unsigned)(want < 8192 ? (want < 1 ? 1 : want) : 8192);
  hipLaunchKernelGGL(copy_probe_kernel, dim3(grid), dim3(kProbeThreads), 0, stream, (const u32x4_t*)src,
                     (u32x4_t*)dst, n);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace fa
