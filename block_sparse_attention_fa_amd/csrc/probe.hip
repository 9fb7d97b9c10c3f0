// Measurement probes: what the chip reaches in practice for the two resources
// the attention kernels are bound by, so their throughput can be reported as a
// fraction of a measured peak as well as of the published one.
//
// mfma_probe_kernel: every wave runs 8 independent accumulation chains of
// v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic in the
// loop), 2 waves per SIMD, the matrix pipe's issue rate being the only limit.
// With random operands every lane holds bf16 values with random signs and
// mantissas, and alternate rounds use two different sets, so the datapath
// switches as it does on real data (and draws the power it does then); with
// constant operands it hardly switches.
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
void mfma_probe_kernel(int iterations, int random_operands, float* sink) {
  const int tid = threadIdx.x;
  // operands that depend on the lane, so nothing folds at compile time
  bf16x8_t a[2], b[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (random_operands) {
        // a 32-bit integer hash of (workgroup, lane, set, element): random sign and
        // mantissa, exponent of [0.5, 1)
        uint32_t h = (uint32_t)(blockIdx.x * 256 + tid) * 0x9E3779B1u + (uint32_t)(16 * s + i) * 0x85EBCA77u;
        h ^= h >> 15;
        h *= 0x2C1B3C6Du;
        h ^= h >> 12;
        const uint16_t bits_a = (uint16_t)(0x3F00u | (h & 0x807Fu));
        const uint16_t bits_b = (uint16_t)(0x3F00u | ((h >> 16) & 0x807Fu));
        a[s][i] = __builtin_bit_cast(__bf16, bits_a);
        b[s][i] = __builtin_bit_cast(__bf16, bits_b);
      } else {
        a[s][i] = (__bf16)(1.0f / (float)(1 + ((tid + i) & 7)));
        b[s][i] = (__bf16)(0.5f / (float)(1 + ((tid * 3 + i) & 7)));
      }
    }
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16_t{};
  for (int it = 0; it < iterations; it += 2) {  // (iterations is rounded up to even)
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], acc[c], 0, 0, 0);
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

// Read-only stream: 16-byte non-temporal loads, four in flight per lane, folded
// into one xor per lane and one word per workgroup (so the loads stay live).
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t* __restrict__ src, long long n,
                                                                   uint32_t* sink) {
  constexpr int U = 4;
  const long long stride = (long long)gridDim.x * kProbeThreads;
  long long i = (long long)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= x[u];
  }
  for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v ^= __shfl_xor(v, off);
  __shared__ uint32_t red[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

int probe_read_workgroups(size_t bytes) {
  const long long n = (long long)(bytes / 16);
  const long long want = (n + kProbeThreads * 4 - 1) / (kProbeThreads * 4);
  return (int)(want < 8192 ? (want < 1 ? 1 : want) : 8192);
}

fa_status launch_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)probe_read_workgroups(bytes)), dim3(kProbeThreads), 0, stream,
                     (const u32x4_t*)src, (long long)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status launch_probe_mfma(int workgroups, int iterations, int random_operands, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream, iterations,
                     random_operands, sink);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

double probe_mfma_flops(int workgroups, int iterations) {
  const double waves = (double)workgroups * (kProbeThreads / 64);
  const int rounds = (iterations + 1) / 2 * 2;  // the kernel runs whole pairs of rounds
  return waves * rounds * kChains * (2.0 * 32 * 32 * 16);
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
