// BlockMask builder (attention-gym "Concepts" page, "BlockMask Internals" and
// "Key attributes"; paper review "Flex Attention: A Programming Model for
// Generating Optimized Attention Kernels", §4.1-4.2).
//
// One workgroup per BlockMask row (b', h', query tile).  Each wave classifies
// whole 128x128 tiles.  Where the mask's structure decides the class exactly
// (linear masks from the tile's corners, documents from the id ranges on each
// side, and/or of decided parts) that answer is taken; otherwise its 64 lanes
// each own up to two key columns of the tile and walk the tile's in-range
// query rows, evaluating the mask_mod per position, and a wave vote gives
// "any position attends" / "every position attends".  A tile is empty when none attends, full when all do, partial
// otherwise.  Wave 0 then appends the tile ids of each class, in ascending
// order, with a ballot + popcount prefix, so every list is written in order
// without atomics.  All integer work: the result is bit-exact by construction.
#include "mods.hpp"

namespace fa {
namespace {

constexpr int kTile = FA_BLOCK;
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 256;  // tiles classified per pass (kChunk / kWaves per wave)

enum : int { kEmpty = kTileEmpty, kPartial = kTilePartial, kFull = kTileFull };

template <class Mask>
__device__ __forceinline__ int classify_tile(const BuildParams& p, int b, int h, int q0, int qn,
                                             int kb, int lane) {
  const int k0 = kb * kTile;
  const int kn = min(kTile, p.Skv - k0);
  const int c = Mask::classify(p.mask, b, h, q0, q0 + qn - 1, k0, k0 + kn - 1, lane);
  if (c != kTileUnknown) return c;
  const bool c0 = lane < kn;
  const bool c1 = lane + 64 < kn;
  bool any = false, all = true;
  for (int i = 0; i < qn; ++i) {
    const auto r = Mask::row(p.mask, b, h, q0 + i);
    if (c0) {
      const bool m = r(k0 + lane);
      any |= m;
      all &= m;
    }
    if (c1) {
      const bool m = r(k0 + 64 + lane);
      any |= m;
      all &= m;
    }
    // Once the wave has seen both an attended and a masked position the
    // tile is partial whatever the remaining rows hold.
    if ((i & 7) == 7 && __any(any) && !__all(all)) return kPartial;
  }
  if (!__any(any)) return kEmpty;
  return __all(all) ? kFull : kPartial;
}

template <class Mask>
__global__ __launch_bounds__(kThreads) void build_block_mask_kernel(BuildParams p) {
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q0 = qb * kTile;
  const int qn = min(kTile, p.Sq - q0);
  const long long row = ((long long)b * p.Hm + h) * p.NQ + qb;
  int* kv_idx = p.kv_idx + row * p.NK;
  int* full_idx = p.full_idx + row * p.NK;

  __shared__ unsigned char cls[kChunk];
  __shared__ int counts[2];
  if (threadIdx.x == 0) {
    counts[0] = 0;
    counts[1] = 0;
  }

  for (int c0 = 0; c0 < p.NK; c0 += kChunk) {
    for (int i = 0; i < kChunk / kWaves; ++i) {
      const int j = i * kWaves + wave;
      const int kb = c0 + j;
      if (kb < p.NK) {
        const int c = classify_tile<Mask>(p, b, h, q0, qn, kb, lane);
        if (lane == 0) cls[j] = (unsigned char)c;
      }
    }
    __syncthreads();
    if (wave == 0) {
      int np = counts[0], nf = counts[1];
      const unsigned long long below = (1ull << lane) - 1ull;
      for (int s = 0; s < kChunk; s += 64) {
        const int kb = c0 + s + lane;
        const int c = kb < p.NK ? (int)cls[s + lane] : kEmpty;
        const bool in_kv = p.separate_full ? (c == kPartial) : (c != kEmpty);
        const bool in_full = c == kFull;
        const unsigned long long mk = __ballot(in_kv);
        const unsigned long long mf = __ballot(in_full);
        if (in_kv) kv_idx[np + __popcll(mk & below)] = kb;
        if (in_full) full_idx[nf + __popcll(mf & below)] = kb;
        np += __popcll(mk);
        nf += __popcll(mf);
      }
      if (lane == 0) {
        counts[0] = np;
        counts[1] = nf;
      }
    }
    __syncthreads();
  }

  const int np = counts[0], nf = counts[1];
  for (int i = threadIdx.x; i < p.NK; i += kThreads) {
    if (i >= np) kv_idx[i] = 0;
    if (i >= nf) full_idx[i] = 0;
  }
  if (threadIdx.x == 0) {
    p.kv_num[row] = np;
    p.full_num[row] = nf;
  }
}

// Transposed view (Concepts "Key attributes": q_num_blocks / q_indices, "used
// in backward"): for KV block kb, the query blocks whose row lists hold kb, in
// ascending order, padded with 0.  One wave per (b', h', kb); its lanes take 64
// query blocks at a time and binary-search kb in their (ascending) row lists,
// so the columns agree with the rows by construction.
__device__ __forceinline__ bool list_has(const int* idx, int n, int kb) {
  int lo = 0, hi = n;  // first entry >= kb in [lo, hi)
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (idx[mid] < kb) lo = mid + 1; else hi = mid;
  }
  return lo < n && idx[lo] == kb;
}

__global__ __launch_bounds__(64) void transpose_block_lists_kernel(BuildParams p) {
  const int kb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const long long bh = (long long)b * p.Hm + h;
  const long long col = bh * p.NK + kb;
  int* q_idx = p.q_idx + col * p.NQ;
  int* full_q_idx = p.full_q_idx + col * p.NQ;
  const unsigned long long below = (1ull << lane) - 1ull;
  int np = 0, nf = 0;
  for (int q0 = 0; q0 < p.NQ; q0 += 64) {
    const int qb = q0 + lane;
    bool in_kv = false, in_full = false;
    if (qb < p.NQ) {
      const long long row = bh * p.NQ + qb;
      in_kv = list_has(p.kv_idx + row * p.NK, p.kv_num[row], kb);
      in_full = list_has(p.full_idx + row * p.NK, p.full_num[row], kb);
    }
    const unsigned long long mk = __ballot(in_kv);
    const unsigned long long mf = __ballot(in_full);
    if (in_kv) q_idx[np + __popcll(mk & below)] = qb;
    if (in_full) full_q_idx[nf + __popcll(mf & below)] = qb;
    np += __popcll(mk);
    nf += __popcll(mf);
  }
  for (int i = lane; i < p.NQ; i += 64) {
    if (i >= np) q_idx[i] = 0;
    if (i >= nf) full_q_idx[i] = 0;
  }
  if (lane == 0) {
    p.q_num[col] = np;
    p.full_q_num[col] = nf;
  }
}

// Work orders (the BlockMask's optional q_order and kv_order): one 1024-thread
// workgroup per (b', h') row sorts the n keys (weight << 14) | i, i < n, in LDS
// with a bitonic network, largest first, and writes their i.  weight = 3 per
// listed tile that runs the mask_mod + 2 per full tile, at most 3 * 16384 <
// 2^16, and i < 2^14, so the keys are distinct and fit 30 bits.  Slots past n
// hold 0, which sorts after every real key except (weight 0, i 0), whose
// decoded i is the same.  For the query blocks the counts are the row lists'
// (ties to the larger query block: key i = qb); for the KV blocks the
// transposed view's (ties to the smaller KV block: key i = n - 1 - kb).
constexpr int kOrderMax = 16384;
constexpr int kOrderThreads = 1024;
struct OrderArgs {
  const int* num;   // [rows, n] tiles that run the mask
  const int* full;  // [rows, n] full tiles
  int* out;         // [rows, n]
  int n;
  int separate_full;
  int reverse;      // key index n - 1 - i (ties to the smaller i)
};
__global__ __launch_bounds__(kOrderThreads) void order_blocks_kernel(OrderArgs a, int Hm) {
  __shared__ uint32_t key[kOrderMax];
  const long long bh = (long long)blockIdx.y * Hm + blockIdx.x;
  int n = 2;
  while (n < a.n) n <<= 1;
  for (int i = threadIdx.x; i < n; i += kOrderThreads) {
    uint32_t k = 0;
    if (i < a.n) {
      const long long at = bh * a.n + i;
      const int w = 3 * a.num[at] + (a.separate_full ? 2 * a.full[at] : 0);
      k = ((uint32_t)w << 14) | (uint32_t)(a.reverse ? a.n - 1 - i : i);
    }
    key[i] = k;
  }
  __syncthreads();
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += kOrderThreads) {
        const int l = i ^ j;
        if (l > i) {
          const uint32_t x = key[i], y = key[l];
          const bool desc = (i & k) == 0;  // this pair's subsequence runs largest first
          if (desc ? x < y : x > y) {
            key[i] = y;
            key[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < a.n; i += kOrderThreads) {
    const int d = (int)(key[i] & 0x3fffu);
    a.out[bh * a.n + i] = a.reverse ? a.n - 1 - d : d;
  }
}

struct LaunchBuild {
  const BuildParams& p;
  hipStream_t stream;
  template <class Mask>
  void operator()() {
    dim3 grid(p.NQ, p.Hm, p.Bm);
    hipLaunchKernelGGL(build_block_mask_kernel<Mask>, grid, dim3(kThreads), 0, stream, p);
    if (p.q_num != nullptr)
      hipLaunchKernelGGL(transpose_block_lists_kernel, dim3(p.NK, p.Hm, p.Bm), dim3(64), 0, stream, p);
    if (p.q_order != nullptr)
      hipLaunchKernelGGL(order_blocks_kernel, dim3(p.Hm, p.Bm), dim3(kOrderThreads), 0, stream,
                         OrderArgs{p.kv_num, p.full_num, p.q_order, p.NQ, p.separate_full, 0}, p.Hm);
    if (p.row_order != nullptr)  // one query block and one head row: the rows' counts are contiguous
      hipLaunchKernelGGL(order_blocks_kernel, dim3(1, 1), dim3(kOrderThreads), 0, stream,
                         OrderArgs{p.kv_num, p.full_num, p.row_order, p.Bm, p.separate_full, 1}, 1);
    if (p.kv_order != nullptr)  // after the transposed view, which it reads
      hipLaunchKernelGGL(order_blocks_kernel, dim3(p.Hm, p.Bm), dim3(kOrderThreads), 0, stream,
                         OrderArgs{p.q_num, p.full_q_num, p.kv_order, p.NK, p.separate_full, 1}, p.Hm);
  }
};

}  // namespace

fa_status launch_block_mask(int mask_kind, const BuildParams& p, hipStream_t stream) {
  LaunchBuild l{p, stream};
  if (!dispatch_mask(mask_kind, l)) return FA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace fa
