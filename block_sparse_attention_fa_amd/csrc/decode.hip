// Split-KV decode with a log-sum-exp merge.
//
// One query token per sequence against a long KV cache; the token of
// sequence b sits at position q_pos[b] (0 without q_pos), which the
// score_mods see as its q index.  Following the
// "Flex Decoding" part of the talk summary "FlexAttention: A Flexible and
// Performant Approach to Transformer Attention", the key axis is split into
// chunks that are processed in parallel and combined by a final reduction;
// the score_mod still applies.  The chunks are cut from the sequence's
// BlockMask row (partial tiles first, then full tiles), so empty tiles past a
// sequence's valid length are never read (Concepts page, "BlockMask
// Internals").  A chunk is every splits-th entry of that list.
//
// decode_partial: one 256-thread workgroup per (split, KV head, batch row).
// It reads each K/V row of its chunk exactly once and serves all G query
// heads of that KV head from it (GQA).  The chunk's tile rows are looked up
// once into LDS, so no row load waits on a block-list read.  Pass 1 computes
// the G scores of every key into LDS (16-byte row loads, a dot product per
// lane over 8 dims and a DPP sum over the lanes of the row), pass 2 takes each
// head's max and exponentials, pass 3 accumulates P.V; in passes 1 and 3 the
// next group of rows is loaded while the current one is used, and the first
// V rows are in flight during pass 2.  Its output is the chunk's normalised
// partial output and base-2 LSE in a caller-provided fp32 workspace.
// decode_merge: LSE = log-sum-exp of the chunk LSEs, O = sum_s e^(LSE_s - LSE) O_s.
#include <mutex>

#include "mods.hpp"

namespace fa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kMaxBps = 8;  // kv tiles per split at most
constexpr int kMaxRows = kMaxBps * FA_BLOCK;
constexpr int kScPad = 16;

struct EvalMask {
  const MaskParams& mp;
  int b, h, q, kv;
  bool result;
  template <class M>
  __device__ void operator()() {
    result = M::row(mp, b, h, q)(kv);
  }
};

__device__ __forceinline__ void unpack8(const u32x4_t& x, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(x[i] << 16);
    f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
  }
}

// Sum over groups of LPR (8 or 16) consecutive lanes, result in every lane of
// the group, with DPP moves (no LDS traffic): quad xor 1, quad xor 2, half-row
// mirror, and for 16 lanes the row mirror.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  if (LPR == 16)
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}

template <int D, int G, class Score, bool PAGED>
__global__ __launch_bounds__(kDecThreads) void decode_partial_kernel(DecodeParams P) {
  constexpr int LPR = D / 8;          // lanes per K/V row (16 bytes each)
  constexpr int RPW = 64 / LPR;       // rows per wave per load
  constexpr int RSTEP = kDecWaves * RPW;
  const FwdParams& p = P.f;
  // with the BlockMask's row order, the grid's sequences run longest first
  const int split = blockIdx.x, hkv = blockIdx.y;
  const int b = P.row_order != nullptr ? min(max(P.row_order[blockIdx.z], 0), (int)gridDim.z - 1) : (int)blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPR, rr = lane / LPR;

  // scores of the chunk's rows per query head; the rows of the G heads are
  // kScPad floats apart beyond a multiple of 64 banks, so the G lanes of a key
  // row that store its G scores hit different banks
  __shared__ float sc[G][kMaxRows + kScPad];
  __shared__ float red[kDecWaves][G];
  __shared__ float osum[kDecWaves][G][D];

  // block list of this sequence (row q-tile 0 of its BlockMask)
  const BlockMaskView& bm = p.bm;
  int n_part, n_full;
  const int* part_idx = nullptr;
  const int* full_idx = nullptr;
  if (bm.dense) {
    n_part = 0;
    n_full = bm.NK;
  } else {
    const int mb = bm.Bm > 1 ? b : 0, mh = bm.Hm > 1 ? hkv * G : 0;
    const long long row = ((long long)mb * bm.Hm + mh) * bm.NQ;
    n_part = bm.kv_num[row];
    part_idx = bm.kv_idx + row * bm.NK;
    if (bm.separate_full) {
      n_full = bm.full_num[row];
      full_idx = bm.full_idx + row * bm.NK;
    } else {
      n_full = 0;
    }
  }
  const int T = n_part + n_full;
  // Tiles are dealt to the splits round-robin (split s takes list entries s,
  // s + splits, ...), so the workgroups that run together read neighbouring
  // tiles instead of addresses a power-of-two stride apart.
  const int n_tiles = T > split ? (T - split + P.splits - 1) / P.splits : 0;
  const long long ws_row0 = ((long long)b * p.Hq + (long long)hkv * G) * P.splits + split;
  if (n_tiles == 0) {  // empty chunk: LSE -inf and a zero row, so the merge needs no branch
    for (int i = tid; i < G * D; i += kDecThreads)
      P.ws_o[(ws_row0 + (long long)(i / D) * P.splits) * D + i % D] = 0.0f;
    if (tid < G) P.ws_lse[ws_row0 + (long long)tid * P.splits] = -INFINITY;
    return;
  }
  const int n_rows = n_tiles * FA_BLOCK;
  // First key of each of this chunk's tiles and whether the tile is partial,
  // looked up once (the row loads below then depend on no global read).
  // With a paged cache (paper review §4.5) the tile's rows come from the page
  // the table gives for its logical block; the mods keep the logical key.
  // (A template parameter, so the per-sequence-cache kernel carries none of it.)
  __shared__ int s_kv0[kMaxBps];
  __shared__ int s_part[kMaxBps];
  __shared__ long long s_koff[kMaxBps], s_voff[kMaxBps];  // first row of the tile, elements from Kp / Vp
  if (tid < n_tiles) {
    const int t = split + tid * P.splits;
    const int kb = t < n_part ? part_idx[t] : (bm.dense ? t - n_part : full_idx[t - n_part]);
    s_kv0[tid] = kb * FA_BLOCK;
    s_part[tid] = t < n_part;
    if constexpr (PAGED) {
      const int pg = min(max(P.page_table[(long long)b * P.pt_stride + kb], 0), P.num_pages - 1);
      s_koff[tid] = (long long)pg * p.ks[0];
      s_voff[tid] = (long long)pg * p.vs[0];
    }
  }

  const uint16_t* Kp = p.k + (PAGED ? 0LL : (long long)b * p.ks[0]) + (long long)hkv * p.ks[1];
  const uint16_t* Vp = p.v + (PAGED ? 0LL : (long long)b * p.vs[0]) + (long long)hkv * p.vs[1];

  // query slices (8 dims per lane) of the G heads
  float qf[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint16_t* Qp = p.q + (long long)b * p.qs[0] + (long long)(hkv * G + g) * p.qs[1];
    unpack8(*(const u32x4_t*)(Qp + 8 * sub), qf[g]);
  }
  // the query's position in its sequence: the q index the mods see
  const int qpos = P.q_pos != nullptr ? P.q_pos[b] : 0;
  typename Score::Row srow[G];
#pragma unroll
  for (int g = 0; g < G; ++g) srow[g] = Score::row(p.score, b, hkv * G + g, qpos);
  __syncthreads();

  // An iteration covers STEP consecutive rows of the chunk (inside one tile):
  // lane group rr of wave w holds rows u * RSTEP + w * RPW + rr, u < U.  The
  // next iteration's rows are loaded while the current ones are used.  Each
  // K/V row is read once per call, so the loads are non-temporal (+5% here).
  constexpr int U = 4;
  constexpr int STEP = RSTEP * U;
  static_assert(FA_BLOCK % STEP == 0, "an iteration stays inside one tile");
  const int my_row = wave * RPW + rr;
  auto load_rows = [&](const uint16_t* X, long long xs, bool v_rows, int base, u32x4_t (&x)[U]) {
    const int t = base / FA_BLOCK, r0 = base % FA_BLOCK + my_row;
    const int kv0 = s_kv0[t] + r0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kv = kv0 + u * RSTEP;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if constexpr (PAGED) {  // row r0 + u RSTEP of the tile's page
        const uint16_t* Xt = X + (v_rows ? s_voff[t] : s_koff[t]);
        if (kv < p.Skv) v = __builtin_nontemporal_load((const u32x4_t*)(Xt + (long long)(r0 + u * RSTEP) * xs + 8 * sub));
      } else {
        if (kv < p.Skv) v = __builtin_nontemporal_load((const u32x4_t*)(X + (long long)kv * xs + 8 * sub));
      }
      x[u] = v;
    }
  };

  // ---- pass 1: scores ---------------------------------------------------------
  auto score_rows = [&](int base, const u32x4_t (&kx)[U]) {
    const int kv0 = s_kv0[base / FA_BLOCK] + base % FA_BLOCK + my_row;
    const bool part = s_part[base / FA_BLOCK];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rl = base + u * RSTEP + my_row;
      const int kv = kv0 + u * RSTEP;
      float kf[8];
      unpack8(kx[u], kf);
      float dot[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaf(qf[g][j], kf[j], a);
        dot[g] = group_sum<LPR>(a);
      }
      bool keep = kv < p.Skv;
      if (keep && part) {
        EvalMask em{p.mask, b, hkv * G, qpos, kv, false};
        dispatch_mask(P.mask_kind, em);
        keep = em.result;
      }
      if (sub < G) {
        float x = -INFINITY;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if (g == sub && keep) x = Score::apply1(srow[g], dot[g], kv, 0);
        }
        sc[sub][rl] = x;
      }
    }
  };
  u32x4_t xa[U], xb[U];
  load_rows(Kp, p.ks[2], false, 0, xa);
  for (int base = 0; base < n_rows; base += 2 * STEP) {
    const bool second = base + STEP < n_rows;
    if (second) load_rows(Kp, p.ks[2], false, base + STEP, xb);
    score_rows(base, xa);
    if (second) {
      if (base + 2 * STEP < n_rows) load_rows(Kp, p.ks[2], false, base + 2 * STEP, xa);
      score_rows(base + STEP, xb);
    }
  }
  __syncthreads();
  // the first V rows in flight during pass 2: two groups with a per-sequence
  // cache (+1%); one with a paged cache, whose kernel would otherwise need
  // more than 128 registers and lose a wave per SIMD (-10%)
  constexpr bool V2 = !PAGED;
  load_rows(Vp, p.vs[2], true, 0, xa);
  if (V2 && STEP < n_rows) load_rows(Vp, p.vs[2], true, STEP, xb);

  // ---- pass 2: per-head max, exponentials, sums --------------------------------
  float m[G], l[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float v = -INFINITY;
    for (int i = tid; i < n_rows; i += kDecThreads) v = fmaxf(v, sc[g][i]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (lane == 0) red[wave][g] = v;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float v = red[0][g];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) v = fmaxf(v, red[w][g]);
    m[g] = v;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float mu = m[g] == -INFINITY ? 0.0f : m[g];
    float s = 0.0f;
    for (int i = tid; i < n_rows; i += kDecThreads) {
      const float e = __builtin_amdgcn_exp2f(sc[g][i] - mu);
      sc[g][i] = e;
      s += e;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) red[wave][g] = s;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) v += red[w][g];
    l[g] = v;
  }

  // ---- pass 3: P.V ------------------------------------------------------------
  float o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < 8; ++j) o[g][j] = 0.0f;
  auto pv_rows = [&](int base, const u32x4_t (&vx)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rl = base + u * RSTEP + my_row;
      float vf[8];
      unpack8(vx[u], vf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pg = sc[g][rl];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] = fmaf(pg, vf[j], o[g][j]);
      }
    }
  };
  for (int base = 0; base < n_rows; base += 2 * STEP) {
    const bool second = base + STEP < n_rows;
    if (second && (!V2 || base > 0)) load_rows(Vp, p.vs[2], true, base + STEP, xb);
    pv_rows(base, xa);
    if (second) {
      if (base + 2 * STEP < n_rows) load_rows(Vp, p.vs[2], true, base + 2 * STEP, xa);
      pv_rows(base + STEP, xb);
    }
  }
  // sum over the row groups of the wave, then over waves
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) o[g][j] += __shfl_xor(o[g][j], off);
  }
  if (rr == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) osum[wave][g][8 * sub + j] = o[g][j];
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kDecThreads) {
    const int g = i / D, d = i % D;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) v += osum[w][g][d];
    const long long wr = ws_row0 + (long long)g * P.splits;
    P.ws_o[wr * D + d] = l[g] > 0.0f ? v / l[g] : 0.0f;
    if (d == 0) P.ws_lse[wr] = l[g] > 0.0f ? m[g] + __log2f(l[g]) : -INFINITY;
  }
}

// One 256-thread workgroup per (b, query head).  The splits are shared out
// over 256 / D groups of D threads (thread = one output dim), each group
// walking every (256 / D)-th split, so several partial rows are read at once.
template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_merge_kernel(DecodeParams P) {
  constexpr int NG = kDecThreads / D;
  const FwdParams& p = P.f;
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = tid % D, grp = tid / D;
  const int b = bh / p.Hq, hq = bh % p.Hq;
  const float* lse = P.ws_lse + (long long)bh * P.splits;
  const float* ws = P.ws_o + (long long)bh * P.splits * D;
  __shared__ float red[kDecWaves];
  __shared__ float part[2][NG][D];

  float m = -INFINITY;
  for (int s = tid; s < P.splits; s += kDecThreads) m = fmaxf(m, lse[s]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) m = fmaxf(m, red[w]);

  float acc = 0.0f, tot = 0.0f;
  if (m > -INFINITY) {
    // every split wrote its row (zeros for an empty one), so the loads are
    // independent of the weights and can all be in flight together
#pragma unroll 8
    for (int s = grp; s < P.splits; s += NG) {
      const float ls = lse[s];
      const float w = ls == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ls - m);
      tot += w;
      acc = fmaf(w, ws[(long long)s * D + d], acc);
    }
  }
  part[0][grp][d] = acc;
  part[1][grp][d] = tot;
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int g = 1; g < NG; ++g) {
      acc += part[0][g][d];
      tot += part[1][g][d];
    }
    const float out = tot > 0.0f ? acc / tot : 0.0f;
    uint16_t* Op = p.o + (long long)b * p.os[0] + (long long)hq * p.os[1];
    Op[d] = __builtin_bit_cast(uint16_t, (__bf16)out);
    if (p.lse != nullptr && d == 0)
      p.lse[(long long)b * p.Hq + hq] = tot > 0.0f ? (m + __log2f(tot)) * kLn2 : -INFINITY;
  }
}

template <int D, int G>
struct LaunchDecode {
  const DecodeParams& P;
  hipStream_t stream;
  template <class Score>
  void operator()() {
    dim3 grid(P.splits, P.f.Hkv, P.f.B);
    if (P.page_table != nullptr)
      hipLaunchKernelGGL((decode_partial_kernel<D, G, Score, true>), grid, dim3(kDecThreads), 0, stream, P);
    else
      hipLaunchKernelGGL((decode_partial_kernel<D, G, Score, false>), grid, dim3(kDecThreads), 0, stream, P);
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(P.f.B * P.f.Hq), dim3(kDecThreads), 0, stream, P);
  }
};

template <int D, int G>
bool launch_dg(int score_kind, const DecodeParams& P, hipStream_t stream) {
  LaunchDecode<D, G> l{P, stream};
  return dispatch_score(score_kind, l);
}

template <int D>
bool launch_d(int G, int score_kind, const DecodeParams& P, hipStream_t stream) {
  switch (G) {
    case 1: return launch_dg<D, 1>(score_kind, P, stream);
    case 2: return launch_dg<D, 2>(score_kind, P, stream);
    case 4: return launch_dg<D, 4>(score_kind, P, stream);
    case 8: return launch_dg<D, 8>(score_kind, P, stream);
    default: return false;
  }
}

}  // namespace

fa_status launch_decode(int D, int G, int score_kind, const DecodeParams& P, hipStream_t stream) {
  bool ok;
  if (D == 128)
    ok = launch_d<128>(G, score_kind, P, stream);
  else if (D == 64)
    ok = launch_d<64>(G, score_kind, P, stream);
  else
    return FA_ERR_UNSUPPORTED;
  if (!ok) return FA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int decode_max_blocks_per_split() { return kMaxBps; }

// The workspace of fa_decode_noalloc: a device array of the library, one per
// GPU.  Host code never passes its name to a kernel (on the host the name
// stands for a host-side shadow, not a device address): the device address is
// looked up with hipGetSymbolAddress on the first call on each device, with
// that device current, and kept per device.
static __device__ __align__(256) float scratch[FA_DECODE_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

fa_status decode_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace fa
