// Fused block-sparse attention forward for CDNA4 (gfx950).
//
// Computes O = softmax(mod(Q K^T * scale)) V (paper review "Flex Attention:
// A Programming Model for Generating Optimized Attention Kernels", §2.1) with
// online softmax (§3.3), skipping empty tiles through the BlockMask and
// evaluating the mask_mod only on partial tiles (§4.2; attention-gym
// "Concepts" page, "BlockMask Internals"), walking the tile lists indirectly
// (§4.3).
//
// Work decomposition: one 256-thread workgroup (4 waves) per (b, hq, 128-row
// query tile); wave w owns query rows 32w..32w+31.  Two workgroups share a CU
// (<= 256 registers per lane, 80 KiB of LDS each at D=128), so one workgroup's
// LDS waits and barriers are covered by the other.
//
// MFMA orientation.  Both products are computed transposed so that every
// lane owns exactly one query row (lane % 32) in both accumulators:
//   S^T[kv, q] = K[kv, :] . Q[q, :]      (A = K tile from LDS, B = Q^T in registers)
//   O^T[d, q] += V^T[d, kv] . P^T[kv, q] (A = V^T read transposed from LDS, B = P^T)
// with v_mfma_f32_32x32x16_bf16.  In a 32x32 accumulator lane l holds column
// l % 32 and rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.  So the softmax row
// max and row sum reduce over the lane's own values plus one swap with lane
// l ^ 32, the O rescale is a per-lane scalar, and the P values leave the S
// accumulator already laid out as the B operand of the PV product: the 16
// keys of a PV k-step sit in lane half h at kv = 4h + {0..3} and 8 + 4h + {0..3}.
// The matching V^T operand comes from row-major V in LDS through
// ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i % 4
// of the 8-byte row pointed to by lane 4j + i/4 (j = 0..3), so lanes pointing
// at a 4-key x 16-dim block of V receive one dim each across the 4 keys.
//
// Software pipeline.  Step j of a wave does the PV product of sub-tile j-1,
// the QK^T product of sub-tile j+1 and the softmax of sub-tile j, in one of
// two orders (chosen per score at compile time):
//  * phased (scores of a few VALU operations per element): the 32 MFMAs of the
//    step first, back to back at raised wave priority with their LDS operands
//    read four MFMAs ahead, then the softmax VALU at normal priority.  The two
//    waves of a SIMD come from different workgroups: while one is in its MFMA
//    stretch the other's VALU issues beside it, and the priority lets the
//    MFMAs go first whenever both are ready.  A wave that mixed the two would
//    hold its own VALU behind every MFMA that waits for the matrix pipe.
//  * interleaved (softcap, with two more transcendentals per score, and the
//    dynamic bias, whose LDS tile reads would sit in the VALU stretch): the
//    score VALU of j beside the PV MFMAs of j-1, the exponentials of j beside
//    the QK^T MFMAs of j+1, so a wave's own MFMAs cover its VALU.
//
// Data movement: K and V sub-tiles go from global memory straight into LDS
// with 16-byte global_load_lds (no registers), row-major with the 16-byte
// chunks of each row XOR-swizzled (bank-conflict-free reads, see
// k_swizzle/v_swizzle), in a 2-deep K ring and a 3-deep V ring.
#pragma once

#include <type_traits>

#include "mods.hpp"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;

constexpr int kFwdThreads = 256;
constexpr int kBM = FA_BLOCK;  // query rows per workgroup
constexpr int kBN = FA_BLOCK;  // keys per tile
// Lazy rescaling: the running max used for the exponentials is only raised
// when a tile's max exceeds it by more than this (base-2 units), so the
// exponentials stay <= 2^8 and the O rescale is skipped for most tiles.
constexpr float kRescaleSlack = 8.0f;

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Give each
// XCD a contiguous range of logical tile ids, so the query tiles of one head
// (which share K/V) run on the same XCD and hit the same L2.
__device__ __forceinline__ int xcd_logical_id(int bid, int total) {
  const int per = total / 8, rem = total % 8;
  const int x = bid % 8, j = bid / 8;
  return x * per + min(x, rem) + j;
}

// The (b * Hq + hq, query tile) unit of this workgroup.  Without a work order
// the last query tiles start first (longest first for causal, window and prefix
// masks) and each XCD takes a contiguous range of units, so the query tiles of
// a head share its L2.  With the BlockMask's q_order (each row's query tiles
// heaviest first) and B * Hq a multiple of 8, XCD x (workgroup id % 8) takes
// the x-th eighth of the (b, hq) heads, a contiguous block (the query heads of
// a GQA group, which read the same K/V, stay on one XCD), and its m-th
// workgroup runs the (m / heads-per-XCD)-th heaviest tile of one of them:
// every XCD starts the longest units of all its heads first.
__device__ __forceinline__ void query_tile_unit(const FwdParams& p, int NQ, int& bh, int& qb) {
  const int BH = p.Hq * p.B;
  if (p.bm.q_order != nullptr && BH % 8 == 0) {
    const int x = blockIdx.x & 7, m = blockIdx.x >> 3, hpx = BH >> 3;
    const int r = m / hpx;
    bh = x * hpx + (m - r * hpx);
    const int mb = p.bm.Bm > 1 ? bh / p.Hq : 0, mh = p.bm.Hm > 1 ? bh % p.Hq : 0;
    qb = min(max(p.bm.q_order[((long long)mb * p.bm.Hm + mh) * NQ + r], 0), NQ - 1);
  } else {
    const int L = xcd_logical_id(blockIdx.x, NQ * BH);
    bh = L / NQ;
    qb = NQ - 1 - L % NQ;
  }
}

// Waits until at most N vector-memory loads of this wave are outstanding
// (loads complete in issue order, so everything older than the N newest is done).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_address(const void* ptr) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)ptr;
}

// 16 bytes per lane from global memory into LDS at lds + 16 * lane (global_load_lds_dwordx4).
// Written as asm so that the compiler does not insert its own conservative
// vmcnt(0) waits before every LDS read; the kernels wait explicitly instead.
// No register is written by the load, only LDS.  No "memory" clobber (it
// would stop the block-list reads from being scalar loads): ordering against
// LDS reads comes from the volatile wait/barrier statements around it, which
// do clobber memory and which volatile asm cannot be reordered with.
// dma16: 64-bit per-lane address.  dma16s: uniform 64-bit base + 32-bit
// per-lane byte offset (one VGPR per lane).  Both set M0 (the LDS base of the
// DMA), which is declared clobbered.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gaddr), "s"(__builtin_amdgcn_readfirstlane(lds)) : "m0");
}
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds)) : "m0");
}
// The same loads with the non-temporal hint, for data read once (the bias
// tiles): they then do not push reused K/V tiles out of L2 and MALL.
__device__ __forceinline__ void dma16_nt(const void* gaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(gaddr), "s"(__builtin_amdgcn_readfirstlane(lds)) : "m0");
}
__device__ __forceinline__ void dma16s_nt(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds)) : "m0");
}
// N loads of 16 bytes per lane into LDS at lds + 4096 i + 16 lane (i < N), from
// sbase + voff[i]: one uniform base and a per-lane offset per load, so a tile's
// loads cost one scalar address for the tile and an M0 write per load.
template <int N>
__device__ __forceinline__ void dma16n(const uint32_t (&voff)[N], const void* sbase, uint32_t lds) {
#pragma unroll
  for (int i = 0; i < N; ++i) dma16s(voff[i], sbase, lds + 4096 * i);
}

// LDS swizzles (16-byte chunk index XOR a function of the row), chosen per
// read pattern so that each group of lanes served together touches distinct
// banks (64 banks of 4 bytes: a 256-byte window):
//  * K, read with ds_read_b128 by 16 lanes = 16 consecutive rows, one chunk:
//    D=128 (one row per window) XOR row % 16; D=64 (two rows per window)
//    XOR (row / 2) % 8.
//  * V, read with ds_read_b64_tr_b16 by 16 lanes = 4 consecutive rows x two
//    adjacent chunks (and by the wave: 8 rows x 4 chunks):
//    D=128 XOR 4 (row % 4); D=64 XOR 4 ((row / 2) % 2).
template <int D>
__device__ __forceinline__ int k_swizzle(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// Marks a register as produced here, after waiting for the load that wrote
// it: later readers then need no wait of their own (without this the
// compiler, unsure whether a load issued on an earlier iteration is still in
// flight, puts a vmcnt(0) before every read, which also waits for the tile
// loads).
__device__ __forceinline__ void loaded(int& x) { asm volatile("" : "+v"(x)); }

// max(x, x of lane l ^ 32) in every lane, with v_permlane32_swap (swaps the
// upper half of one register with the lower half of another; no LDS access).
// Written as asm: the compiler's builtin for it returns the same register for
// both halves of its result.  The s_nop covers the VALU-write hazard.
__device__ __forceinline__ float max_across_halves(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

template <int D, class Mask, class Score>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int KS = D / 16;                  // k-steps of the QK^T product
  constexpr int DT = D / 32;                  // 32-row blocks of O^T
  constexpr int CPR = D / 8;                  // 16-byte chunks per K/V row
  constexpr int HB = 64;                      // keys per step (half a BlockMask tile)
  constexpr int SPT = kBN / HB;               // steps per BlockMask tile
  constexpr int NI = HB * CPR / 64 / 4;       // 16-byte loads per wave per K or V sub-tile
  constexpr int NK = 2, NV = 3;               // ring depths: K of j+1 / j+2, V of j-1 / j / j+1
  // phased or interleaved step (see the header)
  constexpr bool PH = D == 128 && !Score::kReadsMemory && !std::is_base_of<ScoreSoftcap, Score>::value;
  __shared__ __align__(16) uint16_t k_lds[NK][HB * D];
  __shared__ __align__(16) uint16_t v_lds[NV][HB * D];
  // Bias tiles [128 query rows x 64 keys] of steps j and j+1 (only for the
  // staged bias): row r holds its 8 16-byte chunks c at slot c ^ ((r / 2) % 8),
  // so that of the 32 rows one half-wave reads at a time, 16 fall on distinct
  // bank groups (2-way conflicts where the plain c ^ (r % 8) had 4-way).  Each
  // wave loads and reads only its own 32 rows, so a stage is free again for the
  // wave once it has read it, and the tile of step j+2 goes into the stage of
  // step j with no barrier.  Every bias element is read once per launch, so its
  // loads carry the non-temporal hint and leave L2 and MALL to the K/V tiles.
  constexpr bool BL = Score::kStagesBias;
  __shared__ __align__(16) uint16_t b_lds[BL ? 2 : 1][BL ? kBM * HB : 8];
  // Document ids of sub-tiles j, j+1, j+2 (masks that read them, D = 64, where
  // the 768 bytes fit beside two workgroups' rings): the masked pass then reads
  // them from LDS instead of issuing global loads, whose wait would also wait
  // for the tile loads in flight.
  constexpr bool DL = Mask::kReadsMemory && D == 64;
  __shared__ __align__(16) int doc_lds[DL ? 3 : 1][DL ? HB : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lq = lane & 31, hh = lane >> 5;
  const int gi = lane >> 4, si = lane & 15;

  // ---- which (b, hq, query tile) ------------------------------------------
  const int NQ = (p.Sq + kBM - 1) / kBM;
  int bh, qb;
  query_tile_unit(p, NQ, bh, qb);
  const int hq = bh % p.Hq, b = bh / p.Hq;
  const int hkv = hq / p.G;
  const int q0 = qb * kBM;

  // ---- per-lane query row (its loads first: they overlap the list loads) ----
  const uint16_t* Qp = p.q + (long long)b * p.qs[0] + (long long)hq * p.qs[1];
  const int myq = q0 + wave * 32 + lq;
  const bool q_ok = myq < p.Sq;
  const int qc = q_ok ? myq : p.Sq - 1;  // clamped index for mask/score row state
  bf16x8_t qreg[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4_t raw = {0u, 0u, 0u, 0u};
    if (q_ok) raw = *(const u32x4_t*)(Qp + (long long)myq * p.qs[2] + 16 * s + 8 * hh);
    qreg[s] = __builtin_bit_cast(bf16x8_t, raw);
  }

  // ---- this tile's block lists ----------------------------------------------
  const BlockMaskView& bm = p.bm;
  int n_part, n_full;
  const int* part_idx = nullptr;
  const int* full_idx = nullptr;
  if (bm.dense) {
    n_part = 0;
    n_full = bm.NK;
  } else {
    const int mb = bm.Bm > 1 ? b : 0, mh = bm.Hm > 1 ? hq : 0;
    const long long row = ((long long)mb * bm.Hm + mh) * bm.NQ + qb;
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
  // List entry e of this row (partial tiles, then full tiles; 0 past the end).
  auto list_entry = [&](int e) -> int {
    if (e >= T) return 0;
    if (e < n_part) return part_idx[e];
    return bm.dense ? e - n_part : full_idx[e - n_part];
  };
  // A window of 64 list entries lives in one register (lane i: entry win0 + i)
  // and is read back with readlane, so the per-step block lookups touch no
  // memory and never wait on the tile loads in flight.
  // The first window is loaded without waiting for the counts: both lists'
  // first 64 entries (in bounds: lanes past NK read entry NK-1), then lane e
  // takes partial entry e or full entry e - n_part (moved across lanes).
  int win0 = 0;
  int win;
  {
    const int lc = min(lane, bm.NK - 1);
    const int pw = (!bm.dense) ? part_idx[lc] : 0;
    const int fw = (!bm.dense && bm.separate_full) ? full_idx[lc] : 0;
    const int fs = __shfl(fw, lane - n_part);  // full entry lane - n_part (lanes >= n_part use it)
    win = lane >= T ? 0 : lane < n_part ? pw : (bm.dense ? lane - n_part : fs);
  }
  loaded(win);
  auto kb_of = [&](int t) -> int { return __builtin_amdgcn_readlane(win, t - win0); };

  const char* Kp = (const char*)(p.k + (long long)b * p.ks[0] + (long long)hkv * p.ks[1]);
  const char* Vp = (const char*)(p.v + (long long)b * p.vs[0] + (long long)hkv * p.vs[1]);
  const long long ksb = 2 * p.ks[2], vsb = 2 * p.vs[2];  // row strides in bytes

  // ---- global -> LDS sub-tile loads -------------------------------------------
  // Sub-tile j = keys [64 (j % 2), 64 (j % 2) + 64) of BlockMask tile kb_of(j / 2);
  // K of j lives in K stage j % 2, V of j in V stage j % 3.  LDS slot s (16 bytes)
  // of a stage holds row s / CPR, logical chunk (s % CPR) ^ swizzle(row); wave w
  // issues slots [64 (4i + w), +64) for i < NI.  Rows past Skv re-read row Skv-1
  // (finite values whose scores are masked to -inf).  Within one instruction the
  // 64 lanes cover 64 / CPR consecutive rows and the swizzled chunk of a lane does
  // not depend on i, so one per-lane byte offset plus a uniform row step per
  // instruction addresses every load.
  constexpr int RPI = 64 / CPR;
  const int lrow = wave * RPI + lane / CPR;
  const int kchunk = (lane % CPR) ^ k_swizzle<D>(lrow);
  const int vchunk = (lane % CPR) ^ v_swizzle<D>(lrow);
  // per-lane byte offsets of the wave's NI loads inside a sub-tile (row strides
  // below 2^26 bytes are checked by the host, so they fit 32 bits)
  const uint32_t ksb32 = (uint32_t)ksb, vsb32 = (uint32_t)vsb;
  uint32_t k_vo[NI], v_vo[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    k_vo[i] = (uint32_t)(lrow + 4 * RPI * i) * ksb32 + 16 * kchunk;
    v_vo[i] = (uint32_t)(lrow + 4 * RPI * i) * vsb32 + 16 * vchunk;
  }
  auto issue_one = [&](const char* g, long long rsb, const uint16_t* buf, int lchunk, const uint32_t (&vo)[NI], int kv0) {
    const uint32_t base = lds_address(buf) + 16 * 64 * wave;
    if (kv0 + HB <= p.Skv) {
      const char* g0 = g + (uint64_t)(uint32_t)kv0 * (uint32_t)rsb;
      dma16n<NI>(vo, g0, base);
    } else {
      const int last = p.Skv - 1 - kv0;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int rr = min(lrow + 4 * RPI * i, last);
        dma16(g + (kv0 + rr) * rsb + 16 * lchunk, base + 16 * 64 * 4 * i);
      }
    }
  };
  auto kv0_of = [&](int j) { return kb_of(j / SPT) * kBN + HB * (j % SPT); };
  // Document ids of sub-tile j -> doc_lds[j % 3]: 16 lanes of wave 0, 16 bytes
  // each, when the ids are 16-byte aligned and the sub-tile is whole (else the
  // masked pass reads them from global memory).
  const int* doc_row = nullptr;
  if constexpr (DL) doc_row = p.mask.doc + (long long)b * p.mask.doc_stride_b;
  auto issue_k = [&](int j, int jm) {
    issue_one(Kp, ksb, k_lds[jm % NK], kchunk, k_vo, kv0_of(j));
    if constexpr (DL) {
      const int kv0 = kv0_of(j);
      if (p.mask.doc_vec && wave == 0 && kv0 + HB <= p.Skv) {
        if (lane < HB / 4) dma16(doc_row + kv0 + 4 * lane, lds_address(doc_lds[jm % 3]));
      }
    }
  };
  auto issue_v = [&](int j, int jm) { issue_one(Vp, vsb, v_lds[jm % NV], vchunk, v_vo, kv0_of(j)); };
  // Bias tile of sub-tile j -> b_lds[j % 2]: wave w issues slots 64 (4w + i) + lane
  // (i < 4), i.e. row 32 w + 8 i + lane / 8, stored slot lane % 8 holding chunk
  // (lane % 8) ^ ((row / 2) % 8) = (lane % 8) ^ (lane / 16) ^ (4 (i % 2)).
  const int b_row = lane >> 3;  // + 32 w + 8 i
  const int bc0 = (lane & 7) ^ (lane >> 4);  // chunk for even i (odd i: bc0 ^ 4)
  const char* Bbh = nullptr;
  long long bsb = 0;  // bias row stride in bytes
  uint32_t b_voff0 = 0, b_voff1 = 0;
  if constexpr (BL) {
    Bbh = (const char*)(p.score.bias + (long long)b * p.score.bs0 + (long long)hq * p.score.bs1);
    bsb = 2 * p.score.bs2;
    b_voff0 = (uint32_t)(b_row * bsb + 16 * bc0);
    b_voff1 = (uint32_t)(b_row * bsb + 16 * (bc0 ^ 4));
  }
  constexpr int NB = 4;  // bias loads per wave per sub-tile
  auto issue_b = [&](int j, int jm) {
    if constexpr (BL) {
      const int kv0 = kv0_of(j);
      const uint32_t base = lds_address(b_lds[jm % 2]) + 16 * 64 * 4 * wave;
      const int r0 = q0 + 32 * wave;  // first row of the wave
      if (r0 + 32 <= p.Sq && kv0 + HB <= p.Skv) {
        const char* g0 = Bbh + (long long)r0 * bsb + 2 * kv0;
#pragma unroll
        for (int i = 0; i < NB; ++i) dma16s_nt((i & 1) ? b_voff1 : b_voff0, g0 + 8 * i * bsb, base + 16 * 64 * i);
      } else {  // ragged: clamp rows to Sq-1 and chunks to the last one of the row
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int q = min(r0 + 8 * i + b_row, p.Sq - 1);
          const int kc = min(kv0 + 8 * (bc0 ^ (4 * (i & 1))), p.Skv - 8);
          dma16_nt(Bbh + (long long)q * bsb + 2 * kc, base + 16 * 64 * i);
        }
      }
    }
  };
  auto k_off = [](int r, int chunk) { return r * D + ((chunk ^ k_swizzle<D>(r)) * 8); };
  auto v_off = [](int r, int chunk) { return r * D + ((chunk ^ v_swizzle<D>(r)) * 8); };

  const auto mrow = Mask::row(p.mask, b, hq, qc);
  const auto srow = Score::row(p.score, b, hq, qc);
  // Starting value of every QK^T accumulation: zero, or the score's key-offset
  // term (the same for every lane and both 32-key blocks).
  f32x16_t acc0 = f32x16_t{};
  if constexpr (Score::kPreload) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc0[r] = Score::preload(srow, 8 * (r >> 2) + (r & 3));
  }

  // ---- online softmax state (base-2 units) ----------------------------------
  f32x16_t oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16_t{};
  // Reference max of the exponentials: -inf until the row sees a finite score,
  // then only raised when a score exceeds it by more than kRescaleSlack.  Scores
  // are produced relative to it (y = x2 - m_run), so exp2(y) needs no subtraction.
  float m_run = -INFINITY;
  if constexpr (Score::kBounded) m_run = Score::bound(srow);  // fixed reference: no running max
  // This lane's half of the row sum, in four fp32 partial sums of the
  // exponentials (plain adds: on gfx950 a v_dot2 instruction cannot run while
  // an MFMA is in flight, a v_add can).
  float l_run[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

  // Per-lane element offsets of the MFMA operands inside a K or V stage.  The
  // swizzle only depends on the row bits that belong to the lane (32-row
  // blocks of K, 16-row k-steps and the +8 half of V leave them unchanged), so
  // every read is a per-lane register plus a compile-time offset, and a stage
  // change costs one add per register.
  int koff[KS];  // QK A operand, k-step s: row lq (+32 per key block), chunk 2s + hh
#pragma unroll
  for (int s = 0; s < KS; ++s) koff[s] = k_off(lq, 2 * s + hh);
  int voff[DT];  // PV A operand, d block dt: rows 4hh + si/4 (+16 per k-step, +8 for the upper half)
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int d = 32 * dt + 16 * (gi & 1) + 4 * (si & 3);
    voff[dt] = v_off(4 * hh + (si >> 2), d >> 3) + (d & 7);
  }

  // Operand reads take a stage's per-lane byte addresses (one register per k-step
  // of K, one per d block of V, set once per step) plus compile-time offsets.
  uint32_t kaddr[KS], vaddr[DT];
  auto set_k_stage = [&](const uint16_t* kl) {
#pragma unroll
    for (int s = 0; s < KS; ++s) kaddr[s] = lds_address(kl) + 2 * koff[s];
  };
  auto set_v_stage = [&](const uint16_t* vl) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vaddr[dt] = lds_address(vl) + 2 * voff[dt];
  };
  // MFMA i (0..2*KS-1) of S^T = K Q^T for a 64-key sub-tile: (32-key block i % 2, k-step i / 2).
  // The two key blocks alternate, so consecutive MFMAs accumulate into different
  // registers: two independent chains instead of one 8-long chain per block.
  auto qk_mfma = [&](f32x16_t (&acc)[2], int i) {
    const int mt = i & 1, s = i >> 1;
    const bf16x8_t a = ((const lds_bf16x8_t*)(uintptr_t)kaddr[s])[mt * 32 * D / 8];
    acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], s == 0 ? acc0 : acc[mt], 0, 0, 0);
  };
  // MFMA i (0..4*DT-1) of O^T += V^T P^T: (16-key k-step i / DT of the sub-tile, d block i % DT).
  // V^T comes from row-major V through ds_read_b64_tr_b16.
  auto pv_mfma = [&](const bf16x8_t (&pb)[4], int i) {
    const int ks = i / DT, dt = i % DT;
    lds_bf16x4_t* vr = (lds_bf16x4_t*)(uintptr_t)vaddr[dt];
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(vr + ks * 16 * D / 4);
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(vr + (ks * 16 + 8) * D / 4);
    const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], oacc[dt], 0, 0, 0);
  };

  // Software pipeline (per wave), step j:
  //   (phased: O += PV of sub-tile j-1 and S = QK^T of sub-tile j+1, MFMAs only)
  //   B: score_mod / mask / row max of sub-tile j     (interleaved: with O += PV of j-1)
  //   C: (rare) raise the reference max: rescale O (which now includes j-1) and the scores
  //   D: P = exp2(scores) of sub-tile j, row sums     (interleaved: with S = QK^T of j+1)
  // Loads run ahead: K of j+2 and V of j+1 are issued at the start of step j.
  const int J = SPT * T;
  if (J > 0) {
    // V stage 2 stands in for "sub-tile -1" (P = 0) at step 0: clear it
    {
      u32x4_t* vz = (u32x4_t*)v_lds[NV - 1];
      for (int i = tid; i < HB * D / 8; i += kFwdThreads) vz[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
    // The bias tile of sub-tile j is issued two steps ahead (in step j-2, once
    // the wave has read its rows of that stage); in the issue order it sits
    // after K(j) and V(j-1).
    constexpr int NBI = BL ? NB : 0;
    issue_k(0, 0);
    issue_b(0, 0);
    if (J > 1) issue_k(1, 1);
    issue_v(0, 0);
    if (J > 1) issue_b(1, 1);
    if (J > 1)
      wait_vmcnt<2 * NI + NBI>();  // K(0) and the bias of 0 landed (K(1), V(0), bias of 1 may be in flight)
    else
      wait_vmcnt<NI>();
    wait_lds_reads();
    __syncthreads();
    f32x16_t s_a[2], s_b[2];  // (each accumulation starts from acc0)
    set_k_stage(k_lds[0]);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) qk_mfma(s_a, i);
    bf16x8_t p_prev[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p_prev[i] = bf16x8_t{};

    f32x16_t (&s_cur)[2] = s_a;
    f32x16_t (&s_nxt)[2] = s_b;
    // The loop is unrolled by 6 (the least common multiple of the ring depths), so
    // every LDS stage is a compile-time constant: operand reads take it in their
    // immediate offset and the DMA its M0 value.
    auto step = [&](const int j, auto jmc) __attribute__((always_inline)) {
      constexpr int JM = decltype(jmc)::value;
      const int H = JM % SPT;
      // K(j+1), V(j-1) and the bias of j landed for every wave (only V(j) and
      // the bias of j+1 may be in flight), and every wave is done with step
      // j-1: K stage j % 2 and V stage (j+1) % 3 are free.
      if (j + 1 < J)
        wait_vmcnt<NI + NBI>();
      else
        wait_vmcnt<NI>();
      wait_lds_reads();
      __builtin_amdgcn_s_barrier();
      const int t = j / SPT;
      if (t + 1 >= win0 + 64) {  // slide the block-list window (every 64 tiles)
        win0 = t;
        win = list_entry(t + lane);
        loaded(win);
      }
      if (j + 2 < J) issue_k(j + 2, (JM + 2) % 6);
      if (j + 1 < J) issue_v(j + 1, (JM + 1) % 6);

      const int kvt0 = kb_of(t) * kBN + HB * H;
      const bool partial = t < n_part;
      const bool ragged = kvt0 + HB > p.Skv;
      set_v_stage(v_lds[(JM + NV - 1) % NV]);  // V of j-1
      set_k_stage(k_lds[(JM + 1) % NK]);       // K of j+1 (stale on the last step: result unused)

      // ---- phased: PV of j-1 and QK^T of j+1, MFMAs only, at raised priority
      if constexpr (PH) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < 4 * DT; ++i) pv_mfma(p_prev, i);
#pragma unroll
        for (int i = 0; i < 2 * KS; ++i) qk_mfma(s_nxt, i);
        // Instruction order: every MFMA's operands are read PF MFMAs ahead (two
        // ds_read_b64_tr_b16 for a PV MFMA, one ds_read_b128 for a QK^T MFMA).
        // Masks: 0x008 MFMA, 0x100 LDS read.
        constexpr int PF = 4, NPV = 4 * DT, NQK = 2 * KS;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
        for (int i = 0; i < NPV + NQK; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          const int r = i + PF;  // the MFMA whose operands are read now
          if (r < NPV)
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          else if (r < NPV + NQK)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // the softmax VALU stays after the MFMAs
        __builtin_amdgcn_s_setprio(0);
      }

      // ---- B: scores of j  (interleaved: || PV of j-1)
      // Element (mt, r) of this lane holds key kvb + cr, cr = 32 mt + 8 (r/4) + r%4.
      const int kvb = kvt0 + 4 * hh;
      const float m_ref = m_run == -INFINITY ? 0.0f : m_run;
      const auto st = Score::tile(srow, kvb, m_ref);
      const int lim = ragged ? p.Skv - kvb : HB;  // key kvb + cr exists iff cr < lim
      float ymax = -INFINITY;
      // staged bias: chunk g (keys 8g..8g+7) of this lane's row, half hh
      uint32_t bias2[8][2];
      if constexpr (BL) {
        const int br = 32 * wave + lq;
        const uint32_t rowa = lds_address(b_lds[JM % 2]) + 128 * br + 8 * hh;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const uint64_t w =
              *(const __attribute__((address_space(3))) uint64_t*)(uintptr_t)(rowa + 16 * (g ^ ((br >> 1) & 7)));
          bias2[g][0] = (uint32_t)w;
          bias2[g][1] = (uint32_t)(w >> 32);
        }
        // once the wave's rows are in registers (the first LDS reads of the
        // step: nothing else to wait for), its stage takes the tile of j+2
        if (j + 2 < J) {
          wait_lds_reads();
          issue_b(j + 2, (JM + 2) % 6);
        }
      }
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int mt = e >> 4, r = e & 15;
        const int cr = 32 * mt + 8 * (r >> 2) + (r & 3);
        float y;
        if constexpr (BL) {  // element (mt, r) is component r % 4 of chunk 4 mt + r / 4
          const uint32_t w = bias2[4 * mt + (r >> 2)][(r >> 1) & 1];
          y = Score::apply_bits(st, s_cur[mt][r], (r & 1) ? (w >> 16) : (w & 0xffffu));
        } else if constexpr (Score::kPreload) {  // the key-offset term within the block is in the accumulator
          y = Score::apply_pre(st, s_cur[mt][r], mt);
        } else {
          // functors that read memory get an in-bounds key on the ragged tile
          y = Score::apply(st, s_cur[mt][r], Score::kReadsMemory ? min(cr, lim - 1) : cr);
        }
        s_cur[mt][r] = y;
        if constexpr (!Score::kBounded) ymax = fmaxf(ymax, y);
        if constexpr (!PH) {
          if ((e & 1) && (e >> 1) < 4 * DT) pv_mfma(p_prev, e >> 1);
        }
      }
      // Keep the row max of the unmasked scores here, beside the PV MFMAs: left
      // alone, the compiler moves it (and a copy of every score register) past
      // the masked-pass branch, where no MFMA is in flight to cover it.
      if constexpr (!Score::kBounded) asm volatile("" : "+v"(ymax));

      if (partial || ragged) {  // mask_mod on partial tiles, keys past Skv on the ragged tile
        const auto mtl = Mask::tile(mrow, kvb);
        ymax = -INFINITY;
        auto put = [&](int e, bool keep) {  // element e kept or set to -inf, and the row max
          const int mt = e >> 4, r = e & 15;
          const float y = keep ? s_cur[mt][r] : -INFINITY;
          s_cur[mt][r] = y;
          if constexpr (!Score::kBounded) ymax = fmaxf(ymax, y);
        };
        if (Mask::kReadsMemory && DL && p.mask.doc_vec && !ragged) {
          // Document ids from LDS in runs of 4 keys (16 bytes) per lane: all 8
          // runs are read first, then every element is decided and applied at
          // once (a whole tile here, so only the mask decides; a partial tile,
          // since the tile is not ragged).
          typedef int i32x4_t __attribute__((ext_vector_type(4)));
          const uint32_t ids0 = lds_address(doc_lds[DL ? JM % 3 : 0]) + 16 * hh;  // keys kvb = kvt0 + 4 hh
          i32x4_t v[8];
#pragma unroll
          for (int g = 0; g < 8; ++g)  // keys kvb + 32 (g / 4) + 8 (g % 4) + {0..3}
            v[g] = *(const __attribute__((address_space(3))) i32x4_t*)(uintptr_t)(ids0 + 4 * (32 * (g >> 2) + 8 * (g & 3)));
          // (wave-uniform: the parts that read no memory, e.g. causal, decide
          // nothing on the wave's rows x this sub-tile's keys)
          const int wq0 = min(q0 + 32 * wave, p.Sq - 1), wq1 = min(q0 + 32 * wave + 31, p.Sq - 1);
          if (MaskParts<Mask>::rest_full(p.mask, b, hq, wq0, wq1, kvt0, kvt0 + HB - 1)) {
#pragma unroll
            for (int g = 0; g < 8; ++g) {  // elements 4 g .. 4 g + 3
              const int ids[4] = {v[g][0], v[g][1], v[g][2], v[g][3]};
              bool k4[4];
              MaskParts<Mask>::keep4_mem(mtl, 32 * (g >> 2) + 8 * (g & 3), ids, k4);
#pragma unroll
              for (int i = 0; i < 4; ++i) put(4 * g + i, k4[i]);
            }
          } else {
#pragma unroll
            for (int g = 0; g < 8; ++g) {
              const int ids[4] = {v[g][0], v[g][1], v[g][2], v[g][3]};
              bool k4[4];
              Mask::keep4(mtl, 32 * (g >> 2) + 8 * (g & 3), ids, k4);
#pragma unroll
              for (int i = 0; i < 4; ++i) put(4 * g + i, k4[i]);
            }
          }
        } else if constexpr (Mask::kReadsMemory) {
          // A mask that reads memory (document ids) from global memory is
          // evaluated for every element first, in-bounds and without branches,
          // so all its loads are in flight at once.
          bool mk[32];
#pragma unroll
          for (int e = 0; e < 32; ++e) {
            const int mt = e >> 4, r = e & 15;
            mk[e] = Mask::keep(mtl, min(32 * mt + 8 * (r >> 2) + (r & 3), lim - 1));
          }
#pragma unroll
          for (int e = 0; e < 32; ++e) {
            const int mt = e >> 4, r = e & 15;
            const int cr = 32 * mt + 8 * (r >> 2) + (r & 3);
            put(e, cr < lim && (mk[e] || !partial));
          }
        } else {
#pragma unroll
          for (int e = 0; e < 32; ++e) {
            const int mt = e >> 4, r = e & 15;
            const int cr = 32 * mt + 8 * (r >> 2) + (r & 3);
            bool keep = cr < lim;
            if (partial) keep = keep && Mask::keep(mtl, min(cr, lim - 1));
            put(e, keep);
          }
        }
      }

      if constexpr (!PH) {
#pragma unroll
        for (int i = 16; i < 4 * DT; ++i) pv_mfma(p_prev, i);  // (D=128 has 16 PV MFMAs: none left)
      }

      // ---- C: raise the reference max when needed (never for a bounded score)
      if constexpr (!Score::kBounded) ymax = max_across_halves(ymax);
      const bool raise = !Score::kBounded && (ymax > kRescaleSlack || (m_run == -INFINITY && ymax > -INFINITY));
      if (!Score::kBounded && __any(raise)) {
        const float m_new = fmaxf(m_run, m_ref + ymax);
        const float shift = m_new == -INFINITY ? 0.0f : m_ref - m_new;
        const float alpha = m_run == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int k = 0; k < 4; ++k) l_run[k] *= alpha;
#pragma unroll
        for (int i = 0; i < DT; ++i) oacc[i] *= alpha;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) s_cur[mt] += shift;
        m_run = m_new;
      }

      // ---- D: P of j  (interleaved: || S of j+1)
#pragma unroll
      for (int g = 0; g < 4; ++g) {  // 16-key k-step g of the PV product
        const int mt = g >> 1, h8 = 8 * (g & 1);
        bf16x2_t pk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float e0 = __builtin_amdgcn_exp2f(s_cur[mt][h8 + 2 * k]);
          const float e1 = __builtin_amdgcn_exp2f(s_cur[mt][h8 + 2 * k + 1]);
          pk[k][0] = (__bf16)e0;
          pk[k][1] = (__bf16)e1;
          l_run[k] += e0 + e1;
          if constexpr (!PH) {
            if (4 * g + k < 2 * KS) qk_mfma(s_nxt, 4 * g + k);  // D=64 has 8 QK MFMAs
          }
        }
        p_prev[g] = __builtin_shufflevector(__builtin_shufflevector(pk[0], pk[1], 0, 1, 2, 3),
                                            __builtin_shufflevector(pk[2], pk[3], 0, 1, 2, 3),
                                            0, 1, 2, 3, 4, 5, 6, 7);
      }
      if constexpr (!PH) {
#pragma unroll
        for (int i = 16; i < 2 * KS; ++i) qk_mfma(s_nxt, i);  // (D=128 has 16 QK MFMAs: none left)
      }
      s_cur[0] = s_nxt[0];
      s_cur[1] = s_nxt[1];
    };
    typedef std::integral_constant<int, 0> I0;
    typedef std::integral_constant<int, 1> I1;
    typedef std::integral_constant<int, 2> I2;
    typedef std::integral_constant<int, 3> I3;
    typedef std::integral_constant<int, 4> I4;
    typedef std::integral_constant<int, 5> I5;
    for (int j = 0; j < J; j += 6) {
      step(j, I0{});
      if (j + 1 < J) step(j + 1, I1{});
      if (j + 2 < J) step(j + 2, I2{});
      if (j + 3 < J) step(j + 3, I3{});
      if (j + 4 < J) step(j + 4, I4{});
      if (j + 5 < J) step(j + 5, I5{});
    }
    // PV of the last sub-tile
    wait_vmcnt<0>();
    wait_lds_reads();
    __builtin_amdgcn_s_barrier();
    set_v_stage(v_lds[(J - 1) % NV]);
#pragma unroll
    for (int i = 0; i < 4 * DT; ++i) pv_mfma(p_prev, i);
  }

  // ---- epilogue ---------------------------------------------------------------
  const float lh = (l_run[0] + l_run[1]) + (l_run[2] + l_run[3]);
  const float l = lh + __shfl_xor(lh, 32);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  {
    // The lane's row again, from the lane id (mbcnt) and uniform values, so that
    // no per-lane index stays live across the loop for the output address.
    const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int hh = lane_e >> 5;
    const int myq = q0 + wave * 32 + (lane_e & 31);
    const bool q_ok = myq < p.Sq;
    if (q_ok) {
      uint16_t* Op = p.o + (long long)b * p.os[0] + (long long)hq * p.os[1] + (long long)myq * p.os[2];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * dt + 8 * g + 4 * hh;
          bf16x4_t o4;
          o4[0] = (__bf16)(oacc[dt][4 * g + 0] * inv);
          o4[1] = (__bf16)(oacc[dt][4 * g + 1] * inv);
          o4[2] = (__bf16)(oacc[dt][4 * g + 2] * inv);
          o4[3] = (__bf16)(oacc[dt][4 * g + 3] * inv);
          *(bf16x4_t*)(Op + d0) = o4;
        }
      }
      if (p.lse != nullptr && hh == 0) {
        p.lse[((long long)b * p.Hq + hq) * p.Sq + myq] =
            l > 0.0f ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
      }
    }
  }
}

template <int D, class Mask>
struct LaunchFwd {
  const FwdParams& p;
  hipStream_t stream;
  template <class Score>
  void operator()() {
    const int NQ = (p.Sq + kBM - 1) / kBM;
    const long long total = (long long)NQ * p.Hq * p.B;
    if constexpr (std::is_same<Score, ScoreSoftcap>::value) {
      if (p.score.cap_log2 <= kBoundedMaxLog2) {
        hipLaunchKernelGGL((fwd_kernel<D, Mask, ScoreSoftcapBounded>), dim3((unsigned)total), dim3(kFwdThreads), 0,
                           stream, p);
        return;
      }
    }
    if constexpr (std::is_same<Score, ScoreBias>::value) {
      const ScoreParams& s = p.score;
      const bool aligned = ((uintptr_t)s.bias % 16 == 0) && s.bs0 % 8 == 0 && s.bs1 % 8 == 0 &&
                           s.bs2 % 8 == 0 && p.Skv % 8 == 0;
      if (aligned) {
        hipLaunchKernelGGL((fwd_kernel<D, Mask, ScoreBiasTiled>), dim3((unsigned)total), dim3(kFwdThreads), 0,
                           stream, p);
        return;
      }
    }
    hipLaunchKernelGGL((fwd_kernel<D, Mask, Score>), dim3((unsigned)total), dim3(kFwdThreads), 0,
                       stream, p);
  }
};

// Launches the forward for one mask kind, every score kind and both D.
template <class Mask>
fa_status launch_forward_mask(int D, int score_kind, const FwdParams& p, hipStream_t stream) {
  bool ok;
  if (D == 128) {
    LaunchFwd<128, Mask> l{p, stream};
    ok = dispatch_score(score_kind, l);
  } else if (D == 64) {
    LaunchFwd<64, Mask> l{p, stream};
    ok = dispatch_score(score_kind, l);
  } else {
    return FA_ERR_UNSUPPORTED;
  }
  if (!ok) return FA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace fa
