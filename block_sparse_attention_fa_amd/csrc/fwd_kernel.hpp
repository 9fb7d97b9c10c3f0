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
// (<= 256 registers per lane, 64 KiB of LDS each), so one workgroup's matrix
// work overlaps the other's softmax, loads and barriers.
//
// MFMA orientation.  Both products are computed transposed so that every
// lane owns exactly one query row (lane % 32) in both accumulators:
//   S^T[kv, q] = K[kv, :] . Q[q, :]      (A = K tile from LDS, B = Q^T in registers)
//   O^T[d, q] += V^T[d, kv] . P^T[kv, q] (A = V^T read transposed from LDS, B = P^T)
// with v_mfma_f32_32x32x16_bf16.  In a 32x32 accumulator lane l holds column
// l % 32 and rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.  So the softmax row
// max and row sum reduce over the lane's own 64 values plus one swap with
// lane l ^ 32, the O rescale is a per-lane scalar, and the P values leave the
// S accumulator already laid out as the B operand of the PV product: the 16
// keys of a PV k-step sit in lane half h at kv = 4h + {0..3} and 8 + 4h + {0..3}.
// The matching V^T operand comes from row-major V in LDS through
// ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i % 4
// of the 8-byte row pointed to by lane 4j + i/4 (j = 0..3), so lanes pointing
// at a 4-key x 16-dim block of V receive one dim each across the 4 keys.
//
// Data movement: K and V tiles go from global memory straight into LDS with
// 16-byte global_load_lds (no registers), row-major with the 16-byte chunks
// of each row XOR-swizzled (bank-conflict-free reads, see k_swizzle/v_swizzle).  The K tile
// of step t+1 streams in during the softmax and PV of step t; the V tile of
// step t+1 during QK^T and softmax of step t+1.
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
// per-lane byte offset (one VGPR per lane).
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gaddr), "s"(lds));
}
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds));
}

// A pointer the compiler can keep in SGPRs (the value is the same in every lane).
__device__ __forceinline__ const void* uniform_ptr(const void* ptr) {
  const uint64_t v = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
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

template <int D, class Mask, class Score>
__global__ __launch_bounds__(kFwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(FwdParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int KS = D / 16;                  // k-steps of the QK^T product
  constexpr int DT = D / 32;                  // 32-row blocks of O^T
  constexpr int CPR = D / 8;                  // 16-byte chunks per K/V row
  constexpr int HB = 64;                      // keys per sub-tile (half a BlockMask tile)
  constexpr int NI = HB * CPR / 64 / 4;       // 16-byte loads per wave per sub-tile buffer
  // two stages of K and V sub-tiles, row-major, chunks XOR-swizzled by row
  __shared__ __align__(16) uint16_t k_lds[2][HB * D];
  __shared__ __align__(16) uint16_t v_lds[2][HB * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lq = lane & 31, hh = lane >> 5;

  // ---- which (b, hq, query tile) ------------------------------------------
  const int NQ = (p.Sq + kBM - 1) / kBM;
  const int total = NQ * p.Hq * p.B;
  const int L = xcd_logical_id(blockIdx.x, total);
  const int i_in_head = L % NQ;
  const int bh = L / NQ;
  const int hq = bh % p.Hq, b = bh / p.Hq;
  const int qb = NQ - 1 - i_in_head;  // later (heavier, for causal) query tiles first
  const int hkv = hq / p.G;
  const int q0 = qb * kBM;

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
  auto kb_of = [&](int t) -> int {
    if (t < n_part) return part_idx[t];
    return bm.dense ? (t - n_part) : full_idx[t - n_part];
  };

  const uint16_t* Qp = p.q + (long long)b * p.qs[0] + (long long)hq * p.qs[1];
  const uint16_t* Kp = p.k + (long long)b * p.ks[0] + (long long)hkv * p.ks[1];
  const uint16_t* Vp = p.v + (long long)b * p.vs[0] + (long long)hkv * p.vs[1];
  const long long ks2 = p.ks[2], vs2 = p.vs[2];

  // ---- global -> LDS sub-tile loads -------------------------------------------
  // Sub-tile j = keys [64 (j % 2), 64 (j % 2) + 64) of BlockMask tile kb_of(j / 2).
  // LDS slot s (16 bytes) holds row s / CPR, logical chunk (s % CPR) ^ swizzle(row);
  // wave w issues slots [64 (4i + w), +64) for i < NI.  Rows past Skv re-read
  // row Skv-1 (finite values whose scores are masked to -inf).
  // Within one instruction the 64 lanes cover 64 / CPR consecutive rows; the
  // swizzled chunk of a lane does not depend on i (the swizzles only use row
  // bits below 4 * RPI), so a per-lane offset plus a uniform row step per
  // instruction addresses every load.
  constexpr int RPI = 64 / CPR;                                  // rows per instruction
  const int lrow = wave * RPI + lane / CPR;                      // row of this lane in instruction 0
  const int kchunk = (lane % CPR) ^ k_swizzle<D>(lrow);          // logical chunks it loads
  const int vchunk = (lane % CPR) ^ v_swizzle<D>(lrow);
  const uint32_t k_voff = (uint32_t)(2 * lrow * ks2 + 16 * kchunk);  // bytes
  const uint32_t v_voff = (uint32_t)(2 * lrow * vs2 + 16 * vchunk);
  auto issue = [&](const uint16_t* g, long long rs, const uint16_t* buf, int lchunk, uint32_t voff, int j) {
    const int kv0 = kb_of(j >> 1) * kBN + HB * (j & 1);
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(buf)) + 16 * 64 * wave;
    if (kv0 + HB <= p.Skv) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        dma16s(voff, uniform_ptr(g + (long long)(kv0 + 4 * RPI * i) * rs), base + 16 * 64 * 4 * i);
    } else {
      const int last = p.Skv - 1 - kv0;  // rows past Skv re-read row Skv-1
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int rr = min(lrow + 4 * RPI * i, last);
        dma16(g + (long long)(kv0 + rr) * rs + 8 * lchunk, base + 16 * 64 * 4 * i);
      }
    }
  };
  // element offsets of (row, logical chunk) in the K and V stages
  auto k_off = [](int r, int chunk) { return r * D + ((chunk ^ k_swizzle<D>(r)) * 8); };
  auto v_off = [](int r, int chunk) { return r * D + ((chunk ^ v_swizzle<D>(r)) * 8); };

  // ---- per-lane query row ---------------------------------------------------
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
  const auto mrow = Mask::row(p.mask, b, hq, qc);
  const auto srow = Score::row(p.score, b, hq, qc);

  // ---- online softmax state (base-2 units) ----------------------------------
  f32x16_t oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16_t{};
  // Reference max of the exponentials: -inf until the row sees a finite score,
  // then only raised when a score exceeds it by more than kRescaleSlack.  Scores
  // are produced relative to it (y = x2 - m_run), so exp2(y) needs no subtraction.
  float m_run = -INFINITY;
  float l_run = 0.0f;       // this lane's half of the row sum
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones2 = {(__bf16)1.0f, (__bf16)1.0f};

  auto compute_subtile = [&](int j, int kb, bool partial) {
    const int buf = j & 1;
    const int kvt0 = kb * kBN + HB * (j & 1);
    const bool ragged = kvt0 + HB > p.Skv;
    const uint16_t* kl = k_lds[buf];
    const uint16_t* vl = v_lds[buf];

    // S^T = K Q^T  (2 blocks of 32 keys)
    f32x16_t sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = f32x16_t{};
      const int r = 32 * mt + lq;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8_t a = *(const bf16x8_t*)&kl[k_off(r, 2 * s + hh)];
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc[mt], 0, 0, 0);
      }
    }

    // Element (mt, r) of this lane holds key kvb + cr, cr = 32 mt + 8 (r/4) + r%4.
    // score_mod everywhere; mask_mod on partial tiles; keys past Skv on the ragged tile.
    const int kvb = kvt0 + 4 * hh;
    const float m_ref = m_run == -INFINITY ? 0.0f : m_run;
    const auto st = Score::tile(srow, kvb, m_ref);
    float ymax = -INFINITY;
    if (!partial && !ragged) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cr = 32 * mt + 8 * (r >> 2) + (r & 3);
          const float y = Score::apply(st, sacc[mt][r], cr);
          sacc[mt][r] = y;
          ymax = fmaxf(ymax, y);
        }
      }
    } else {
      const auto mtl = Mask::tile(mrow, kvb);
      const int lim = ragged ? p.Skv - kvb : HB;  // key kvb + cr exists iff cr < lim
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cr = 32 * mt + 8 * (r >> 2) + (r & 3);
          const int crs = min(cr, lim - 1);  // in-bounds index for functors that load
          bool keep = cr < lim;
          if (partial) keep = keep && Mask::keep(mtl, crs);
          const float y = keep ? Score::apply(st, sacc[mt][r], crs) : -INFINITY;
          sacc[mt][r] = y;
          ymax = fmaxf(ymax, y);
        }
      }
    }
    ymax = fmaxf(ymax, __shfl_xor(ymax, 32));
    const bool raise = ymax > kRescaleSlack || (m_run == -INFINITY && ymax > -INFINITY);
    if (__any(raise)) {
      const float m_new = fmaxf(m_run, m_ref + ymax);
      const float shift = m_new == -INFINITY ? 0.0f : m_ref - m_new;
      const float alpha = m_run == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i) oacc[i] *= alpha;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) sacc[mt] += shift;
      m_run = m_new;
    }

    // P = exp2(y) in bf16; the row sum adds the rounded values (v_dot2 with ones)
    bf16x8_t pb[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x2_t pk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          pk[k][0] = (__bf16)__builtin_amdgcn_exp2f(sacc[mt][8 * s + 2 * k]);
          pk[k][1] = (__bf16)__builtin_amdgcn_exp2f(sacc[mt][8 * s + 2 * k + 1]);
          l_run = __builtin_amdgcn_fdot2_f32_bf16(pk[k], ones2, l_run, false);
        }
        pb[mt][s] = __builtin_shufflevector(__builtin_shufflevector(pk[0], pk[1], 0, 1, 2, 3),
                                            __builtin_shufflevector(pk[2], pk[3], 0, 1, 2, 3),
                                            0, 1, 2, 3, 4, 5, 6, 7);
      }
    }

    // O^T += V^T P^T
    const int gi = lane >> 4, si = lane & 15;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int row0 = 32 * mt + 16 * s + 4 * hh + (si >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int d = 32 * dt + 16 * (gi & 1) + 4 * (si & 3);
          const int off_lo = v_off(row0, d >> 3) + (d & 7);
          const int off_hi = v_off(row0 + 8, d >> 3) + (d & 7);
          const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(vl + off_lo));
          const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(vl + off_hi));
          const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[mt][s], oacc[dt], 0, 0, 0);
        }
      }
    }
  };

  const int J = 2 * T;
  if (J > 0) {
    issue(Kp, ks2, k_lds[0], kchunk, k_voff, 0);
    issue(Vp, vs2, v_lds[0], vchunk, v_voff, 0);
    issue(Kp, ks2, k_lds[1], kchunk, k_voff, 1);
    issue(Vp, vs2, v_lds[1], vchunk, v_voff, 1);
    for (int j = 0; j < J; ++j) {
      // K(j), V(j) landed for every wave; K(j+1), V(j+1) may still be in flight
      if (j + 1 < J)
        wait_vmcnt<2 * NI>();
      else
        wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      const int t = j >> 1;
      compute_subtile(j, kb_of(t), t < n_part);
      // every wave is done reading stage j % 2: refill it with sub-tile j + 2
      wait_lds_reads();
      __builtin_amdgcn_s_barrier();
      if (j + 2 < J) {
        issue(Kp, ks2, k_lds[j & 1], kchunk, k_voff, j + 2);
        issue(Vp, vs2, v_lds[j & 1], vchunk, v_voff, j + 2);
      }
    }
  }

  // ---- epilogue ---------------------------------------------------------------
  const float l = l_run + __shfl_xor(l_run, 32);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
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

template <int D, class Mask>
struct LaunchFwd {
  const FwdParams& p;
  hipStream_t stream;
  template <class Score>
  void operator()() {
    const int NQ = (p.Sq + kBM - 1) / kBM;
    const long long total = (long long)NQ * p.Hq * p.B;
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
