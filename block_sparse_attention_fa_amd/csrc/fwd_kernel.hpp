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
// query tile).  Wave w owns query rows 32w..32w+31 of the tile.
//
// MFMA orientation.  Both products are computed transposed so that every
// lane owns exactly one query row (lane % 32) in both accumulators:
//   S^T[kv, q] = K[kv, :] . Q[q, :]      (A = K tile from LDS, B = Q^T in registers)
//   O^T[d, q] += V^T[d, kv] . P^T[kv, q] (A = V^T tile from LDS, B = P^T in registers)
// with v_mfma_f32_32x32x16_bf16.  In a 32x32 accumulator lane l holds column
// l % 32 and rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.  So the row max and
// row sum of the softmax reduce over the lane's own 64 values and then one
// swap with lane l ^ 32, the O rescale is a per-lane scalar, and the P
// values come out of the S accumulator already in the B-operand layout of
// the PV product (the k index is a permutation of the 16 keys of each step,
// which V^T in LDS is stored to match).
//
// LDS: the K tile row-major [128][D+8] and V transposed [D][128+8] (both
// padded by 16 bytes per row against bank conflicts).  The next tile's K/V
// rows are loaded into registers while the current tile is computed.
#pragma once

#include <type_traits>

#include "mods.hpp"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kFwdThreads = 256;
constexpr int kBM = FA_BLOCK;  // query rows per workgroup
constexpr int kBN = FA_BLOCK;  // keys per tile

template <int D>
struct FwdSmem {
  static constexpr int KSTR = D + 8;    // elements per K row
  static constexpr int VSTR = kBN + 8;  // elements per V^T row
  uint16_t k[kBN * KSTR];
  uint16_t vt[D * VSTR];
};

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Give each
// XCD a contiguous range of logical tile ids, so the query tiles of one head
// (which share K/V) run on the same XCD and hit the same L2.
__device__ __forceinline__ int xcd_logical_id(int bid, int total) {
  const int per = total / 8, rem = total % 8;
  const int x = bid % 8, j = bid / 8;
  return x * per + min(x, rem) + j;
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);  // (a.lo16, b.lo16)
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);  // (a.hi16, b.hi16)
}

template <int D, class Mask, class Score>
__global__ __launch_bounds__(kFwdThreads) void fwd_kernel(FwdParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int KS = D / 16;        // k-steps of the QK^T product
  constexpr int DT = D / 32;        // 32-row blocks of O^T
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int KCH = kBN * CPR / kFwdThreads;  // K chunks staged per thread
  constexpr int VTHREADS = 2 * D;   // threads that stage V (8 rows x 8 d each)
  using Smem = FwdSmem<D>;
  __shared__ __align__(16) Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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

  const uint16_t* Qp = p.q + (long long)b * p.qs[0] + (long long)hq * p.qs[1];
  const uint16_t* Kp = p.k + (long long)b * p.ks[0] + (long long)hkv * p.ks[1];
  const uint16_t* Vp = p.v + (long long)b * p.vs[0] + (long long)hkv * p.vs[1];
  const long long ks2 = p.ks[2], vs2 = p.vs[2];

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

  // ---- staging of K/V tiles through registers -------------------------------
  u32x4_t kreg[KCH];
  u32x4_t vreg[8];
  const int vc = tid % CPR;                 // d chunk this thread stages for V
  const int vhalf = (tid / CPR) & 1;
  const int vg = tid / (2 * CPR);           // 16-key group
  auto kb_of = [&](int t) -> int {
    if (t < n_part) return part_idx[t];
    return bm.dense ? (t - n_part) : full_idx[t - n_part];
  };
  auto load_tile = [&](int kb) {
    const int kv0 = kb * kBN;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ci = tid + kFwdThreads * i;
      const int r = ci / CPR, c = ci % CPR;
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (kv0 + r < p.Skv) x = *(const u32x4_t*)(Kp + (long long)(kv0 + r) * ks2 + 8 * c);
      kreg[i] = x;
    }
    if (tid < VTHREADS) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 16 * vg + 4 * vhalf + (j & 3) + 8 * (j >> 2);
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (kv0 + r < p.Skv) x = *(const u32x4_t*)(Vp + (long long)(kv0 + r) * vs2 + 8 * vc);
        vreg[j] = x;
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ci = tid + kFwdThreads * i;
      const int r = ci / CPR, c = ci % CPR;
      *(u32x4_t*)&sm.k[r * Smem::KSTR + 8 * c] = kreg[i];
    }
    if (tid < VTHREADS) {
      // 8 keys x 8 dims -> 8 dims x 8 keys.  The keys of this thread are, in
      // order, 16g + 4*half + {0..3} and 16g + 8 + 4*half + {0..3}; they land at
      // positions 16g + 8*half + {0..7} of each V^T row, the order in which
      // the P^T operand lists its keys.
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int w = dd >> 1;
        u32x4_t o;
        if (dd & 1) {
          o[0] = pack_hi(vreg[0][w], vreg[1][w]);
          o[1] = pack_hi(vreg[2][w], vreg[3][w]);
          o[2] = pack_hi(vreg[4][w], vreg[5][w]);
          o[3] = pack_hi(vreg[6][w], vreg[7][w]);
        } else {
          o[0] = pack_lo(vreg[0][w], vreg[1][w]);
          o[1] = pack_lo(vreg[2][w], vreg[3][w]);
          o[2] = pack_lo(vreg[4][w], vreg[5][w]);
          o[3] = pack_lo(vreg[6][w], vreg[7][w]);
        }
        *(u32x4_t*)&sm.vt[(8 * vc + dd) * Smem::VSTR + 16 * vg + 8 * vhalf] = o;
      }
    }
  };

  // ---- online softmax state (base-2 units) ----------------------------------
  f32x16_t oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16_t{};
  float m_run = -INFINITY;
  float l_run = 0.0f;  // this lane's half of the row sum

  auto compute_tile = [&](int kb, auto partial_tag) {
    constexpr bool kPartialTile = decltype(partial_tag)::value;
    const int kvt0 = kb * kBN;
    const bool ragged = kvt0 + kBN > p.Skv;

    // S^T = K Q^T
    f32x16_t sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sacc[mt] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8_t a = *(const bf16x8_t*)&sm.k[(32 * mt + lq) * Smem::KSTR + 16 * s + 8 * hh];
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc[mt], 0, 0, 0);
      }
    }

    // score_mod, mask_mod (partial tiles only), out-of-range keys
    float mloc = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kv = kvt0 + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
        bool keep = true;
        if (ragged) keep = kv < p.Skv;
        if constexpr (kPartialTile) keep = keep && mrow(kv);
        const float x = keep ? Score::apply1(srow, sacc[mt][r], kv, 0) : -INFINITY;
        sacc[mt][r] = x;
        mloc = fmaxf(mloc, x);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;

    float lsum = 0.0f;
    bf16x8_t pb[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(sacc[mt][r] - m_use);
        lsum += e;
        pb[mt][r >> 3][r & 7] = (__bf16)e;
      }
    }
    l_run = fmaf(l_run, alpha, lsum);
#pragma unroll
    for (int i = 0; i < DT; ++i) oacc[i] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8_t a =
              *(const bf16x8_t*)&sm.vt[(32 * dt + lq) * Smem::VSTR + 16 * (2 * mt + s) + 8 * hh];
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[mt][s], oacc[dt], 0, 0, 0);
        }
      }
    }
  };

  if (T > 0) load_tile(kb_of(0));
  for (int t = 0; t < T; ++t) {
    const int kb = kb_of(t);
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < T) load_tile(kb_of(t + 1));
    if (t < n_part)
      compute_tile(kb, std::true_type{});
    else
      compute_tile(kb, std::false_type{});
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
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
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
