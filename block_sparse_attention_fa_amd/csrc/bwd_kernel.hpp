// Block-sparse attention backward for CDNA4 (gfx950).
//
// The pages name a backward pass and the transposed BlockMask view it walks
// (attention-gym "Concepts" page, "Key attributes": q_num_blocks / q_indices,
// "used in backward"; paper review "Flex Attention: A Programming Model for
// Generating Optimized Attention Kernels", kernel-template diagram) without
// printing its formulas, so this is the gradient of the forward definition:
// with S = Q K^T * scale, S' = mod(S) where the mask keeps (else -inf),
// P = softmax(S') and O = P V,
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - Delta) * mod'(S),
//     dQ = scale * dS K,   dK = scale * dS^T Q,   Delta = rowsum(dO * O),
// with P recomputed from the forward's log-sum-exp (no online softmax).
//
// Three kernels:
//  * bwd_prep:  Delta and the base-2 LSE per query row, into a workspace padded
//    to whole 128-row tiles (padded rows and rows that attend nothing get
//    LSE = +inf, so their P is 0).
//  * bwd_dq:    one workgroup per (b, hq, 128-row query tile), the forward's
//    layout (4 waves x 32 query rows, a lane per query row): for every listed
//    key tile, S^T = K Q^T and dP^T = V dO^T, then dQ^T += K^T dS^T with K^T
//    read transposed from LDS (as the forward reads V^T).  Partial tiles
//    evaluate the mask_mod, full tiles do not.
//  * bwd_dkdv:  one workgroup per (b, hkv, 128-key tile), 4 waves x 32 keys, a
//    lane per key; K and V stay in registers as MFMA B operands while the query
//    tiles of the transposed lists (for every query head of the GQA group) stream
//    through LDS: S = Q K^T, dP = dO V^T, then dV^T += dO^T P and
//    dK^T += Q^T dS with dO^T and Q^T read transposed.  Its accumulators need
//    more than 256 registers, so it runs one wave per SIMD.
// No atomics: dQ and dK/dV come from separate passes (S and dP are computed
// in both).
#pragma once

#include "fwd_kernel.hpp"

namespace fa {

constexpr int kBwdThreads = 256;

// LDS chunk swizzle for tiles that are read both by rows (ds_read_b128: 16
// lanes = 16 consecutive rows, one 16-byte chunk) and transposed
// (ds_read_b64_tr_b16: 32 lanes = 4 consecutive rows x 4 adjacent chunks).
// Rows are 256 bytes (D = 128, one pass over the 64 banks) or 128 bytes
// (D = 64, two rows per pass).  The swizzle is a bijection on the 16 rows of
// a row read, and it maps the 4 x 4 chunks of a transposed read to 16
// distinct bank groups, so neither read pattern has bank conflicts.  (The
// forward's K and V swizzles each serve one of the two patterns.)
template <int D>
__device__ __forceinline__ int rt_swizzle(int r) {
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// A block-list entry at a wave-uniform address, read through the constant
// address space so that it becomes a scalar load (the lists are written by an
// earlier launch and do not change during this one).  A plain load here would
// be a vector load, and the compiler's wait for it would also wait for the
// LDS DMA in flight, which it cannot see.
__device__ __forceinline__ int load_list(const int* p, long long i) {
  return *(const __attribute__((address_space(4))) int*)(uintptr_t)(p + i);
}

// ---- bwd_prep: Delta = rowsum(dO * O) and LSE * log2(e) per query row --------------
// D / 8 lanes per row, 16 bytes of O and of dO each; 64 / (D / 8) rows per wave.
template <int D>
constexpr int kPrepRowsPerWave = 64 / (D / 8);

template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_prep_kernel(BwdParams P) {
  constexpr int LPR = D / 8;
  const FwdParams& p = P.f;
  const int lane = threadIdx.x & 63;
  const long long gw = (long long)blockIdx.x * (kBwdThreads / 64) + (threadIdx.x >> 6);
  const long long gr = gw * kPrepRowsPerWave<D> + lane / LPR;  // padded row [b, h, q]
  const int Sp = P.sq_pad;
  const bool live = gr < (long long)p.B * p.Hq * Sp;
  const int q = (int)(gr % Sp);
  const int bh = (int)(gr / Sp);
  const int b = bh / p.Hq, hq = bh % p.Hq;
  float acc = 0.0f, lse2 = INFINITY;
  if (live && q < p.Sq) {
    const int d0 = 8 * (lane % LPR);
    const u32x4_t o = *(const u32x4_t*)(p.o + (long long)b * p.os[0] + (long long)hq * p.os[1] + (long long)q * p.os[2] + d0);
    const u32x4_t g = *(const u32x4_t*)(P.dout + (long long)b * P.dos[0] + (long long)hq * P.dos[1] + (long long)q * P.dos[2] + d0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_bits_to_float(o[i] & 0xffffu), bf16_bits_to_float(g[i] & 0xffffu), acc);
      acc = fmaf(bf16_bits_to_float(o[i] >> 16), bf16_bits_to_float(g[i] >> 16), acc);
    }
    const float l = p.lse[((long long)b * p.Hq + hq) * p.Sq + q];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (live && lane % LPR == 0) {
    P.ws_delta[gr] = acc;
    P.ws_lse2[gr] = lse2;
  }
}

// ---- bwd_dq ----------------------------------------------------------------------
template <int D, class Mask, class Score>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(BwdParams P) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int CPR = D / 8;
  constexpr int HB = 64;
  constexpr int SPT = kBN / HB;
  constexpr int NI = HB * CPR / 64 / 4;
  const FwdParams& p = P.f;
  // K and V sub-tiles, row-major with the row/transposed swizzle, 2-deep ring
  __shared__ __align__(16) uint16_t k_lds[2][HB * D];
  __shared__ __align__(16) uint16_t v_lds[2][HB * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hh = lane >> 5;
  const int gi = lane >> 4, si = lane & 15;

  const int NQ = (p.Sq + kBM - 1) / kBM;
  int bh, qb;
  query_tile_unit(p, NQ, bh, qb);  // the forward's order, q_order included
  const int hq = bh % p.Hq, b = bh / p.Hq;
  const int hkv = hq / p.G;
  const int q0 = qb * kBM;

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
    n_part = load_list(bm.kv_num, row);
    part_idx = bm.kv_idx + row * bm.NK;
    if (bm.separate_full) {
      n_full = load_list(bm.full_num, row);
      full_idx = bm.full_idx + row * bm.NK;
    } else {
      n_full = 0;
    }
  }
  const int T = n_part + n_full;
  auto kb_of = [&](int t) -> int {
    if (t < n_part) return load_list(part_idx, t);
    return bm.dense ? t - n_part : load_list(full_idx, t - n_part);
  };

  const char* Kp = (const char*)(p.k + (long long)b * p.ks[0] + (long long)hkv * p.ks[1]);
  const char* Vp = (const char*)(p.v + (long long)b * p.vs[0] + (long long)hkv * p.vs[1]);
  const long long ksb = 2 * p.ks[2], vsb = 2 * p.vs[2];
  constexpr int RPI = 64 / CPR;
  const int lrow = wave * RPI + lane / CPR;
  const int kchunk = (lane % CPR) ^ rt_swizzle<D>(lrow);
  const uint32_t k_voff = (uint32_t)(lrow * ksb + 16 * kchunk);
  const uint32_t v_voff = (uint32_t)(lrow * vsb + 16 * kchunk);
  auto issue_one = [&](const char* g, long long rsb, const uint16_t* buf, uint32_t voff, int kv0) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(buf) + 16 * 64 * wave);
    if (kv0 + HB <= p.Skv) {
      const char* g0 = g + kv0 * rsb;
#pragma unroll
      for (int i = 0; i < NI; ++i) dma16s(voff, g0 + 4 * RPI * i * rsb, base + 16 * 64 * 4 * i);
    } else {
      const int last = p.Skv - 1 - kv0;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int rr = min(lrow + 4 * RPI * i, last);
        dma16(g + (kv0 + rr) * rsb + 16 * kchunk, base + 16 * 64 * 4 * i);
      }
    }
  };
  auto kv0_of = [&](int j) { return kb_of(j / SPT) * kBN + HB * (j % SPT); };
  auto issue = [&](int kv0, int j) {
    issue_one(Kp, ksb, k_lds[j % 2], k_voff, kv0);
    issue_one(Vp, vsb, v_lds[j % 2], v_voff, kv0);
  };
  auto k_off = [](int r, int chunk) { return r * D + ((chunk ^ rt_swizzle<D>(r)) * 8); };

  // ---- this lane's query row: Q and dO as B operands, its LSE and Delta ----
  const int myq = q0 + wave * 32 + lq;
  const bool q_ok = myq < p.Sq;
  const int qc = q_ok ? myq : p.Sq - 1;
  bf16x8_t qreg[KS], doreg[KS];
  {
    const uint16_t* Qp = p.q + (long long)b * p.qs[0] + (long long)hq * p.qs[1] + (long long)qc * p.qs[2];
    const uint16_t* Gp = P.dout + (long long)b * P.dos[0] + (long long)hq * P.dos[1] + (long long)qc * P.dos[2];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qreg[s] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(Qp + 16 * s + 8 * hh));
      doreg[s] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(Gp + 16 * s + 8 * hh));
    }
  }
  const long long wrow = ((long long)b * p.Hq + hq) * P.sq_pad + myq;  // padded rows exist
  const float lse2 = P.ws_lse2[wrow];      // +inf: the row attends nothing (P = 0)
  const float delta = P.ws_delta[wrow];
  const auto mrow = Mask::row(p.mask, b, hq, qc);
  const auto srow = Score::row(p.score, b, hq, qc);

  int koff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) koff[s] = k_off(lq, 2 * s + hh);
  // K^T operand (transposed reads, as the forward reads V^T): rows 4hh + si/4
  // (+16 per k-step), lower and upper 8 rows, d block dt
  int ktlo[DT], kthi[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int d = 32 * dt + 16 * (gi & 1) + 4 * (si & 3);
    ktlo[dt] = k_off(4 * hh + (si >> 2), d >> 3) + (d & 7);
    kthi[dt] = k_off(4 * hh + (si >> 2) + 8, d >> 3) + (d & 7);
  }

  f32x16_t dq[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) dq[i] = f32x16_t{};
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

  // One sub-tile; the ring stage j % 2 is a compile-time constant (the loop
  // below is unrolled by 2) so that LDS reads take immediate offsets.
  const int J = SPT * T;
  // first keys of sub-tiles j + 1 and j + 2: the list entry read in step j is
  // in hand when step j + 1 issues its loads
  int kv_nxt = 0, kv_nx2 = 0;
  auto step = [&](int j, auto stage) {
    constexpr int stg = decltype(stage)::value;
    wait_vmcnt<0>();
    wait_lds_reads();
    __syncthreads();  // sub-tile j landed for every wave; every wave is done with j-1
    const int kvt0 = kv_nxt;
    kv_nxt = kv_nx2;
    if (j + 1 < J) issue(kv_nxt, j + 1);
    if (j + 2 < J) kv_nx2 = kv0_of(j + 2);
    const int t = j / SPT;
    const bool partial = t < n_part;
    const bool ragged = kvt0 + HB > p.Skv;
    const uint32_t kbase = lds_address(k_lds[stg]), vbase = lds_address(v_lds[stg]);

    // S^T = K Q^T and dP^T = V dO^T for this 64-key sub-tile: key block 0
    // first; block 1 beside the element-wise work of block 0, and dQ's first
    // two k-steps (which need only block 0's dS) beside that of block 1
    f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}}, dpacc[2] = {f32x16_t{}, f32x16_t{}};
    auto sdp_mfma = [&](int i) {
      const int mt = i / KS, s = i % KS;
      const bf16x8_t ak = *(const lds_bf16x8_t*)(uintptr_t)(kbase + 2 * (koff[s] + mt * 32 * D));
      const bf16x8_t av = *(const lds_bf16x8_t*)(uintptr_t)(vbase + 2 * (koff[s] + mt * 32 * D));
      sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[s], sacc[mt], 0, 0, 0);
      dpacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, doreg[s], dpacc[mt], 0, 0, 0);
    };
    bf16x8_t dsb[4];
    auto dq_mfma = [&](int i) {  // dQ^T += K^T dS^T, k-step i / DT, d block i % DT
      const int ks = i / DT, dt = i % DT;
      const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4_t*)(uintptr_t)(kbase + 2 * (ktlo[dt] + ks * 16 * D)));
      const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4_t*)(uintptr_t)(kbase + 2 * (kthi[dt] + ks * 16 * D)));
      const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[ks], dq[dt], 0, 0, 0);
    };
#pragma unroll
    for (int i = 0; i < KS; ++i) sdp_mfma(i);

    // dS^T = P (dP - Delta) mod'(S); element (mt, r) is key kvb + cr.  Each
    // block is computed for every element first (no branches), then the mask
    // and the ragged tail are zeroed on the tiles that have them.
    const int kvb = kvt0 + 4 * hh;
    const int lim = ragged ? p.Skv - kvb : HB;
    const float m_ref = lse2;
    const auto st = Score::tile(srow, kvb, m_ref);
    const auto mtl = Mask::tile(mrow, kvb);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int cr = 32 * mt + 8 * (r >> 2) + (r & 3);
        const int crs = Score::kReadsMemory ? min(cr, lim - 1) : cr;  // in-bounds key for functors that read memory
        const float sv = sacc[mt][r];
        const float pv = __builtin_amdgcn_exp2f(Score::apply(st, sv, crs));
        dpacc[mt][r] = pv * (dpacc[mt][r] - delta) * Score::dmod1(srow, sv, kvb + crs);
        if (mt == 0 && r % (16 / KS) == 16 / KS - 1) sdp_mfma(KS + r / (16 / KS));
        if (mt == 1 && r % (8 / DT) == 8 / DT - 1) dq_mfma(r / (8 / DT));
      }
      if (partial || ragged) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int cr = 32 * mt + 8 * (r >> 2) + (r & 3);
          bool keep = cr < lim;
          if (partial) keep = keep && Mask::keep(mtl, min(cr, lim - 1));
          dpacc[mt][r] = keep ? dpacc[mt][r] : 0.0f;
        }
      }
#pragma unroll
      for (int g = 2 * mt; g < 2 * mt + 2; ++g)
#pragma unroll
        for (int k = 0; k < 8; ++k) dsb[g][k] = (__bf16)dpacc[mt][8 * (g & 1) + k];
    }
#pragma unroll
    for (int i = 2 * DT; i < 4 * DT; ++i) dq_mfma(i);
  };
  if (J > 0) {
    kv_nxt = kv0_of(0);
    issue(kv_nxt, 0);
  }
  if (J > 1) kv_nx2 = kv0_of(1);
  for (int j = 0; j < J; j += 2) {
    step(j, std::integral_constant<int, 0>{});
    if (j + 1 < J) step(j + 1, std::integral_constant<int, 1>{});
  }

  if (q_ok) {
    const float sc = p.score.scale;
    uint16_t* Gq = P.dq + (long long)b * P.dqs[0] + (long long)hq * P.dqs[1] + (long long)myq * P.dqs[2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4_t o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = (__bf16)(dq[dt][4 * g + i] * sc);
        *(bf16x4_t*)(Gq + 32 * dt + 8 * g + 4 * hh) = o4;
      }
    }
  }
}

// ---- bwd_dkdv ------------------------------------------------------------------------
// One 512-thread workgroup (8 waves, two per SIMD) per (b, hkv, 128-key tile).
// Wave w and wave w + 4 (the same SIMD) own the same 32 keys (a lane per key)
// and split the work of every 64-row query sub-step j, one barrier per sub-step:
//  * P role (waves 0-3): S = Q K^T of j beside dV^T += dO^T P of j - 1 (MFMAs),
//    then P = exp2(S' - LSE) of j with the mask and the rows past Sq zeroed,
//    P mod'(S) to LDS (bf16) and P kept (bf16) for the next sub-step (VALU).
//  * dS role (waves 4-7): dS = P mod'(S) (dP - Delta) of j - 1 from the P
//    role's copy (VALU), then dK^T += Q^T dS of j - 1 beside dP = dO V^T of j
//    (MFMAs); it also issues every tile load, since its sub-step starts with
//    element-wise work, not with MFMAs waiting for their operands.
// The two orders are complementary: the P role's MFMAs run beside the dS
// role's element-wise work, and the other way round.  Each role holds one of
// K / V and one of the dK / dV accumulators, so both fit in the registers of
// two waves per SIMD.
constexpr int kDkdvThreads = 512;

template <int D, class Mask, class Score>
__global__ __launch_bounds__(kDkdvThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdParams P) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int CPR = D / 8;
  constexpr int HB = 64;                 // query rows per sub-step
  constexpr int SPT = kBM / HB;
  constexpr int NI = HB * CPR / 64 / 4;  // 16-byte loads per wave of a Q or dO sub-tile (4 waves a tile)
  const FwdParams& p = P.f;
  // Q and dO sub-tiles, row-major with the row/transposed swizzle, 3-deep ring:
  // sub-step j reads stage j % 3 (and Q of j - 1) while j + 1 loads
  __shared__ __align__(16) uint16_t q_lds[3][HB * D];
  __shared__ __align__(16) uint16_t g_lds[3][HB * D];
  // base-2 LSE (first HB floats) and Delta (next HB) of the sub-tile's query rows
  __shared__ __align__(16) float ld_lds[3][2 * HB];
  // P mod'(S) of sub-step j for the dS role, in buffer j % 2: per wave, four
  // groups of 64 lanes x 16 bytes (elements 8 g .. 8 g + 7 of the lane)
  __shared__ __align__(16) uint16_t p_lds[2][4][64 * 32];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 3;         // 32-key block of the wave
  const bool ds_role = wave >= 4;  // uniform per wave
  const int lq = lane & 31, hh = lane >> 5;
  const int gi = lane >> 4, si = lane & 15;

  const int NK = (p.Skv + kBN - 1) / kBN;
  const int BHk = p.Hkv * p.B;
  int bh, kb;
  if (P.kv_order != nullptr && p.bm.Hm == 1 && BHk % 8 == 0) {
    // The BlockMask orders each column's KV blocks heaviest first (one order for
    // every head, Hm = 1).  XCD x (workgroup id % 8) takes the x-th eighth of
    // the (b, hkv) heads, a contiguous block, and its m-th workgroup runs the
    // (m / heads-per-XCD)-th heaviest KV block of one of them.
    const int x = blockIdx.x & 7, m = blockIdx.x >> 3, hpx = BHk >> 3;
    const int r = m / hpx;
    bh = x * hpx + (m - r * hpx);
    const int mb = p.bm.Bm > 1 ? bh / p.Hkv : 0;
    kb = min(max(P.kv_order[(long long)mb * NK + r], 0), NK - 1);
  } else {
    // first KV blocks first: longest first for causal masks
    const int L = xcd_logical_id(blockIdx.x, NK * BHk);
    kb = L % NK;
    bh = L / NK;
  }
  const int hkv = bh % p.Hkv, b = bh / p.Hkv;
  const int k0 = kb * kBN;

  // ---- this lane's key row: K (P role) or V (dS role) as B operands ----
  const int mykv = k0 + kw * 32 + lq;
  const bool kv_ok = mykv < p.Skv;
  const bool kv_all = k0 + kBN <= p.Skv;  // every key of the block exists
  const int kvc = kv_ok ? mykv : p.Skv - 1;
  bf16x8_t xreg[KS];
  {
    const uint16_t* Xr = ds_role
        ? p.v + (long long)b * p.vs[0] + (long long)hkv * p.vs[1] + (long long)kvc * p.vs[2]
        : p.k + (long long)b * p.ks[0] + (long long)hkv * p.ks[1] + (long long)kvc * p.ks[2];
#pragma unroll
    for (int s = 0; s < KS; ++s) xreg[s] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(Xr + 16 * s + 8 * hh));
  }

  // ---- the query tiles to visit: for each head of the group, its column lists ----
  const BlockMaskView& bm = p.bm;
  auto col_counts = [&](int hq, int& np, int& nf) {
    if (bm.dense) {
      np = 0;
      nf = bm.NQ;
      return;
    }
    const int mb = bm.Bm > 1 ? b : 0, mh = bm.Hm > 1 ? hq : 0;
    const long long col = ((long long)mb * bm.Hm + mh) * bm.NK + kb;
    np = load_list(P.q_num, col);
    nf = bm.separate_full ? load_list(P.full_q_num, col) : 0;
  };
  // Sub-steps: the group's heads in order, each head's column list (partial
  // entries, then full ones), SPT sub-steps per entry.
  int Jtot = 0;
  for (int g = 0; g < p.G; ++g) {
    int np, nf;
    col_counts(hkv * p.G + g, np, nf);
    Jtot += SPT * (np + nf);
  }
  // A cursor walks them in order (sub-steps are described one after another):
  // head cg with cnp partial and cnt entries in all, entry ct, half ch, and
  // the head's two lists.
  int cg = -1, cnp = 0, cnt = 0, ct = 0, ch = 0;
  const int* plist = nullptr;
  const int* flist = nullptr;
  auto next_head = [&]() {  // the next head with a non-empty list (the caller knows one exists)
    do {
      ++cg;
      int nf;
      col_counts(hkv * p.G + cg, cnp, nf);
      cnt = cnp + nf;
    } while (cnt == 0);
    if (!bm.dense) {
      const int mb = bm.Bm > 1 ? b : 0, mh = bm.Hm > 1 ? hkv * p.G + cg : 0;
      const long long col = ((long long)mb * bm.Hm + mh) * bm.NK + kb;
      plist = P.q_idx + col * bm.NQ;
      flist = P.full_q_idx + col * bm.NQ;
    }
    ct = 0;
    ch = 0;
  };

  // Loads: the dS-role waves bring the Q and dO sub-tiles (each 4 waves x NI
  // loads), wave 4 the LSE / Delta rows.
  constexpr int RPI = 64 / CPR;
  const int lrow = kw * RPI + lane / CPR;
  const int kchunk = (lane % CPR) ^ rt_swizzle<D>(lrow);
  const long long gsb = 2 * P.dos[2], qsb = 2 * p.qs[2];
  const uint32_t g_voff = (uint32_t)(lrow * gsb + 16 * kchunk), q_voff = (uint32_t)(lrow * qsb + 16 * kchunk);
  auto issue_one = [&](const char* g, long long rsb, const uint16_t* buf, uint32_t voff, int r0) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(buf) + 16 * 64 * kw);
    if (r0 + HB <= p.Sq) {
      const char* g0 = g + r0 * rsb;
#pragma unroll
      for (int i = 0; i < NI; ++i) dma16s(voff, g0 + 4 * RPI * i * rsb, base + 16 * 64 * 4 * i);
    } else {
      const int last = p.Sq - 1 - r0;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int rr = min(lrow + 4 * RPI * i, last);
        dma16(g + (r0 + rr) * rsb + 16 * kchunk, base + 16 * 64 * 4 * i);
      }
    }
  };
  // sub-step j: its query head, first query row and whether its tile is partial
  struct Sub {
    int hq, qs0;
    bool partial;
  };
  auto describe = [&]() -> Sub {  // the sub-step after the last one described
    if (ch == SPT) {
      ch = 0;
      ++ct;
    }
    if (cg < 0 || ct == cnt) next_head();
    const int qt = bm.dense ? ct : (ct < cnp ? load_list(plist, ct) : load_list(flist, ct - cnp));
    const Sub s{hkv * p.G + cg, qt * kBM + HB * ch, ct < cnp};
    ++ch;
    return s;
  };
  auto issue = [&](const Sub& s, int j) {
    const int r0 = s.qs0;
    if (ds_role) {
      const char* Gh = (const char*)(P.dout + (long long)b * P.dos[0] + (long long)s.hq * P.dos[1]);
      const char* Qh = (const char*)(p.q + (long long)b * p.qs[0] + (long long)s.hq * p.qs[1]);
      issue_one(Qh, qsb, q_lds[j % 3], q_voff, r0);
      issue_one(Gh, gsb, g_lds[j % 3], g_voff, r0);
    }
    if (wave == 4 && lane < 2 * HB / 4) {  // 16 bytes a lane; the workspace rows are padded
      const long long w0 = ((long long)b * p.Hq + s.hq) * P.sq_pad + r0 + 4 * (lane % (HB / 4));
      dma16((lane < HB / 4 ? P.ws_lse2 : P.ws_delta) + w0, lds_address(ld_lds[j % 3]));
    }
  };
  auto k_off = [](int r, int chunk) { return r * D + ((chunk ^ rt_swizzle<D>(r)) * 8); };
  int aoff[KS];  // Q / dO rows as A operands: row lq (+32 per query block), chunk 2s + hh
#pragma unroll
  for (int s = 0; s < KS; ++s) aoff[s] = k_off(lq, 2 * s + hh);
  int ttlo[DT], tthi[DT];  // Q^T / dO^T through transposed reads
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int d = 32 * dt + 16 * (gi & 1) + 4 * (si & 3);
    ttlo[dt] = k_off(4 * hh + (si >> 2), d >> 3) + (d & 7);
    tthi[dt] = k_off(4 * hh + (si >> 2) + 8, d >> 3) + (d & 7);
  }
  auto tr_read = [&](uint32_t base, int dt, int ks) {
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_t*)(uintptr_t)(base + 2 * (ttlo[dt] + ks * 16 * D)));
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_t*)(uintptr_t)(base + 2 * (tthi[dt] + ks * 16 * D)));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // this lane's four 16-byte groups in the P mod'(S) buffer
  const uint32_t pbase = lds_address(p_lds[0][kw]) + 16 * lane;
  constexpr uint32_t kPBuf = 4 * 64 * 32 * 2;  // bytes between the two buffers
  auto p_addr = [&](int j, int g) { return pbase + ((j & 1) ? kPBuf : 0u) + 1024 * g; };

  f32x16_t acc[DT];  // dV (P role) or dK (dS role)
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x16_t{};
  typedef float f32x4_t __attribute__((ext_vector_type(4)));

  // dK^T += Q^T dS for a sub-step whose Q is at qb, dS in dsb; MFMA i is
  // k-step i / DT (16 query rows), d block i % DT
  bf16x8_t dsb[4];  // (dS role) dS of the last sub-step, bf16 B operands
  auto dk_mfma = [&](uint32_t qb, int i, bf16x8_t (&tq)[2]) {
    if (i + 1 < 4 * DT) tq[(i + 1) & 1] = tr_read(qb, (i + 1) % DT, (i + 1) / DT);
    acc[i % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[i & 1], dsb[i / DT], acc[i % DT], 0, 0, 0);
  };

  // dV^T += dO^T P for a sub-step whose dO is at gb, P (bf16) in bo; MFMA i is
  // k-step i / DT (16 query rows), d block i % DT
  bf16x8_t bo[4];  // (P role) P of the last sub-step, bf16 B operands
  auto dv_mfma = [&](uint32_t gb, int i, bf16x8_t (&tg)[2]) {
    if (i + 1 < 4 * DT) tg[(i + 1) & 1] = tr_read(gb, (i + 1) % DT, (i + 1) / DT);
    acc[i % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tg[i & 1], bo[i / DT], acc[i % DT], 0, 0, 0);
  };
  // dS role: dS = P mod'(S) (dP - Delta) of sub-step jj as bf16 B operands (k =
  // query row; k-step g holds elements 8 g .. 8 g + 7), from the P role's copy in
  // LDS, dP in sd and Delta at ldp
  f32x16_t sd[2] = {f32x16_t{}, f32x16_t{}};  // S then P (P role), dP (dS role)
  auto make_ds = [&](int jj, uint32_t ldp) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int mt = g >> 1, h8 = 8 * (g & 1);
      const u32x4_t pm = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)p_addr(jj, g);
      // elements h8 .. h8 + 7 are rows 2 h8 + {0..3} and 2 h8 + 8 + {0..3} of the block (+ 4 hh)
      const f32x4_t d0 = *(const __attribute__((address_space(3))) f32x4_t*)(uintptr_t)(ldp + 4 * (32 * mt + 2 * h8));
      const f32x4_t d1 =
          *(const __attribute__((address_space(3))) f32x4_t*)(uintptr_t)(ldp + 4 * (32 * mt + 2 * h8 + 8));
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t w = pm[k >> 1];
        const float pv = bf16_bits_to_float((k & 1) ? (w >> 16) : (w & 0xffffu));
        const float dl = (k < 4) ? d0[k] : d1[k - 4];
        dsb[g][k] = (__bf16)(pv * (sd[mt][h8 + k] - dl));
      }
    }
  };

  // One sub-step j, one barrier.  The two waves of a SIMD run complementary
  // orders, so that each one's MFMAs run beside the other's element-wise work:
  //  * P role: S = Q K^T of j and dV^T += dO^T P of j - 1 (MFMAs), then P of j
  //    and P mod'(S) to LDS buffer j % 2 (VALU), P kept as bf16 for step j + 1;
  //  * dS role: dS of j - 1 from LDS buffer (j - 1) % 2 (VALU), then
  //    dK^T += Q^T dS of j - 1 and dP = dO V^T of j (MFMAs).
  // The ring stage j % 3 is a compile-time constant (the loop below is unrolled
  // by 3) so that every LDS read address is a per-lane register plus an
  // immediate offset.  Sub-step descriptors run two ahead.
  Sub nxt{0, 0, false}, nx2{0, 0, false};
  // (the role is a compile-time constant of each copy, so the two roles'
  // registers are allocated apart; both pass the same barriers)
  auto step = [&](int j, auto stage, auto role) {
    constexpr int st = decltype(stage)::value, sp = (st + 2) % 3;
    constexpr bool ds_role = decltype(role)::value;
    wait_vmcnt<0>();
    wait_lds_reads();  // (lgkmcnt covers the LDS writes too)
    // sub-step j landed and P mod'(S) of j - 1 is in LDS; every wave is done
    // with step j - 1, so stage j + 1 (last used for j - 2) and P buffer j % 2
    // (last read for j - 2) are free
    __syncthreads();
    const Sub cur = nxt;
    nxt = nx2;
    if (j + 1 < Jtot) issue(nxt, j + 1);
    if (j + 2 < Jtot) nx2 = describe();
    const uint32_t gbase = lds_address(g_lds[st]);
    const uint32_t qbase = lds_address(q_lds[st]);
    constexpr int PF = 4;  // A-operand reads run PF MFMAs ahead
    // S = Q K^T (P role) or dP = dO V^T (dS role) of j: MFMA i is query block
    // i % 2, k-step i / 2 (two accumulation chains)
    const uint32_t abase = ds_role ? gbase : qbase;
    auto rd_a = [&](int i) {
      return *(const lds_bf16x8_t*)(uintptr_t)(abase + 2 * (aoff[i >> 1] + (i & 1) * 32 * D));
    };
    if constexpr (ds_role) {
      if (j > 0) make_ds(j - 1, lds_address(ld_lds[sp]) + 16 * hh + 4 * HB);
    }
    {
      static_assert(2 * KS == 4 * DT, "S/dP and dV/dK MFMAs pair up");
      // the MFMAs of j - 1: dV (P role, operand dO^T of j - 1) or dK (dS role, Q^T of j - 1)
      const bool with_prev = j > 0;
      // (stage sp of the ring as an offset from stage st: both are compile-time)
      const uint32_t pb = ds_role ? qbase + (uint32_t)(sp - st) * (uint32_t)sizeof(q_lds[0])
                                  : gbase + (uint32_t)(sp - st) * (uint32_t)sizeof(g_lds[0]);
      bf16x8_t aq[2 * KS], tq[2];
#pragma unroll
      for (int i = 0; i < PF; ++i) aq[i] = rd_a(i);
      if (with_prev) tq[0] = tr_read(pb, 0, 0);
      sd[0] = f32x16_t{};
      sd[1] = f32x16_t{};
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) {
        if (i + PF < 2 * KS) aq[i + PF] = rd_a(i + PF);
        sd[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[i], xreg[i >> 1], sd[i & 1], 0, 0, 0);
        if (with_prev) {
          if constexpr (ds_role)
            dk_mfma(pb, i, tq);
          else
            dv_mfma(pb, i, tq);
        }
      }
    }
    if constexpr (!ds_role) {
      // ---- P role: P of j, P mod'(S) to LDS, P as bf16 for step j + 1 ----
      const int hq = cur.hq, qs0 = cur.qs0;  // query head, first query row of the sub-step
      const bool partial = cur.partial;
      const auto scol = Score::col(p.score, Score::row(p.score, b, hq, 0), qs0 + 4 * hh, kvc);
      const int qlast = p.Sq - 1 - (qs0 + 4 * hh);
      const bool fix = partial | (qs0 + HB > p.Sq) | !kv_all;  // needs the zeroing pass below
      const uint32_t ldb = lds_address(ld_lds[st]) + 16 * hh;
      // element (mt, r): query row qs0 + 32 mt + 8 (r / 4) + 4 hh + r % 4
      float pm[2][16];
      f32x4_t l4;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int mt = e >> 4, r = e & 15;
        const int dr = 32 * mt + 8 * (r >> 2) + (r & 3);
        if ((r & 3) == 0)
          l4 = *(const __attribute__((address_space(3))) f32x4_t*)(uintptr_t)(ldb + 4 * (32 * mt + 8 * (r >> 2)));
        const float sv = sd[mt][r];
        // functors that read memory get an in-bounds row past Sq (zeroed below)
        const float pv = __builtin_amdgcn_exp2f(
            Score::apply_col(scol, sv, Score::kReadsMemory ? min(dr, qlast) : dr) - l4[r & 3]);
        pm[mt][r] = pv * Score::dmod_col(scol, sv);
        sd[mt][r] = pv;
      }
      // Zero what the mask drops (partial tiles), rows past Sq and a key past Skv
      if (fix) {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const int mt = e >> 4, r = e & 15;
          const int q = qs0 + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
          bool keep = kv_ok && q < p.Sq;
          if (partial) keep = keep && Mask::row(p.mask, b, hq, min(q, p.Sq - 1))(kvc);
          sd[mt][r] = keep ? sd[mt][r] : 0.0f;
          pm[mt][r] = keep ? pm[mt][r] : 0.0f;
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int mt = g >> 1, h8 = 8 * (g & 1);
        bf16x8_t pmb;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          pmb[k] = (__bf16)pm[mt][h8 + k];
          bo[g][k] = (__bf16)sd[mt][h8 + k];
        }
        *(__attribute__((address_space(3))) u32x4_t*)(uintptr_t)p_addr(j, g) = __builtin_bit_cast(u32x4_t, pmb);
      }
    }
  };
  if (Jtot > 0) {
    nxt = describe();
    issue(nxt, 0);
  }
  if (Jtot > 1) nx2 = describe();
  auto run = [&](auto role) {
    for (int j = 0; j < Jtot; j += 3) {
      step(j, std::integral_constant<int, 0>{}, role);
      if (j + 1 < Jtot) step(j + 1, std::integral_constant<int, 1>{}, role);
      if (j + 2 < Jtot) step(j + 2, std::integral_constant<int, 2>{}, role);
    }
  };
  if (ds_role)
    run(std::true_type{});
  else
    run(std::false_type{});
  if (Jtot > 0) {  // the MFMAs of the last sub-step (its stages are still intact)
    wait_lds_reads();
    __syncthreads();  // P mod'(S) of the last sub-step is in LDS
    const int jl = Jtot - 1, sl = jl % 3;
    bf16x8_t tq[2];
    if (ds_role) {
      make_ds(jl, lds_address(ld_lds[0]) + sl * (uint32_t)sizeof(ld_lds[0]) + 16 * hh + 4 * HB);
      const uint32_t ql = lds_address(q_lds[0]) + sl * (uint32_t)sizeof(q_lds[0]);
      tq[0] = tr_read(ql, 0, 0);
#pragma unroll
      for (int i = 0; i < 4 * DT; ++i) dk_mfma(ql, i, tq);
    } else {
      const uint32_t gl = lds_address(g_lds[0]) + sl * (uint32_t)sizeof(g_lds[0]);
      tq[0] = tr_read(gl, 0, 0);
#pragma unroll
      for (int i = 0; i < 4 * DT; ++i) dv_mfma(gl, i, tq);
    }
  }

  if (kv_ok) {  // dV from the P role, dK (times the scale) from the dS role
    const float sc = ds_role ? p.score.scale : 1.0f;
    uint16_t* G = ds_role
        ? P.dk + (long long)b * P.dks[0] + (long long)hkv * P.dks[1] + (long long)mykv * P.dks[2]
        : P.dv + (long long)b * P.dvs[0] + (long long)hkv * P.dvs[1] + (long long)mykv * P.dvs[2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4_t o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = (__bf16)(acc[dt][4 * g + i] * sc);
        *(bf16x4_t*)(G + 32 * dt + 8 * g + 4 * hh) = o4;
      }
    }
  }
}

template <int D, class Mask>
struct LaunchBwd {
  const BwdParams& P;
  hipStream_t stream;
  template <class Score>
  void operator()() {
    const FwdParams& p = P.f;
    const int NQ = (p.Sq + kBM - 1) / kBM, NK = (p.Skv + kBN - 1) / kBN;
    hipLaunchKernelGGL((bwd_dq_kernel<D, Mask, Score>), dim3((unsigned)(NQ * p.Hq * p.B)), dim3(kBwdThreads), 0,
                       stream, P);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, Mask, Score>), dim3((unsigned)(NK * p.Hkv * p.B)),
                       dim3(kDkdvThreads), 0, stream, P);
  }
};

// Launches the backward (after the prep kernel) for one mask kind, every score kind and both D.
template <class Mask>
fa_status launch_backward_mask(int D, int score_kind, const BwdParams& P, hipStream_t stream) {
  bool ok;
  if (D == 128) {
    LaunchBwd<128, Mask> l{P, stream};
    ok = dispatch_score(score_kind, l);
  } else if (D == 64) {
    LaunchBwd<64, Mask> l{P, stream};
    ok = dispatch_score(score_kind, l);
  } else {
    return FA_ERR_UNSUPPORTED;
  }
  if (!ok) return FA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace fa
