// Compile-time mask_mod and score_mod functors.
//
// A mask_mod decides from positions alone whether a query attends to a key
// (attention-gym "Concepts" page, "mask_mod"); a score_mod rewrites the scaled
// score (Concepts, "score_mod"; paper review "Flex Attention: A Programming
// Model for Generating Optimized Attention Kernels", §2.1-2.2).  Both are
// written once here and instantiated into the builder, forward and decode
// kernels; their runtime parameters (window, prefix, document ids, lengths,
// slopes, cap, bias tensor) are kernel arguments, so changing them never needs
// a rebuild.
//
// Every functor is split into a per-query-row part (`row`) evaluated once per
// lane and a per-key part evaluated per element, because each lane of the
// kernels owns one query row.  The forward additionally uses a per-tile form:
// `tile(row, kvb)` folds everything that is constant over a tile, and the
// per-element call takes the key as kvb + cr with cr a compile-time offset.
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "fa_internal.hpp"

namespace fa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// A read-only parameter at a wave-uniform address, read through the constant
// address space (a scalar load).
__device__ __forceinline__ float load_param(const float* p) {
  return *(const __attribute__((address_space(4))) float*)(uintptr_t)p;
}

// ---------------------------------------------------------------------------
// mask_mods
//
// classify(p, b, h, q0, q1, k0, k1, lane) gives the exact class of the
// in-range rectangle [q0, q1] x [k0, k1] (inclusive) when the mask's structure
// decides it, and kTileUnknown otherwise (the BlockMask builder then votes
// position by position).  Every lane of a wave calls it with the same
// arguments; the value is the same in every lane.
// ---------------------------------------------------------------------------

enum : int { kTileEmpty = 0, kTilePartial = 1, kTileFull = 2, kTileUnknown = 3 };

// Class of a mask that attends exactly where an integer quantity x >= 0, x
// taking every integer value between its minimum and maximum over the tile.
__device__ __forceinline__ int classify_threshold(long long xmin, long long xmax) {
  if (xmin >= 0) return kTileFull;
  if (xmax < 0) return kTileEmpty;
  return kTilePartial;
}

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = min(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off));
  return x;
}

struct MaskNone {
  static constexpr bool kBatchDependent = false;
  static constexpr bool kReadsMemory = false;
  struct Row {
    __device__ __forceinline__ bool operator()(int) const { return true; }
  };
  static __device__ __forceinline__ Row row(const MaskParams&, int, int, int) { return {}; }
  struct Tile {};
  static __device__ __forceinline__ Tile tile(const Row&, int) { return {}; }
  static __device__ __forceinline__ bool keep(const Tile&, int) { return true; }
  static __device__ __forceinline__ void keep4(const Tile&, int, const int (&)[4], bool (&k)[4]) {
    k[0] = k[1] = k[2] = k[3] = true;
  }
  static __device__ __forceinline__ int classify(const MaskParams&, int, int, int, int, int, int, int) {
    return kTileFull;
  }
};

// Concepts "mask_mod": causal, q >= kv.
struct MaskCausal {
  static constexpr bool kBatchDependent = false;
  static constexpr bool kReadsMemory = false;
  struct Row {
    int q;
    __device__ __forceinline__ bool operator()(int kv) const { return q >= kv; }
  };
  static __device__ __forceinline__ Row row(const MaskParams&, int, int, int q) { return {q}; }
  struct Tile {
    int dq;  // q - kvb
  };
  static __device__ __forceinline__ Tile tile(const Row& r, int kvb) { return {r.q - kvb}; }
  static __device__ __forceinline__ bool keep(const Tile& t, int cr) { return cr <= t.dq; }
  static __device__ __forceinline__ void keep4(const Tile& t, int cr, const int (&)[4], bool (&k)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = keep(t, cr + i);
  }
  static __device__ __forceinline__ int classify(const MaskParams&, int, int, int q0, int q1, int k0, int k1, int) {
    return classify_threshold((long long)q0 - k1, (long long)q1 - k0);  // x = q - kv
  }
};

// The window term of Concepts "Composing masks": q - kv <= window.
struct MaskWindow {
  static constexpr bool kBatchDependent = false;
  static constexpr bool kReadsMemory = false;
  struct Row {
    int lo;  // smallest kv with q - kv <= window
    __device__ __forceinline__ bool operator()(int kv) const { return kv >= lo; }
  };
  static __device__ __forceinline__ Row row(const MaskParams& p, int, int, int q) {
    return {q - p.window};
  }
  struct Tile {
    int lo;  // q - window - kvb
  };
  static __device__ __forceinline__ Tile tile(const Row& r, int kvb) { return {r.lo - kvb}; }
  static __device__ __forceinline__ bool keep(const Tile& t, int cr) { return cr >= t.lo; }
  static __device__ __forceinline__ void keep4(const Tile& t, int cr, const int (&)[4], bool (&k)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = keep(t, cr + i);
  }
  static __device__ __forceinline__ int classify(const MaskParams& p, int, int, int q0, int q1, int k0, int k1, int) {
    return classify_threshold((long long)k0 - q1 + p.window, (long long)k1 - q0 + p.window);  // x = kv - q + window
  }
};

// Talk summary (variant list) / paper review §5.3: same document only.
struct MaskDocument {
  static constexpr bool kBatchDependent = true;
  static constexpr bool kReadsMemory = true;
  struct Row {
    const int* doc;
    int dq;
    __device__ __forceinline__ bool operator()(int kv) const { return doc[kv] == dq; }
  };
  static __device__ __forceinline__ Row row(const MaskParams& p, int b, int, int q) {
    const int* d = p.doc + (long long)b * p.doc_stride_b;
    return {d, d[q]};
  }
  struct Tile {
    const int* doc;  // doc + kvb
    int dq;
  };
  static __device__ __forceinline__ Tile tile(const Row& r, int kvb) { return {r.doc + kvb, r.dq}; }
  static __device__ __forceinline__ bool keep(const Tile& t, int cr) { return t.doc[cr] == t.dq; }
  // Keys cr..cr+3 given their document ids (read by the caller, e.g. from a
  // copy of the tile's ids in LDS).
  static __device__ __forceinline__ void keep4(const Tile& t, int, const int (&ids)[4], bool (&k)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = ids[i] == t.dq;
  }
  // One document on each side decides the tile; so do disjoint id ranges.
  static __device__ int classify(const MaskParams& p, int b, int, int q0, int q1, int k0, int k1, int lane) {
    const int* d = p.doc + (long long)b * p.doc_stride_b;
    int qmin = INT_MAX, qmax = INT_MIN, kmin = INT_MAX, kmax = INT_MIN;
    for (int i = q0 + lane; i <= q1; i += 64) {
      qmin = min(qmin, d[i]);
      qmax = max(qmax, d[i]);
    }
    for (int i = k0 + lane; i <= k1; i += 64) {
      kmin = min(kmin, d[i]);
      kmax = max(kmax, d[i]);
    }
    qmin = wave_min(qmin);
    qmax = wave_max(qmax);
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
    if (qmax < kmin || kmax < qmin) return kTileEmpty;
    if (qmin == qmax && kmin == kmax) return kTileFull;  // (ids equal: the ranges overlap)
    return kTileUnknown;
  }
};

// The prefix term of paper review §4.4: keys before prefix_len are visible to all.
struct MaskPrefix {
  static constexpr bool kBatchDependent = false;
  static constexpr bool kReadsMemory = false;
  struct Row {
    int n;
    __device__ __forceinline__ bool operator()(int kv) const { return kv < n; }
  };
  static __device__ __forceinline__ Row row(const MaskParams& p, int, int, int) { return {p.prefix_len}; }
  struct Tile {
    int n;  // prefix_len - kvb
  };
  static __device__ __forceinline__ Tile tile(const Row& r, int kvb) { return {r.n - kvb}; }
  static __device__ __forceinline__ bool keep(const Tile& t, int cr) { return cr < t.n; }
  static __device__ __forceinline__ void keep4(const Tile& t, int cr, const int (&)[4], bool (&k)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = keep(t, cr + i);
  }
  static __device__ __forceinline__ int classify(const MaskParams& p, int, int, int, int, int k0, int k1, int) {
    return classify_threshold((long long)p.prefix_len - 1 - k1, (long long)p.prefix_len - 1 - k0);
  }
};

// Valid prefix of a KV cache: kv < kv_len[b].
struct MaskKvLen {
  static constexpr bool kBatchDependent = true;
  static constexpr bool kReadsMemory = false;
  struct Row {
    int n;
    __device__ __forceinline__ bool operator()(int kv) const { return kv < n; }
  };
  static __device__ __forceinline__ Row row(const MaskParams& p, int b, int, int) { return {p.kv_len[b]}; }
  struct Tile {
    int n;  // kv_len[b] - kvb
  };
  static __device__ __forceinline__ Tile tile(const Row& r, int kvb) { return {r.n - kvb}; }
  static __device__ __forceinline__ bool keep(const Tile& t, int cr) { return cr < t.n; }
  static __device__ __forceinline__ void keep4(const Tile& t, int cr, const int (&)[4], bool (&k)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = keep(t, cr + i);
  }
  static __device__ __forceinline__ int classify(const MaskParams& p, int b, int, int, int, int k0, int k1, int) {
    const int n = p.kv_len[b];
    return classify_threshold((long long)n - 1 - k1, (long long)n - 1 - k0);
  }
};

// Logical fusion (paper review §4.4; Concepts "Composing masks").
template <class A, class B>
struct MaskAnd {
  static constexpr bool kBatchDependent = A::kBatchDependent || B::kBatchDependent;
  static constexpr bool kReadsMemory = A::kReadsMemory || B::kReadsMemory;
  struct Row {
    typename A::Row a;
    typename B::Row b;
    __device__ __forceinline__ bool operator()(int kv) const { return a(kv) && b(kv); }
  };
  static __device__ __forceinline__ Row row(const MaskParams& p, int b, int h, int q) {
    return {A::row(p, b, h, q), B::row(p, b, h, q)};
  }
  struct Tile {
    typename A::Tile a;
    typename B::Tile b;
  };
  static __device__ __forceinline__ Tile tile(const Row& r, int kvb) { return {A::tile(r.a, kvb), B::tile(r.b, kvb)}; }
  static __device__ __forceinline__ bool keep(const Tile& t, int cr) { return A::keep(t.a, cr) && B::keep(t.b, cr); }
  static __device__ __forceinline__ void keep4(const Tile& t, int cr, const int (&ids)[4], bool (&k)[4]) {
    bool ka[4], kb[4];
    A::keep4(t.a, cr, ids, ka);
    B::keep4(t.b, cr, ids, kb);
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = ka[i] && kb[i];
  }
  static __device__ int classify(const MaskParams& p, int b, int h, int q0, int q1, int k0, int k1, int lane) {
    const int ca = A::classify(p, b, h, q0, q1, k0, k1, lane);
    if (ca == kTileEmpty) return kTileEmpty;
    const int cb = B::classify(p, b, h, q0, q1, k0, k1, lane);
    if (cb == kTileEmpty) return kTileEmpty;
    if (ca == kTileFull) return cb;
    if (cb == kTileFull) return ca;
    return kTileUnknown;  // partial AND partial can be anything
  }
};

template <class A, class B>
struct MaskOr {
  static constexpr bool kBatchDependent = A::kBatchDependent || B::kBatchDependent;
  static constexpr bool kReadsMemory = A::kReadsMemory || B::kReadsMemory;
  struct Row {
    typename A::Row a;
    typename B::Row b;
    __device__ __forceinline__ bool operator()(int kv) const { return a(kv) || b(kv); }
  };

  static __device__ __forceinline__ Row row(const MaskParams& p, int b, int h, int q) {
    return {A::row(p, b, h, q), B::row(p, b, h, q)};
  }
  struct Tile {
    typename A::Tile a;
    typename B::Tile b;
  };
  static __device__ __forceinline__ Tile tile(const Row& r, int kvb) { return {A::tile(r.a, kvb), B::tile(r.b, kvb)}; }
  static __device__ __forceinline__ bool keep(const Tile& t, int cr) { return A::keep(t.a, cr) || B::keep(t.b, cr); }
  static __device__ __forceinline__ void keep4(const Tile& t, int cr, const int (&ids)[4], bool (&k)[4]) {
    bool ka[4], kb[4];
    A::keep4(t.a, cr, ids, ka);
    B::keep4(t.b, cr, ids, kb);
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = ka[i] || kb[i];
  }
  static __device__ int classify(const MaskParams& p, int b, int h, int q0, int q1, int k0, int k1, int lane) {
    const int ca = A::classify(p, b, h, q0, q1, k0, k1, lane);
    if (ca == kTileFull) return kTileFull;
    const int cb = B::classify(p, b, h, q0, q1, k0, k1, lane);
    if (cb == kTileFull) return kTileFull;
    if (ca == kTileEmpty) return cb;
    if (cb == kTileEmpty) return ca;
    return kTileUnknown;  // partial OR partial can be anything
  }
};

// The parts of a mask that read memory, and whether the others decide nothing
// on a rectangle: where rest_full holds, keep4_mem gives the same answer as
// keep4 with fewer compares (a document mask ANDed with causal, on a tile below
// the diagonal: only the document ids decide).  Leaf masks: a memory-reading
// mask is all of its own memory part; the others are their structural class.
template <class M>
struct MaskParts {
  static __device__ __forceinline__ bool rest_full(const MaskParams& p, int b, int h, int q0, int q1, int k0, int k1) {
    if constexpr (M::kReadsMemory)
      return true;
    else
      return M::classify(p, b, h, q0, q1, k0, k1, 0) == kTileFull;
  }
  static __device__ __forceinline__ void keep4_mem(const typename M::Tile& t, int cr, const int (&ids)[4],
                                                   bool (&k)[4]) {
    if constexpr (M::kReadsMemory) {
      M::keep4(t, cr, ids, k);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) k[i] = true;
    }
  }
};
template <class A, class B>
struct MaskParts<MaskAnd<A, B>> {
  static __device__ __forceinline__ bool rest_full(const MaskParams& p, int b, int h, int q0, int q1, int k0, int k1) {
    return MaskParts<A>::rest_full(p, b, h, q0, q1, k0, k1) && MaskParts<B>::rest_full(p, b, h, q0, q1, k0, k1);
  }
  static __device__ __forceinline__ void keep4_mem(const typename MaskAnd<A, B>::Tile& t, int cr, const int (&ids)[4],
                                                   bool (&k)[4]) {
    bool ka[4], kb[4];
    MaskParts<A>::keep4_mem(t.a, cr, ids, ka);
    MaskParts<B>::keep4_mem(t.b, cr, ids, kb);
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = ka[i] && kb[i];
  }
};
template <class A, class B>
struct MaskParts<MaskOr<A, B>> {  // (no shortcut: a full structural part would decide everything)
  static __device__ __forceinline__ bool rest_full(const MaskParams&, int, int, int, int, int, int) { return false; }
  static __device__ __forceinline__ void keep4_mem(const typename MaskOr<A, B>::Tile& t, int cr, const int (&ids)[4],
                                                   bool (&k)[4]) {
    MaskOr<A, B>::keep4(t, cr, ids, k);
  }
};

using MaskSlidingCausal = MaskAnd<MaskCausal, MaskWindow>;
using MaskDocumentCausal = MaskAnd<MaskDocument, MaskCausal>;
using MaskPrefixLM = MaskOr<MaskPrefix, MaskCausal>;

// Calls f.template operator()<MaskType>() for a runtime fa_mask_kind.
template <class F>
__host__ __device__ inline bool dispatch_mask(int kind, F&& f) {
  switch (kind) {
    case FA_MASK_NONE: f.template operator()<MaskNone>(); return true;
    case FA_MASK_CAUSAL: f.template operator()<MaskCausal>(); return true;
    case FA_MASK_SLIDING_WINDOW: f.template operator()<MaskWindow>(); return true;
    case FA_MASK_SLIDING_CAUSAL: f.template operator()<MaskSlidingCausal>(); return true;
    case FA_MASK_DOCUMENT: f.template operator()<MaskDocument>(); return true;
    case FA_MASK_DOCUMENT_CAUSAL: f.template operator()<MaskDocumentCausal>(); return true;
    case FA_MASK_PREFIX_LM: f.template operator()<MaskPrefixLM>(); return true;
    case FA_MASK_KV_LEN: f.template operator()<MaskKvLen>(); return true;
    default: return false;
  }
}

// ---------------------------------------------------------------------------
// score_mods, producing base-2 scores x2 = mod(s) * log2(e).
//
// `s` is the raw dot product Q.K (not yet scaled).  apply1(row, s, kv) gives
// x2 for one key.  The forward's tile form gives y = x2 - m_ref directly,
// folding the softmax reference max m_ref into the additive term, so the
// exponential needs no separate subtraction: tile(row, kvb, m_ref), then
// apply(tile, s, cr) for key kvb + cr.  at(p, row(p, b, h, 0), q) equals
// row(p, b, h, q) with only the per-query part recomputed.  The column form
// serves kernels where a lane holds one key kv and walks query rows q0 + dr:
// col(p, row(p, b, h, 0), q0, kv) folds what is constant over the column,
// apply_col(c, s, dr) gives x2 for query q0 + dr and dmod_col(c, s) the
// derivative of the mod with respect to s (scaled scores, log2(e) excluded).
//
// Functors whose score is linear in s plus a term linear in the key offset set
// kPreload: the forward then starts each QK^T accumulation from preload(row, c)
// (c = key offset inside a 32-key block, 0..31) and applies apply_pre(tile, acc,
// mt) = apply(tile, s, 32 mt + c), one multiply-add per element.
// ---------------------------------------------------------------------------

struct ScoreNone {
  static constexpr bool kReadsMemory = false;
  static constexpr bool kPreload = false;
  static constexpr bool kStagesBias = false;
  static constexpr bool kBounded = false;
  struct Row {
    float c;
  };
  static __device__ __forceinline__ Row row(const ScoreParams& p, int, int, int) { return {p.scale_log2}; }
  static __device__ __forceinline__ Row at(const ScoreParams&, const Row& r0, int) { return r0; }
  static __device__ __forceinline__ float apply1(const Row& r, float s, int, int) { return s * r.c; }
  using Col = Row;
  static __device__ __forceinline__ Col col(const ScoreParams&, const Row& r0, int, int) { return r0; }
  static __device__ __forceinline__ float apply_col(const Col& c, float s, int) { return s * c.c; }
  static __device__ __forceinline__ float dmod_col(const Col&, float) { return 1.0f; }
  struct Tile {
    float c, add;
  };
  static __device__ __forceinline__ Tile tile(const Row& r, int, float m_ref) { return {r.c, -m_ref}; }
  static __device__ __forceinline__ float apply(const Tile& t, float s, int) { return fmaf(s, t.c, t.add); }
  // d mod / d (scaled score), for the backward: 1 for every additive mod
  static __device__ __forceinline__ float dmod1(const Row&, float, int) { return 1.0f; }
};

// Concepts "score_mod": s + slope[h] * (kv - q).
struct ScoreAlibi {
  static constexpr bool kReadsMemory = false;
  static constexpr bool kPreload = true;
  static constexpr bool kStagesBias = false;
  static constexpr bool kBounded = false;
  struct Row {
    float c;    // scale * log2e
    float sl;   // slope[h] * log2e
    int q;
  };
  static __device__ __forceinline__ Row row(const ScoreParams& p, int, int h, int q) {
    float slope = p.slopes ? load_param(p.slopes + h) : exp2f(-8.0f * (float)(h + 1) / (float)p.Hq);
    return {p.scale_log2, slope * kLog2e, q};
  }
  static __device__ __forceinline__ Row at(const ScoreParams&, const Row& r0, int q) { return {r0.c, r0.sl, q}; }
  static __device__ __forceinline__ float apply1(const Row& r, float s, int kv, int) {
    return fmaf(s, r.c, r.sl * (float)(kv - r.q));
  }
  struct Col {
    float c, nsl, add;  // add = sl * (kv - q0)
  };
  static __device__ __forceinline__ Col col(const ScoreParams&, const Row& r0, int q0, int kv) {
    return {r0.c, -r0.sl, r0.sl * (float)(kv - q0)};
  }
  static __device__ __forceinline__ float apply_col(const Col& c, float s, int dr) {
    return fmaf(s, c.c, fmaf(c.nsl, (float)dr, c.add));
  }
  static __device__ __forceinline__ float dmod_col(const Col&, float) { return 1.0f; }
  struct Tile {
    float c, sl, add;  // add = sl * (kvb - q) - m_ref
  };
  static __device__ __forceinline__ Tile tile(const Row& r, int kvb, float m_ref) {
    return {r.c, r.sl, fmaf(r.sl, (float)(kvb - r.q), -m_ref)};
  }
  static __device__ __forceinline__ float apply(const Tile& t, float s, int cr) {
    return fmaf(s, t.c, fmaf(t.sl, (float)cr, t.add));
  }
  // s + sl c / (scale log2e): the key-offset term in units of the raw dot product
  static __device__ __forceinline__ float preload(const Row& r, int c) { return r.sl * (float)c / r.c; }
  static __device__ __forceinline__ float apply_pre(const Tile& t, float acc, int mt) {
    return fmaf(acc, t.c, fmaf(t.sl, (float)(32 * mt), t.add));
  }
  static __device__ __forceinline__ float dmod1(const Row&, float, int) { return 1.0f; }
};

// Softcapping (paper review §2.1 table): cap * tanh(s / cap), with
// tanh(y) = 1 - 2 / (1 + e^{2y}) evaluated with the hardware exp2 and
// reciprocal; the error this adds is measured against fp64 tanh in the tests.
struct ScoreSoftcap {
  static constexpr bool kReadsMemory = false;
  static constexpr bool kPreload = false;
  static constexpr bool kStagesBias = false;
  static constexpr bool kBounded = false;
  struct Row {
    float k;     // 2 * scale / cap * log2e
    float c2;    // cap * log2e
  };
  static __device__ __forceinline__ Row row(const ScoreParams& p, int, int, int) {
    return {p.tanh_k, p.cap_log2};
  }
  static __device__ __forceinline__ Row at(const ScoreParams&, const Row& r0, int) { return r0; }
  static __device__ __forceinline__ float apply1(const Row& r, float s, int, int) {
    float e = __builtin_amdgcn_exp2f(s * r.k);
    return fmaf(-2.0f * r.c2, __builtin_amdgcn_rcpf(1.0f + e), r.c2);
  }
  using Col = Row;
  static __device__ __forceinline__ Col col(const ScoreParams&, const Row& r0, int, int) { return r0; }
  static __device__ __forceinline__ float apply_col(const Col& c, float s, int) { return apply1(c, s, 0, 0); }
  static __device__ __forceinline__ float dmod_col(const Col& c, float s) { return dmod1(c, s, 0); }
  struct Tile {
    float k, neg2c2, add;  // add = cap*log2e - m_ref
  };
  static __device__ __forceinline__ Tile tile(const Row& r, int, float m_ref) {
    return {r.k, -2.0f * r.c2, r.c2 - m_ref};
  }
  static __device__ __forceinline__ float apply(const Tile& t, float s, int) {
    const float e = __builtin_amdgcn_exp2f(s * t.k);
    return fmaf(t.neg2c2, __builtin_amdgcn_rcpf(1.0f + e), t.add);
  }
  // d (cap tanh(x / cap)) / dx = 1 - tanh^2, with the same tanh as above
  static __device__ __forceinline__ float dmod1(const Row& r, float s, int) {
    const float th = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(s * r.k));
    return fmaf(-th, th, 1.0f);
  }
};

// Talk summary (score mode) / Concepts "Debugging score_mods": s + (q - kv).
struct ScoreRelPos {
  static constexpr bool kReadsMemory = false;
  static constexpr bool kPreload = true;
  static constexpr bool kStagesBias = false;
  static constexpr bool kBounded = false;
  struct Row {
    float c;
    int q;
  };
  static __device__ __forceinline__ Row row(const ScoreParams& p, int, int, int q) { return {p.scale_log2, q}; }
  static __device__ __forceinline__ Row at(const ScoreParams&, const Row& r0, int q) { return {r0.c, q}; }
  static __device__ __forceinline__ float apply1(const Row& r, float s, int kv, int) {
    return fmaf(s, r.c, kLog2e * (float)(r.q - kv));
  }
  struct Col {
    float c, add;  // add = log2e * (q0 - kv)
  };
  static __device__ __forceinline__ Col col(const ScoreParams&, const Row& r0, int q0, int kv) {
    return {r0.c, kLog2e * (float)(q0 - kv)};
  }
  static __device__ __forceinline__ float apply_col(const Col& c, float s, int dr) {
    return fmaf(s, c.c, fmaf(kLog2e, (float)dr, c.add));
  }
  static __device__ __forceinline__ float dmod_col(const Col&, float) { return 1.0f; }
  struct Tile {
    float c, add;  // add = log2e * (q - kvb) - m_ref
  };
  static __device__ __forceinline__ Tile tile(const Row& r, int kvb, float m_ref) {
    return {r.c, fmaf(kLog2e, (float)(r.q - kvb), -m_ref)};
  }
  static __device__ __forceinline__ float apply(const Tile& t, float s, int cr) {
    return fmaf(s, t.c, fmaf(-kLog2e, (float)cr, t.add));
  }
  static __device__ __forceinline__ float preload(const Row& r, int c) { return -kLog2e * (float)c / r.c; }
  static __device__ __forceinline__ float apply_pre(const Tile& t, float acc, int mt) {
    return fmaf(acc, t.c, fmaf(-kLog2e, (float)(32 * mt), t.add));
  }
  static __device__ __forceinline__ float dmod1(const Row&, float, int) { return 1.0f; }
};

// Dynamic-bias feature request (attention-gym issue 123): s + bias[b,h,q,kv].
struct ScoreBias {
  static constexpr bool kReadsMemory = true;
  static constexpr bool kPreload = false;
  static constexpr bool kStagesBias = false;
  static constexpr bool kBounded = false;
  struct Row {
    float c;
    const uint16_t* row;  // bias[b, h, q, :]
  };
  static __device__ __forceinline__ Row row(const ScoreParams& p, int b, int h, int q) {
    return {p.scale_log2, p.bias + (long long)b * p.bs0 + (long long)h * p.bs1 + (long long)q * p.bs2};
  }
  static __device__ __forceinline__ Row at(const ScoreParams& p, const Row& r0, int q) {
    return {r0.c, r0.row + (long long)q * p.bs2};
  }
  static __device__ __forceinline__ float apply1(const Row& r, float s, int kv, int) {
    return fmaf(kLog2e, bf16_bits_to_float(r.row[kv]), s * r.c);
  }
  struct Col {
    float c;
    const uint16_t* at;  // &bias[b, h, q0, kv]
    long long rs;        // row stride (elements)
  };
  static __device__ __forceinline__ Col col(const ScoreParams& p, const Row& r0, int q0, int kv) {
    return {r0.c, r0.row + (long long)q0 * p.bs2 + kv, p.bs2};
  }
  static __device__ __forceinline__ float apply_col(const Col& c, float s, int dr) {
    return fmaf(kLog2e, bf16_bits_to_float(c.at[dr * c.rs]), s * c.c);
  }
  static __device__ __forceinline__ float dmod_col(const Col&, float) { return 1.0f; }
  struct Tile {
    float c, add;
    const uint16_t* row;  // bias[b, h, q, kvb:]
  };
  static __device__ __forceinline__ Tile tile(const Row& r, int kvb, float m_ref) {
    return {r.c, -m_ref, r.row + kvb};
  }
  static __device__ __forceinline__ float apply(const Tile& t, float s, int cr) {
    return fmaf(s, t.c, fmaf(kLog2e, bf16_bits_to_float(t.row[cr]), t.add));
  }
  static __device__ __forceinline__ float dmod1(const Row&, float, int) { return 1.0f; }
};

// The dynamic bias with the forward staging each step's [128 query x 64 key]
// bias tile in LDS (coalesced 16-byte loads) instead of every lane reading its
// own row element by element.  Same arithmetic as ScoreBias; used when the
// bias layout is 16-byte aligned (base, row strides and Skv multiples of 8
// elements).
struct ScoreBiasTiled : ScoreBias {
  static constexpr bool kStagesBias = true;
  // x2 - m_ref for raw score s and a bias value b (bf16 bits).
  static __device__ __forceinline__ float apply_bits(const Tile& t, float s, uint32_t b) {
    return fmaf(s, t.c, fmaf(kLog2e, bf16_bits_to_float(b), t.add));
  }
};

// Softcapping with the softmax reference fixed at the cap: |cap tanh(x)| <= cap,
// so with the reference max at cap * log2(e) every exponent lies in
// [-2 cap log2(e), 0] and no running max is needed (softmax is unchanged by the
// shift).  Chosen by the launch when cap log2(e) <= kBoundedMaxLog2: every
// weight is then >= 2^-112, normal in fp32 and bf16, and so are its products
// with any V element of magnitude >= 2^-14.
//
// Relative to the bound, the score is y = cap log2(e) (tanh(x) - 1) =
// -2 cap log2(e) / (1 + e^{2x}), computed as 1 / (a (1 + e^{2x})) with
// a = -1 / (2 cap log2(e)): one multiply-add and a reciprocal after the exp2.
struct ScoreSoftcapBounded : ScoreSoftcap {
  static constexpr bool kBounded = true;
  static __device__ __forceinline__ float bound(const Row& r) { return r.c2; }
  struct Tile {
    float k, a;
  };
  static __device__ __forceinline__ Tile tile(const Row& r, int, float) { return {r.k, -0.5f / r.c2}; }
  static __device__ __forceinline__ float apply(const Tile& t, float s, int) {
    const float e = __builtin_amdgcn_exp2f(s * t.k);
    return __builtin_amdgcn_rcpf(fmaf(e, t.a, t.a));
  }
};
constexpr float kBoundedMaxLog2 = 56.0f;

template <class F>
__host__ __device__ inline bool dispatch_score(int kind, F&& f) {
  switch (kind) {
    case FA_SCORE_NONE: f.template operator()<ScoreNone>(); return true;
    case FA_SCORE_ALIBI: f.template operator()<ScoreAlibi>(); return true;
    case FA_SCORE_SOFTCAP: f.template operator()<ScoreSoftcap>(); return true;
    case FA_SCORE_REL_POS: f.template operator()<ScoreRelPos>(); return true;
    case FA_SCORE_BIAS: f.template operator()<ScoreBias>(); return true;
    default: return false;
  }
}

}  // namespace fa
