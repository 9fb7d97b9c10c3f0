// Host side of the C ABI declared in include/fa.h: argument validation,
// folding of score_mod constants, choice of the compiled instantiation and
// launch on the caller's stream.  No device memory is allocated here.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "fa_internal.hpp"

namespace fa {
// Measurement probes (probe.hip).
int probe_read_workgroups(size_t bytes);
fa_status launch_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

namespace {

thread_local char g_last_error[512] = "";

fa_status fail(fa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

constexpr float kLog2eHost = 1.4426950408889634f;
constexpr int64_t kMaxRowStride = (int64_t)1 << 25;  // K/V row strides in elements (64 MiB)

int ceil_div(int a, int b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Masks whose value depends on the batch row.
bool mask_batch_dependent(const fa_mask_desc& m) {
  switch (m.kind) {
    case FA_MASK_DOCUMENT:
    case FA_MASK_DOCUMENT_CAUSAL: return m.doc_stride_b != 0;
    case FA_MASK_KV_LEN: return true;
    default: return false;
  }
}

fa_status check_mask(const fa_mask_desc& m, int Sq, int Skv) {
  if (m.kind < 0 || m.kind >= FA_MASK_KIND_COUNT) return fail(FA_ERR_UNSUPPORTED, "unknown mask kind %d", m.kind);
  if ((m.kind == FA_MASK_SLIDING_WINDOW || m.kind == FA_MASK_SLIDING_CAUSAL) && m.window < 0)
    return fail(FA_ERR_SHAPE, "sliding window %d < 0", m.window);
  if (m.kind == FA_MASK_PREFIX_LM && m.prefix_len < 0)
    return fail(FA_ERR_SHAPE, "prefix_len %d < 0", m.prefix_len);
  if (m.kind == FA_MASK_DOCUMENT || m.kind == FA_MASK_DOCUMENT_CAUSAL) {
    if (m.doc_ids == nullptr) return fail(FA_ERR_NULL, "document mask without doc_ids");
    if (m.doc_stride_b < 0) return fail(FA_ERR_SHAPE, "doc_stride_b < 0");
    if (Sq != Skv) return fail(FA_ERR_SHAPE, "document masks need Sq == Skv (got %d, %d)", Sq, Skv);
  }
  if (m.kind == FA_MASK_KV_LEN && m.kv_len == nullptr) return fail(FA_ERR_NULL, "kv_len mask without kv_len");
  return FA_OK;
}

MaskParams mask_params(const fa_mask_desc& m) {
  MaskParams p;
  p.window = m.window;
  p.prefix_len = m.prefix_len;
  p.doc = m.doc_ids;
  p.doc_stride_b = m.doc_stride_b;
  p.kv_len = m.kv_len;
  p.doc_vec = m.doc_ids != nullptr && aligned16(m.doc_ids) && m.doc_stride_b % 4 == 0;
  return p;
}

fa_status check_strides(const char* name, const int64_t* s, const void* ptr) {
  if (s[3] != 1) return fail(FA_ERR_UNSUPPORTED, "%s: d stride must be 1 (got %lld)", name, (long long)s[3]);
  for (int i = 0; i < 3; ++i) {
    if (s[i] < 0) return fail(FA_ERR_SHAPE, "%s: negative stride", name);
    if (s[i] % 8 != 0) return fail(FA_ERR_UNSUPPORTED, "%s: stride[%d]=%lld not a multiple of 8", name, i, (long long)s[i]);
  }
  if (!aligned16(ptr)) return fail(FA_ERR_UNSUPPORTED, "%s: pointer not 16-byte aligned", name);
  return FA_OK;
}

// Validation shared by fa_forward and fa_decode; fills `p` on success.
fa_status prepare(const fa_attn_args* a, bool decode, FwdParams& p, int& mask_kind) {
  if (a == nullptr) return fail(FA_ERR_NULL, "args is NULL");
  if (!a->q || !a->k || !a->v || !a->o) return fail(FA_ERR_NULL, "q, k, v and o must be non-NULL");
  if (a->B <= 0 || a->Hq <= 0 || a->Hkv <= 0 || a->Sq <= 0 || a->Skv <= 0 || a->D <= 0)
    return fail(FA_ERR_SHAPE, "sizes must be positive");
  if (a->Hq % a->Hkv != 0) return fail(FA_ERR_SHAPE, "Hq %% Hkv != 0 (%d, %d)", a->Hq, a->Hkv);
  if (a->D != 64 && a->D != 128) return fail(FA_ERR_UNSUPPORTED, "D=%d (supported: 64, 128)", a->D);
  if (decode && a->Sq != 1) return fail(FA_ERR_SHAPE, "decode needs Sq == 1 (got %d)", a->Sq);
  if (!decode && a->q_pos != nullptr) return fail(FA_ERR_UNSUPPORTED, "q_pos is an argument of fa_decode only");
  if (a->page_table != nullptr) {
    if (!decode) return fail(FA_ERR_UNSUPPORTED, "a paged KV cache is supported by fa_decode only");
    if (a->num_pages <= 0) return fail(FA_ERR_SHAPE, "num_pages must be positive (got %d)", a->num_pages);
    if (a->page_table_stride < ceil_div(a->Skv, FA_BLOCK))
      return fail(FA_ERR_SHAPE, "page_table_stride %lld < ceil(Skv/128) = %d", (long long)a->page_table_stride,
                  ceil_div(a->Skv, FA_BLOCK));
  }
  fa_status st;
  if ((st = check_strides("q", a->q_stride, a->q)) != FA_OK) return st;
  if ((st = check_strides("k", a->k_stride, a->k)) != FA_OK) return st;
  if ((st = check_strides("v", a->v_stride, a->v)) != FA_OK) return st;
  if ((st = check_strides("o", a->o_stride, a->o)) != FA_OK) return st;
  // the kernels address the rows of a 64-key K/V sub-tile with 32-bit offsets
  if (a->k_stride[2] >= kMaxRowStride || a->v_stride[2] >= kMaxRowStride)
    return fail(FA_ERR_UNSUPPORTED, "k/v row stride must be below %lld elements", (long long)kMaxRowStride);
  if (!(isfinite(a->scale)) || a->scale < 0.0f) return fail(FA_ERR_SHAPE, "scale must be finite and >= 0");
  if (a->scale > 0.0f && a->scale < 1e-20f) return fail(FA_ERR_SHAPE, "scale must be 0 (default) or >= 1e-20");

  const int NQ = ceil_div(a->Sq, FA_BLOCK), NK = ceil_div(a->Skv, FA_BLOCK);
  if ((long long)NQ * a->Hq * a->B > 0x7fffffffLL) return fail(FA_ERR_SHAPE, "too many query tiles");
  if (a->B > 65535 || a->Hkv > 65535) return fail(FA_ERR_SHAPE, "B and Hkv must be <= 65535");

  memset(&p, 0, sizeof(p));
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  for (int i = 0; i < 4; ++i) {
    p.qs[i] = a->q_stride[i];
    p.ks[i] = a->k_stride[i];
    p.vs[i] = a->v_stride[i];
    p.os[i] = a->o_stride[i];
  }
  p.B = a->B;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.Sq = a->Sq;
  p.Skv = a->Skv;
  p.G = a->Hq / a->Hkv;

  // BlockMask
  mask_kind = FA_MASK_NONE;
  const fa_block_mask* bm = a->block_mask;
  if (bm == nullptr) {
    p.bm.dense = 1;
    p.bm.NK = NK;
    p.bm.NQ = NQ;
    p.bm.Bm = p.bm.Hm = 1;
    p.bm.separate_full = 1;
    p.bm.q_order = nullptr;
  } else {
    if (bm->block_q != FA_BLOCK || bm->block_kv != FA_BLOCK)
      return fail(FA_ERR_UNSUPPORTED, "BlockMask block size %dx%d (supported: 128x128)", bm->block_q, bm->block_kv);
    if (!bm->kv_num_blocks || !bm->kv_indices || !bm->full_kv_num_blocks || !bm->full_kv_indices)
      return fail(FA_ERR_NULL, "BlockMask tensors must be non-NULL");
    if (bm->NQ != NQ || bm->NK != NK)
      return fail(FA_ERR_SHAPE, "BlockMask dims %dx%d do not match ceil(S/128) = %dx%d", bm->NQ, bm->NK, NQ, NK);
    if (bm->Sq != a->Sq || bm->Skv != a->Skv)
      return fail(FA_ERR_SHAPE, "BlockMask was built for Sq=%d Skv=%d, call has %d, %d", bm->Sq, bm->Skv, a->Sq, a->Skv);
    if (!(bm->Bm == 1 || bm->Bm == a->B)) return fail(FA_ERR_SHAPE, "BlockMask Bm=%d not in {1, B=%d}", bm->Bm, a->B);
    if (!(bm->Hm == 1 || bm->Hm == a->Hq)) return fail(FA_ERR_SHAPE, "BlockMask Hm=%d not in {1, Hq=%d}", bm->Hm, a->Hq);
    if ((st = check_mask(bm->mask, a->Sq, a->Skv)) != FA_OK) return st;
    if (bm->Bm == 1 && a->B > 1 && mask_batch_dependent(bm->mask))
      return fail(FA_ERR_SHAPE, "mask depends on the batch row but the BlockMask has Bm=1 and B=%d", a->B);
    if (bm->separate_full != 0 && bm->separate_full != 1) return fail(FA_ERR_SHAPE, "separate_full must be 0 or 1");
    p.bm.kv_num = bm->kv_num_blocks;
    p.bm.kv_idx = bm->kv_indices;
    p.bm.full_num = bm->full_kv_num_blocks;
    p.bm.full_idx = bm->full_kv_indices;
    p.bm.Bm = bm->Bm;
    p.bm.Hm = bm->Hm;
    p.bm.NQ = NQ;
    p.bm.NK = NK;
    p.bm.dense = 0;
    p.bm.separate_full = bm->separate_full;
    p.bm.q_order = bm->q_order;
    p.mask = mask_params(bm->mask);
    mask_kind = bm->mask.kind;
  }

  // score_mod constants
  const fa_score_desc& sd = a->score;
  if (sd.kind < 0 || sd.kind >= FA_SCORE_KIND_COUNT) return fail(FA_ERR_UNSUPPORTED, "unknown score kind %d", sd.kind);
  const float scale = a->scale > 0.0f ? a->scale : 1.0f / sqrtf((float)a->D);
  p.score.scale = scale;
  p.score.scale_log2 = scale * kLog2eHost;
  p.score.Hq = a->Hq;
  p.score.slopes = sd.alibi_slopes;
  if (sd.kind == FA_SCORE_SOFTCAP) {
    if (!(sd.softcap > 0.0f) || !isfinite(sd.softcap)) return fail(FA_ERR_SHAPE, "softcap must be finite and > 0");
    p.score.cap_log2 = sd.softcap * kLog2eHost;
    p.score.tanh_k = 2.0f * scale / sd.softcap * kLog2eHost;
  }
  if (sd.kind == FA_SCORE_BIAS) {
    if (sd.bias == nullptr) return fail(FA_ERR_NULL, "bias score without a bias tensor");
    if (sd.bias_stride[3] != 1) return fail(FA_ERR_UNSUPPORTED, "bias kv stride must be 1");
    for (int i = 0; i < 3; ++i)
      if (sd.bias_stride[i] < 0) return fail(FA_ERR_SHAPE, "negative bias stride");
    if (((uintptr_t)sd.bias & 1u) != 0) return fail(FA_ERR_UNSUPPORTED, "bias pointer not 2-byte aligned");
    p.score.bias = sd.bias;
    p.score.bs0 = sd.bias_stride[0];
    p.score.bs1 = sd.bias_stride[1];
    p.score.bs2 = sd.bias_stride[2];
  }
  return FA_OK;
}

struct DecodePlan {
  int splits;
  int bps;
};

DecodePlan decode_plan(const fa_attn_args* a) {
  const int NK = ceil_div(a->Skv, FA_BLOCK);
  int bps;
  if (a->num_splits > 0) {
    bps = ceil_div(NK, a->num_splits);
  } else {
    // Seven tiles per chunk (measured best for long caches with the longest
    // sequences first; 6 and 8 within 1-1.5%), fewer while the grid would not
    // cover the 256 CUs many times over.
    bps = 7;
    while (bps > 1 && (long long)a->B * a->Hkv * ceil_div(NK, bps) < 4096) --bps;
  }
  if (bps < 1) bps = 1;
  if (bps > 8) bps = 8;
  return {ceil_div(NK, bps), bps};
}

fa_status prepare_decode(const fa_attn_args* a, FwdParams& p, int& mask_kind, DecodePlan& plan, size_t& bytes) {
  fa_status st = prepare(a, true, p, mask_kind);
  if (st != FA_OK) return st;
  const int G = a->Hq / a->Hkv;
  if (!(G == 1 || G == 2 || G == 4 || G == 8))
    return fail(FA_ERR_UNSUPPORTED, "decode GQA group %d (supported: 1, 2, 4, 8)", G);
  if (a->block_mask && a->block_mask->Hm > 1 && G != 1)
    return fail(FA_ERR_UNSUPPORTED, "decode with a per-head BlockMask needs group size 1");
  // The decode BlockMask has one query row (built with Sq = 1, the query at
  // index 0), so a mask that depends on the query position would be
  // classified for the wrong query; kv_len expresses a causal cache.
  if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_KV_LEN)
    return fail(FA_ERR_UNSUPPORTED, "decode supports the none and kv_len masks only (got kind %d): the "
                                    "BlockMask's one query row cannot follow the query position", mask_kind);
  if (a->num_splits < 0) return fail(FA_ERR_SHAPE, "num_splits < 0");
  plan = decode_plan(a);
  if ((long long)plan.splits > 0x7fffffffLL) return fail(FA_ERR_SHAPE, "too many splits");
  bytes = (size_t)plan.splits * a->B * a->Hq * (size_t)(a->D + 1) * sizeof(float);
  return FA_OK;
}

fa_status prepare_backward(const fa_attn_args* a, const fa_grad_args* g, BwdParams& P, int& mask_kind,
                           size_t& bytes) {
  fa_status st = prepare(a, false, P.f, mask_kind);
  if (st != FA_OK) return st;
  if (a->lse == nullptr) return fail(FA_ERR_NULL, "the backward needs the forward's LSE (lse)");
  const fa_block_mask* bm = a->block_mask;
  if (bm != nullptr && (!bm->q_num_blocks || !bm->q_indices || !bm->full_q_num_blocks || !bm->full_q_indices))
    return fail(FA_ERR_NULL, "the backward needs the BlockMask's transposed view (q_num_blocks, q_indices, "
                             "full_q_num_blocks, full_q_indices)");
  const int NQ = ceil_div(a->Sq, FA_BLOCK);
  P.sq_pad = NQ * FA_BLOCK;
  bytes = 2 * sizeof(float) * (size_t)a->B * a->Hq * P.sq_pad;
  if (g == nullptr) return FA_OK;  // size query
  if (!g->dout || !g->dq || !g->dk || !g->dv) return fail(FA_ERR_NULL, "dout, dq, dk and dv must be non-NULL");
  if ((st = check_strides("dout", g->dout_stride, g->dout)) != FA_OK) return st;
  if ((st = check_strides("dq", g->dq_stride, g->dq)) != FA_OK) return st;
  if ((st = check_strides("dk", g->dk_stride, g->dk)) != FA_OK) return st;
  if ((st = check_strides("dv", g->dv_stride, g->dv)) != FA_OK) return st;
  P.dout = g->dout;
  P.dq = g->dq;
  P.dk = g->dk;
  P.dv = g->dv;
  for (int i = 0; i < 4; ++i) {
    P.dos[i] = g->dout_stride[i];
    P.dqs[i] = g->dq_stride[i];
    P.dks[i] = g->dk_stride[i];
    P.dvs[i] = g->dv_stride[i];
  }
  P.q_num = bm ? bm->q_num_blocks : nullptr;
  P.q_idx = bm ? bm->q_indices : nullptr;
  P.full_q_num = bm ? bm->full_q_num_blocks : nullptr;
  P.kv_order = bm ? bm->kv_order : nullptr;
  P.full_q_idx = bm ? bm->full_q_indices : nullptr;
  return FA_OK;
}

fa_status run_decode(const fa_attn_args* a, const FwdParams& p, int mask_kind, const DecodePlan& plan,
                     void* workspace, hipStream_t stream) {
  DecodeParams P;
  P.f = p;
  P.mask_kind = mask_kind;
  P.splits = plan.splits;
  P.blocks_per_split = plan.bps;
  P.ws_o = (float*)workspace;
  P.ws_lse = P.ws_o + (size_t)plan.splits * a->B * a->Hq * a->D;
  P.page_table = a->page_table;
  P.pt_stride = a->page_table_stride;
  P.num_pages = a->num_pages;
  P.q_pos = a->q_pos;
  const fa_block_mask* bm = a->block_mask;
  P.row_order = (bm != nullptr && bm->row_order != nullptr && bm->Bm == a->B && bm->NQ == 1 && bm->Hm == 1)
                    ? bm->row_order : nullptr;
  const fa_status st = launch_decode(a->D, a->Hq / a->Hkv, a->score.kind, P, stream);
  if (st != FA_OK) return fail(st, "decode launch failed");
  return FA_OK;
}

}  // namespace

fa_status launch_backward(int D, int mask_kind, int score_kind, const BwdParams& p, hipStream_t s) {
  switch (mask_kind) {
    case FA_MASK_NONE: return launch_backward_none(D, score_kind, p, s);
    case FA_MASK_CAUSAL: return launch_backward_causal(D, score_kind, p, s);
    case FA_MASK_SLIDING_WINDOW: return launch_backward_window(D, score_kind, p, s);
    case FA_MASK_SLIDING_CAUSAL: return launch_backward_sliding_causal(D, score_kind, p, s);
    case FA_MASK_DOCUMENT: return launch_backward_document(D, score_kind, p, s);
    case FA_MASK_DOCUMENT_CAUSAL: return launch_backward_document_causal(D, score_kind, p, s);
    case FA_MASK_PREFIX_LM: return launch_backward_prefix_lm(D, score_kind, p, s);
    case FA_MASK_KV_LEN: return launch_backward_kv_len(D, score_kind, p, s);
    default: return FA_ERR_UNSUPPORTED;
  }
}

fa_status launch_forward(int D, int mask_kind, int score_kind, const FwdParams& p, hipStream_t s) {
  switch (mask_kind) {
    case FA_MASK_NONE: return launch_forward_none(D, score_kind, p, s);
    case FA_MASK_CAUSAL: return launch_forward_causal(D, score_kind, p, s);
    case FA_MASK_SLIDING_WINDOW: return launch_forward_window(D, score_kind, p, s);
    case FA_MASK_SLIDING_CAUSAL: return launch_forward_sliding_causal(D, score_kind, p, s);
    case FA_MASK_DOCUMENT: return launch_forward_document(D, score_kind, p, s);
    case FA_MASK_DOCUMENT_CAUSAL: return launch_forward_document_causal(D, score_kind, p, s);
    case FA_MASK_PREFIX_LM: return launch_forward_prefix_lm(D, score_kind, p, s);
    case FA_MASK_KV_LEN: return launch_forward_kv_len(D, score_kind, p, s);
    default: return FA_ERR_UNSUPPORTED;
  }
}

}  // namespace fa

using namespace fa;

extern "C" {

int32_t fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    default: return "FA_ERR_UNKNOWN";
  }
}

const char* fa_last_error(void) { return g_last_error; }

fa_status fa_block_mask_dims(int32_t Sq, int32_t Skv, int32_t block_q, int32_t block_kv, int32_t* NQ, int32_t* NK) {
  if (NQ == nullptr || NK == nullptr) return fail(FA_ERR_NULL, "NQ/NK outputs are NULL");
  if (Sq <= 0 || Skv <= 0) return fail(FA_ERR_SHAPE, "sequence lengths must be positive");
  if (block_q != FA_BLOCK || block_kv != FA_BLOCK)
    return fail(FA_ERR_UNSUPPORTED, "block size %dx%d (supported: 128x128)", block_q, block_kv);
  *NQ = ceil_div(Sq, block_q);
  *NK = ceil_div(Skv, block_kv);
  return FA_OK;
}

fa_status fa_build_block_mask(fa_block_mask* bm, int32_t Sq, int32_t Skv, void* stream) {
  if (bm == nullptr) return fail(FA_ERR_NULL, "BlockMask is NULL");
  if (!bm->kv_num_blocks || !bm->kv_indices || !bm->full_kv_num_blocks || !bm->full_kv_indices)
    return fail(FA_ERR_NULL, "BlockMask tensors must be non-NULL");
  if (bm->block_q != FA_BLOCK || bm->block_kv != FA_BLOCK)
    return fail(FA_ERR_UNSUPPORTED, "block size %dx%d (supported: 128x128)", bm->block_q, bm->block_kv);
  if (Sq <= 0 || Skv <= 0) return fail(FA_ERR_SHAPE, "sequence lengths must be positive");
  if (bm->NQ != ceil_div(Sq, FA_BLOCK) || bm->NK != ceil_div(Skv, FA_BLOCK))
    return fail(FA_ERR_SHAPE, "BlockMask dims %dx%d do not match ceil(S/128)", bm->NQ, bm->NK);
  if (bm->Bm < 1 || bm->Hm < 1 || bm->Bm > 65535 || bm->Hm > 65535)
    return fail(FA_ERR_SHAPE, "Bm and Hm must be in [1, 65535]");
  if (bm->separate_full != 0 && bm->separate_full != 1) return fail(FA_ERR_SHAPE, "separate_full must be 0 or 1");
  const int n_transposed = (bm->q_num_blocks != nullptr) + (bm->q_indices != nullptr) +
                           (bm->full_q_num_blocks != nullptr) + (bm->full_q_indices != nullptr);
  if (n_transposed != 0 && n_transposed != 4)
    return fail(FA_ERR_NULL, "the transposed view needs all four of q_num_blocks, q_indices, "
                             "full_q_num_blocks and full_q_indices (or none)");
  if (bm->q_order != nullptr && bm->NQ > 16384)
    return fail(FA_ERR_UNSUPPORTED, "q_order needs NQ <= 16384 (got %d)", bm->NQ);
  if (bm->kv_order != nullptr && n_transposed != 4)
    return fail(FA_ERR_NULL, "kv_order is built from the transposed view, which is not requested");
  if (bm->kv_order != nullptr && bm->NK > 16384)
    return fail(FA_ERR_UNSUPPORTED, "kv_order needs NK <= 16384 (got %d)", bm->NK);
  if (bm->row_order != nullptr && (bm->NQ != 1 || bm->Hm != 1))
    return fail(FA_ERR_SHAPE, "row_order needs one query block and one head row (NQ = %d, Hm = %d)", bm->NQ, bm->Hm);
  if (bm->row_order != nullptr && bm->Bm > 16384)
    return fail(FA_ERR_UNSUPPORTED, "row_order needs Bm <= 16384 (got %d)", bm->Bm);
  fa_status st = check_mask(bm->mask, Sq, Skv);
  if (st != FA_OK) return st;

  BuildParams p;
  p.kv_num = bm->kv_num_blocks;
  p.kv_idx = bm->kv_indices;
  p.full_num = bm->full_kv_num_blocks;
  p.full_idx = bm->full_kv_indices;
  p.q_num = bm->q_num_blocks;
  p.q_idx = bm->q_indices;
  p.full_q_num = bm->full_q_num_blocks;
  p.full_q_idx = bm->full_q_indices;
  p.q_order = bm->q_order;
  p.kv_order = bm->kv_order;
  p.row_order = bm->row_order;
  p.Bm = bm->Bm;
  p.Hm = bm->Hm;
  p.NQ = bm->NQ;
  p.NK = bm->NK;
  p.Sq = Sq;
  p.Skv = Skv;
  p.separate_full = bm->separate_full;
  p.mask = mask_params(bm->mask);
  st = launch_block_mask(bm->mask.kind, p, (hipStream_t)stream);
  if (st != FA_OK) return fail(st, "block mask launch failed");
  bm->Sq = Sq;
  bm->Skv = Skv;
  return FA_OK;
}

fa_status fa_forward(const fa_attn_args* a, void* stream) {
  FwdParams p;
  int mask_kind;
  fa_status st = prepare(a, false, p, mask_kind);
  if (st != FA_OK) return st;
  st = launch_forward(a->D, mask_kind, a->score.kind, p, (hipStream_t)stream);
  if (st != FA_OK) return fail(st, "forward launch failed");
  return FA_OK;
}

fa_status fa_decode_workspace_size(const fa_attn_args* a, size_t* bytes) {
  if (bytes == nullptr) return fail(FA_ERR_NULL, "bytes is NULL");
  FwdParams p;
  int mask_kind;
  DecodePlan plan;
  return prepare_decode(a, p, mask_kind, plan, *bytes);
}

fa_status fa_decode_noalloc(const fa_attn_args* a, void* stream) {
  FwdParams p;
  int mask_kind;
  DecodePlan plan;
  size_t need;
  fa_status st = prepare_decode(a, p, mask_kind, plan, need);
  if (st != FA_OK) return st;
  if (need > (size_t)FA_DECODE_SCRATCH_BYTES)
    return fail(FA_ERR_WORKSPACE, "decode needs %zu bytes of workspace, above the %u bytes of the library's "
                                  "scratch (use fa_decode with a workspace)", need, (unsigned)FA_DECODE_SCRATCH_BYTES);
  void* ws = nullptr;
  st = decode_scratch(&ws);
  if (st != FA_OK) return fail(st, "decode scratch address lookup failed");
  return run_decode(a, p, mask_kind, plan, ws, (hipStream_t)stream);
}

fa_status fa_decode(const fa_attn_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  FwdParams p;
  int mask_kind;
  DecodePlan plan;
  size_t need;
  fa_status st = prepare_decode(a, p, mask_kind, plan, need);
  if (st != FA_OK) return st;
  if (workspace == nullptr) return fail(FA_ERR_WORKSPACE, "decode workspace is NULL");
  if (workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "decode workspace %zu bytes < %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace & 3u) != 0) return fail(FA_ERR_WORKSPACE, "decode workspace not 4-byte aligned");
  return run_decode(a, p, mask_kind, plan, workspace, (hipStream_t)stream);
}

fa_status fa_backward_workspace_size(const fa_attn_args* a, size_t* bytes) {
  if (bytes == nullptr) return fail(FA_ERR_NULL, "bytes is NULL");
  BwdParams P;
  int mask_kind;
  return prepare_backward(a, nullptr, P, mask_kind, *bytes);
}

fa_status fa_backward(const fa_attn_args* a, const fa_grad_args* g, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (g == nullptr) return fail(FA_ERR_NULL, "gradient args are NULL");
  BwdParams P;
  int mask_kind;
  size_t need;
  fa_status st = prepare_backward(a, g, P, mask_kind, need);
  if (st != FA_OK) return st;
  if (workspace == nullptr) return fail(FA_ERR_WORKSPACE, "backward workspace is NULL");
  if (workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "backward workspace %zu bytes < %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace & 15u) != 0) return fail(FA_ERR_WORKSPACE, "backward workspace not 16-byte aligned");
  P.ws_lse2 = (float*)workspace;
  P.ws_delta = P.ws_lse2 + (size_t)a->B * a->Hq * P.sq_pad;
  st = launch_backward_prep(a->D, P, (hipStream_t)stream);
  if (st != FA_OK) return fail(st, "backward prep launch failed");
  st = launch_backward(a->D, mask_kind, a->score.kind, P, (hipStream_t)stream);
  if (st != FA_OK) return fail(st, "backward launch failed");
  return FA_OK;
}

fa_status fa_probe_mfma(int32_t workgroups, int32_t iterations, int32_t random_operands, float* sink, double* flops,
                        void* stream) {
  if (sink == nullptr || flops == nullptr) return fail(FA_ERR_NULL, "sink and flops must be non-NULL");
  if (workgroups < 1 || iterations < 1) return fail(FA_ERR_SHAPE, "workgroups and iterations must be >= 1");
  *flops = probe_mfma_flops(workgroups, iterations);
  const fa_status st = launch_probe_mfma(workgroups, iterations, random_operands != 0, sink, (hipStream_t)stream);
  return st == FA_OK ? FA_OK : fail(st, "MFMA probe launch failed");
}

fa_status fa_probe_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, void* stream) {
  if (src == nullptr || sink == nullptr) return fail(FA_ERR_NULL, "src and sink must be non-NULL");
  if (bytes == 0 || bytes % 16 != 0) return fail(FA_ERR_SHAPE, "bytes must be a positive multiple of 16");
  if (!aligned16(src)) return fail(FA_ERR_UNSUPPORTED, "src must be 16-byte aligned");
  if (sink_words < (size_t)probe_read_workgroups(bytes))
    return fail(FA_ERR_SHAPE, "sink holds %zu words, the probe writes %d", sink_words, probe_read_workgroups(bytes));
  const fa_status st = launch_probe_read(src, bytes, sink, (hipStream_t)stream);
  return st == FA_OK ? FA_OK : fail(st, "read probe launch failed");
}

fa_status fa_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr) return fail(FA_ERR_NULL, "src and dst must be non-NULL");
  if (bytes == 0 || bytes % 16 != 0) return fail(FA_ERR_SHAPE, "bytes must be a positive multiple of 16");
  if (!aligned16(src) || !aligned16(dst)) return fail(FA_ERR_UNSUPPORTED, "src and dst must be 16-byte aligned");
  const fa_status st = launch_probe_copy(src, dst, bytes, (hipStream_t)stream);
  return st == FA_OK ? FA_OK : fail(st, "copy probe launch failed");
}

}  // extern "C"
