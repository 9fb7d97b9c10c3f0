// Internal declarations shared by the host dispatch (fa_api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa.h"

namespace fa {

// Runtime parameters of the mask_mods (see fa_mask_desc).
struct MaskParams {
  int window;
  int prefix_len;
  const int* doc;
  long long doc_stride_b;
  const int* kv_len;
  int doc_vec;  // doc (and every batch row of it) 16-byte aligned: ids can be read 4 at a time
};

// Runtime parameters of the score_mods, with host-folded constants.
// Scores inside the kernels are kept in base-2 units: x2 = mod(s) * log2(e),
// so that the softmax exponentials are single exp2 instructions.
struct ScoreParams {
  float scale;        // 1/sqrt(D) unless given
  float scale_log2;   // scale * log2(e)
  float cap_log2;     // softcap * log2(e)
  float tanh_k;       // 2 * scale / softcap * log2(e): exp2 argument of tanh's identity
  const float* slopes;  // ALiBi slopes [Hq] or nullptr (default geometric slopes)
  int Hq;
  const uint16_t* bias;
  long long bs0, bs1, bs2;  // bias strides for b, h, q (kv stride is 1)
};

struct BlockMaskView {
  const int* kv_num;
  const int* kv_idx;
  const int* full_num;
  const int* full_idx;
  int Bm, Hm, NQ, NK;
  int dense;          // no BlockMask: every kv tile is treated as full
  int separate_full;  // 0: kv_* already holds every non-empty tile
  const int* q_order; // nullptr, or each row's query blocks heaviest first [Bm,Hm,NQ]
};

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  long long qs[4], ks[4], vs[4], os[4];
  int B, Hq, Hkv, Sq, Skv, G;
  BlockMaskView bm;
  MaskParams mask;
  ScoreParams score;
};

struct DecodeParams {
  FwdParams f;          // Sq == 1
  int mask_kind;        // decode evaluates the mask through a runtime switch
  int splits;           // splits per (b, hkv) row = grid.x
  int blocks_per_split; // kv tiles per split
  float* ws_o;          // [B, Hq, splits, D] fp32 (normalised partial outputs)
  float* ws_lse;        // [B, Hq, splits] fp32 base-2 LSE of each split
  const int* page_table;  // nullptr: per-sequence caches; else page of (b, logical block)
  long long pt_stride;    // page-table entries between sequences
  int num_pages;
  const int* q_pos;       // nullptr: query position 0; else position of sequence b's query
  const int* row_order;   // nullptr, or the sequences longest first [B] (grid z -> b)
};

struct BwdParams {
  FwdParams f;            // q, k, v, o (the forward's output), lse (its natural-log LSE), masks, scores
  const uint16_t* dout;   // dO [B, Hq, Sq, D]
  long long dos[4];
  uint16_t* dq;           // outputs, bf16
  uint16_t* dk;
  uint16_t* dv;
  long long dqs[4], dks[4], dvs[4];
  const int* q_num;       // transposed BlockMask view (nullptr for dense)
  const int* q_idx;
  const int* full_q_num;
  const int* full_q_idx;
  const int* kv_order;    // nullptr, or each column's KV blocks heaviest first [Bm,Hm,NK]
  float* ws_lse2;         // [B, Hq, sq_pad] base-2 LSE, +inf for rows without keys
  float* ws_delta;        // [B, Hq, sq_pad] rowsum(dO * O)
  int sq_pad;             // Sq rounded up to whole 128-row tiles
};

struct BuildParams {
  int* kv_num;
  int* kv_idx;
  int* full_num;
  int* full_idx;
  int* q_num;       // transposed view, all four nullptr when not requested
  int* q_idx;
  int* full_q_num;
  int* full_q_idx;
  int* q_order;     // work order of the query blocks, nullptr when not requested
  int* kv_order;    // work order of the KV blocks (from the transposed view), nullptr when not requested
  int* row_order;   // work order of the batch rows (NQ = Hm = 1), nullptr when not requested
  int Bm, Hm, NQ, NK, Sq, Skv;
  int separate_full;
  MaskParams mask;
};

fa_status launch_block_mask(int mask_kind, const BuildParams& p, hipStream_t stream);
fa_status launch_probe_mfma(int workgroups, int iterations, int random_operands, float* sink, hipStream_t stream);
double probe_mfma_flops(int workgroups, int iterations);
fa_status launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);
fa_status launch_forward(int D, int mask_kind, int score_kind, const FwdParams& p, hipStream_t stream);
// One translation unit per mask kind (compiled in parallel).
fa_status launch_forward_none(int D, int score_kind, const FwdParams& p, hipStream_t stream);
fa_status launch_forward_causal(int D, int score_kind, const FwdParams& p, hipStream_t stream);
fa_status launch_forward_window(int D, int score_kind, const FwdParams& p, hipStream_t stream);
fa_status launch_forward_sliding_causal(int D, int score_kind, const FwdParams& p, hipStream_t stream);
fa_status launch_forward_document(int D, int score_kind, const FwdParams& p, hipStream_t stream);
fa_status launch_forward_document_causal(int D, int score_kind, const FwdParams& p, hipStream_t stream);
fa_status launch_forward_prefix_lm(int D, int score_kind, const FwdParams& p, hipStream_t stream);
fa_status launch_forward_kv_len(int D, int score_kind, const FwdParams& p, hipStream_t stream);
fa_status launch_decode(int D, int G, int score_kind, const DecodeParams& p, hipStream_t stream);
// Device address of the current device's decode scratch (FA_DECODE_SCRATCH_BYTES).
fa_status decode_scratch(void** ptr);
fa_status launch_backward(int D, int mask_kind, int score_kind, const BwdParams& p, hipStream_t stream);
fa_status launch_backward_prep(int D, const BwdParams& p, hipStream_t stream);
fa_status launch_backward_none(int D, int score_kind, const BwdParams& p, hipStream_t stream);
fa_status launch_backward_causal(int D, int score_kind, const BwdParams& p, hipStream_t stream);
fa_status launch_backward_window(int D, int score_kind, const BwdParams& p, hipStream_t stream);
fa_status launch_backward_sliding_causal(int D, int score_kind, const BwdParams& p, hipStream_t stream);
fa_status launch_backward_document(int D, int score_kind, const BwdParams& p, hipStream_t stream);
fa_status launch_backward_document_causal(int D, int score_kind, const BwdParams& p, hipStream_t stream);
fa_status launch_backward_prefix_lm(int D, int score_kind, const BwdParams& p, hipStream_t stream);
fa_status launch_backward_kv_len(int D, int score_kind, const BwdParams& p, hipStream_t stream);

}  // namespace fa
