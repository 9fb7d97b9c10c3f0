/*
 * fa.h — C ABI of the MI355X (gfx950) block-sparse FlexAttention library (libfa.so).
 *
 * What the library computes is fixed by the FlexAttention pages:
 *   O = softmax(mod(Q K^T / sqrt(d))) V
 * (paper review "Flex Attention: A Programming Model for Generating Optimized
 * Attention Kernels", §2.1), where the mod is a score_mod applied to the
 * scaled score and a mask_mod that removes positions (attention-gym
 * "Concepts" page, sections "mask_mod", "score_mod", "When to use which?").
 * Masked positions count as -inf; the score_mod is only applied where the
 * mask keeps the position.  Work is skipped per 128x128 tile through a
 * BlockMask (Concepts, "BlockMask Internals" and "Key attributes"; paper
 * review §4.1-4.3).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates and frees no memory; decode's workspace is caller-provided.
 *  - bfloat16 tensors are passed as uint16_t bit patterns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls are asynchronous and ordered on that stream.
 *  - Arguments are validated on the host before any HIP call; a failed
 *    check returns a status and launches nothing.  fa_last_error() then
 *    returns a message naming the failed check (per calling thread).
 *  - Launch failures return FA_ERR_HIP.  Faults inside a kernel surface at
 *    the caller's next synchronisation, as for any HIP kernel.
 *  - The only global state is the last-error message (per thread) and, for
 *    fa_decode_noalloc, a per-device pointer set once under a lock: calls may be
 *    made from several threads at once (fa_decode_noalloc calls on one GPU
 *    share its scratch and must not overlap).
 *  - Changing any runtime parameter (window, prefix length, document ids,
 *    lengths, slopes, cap, bias tensor, BlockMask contents) never needs a
 *    rebuild: only the mask/score *kind* selects compiled code (Concepts,
 *    "Changing BlockMask doesn't require recompilation"; the dynamic-bias
 *    feature request, attention-gym issue 123).
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 6
#define FA_BLOCK 128 /* the only supported BLOCK_SIZE (Concepts, "BlockMask Internals": default 128x128) */

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* sizes, strides or BlockMask dims are inconsistent */
  FA_ERR_UNSUPPORTED = 3, /* valid request outside what is compiled (D, block size, kind, alignment) */
  FA_ERR_WORKSPACE = 4,   /* decode workspace missing or too small */
  FA_ERR_HIP = 5          /* a HIP launch failed */
} fa_status;

/* mask_mod kinds (Concepts "mask_mod" / "Composing masks"; paper review §2.2, §4.4;
 * talk summary "FlexAttention: A Flexible and Performant Approach to Transformer
 * Attention", variant list).  q and kv are absolute token indices; b is the batch row. */
typedef enum {
  FA_MASK_NONE = 0,            /* every position attends */
  FA_MASK_CAUSAL = 1,          /* q >= kv */
  FA_MASK_SLIDING_WINDOW = 2,  /* q - kv <= window (the window term alone) */
  FA_MASK_SLIDING_CAUSAL = 3,  /* AND(causal, window): 0 <= q - kv <= window */
  FA_MASK_DOCUMENT = 4,        /* doc[b][q] == doc[b][kv] */
  FA_MASK_DOCUMENT_CAUSAL = 5, /* AND(document, causal) */
  FA_MASK_PREFIX_LM = 6,       /* OR(kv < prefix_len, causal) */
  FA_MASK_KV_LEN = 7,          /* kv < kv_len[b] (valid prefix of a KV cache) */
  FA_MASK_KIND_COUNT = 8
} fa_mask_kind;

typedef struct {
  int32_t kind;            /* fa_mask_kind */
  int32_t window;          /* SLIDING_*: inclusive window, >= 0 */
  int32_t prefix_len;      /* PREFIX_LM: keys [0, prefix_len) are visible to every query, >= 0 */
  int32_t reserved0;
  const int32_t* doc_ids;  /* DOCUMENT*: device int32; token t of batch row b has id
                              doc_ids[b * doc_stride_b + t]; shared by queries and keys, so
                              these kinds need Sq == Skv */
  int64_t doc_stride_b;    /* elements; 0 = one layout for every batch row */
  const int32_t* kv_len;   /* KV_LEN: device int32 [B] valid lengths */
} fa_mask_desc;

/* score_mod kinds (Concepts "score_mod"; paper review §2.1 table; talk summary;
 * dynamic-bias feature request).  `s` is the scaled score Q.K * scale. */
typedef enum {
  FA_SCORE_NONE = 0,    /* s */
  FA_SCORE_ALIBI = 1,   /* s + slope[h] * (kv - q) */
  FA_SCORE_SOFTCAP = 2, /* softcap * tanh(s / softcap) */
  FA_SCORE_REL_POS = 3, /* s + (q - kv) */
  FA_SCORE_BIAS = 4,    /* s + bias[b, h, q, kv] (bf16 tensor, read per element) */
  FA_SCORE_KIND_COUNT = 5
} fa_score_kind;

typedef struct {
  int32_t kind;                /* fa_score_kind */
  float softcap;               /* SOFTCAP: cap > 0 */
  const float* alibi_slopes;   /* ALIBI: device fp32 [Hq], or NULL for slope[h] = 2^(-8(h+1)/Hq) */
  const uint16_t* bias;        /* BIAS: device bf16; element (b,h,q,kv) at
                                  b*s[0] + h*s[1] + q*s[2] + kv*s[3] */
  int64_t bias_stride[4];      /* elements, >= 0; 0 broadcasts a dim; s[3] must be 1 */
} fa_score_desc;

/* BlockMask (Concepts "Key attributes"; paper review §4.1).  All four index
 * tensors are caller-allocated device int32, written by fa_build_block_mask:
 *   kv_num_blocks [Bm,Hm,NQ], kv_indices [Bm,Hm,NQ,NK],
 *   full_kv_num_blocks [Bm,Hm,NQ], full_kv_indices [Bm,Hm,NQ,NK],
 * contiguous, NQ = ceil(Sq/128), NK = ceil(Skv/128).  Lists are ascending and
 * padded with 0.  With separate_full = 1 (canonical) kv_* lists the partial
 * tiles and full_* the full tiles (disjoint); with separate_full = 0, kv_*
 * lists every non-empty tile and full_* the full ones among them, and the
 * forward then evaluates the mask on every listed tile.  A tile is full when
 * every in-range position attends, empty when none does (Concepts,
 * "BlockMask Internals"; paper review §4.2).  Bm is 1 or B and Hm is 1 or Hq;
 * a dim of 1 is shared by every batch row / head.  The mask descriptor is
 * carried with the tensors and is evaluated on partial tiles. */
typedef struct {
  int32_t* kv_num_blocks;
  int32_t* kv_indices;
  int32_t* full_kv_num_blocks;
  int32_t* full_kv_indices;
  int32_t Bm, Hm, NQ, NK;
  int32_t block_q, block_kv; /* must both be FA_BLOCK */
  int32_t separate_full;     /* 1 = disjoint lists (canonical), 0 = superset */
  int32_t Sq, Skv;           /* set by fa_build_block_mask; fa_forward checks them */
  fa_mask_desc mask;
  /* Transposed view (Concepts "Key attributes": q_num_blocks / q_indices, used by
   * the backward): for each KV block, the query blocks of the lists above, in
   * ascending order and padded with 0.  q_* is the view of kv_* (partial tiles,
   * or every non-empty one when separate_full = 0) and full_q_* the view of
   * full_kv_*.  Optional: either all four are NULL, or all four are device
   * buffers that fa_build_block_mask fills.
   * q_num_blocks, full_q_num_blocks: [Bm,Hm,NK]; q_indices, full_q_indices: [Bm,Hm,NK,NQ]. */
  int32_t* q_num_blocks;
  int32_t* q_indices;
  int32_t* full_q_num_blocks;
  int32_t* full_q_indices;
  /* Work order of the query blocks (optional; NULL = none): [Bm,Hm,NQ] device
   * int32 that fa_build_block_mask fills with each row's query blocks sorted
   * by their work, heaviest first: weight 3 per tile that runs the mask (the
   * kv_* tiles) plus 2 per tile of full_kv_* (with separate_full = 1), ties
   * broken by the larger query block; NQ <= 16384.  When it is present and
   * B*Hq is a multiple of 8, the forward (and the backward's dQ pass, which
   * has the same units) starts its (b, h, query tile) units
   * in that order, the heaviest tiles of every head of an XCD first (paper
   * review §4.3: a query tile's work is the length of its lists).  Without it
   * the forward starts the last query tiles first, which is longest-first for
   * masks whose work grows with the query index (causal, windows, prefix);
   * document masks, whose work follows the position inside a document, gain
   * from the order (about 10% at 16K tokens with ~1.6K-token documents), the
   * others do not (one more dependent load per workgroup).  The order changes
   * no result, only which workgroups run together. */
  int32_t* q_order;
  /* Work order of the KV blocks (optional; NULL = none): [Bm,Hm,NK] device int32
   * that fa_build_block_mask fills from the transposed view (which must then be
   * requested too) with each column's KV blocks sorted by their work, heaviest
   * first: 3 per entry of q_* and 2 per entry of full_q_* (with separate_full =
   * 1), ties broken by the smaller KV block; NK <= 16384.  The backward's dK/dV
   * pass, whose units are (b, hkv, KV block), starts them in that order when
   * Hm = 1 and B*Hkv is a multiple of 8, the heaviest blocks of every head of
   * an XCD first.  Like q_order it changes no result, and it pays off for
   * document masks (the natural order, first KV blocks first, is already
   * longest-first for causal masks). */
  int32_t* kv_order;
  /* Work order of the batch rows (optional; NULL = none), for BlockMasks of one
   * query block and one head row (NQ = 1, Hm = 1: the decode masks): [Bm]
   * device int32 that fa_build_block_mask fills with the rows sorted by their
   * listed tiles, heaviest first (3 per kv_* tile, 2 per full_kv_* tile with
   * separate_full = 1), ties to the smaller row; Bm <= 16384.  fa_decode with
   * Bm = B starts the longest sequences' workgroups first, so that the short
   * ones, not the long ones, run at the end of the launch (the talk summary's
   * Flex Decoding: the key axis of each sequence split into chunks).  Changes
   * no result.  Errors: FA_ERR_SHAPE for NQ > 1 or Hm > 1. */
  int32_t* row_order;
} fa_block_mask;

/* Attention call arguments.  Q/O are [B,Hq,Sq,D], K/V are [B,Hkv,Skv,D]
 * (for decode: the KV cache, Skv = its capacity).  Strides are in elements
 * for dims (b, h, s, d); the d stride must be 1, other strides multiples of 8,
 * the K/V row (s) strides below 2^25, base pointers 16-byte aligned.  GQA: query head hq reads KV head
 * hq / (Hq / Hkv) (paper review §3.3 lists GQA support). */
typedef struct {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;                 /* optional fp32 [B,Hq,Sq] contiguous, natural-log LSE; -inf for empty rows */
  int64_t q_stride[4], k_stride[4], v_stride[4], o_stride[4];
  int32_t B, Hq, Hkv, Sq, Skv, D; /* D in {64, 128} */
  float scale;                /* 0 => 1/sqrt(D); otherwise >= 1e-20 */
  const fa_block_mask* block_mask; /* NULL => dense attention without a mask */
  fa_score_desc score;
  int32_t num_splits;         /* decode: max KV splits per sequence, 0 = auto; ignored by fa_forward */
  /* Paged KV cache, fa_decode only (paper review §4.5 "PagedAttention support"
   * and §5.4; talk summary, "Page Attention"): a compact pool of fixed-size pages
   * reached through a page table.  NULL => k and v hold each sequence's cache
   * [B,Hkv,Skv,D] as above.  Otherwise k and v point at page pools
   * [num_pages, Hkv, FA_BLOCK, D] whose k_stride / v_stride are the (page, head,
   * row, d) strides, and logical 128-key block j of sequence b is stored in page
   * page_table[b * page_table_stride + j].  Skv is then the logical capacity
   * (the BlockMask's KV length); the BlockMask, mask_mods and score_mods all see
   * logical positions, and only blocks the BlockMask lists are looked up.
   * Sequences may share pages.  Page ids outside [0, num_pages) are clamped into
   * range (no fault, wrong values): the caller owns the table's validity. */
  const int32_t* page_table;  /* device int32, >= B rows of page_table_stride entries */
  int64_t page_table_stride;  /* entries between sequences, >= ceil(Skv / FA_BLOCK) */
  int32_t num_pages;          /* pages in each pool */
  /* fa_decode only: the position of each sequence's query token, the q index
   * the score_mods see (talk summary, "Flex Decoding": the score_mod still
   * applies; Concepts "score_mod": ALiBi reads q_idx).  Device int32 [B], or
   * NULL for position 0 in every sequence.  For a cache holding len[b] tokens
   * and the newest token as query, pass len[b] - 1.  fa_forward requires NULL. */
  const int32_t* q_pos;
} fa_attn_args;

/* Backward pass: the gradient buffers.  Strides are in elements for (b, h, s, d),
 * with the same rules as the forward's tensors (d stride 1, others multiples of 8,
 * 16-byte aligned bases). */
typedef struct {
  const uint16_t* dout;       /* dO, bf16 [B,Hq,Sq,D]: the gradient of the loss at O */
  int64_t dout_stride[4];
  uint16_t* dq;               /* written: bf16 [B,Hq,Sq,D] */
  uint16_t* dk;               /* written: bf16 [B,Hkv,Skv,D] (summed over the GQA group) */
  uint16_t* dv;               /* written: bf16 [B,Hkv,Skv,D] */
  int64_t dq_stride[4], dk_stride[4], dv_stride[4];
} fa_grad_args;

/* Version of this ABI (FA_ABI_VERSION). */
int32_t fa_abi_version(void);

/* Human-readable name of a status code.  Never NULL. */
const char* fa_status_string(fa_status s);

/* Message describing the last non-OK status returned on the calling thread. */
const char* fa_last_error(void);

/* Host only.  NQ = ceil(Sq/block_q), NK = ceil(Skv/block_kv).
 * Errors: NULL outputs, sizes <= 0, a block size other than FA_BLOCK. */
fa_status fa_block_mask_dims(int32_t Sq, int32_t Skv, int32_t block_q, int32_t block_kv,
                             int32_t* NQ, int32_t* NK);

/* Build a BlockMask on the device (Concepts "BlockMask Internals": every
 * 128x128 tile is classified full / partial / empty from the mask_mod, then
 * compacted into the four index tensors).  `bm` is host memory with the four
 * device pointers, Bm, Hm, NQ, NK, block sizes, separate_full and the mask
 * descriptor filled in; on success bm->Sq and bm->Skv are set.  Every entry
 * of the four tensors is written (padding included).  The mask is evaluated
 * for b' < Bm and h' < Hm.
 * The optional work orders (q_order, kv_order, row_order) are written when
 * their pointers are set.
 * Errors: FA_ERR_NULL (tensor pointers, doc_ids/kv_len needed by the kind,
 * kv_order without the transposed view), FA_ERR_SHAPE (NQ/NK not matching
 * Sq/Skv, Bm or Hm < 1, Sq != Skv for a document kind, negative
 * window/prefix, row_order with NQ > 1 or Hm > 1), FA_ERR_UNSUPPORTED (block
 * size, unknown kind, an order longer than 16384), FA_ERR_HIP. */
fa_status fa_build_block_mask(fa_block_mask* bm, int32_t Sq, int32_t Skv, void* stream);

/* Fused block-sparse attention forward (paper review §2.1, §3.3, §4.2-4.3):
 * for each (b, hq, 128-row query tile) one workgroup walks the tile's
 * partial list (mask evaluated per element) and then its full list (no mask),
 * with online softmax, writing O (bf16) and optionally LSE.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (sizes, Hq % Hkv, strides, BlockMask dims,
 * Bm/Hm not in {1,B}/{1,Hq}, a batch-dependent mask with Bm = 1 < B, a BlockMask
 * built for other lengths), FA_ERR_UNSUPPORTED (D, alignment, kinds, bias
 * stride[3] != 1, a K/V row stride of 2^25 or more, a page table), FA_ERR_HIP. */
fa_status fa_forward(const fa_attn_args* a, void* stream);

/* Host only.  Bytes of decode workspace fa_decode needs for these arguments
 * (fp32 partial outputs and LSEs of every split).  Same validation as fa_decode. */
fa_status fa_decode_workspace_size(const fa_attn_args* a, size_t* bytes);

/* Split-KV decode (talk summary, "Flex Decoding": split along the key axis
 * for parallelism, then a final reduction; score_mod still applies).  Sq must
 * be 1; the query of sequence b sits at q index q_pos[b] (0 when q_pos is
 * NULL), which is the q the score_mods see.  The BlockMask is the one-row
 * BlockMask of the KV axis (built with Sq = 1), so its mask must not depend on
 * the query position: only FA_MASK_NONE and FA_MASK_KV_LEN are accepted (a
 * causal cache of len[b] tokens is kv < len[b]).  Each sequence's block list (its
 * BlockMask row) is dealt round-robin into chunks (chunk s holds entries s,
 * s + splits, s + 2 splits, ...); one workgroup per (chunk, KV head, batch
 * row) computes all Hq/Hkv query heads of that KV head against the chunk, and
 * a merge kernel combines the chunks through their log-sum-exp.  The result
 * does not depend on the split count beyond fp32 rounding.  The GQA group
 * size Hq/Hkv must be 1, 2, 4 or 8, and 1 when Hm > 1.  num_splits (0 = auto)
 * sets how many chunks a sequence is cut into; a chunk holds 1 to 8 tiles, so
 * the split count used is ceil(NK / clamp(ceil(NK / num_splits), 1, 8)).
 * With a page table (see fa_attn_args) the K/V rows of each listed block are
 * read from its page; the arithmetic is otherwise unchanged.
 * Errors: as fa_forward, plus FA_ERR_SHAPE for Sq != 1, num_pages <= 0 or
 * page_table_stride < ceil(Skv / FA_BLOCK), FA_ERR_UNSUPPORTED for a mask kind
 * other than NONE / KV_LEN, and FA_ERR_WORKSPACE. */
fa_status fa_decode(const fa_attn_args* a, void* workspace, size_t workspace_bytes, void* stream);

/* Scratch size of fa_decode_noalloc: decode calls whose workspace
 * (fa_decode_workspace_size) exceeds this are rejected by it. */
#define FA_DECODE_SCRATCH_BYTES (32u << 20)

/* fa_decode without a workspace argument, for callers that cannot allocate
 * device memory around the call (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, kernels and result
 * as fa_decode; the split partial outputs and LSEs go to a device array
 * inside the library (FA_DECODE_SCRATCH_BYTES per GPU, held by every GPU the
 * library runs on until the process ends; its address is looked up on the first
 * call on each device).  Nothing is allocated or freed by the call.  Every call
 * on one GPU shares that array, so calls that overlap in time on one GPU (on
 * different streams, or from several threads) race and must be ordered by the
 * caller; the array needs no clearing between calls (every split writes its
 * whole row before the merge reads it).
 * Errors: as fa_decode, with FA_ERR_WORKSPACE when the workspace fa_decode
 * would need exceeds FA_DECODE_SCRATCH_BYTES (checked before any HIP call). */
fa_status fa_decode_noalloc(const fa_attn_args* a, void* stream);

/* Host only.  Bytes of workspace fa_backward needs: two fp32 values (base-2
 * LSE and Delta = rowsum(dO * O)) per query row, rows padded to whole tiles.
 * Same validation as fa_backward. */
fa_status fa_backward_workspace_size(const fa_attn_args* a, size_t* bytes);

/* Backward pass (dQ, dK, dV) of fa_forward for the same arguments: the
 * gradient of the forward definition, O = softmax(mod(Q K^T * scale)) V with
 * the mask.  The pages name a backward pass that walks the transposed
 * BlockMask view (Concepts "Key attributes": q_num_blocks / q_indices, "used in
 * backward") without giving its formulas; with P recomputed from the forward's
 * LSE, Delta = rowsum(dO * O), dS = P * (dP - Delta) * mod'(S) and dP = dO V^T:
 * dV = P^T dO, dQ = scale * dS K, dK = scale * dS^T Q.  For the bias score the
 * bias is an input, not a learned parameter: no bias gradient is produced.
 * a->o must hold fa_forward's output and a->lse its LSE (both required).  A
 * BlockMask must carry its transposed view (all four q_* buffers, built by
 * fa_build_block_mask); NULL means dense.  No page table.
 * Kernels: a prep kernel (LSE, Delta), a query-parallel dQ kernel walking the
 * row lists and a key-parallel dK/dV kernel walking the column lists of every
 * query head of the GQA group; no atomics.
 * Errors: as fa_forward, plus FA_ERR_NULL (o, lse, dO, dQ, dK, dV or the
 * transposed view missing) and FA_ERR_WORKSPACE. */
fa_status fa_backward(const fa_attn_args* a, const fa_grad_args* g, void* workspace, size_t workspace_bytes,
                      void* stream);

/* ---- Measurement probes (not part of the attention path) ----------------
 * Kernels whose rate is what the chip reaches in practice, so that a kernel's
 * throughput can be given as a fraction of a measured peak beside the
 * published one (bf16 matrix peak, HBM bandwidth). */

/* Dense bf16 MFMA loop: `workgroups` workgroups of 256 threads; every wave runs
 * `iterations` rounds (rounded up to even) of 8 independent
 * v_mfma_f32_32x32x16_bf16 chains on register operands (32768 flops per
 * instruction).  random_operands = 0: constant operands (the datapath hardly
 * switches); 1: random bf16 signs and mantissas, two operand sets alternating
 * between rounds (switching as on real data, which costs power).  *flops
 * receives the flop count of the launch; `sink` (device fp32, workgroups * 256
 * entries) receives one value per lane so the work is not optimised away.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (workgroups or iterations < 1), FA_ERR_HIP. */
fa_status fa_probe_mfma(int32_t workgroups, int32_t iterations, int32_t random_operands, float* sink, double* flops,
                        void* stream);

/* Read-only stream over `bytes` bytes at src (a device pointer, 16-byte
 * aligned, bytes a multiple of 16): 16-byte loads, each byte read once, folded
 * into one 32-bit word per workgroup written to `sink` (device, sink_words
 * entries; the probe uses min(8192, ceil(bytes / 16384)) workgroups).
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (bytes, or a sink too small), FA_ERR_UNSUPPORTED
 * (alignment), FA_ERR_HIP. */
fa_status fa_probe_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, void* stream);

/* Streaming copy of `bytes` bytes from src to dst (device pointers, 16-byte
 * aligned, bytes a multiple of 16): 16-byte loads and stores, each byte read
 * and written once.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (bytes 0 or not a multiple of 16),
 * FA_ERR_UNSUPPORTED (alignment), FA_ERR_HIP. */
fa_status fa_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
