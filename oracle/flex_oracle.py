"""Dense fp64 CPU oracle for block-sparse FlexAttention — TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It is plain, slow and written to be checked by eye
against the pages; it shares no code with the HIP library and imports
nothing from it.  Inputs are bfloat16 bit patterns (uint16), widened here
exactly to float64, so the oracle sees the same values as the GPU.

Sources (cited by title and section):
  * "Concepts" page of attention-gym (meta-pytorch.org/attention-gym/concepts):
    sections "mask_mod", "score_mod", "When to use which?", "Composing masks",
    "BlockMask Internals", "Key attributes", "Inspecting a BlockMask".
  * Paper review "Flex Attention: A Programming Model for Generating
    Optimized Attention Kernels" (xllm-io): §2.1 (formula), §2.2 (mod
    signatures), §3.3 (online softmax, GQA), §4.1 (BlockMask), §4.2
    (full/partial blocks), §4.4 (logical fusion), §6.1 (variant list).
  * Talk summary "FlexAttention: A Flexible and Performant Approach to
    Transformer Attention" (rocketrecap): variant list at 1:33, score/mask
    mode mechanism, Flex Decoding (split along K plus a final reduction).
  * Feature request "Support for Dynamic Bias Tensor in FlexAttention
    Without Recompilation" (attention-gym issue 123): a [B,H,S,S] bias added
    to the scores.

What is computed (paper review §2.1, Concepts "When to use which?"):
    O = softmax(mod(Q K^T / sqrt(d))) V
with the 1/sqrt(d) scale applied before the mod, the score_mod applied only
at positions the mask_mod keeps, and masked positions set to -inf.

Readings taken where the pages are silent (each is listed in the design doc):
  * a row whose every position is masked gives O = 0 and LSE = -inf;
  * GQA: query head hq reads KV head hq // (Hq // Hkv);
  * the `h` handed to the mods is the query-head index;
  * BlockMask lists are ascending, padded with 0, int32, last dim NK;
    canonical encoding keeps partial and full blocks in disjoint lists;
  * ragged edges: a tile is classified over its in-range positions only;
  * ALiBi slope default 2^(-8(h+1)/H); softcap is cap*tanh(s/cap) with the
    exact tanh; the relative-position bias is the float (q - kv).

Parity pins for every function here live in tests/test_oracle_pins.py.
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# Input decoding
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64, exactly (bf16 is the top half of fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _values(x) -> np.ndarray:
    """Tensor values as float64: bfloat16 bit patterns are decoded, float64
    arrays (used by the finite-difference pins) are taken as they are."""
    x = np.asarray(x)
    return x if x.dtype == np.float64 else bf16_to_f64(x)


# ---------------------------------------------------------------------------
# mask_mods: mask(b, h, q_idx, kv_idx) -> bool, True = attend.
# Signature from Concepts "mask_mod" and paper review §2.2; indices are
# numpy integer arrays that broadcast against each other.
# ---------------------------------------------------------------------------

def no_mask():
    return lambda b, h, q, kv: np.ones(np.broadcast(q, kv).shape, dtype=bool)


def causal():
    """Concepts "mask_mod": a query attends to keys at or before it."""
    return lambda b, h, q, kv: q >= kv


def sliding_window(window: int):
    """The window term of Concepts "Composing masks": q - kv <= window (inclusive).

    On its own it only bounds how far back a key may lie, so every later key
    (kv > q) is kept; the page ANDs it with causal to get the sliding band."""
    return lambda b, h, q, kv: (q - kv) <= window


def and_masks(*masks):
    """Concepts "Composing masks" / paper review §4.4: logical AND of mask_mods."""
    def m(b, h, q, kv):
        out = masks[0](b, h, q, kv)
        for x in masks[1:]:
            out = out & x(b, h, q, kv)
        return out
    return m


def or_masks(*masks):
    """Paper review §4.4: logical OR of mask_mods."""
    def m(b, h, q, kv):
        out = masks[0](b, h, q, kv)
        for x in masks[1:]:
            out = out | x(b, h, q, kv)
        return out
    return m


def sliding_causal(window: int):
    """Concepts "Composing masks": causal AND sliding window."""
    return and_masks(causal(), sliding_window(window))


def document(doc_ids):
    """Talk summary 1:33 / paper review §5.3: attend only within the same document.

    doc_ids is int [B, S] (one id per token, shared by queries and keys).
    """
    doc = np.asarray(doc_ids)
    return lambda b, h, q, kv: doc[b, q] == doc[b, kv]


def document_causal(doc_ids):
    return and_masks(document(doc_ids), causal())


def prefix(prefix_len: int):
    """The prefix term of paper review §4.4: keys inside the prefix are visible to all."""
    return lambda b, h, q, kv: np.broadcast_to(kv < prefix_len, np.broadcast(q, kv).shape)


def prefix_lm(prefix_len: int):
    """Paper review §4.4: PrefixLM = prefix OR causal."""
    return or_masks(prefix(prefix_len), causal())


def kv_length(lengths):
    """Only the first lengths[b] keys of batch row b are valid."""
    ln = np.asarray(lengths)
    return lambda b, h, q, kv: np.broadcast_to(kv < ln[b], np.broadcast(q, kv).shape)


# ---------------------------------------------------------------------------
# score_mods: score_mod(score, b, h, q_idx, kv_idx) -> score (float64).
# Signature from Concepts "score_mod" and paper review §2.2.
# ---------------------------------------------------------------------------

def default_alibi_slopes(H: int) -> np.ndarray:
    """Geometric ALiBi slopes 2^(-8(h+1)/H), h = 0..H-1."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float64)


def _with_grad(mod, grad):
    """Attach d mod / d s (used by the backward; the forward never calls it)."""
    mod.grad = grad
    return mod


def _unit_grad(s, b, h, q, kv):
    """Derivative of an additive score_mod (s + something that does not depend on s)."""
    return np.ones_like(np.asarray(s, dtype=np.float64))


def alibi(slopes):
    """Concepts "score_mod": score + slope[h] * (kv - q)."""
    sl = np.asarray(slopes, dtype=np.float64)
    return _with_grad(lambda s, b, h, q, kv: s + sl[h] * (kv - q), _unit_grad)


def softcap(cap: float):
    """Paper review §2.1 table (Softcapping), Concepts notebook list: cap * tanh(s / cap).
    Its derivative is 1 - tanh(s / cap)^2."""
    return _with_grad(lambda s, b, h, q, kv: cap * np.tanh(s / cap),
                      lambda s, b, h, q, kv: 1.0 - np.tanh(s / cap) ** 2)


def rel_pos():
    """Talk summary (score mode) / Concepts "Debugging score_mods": score + (q - kv)."""
    return _with_grad(lambda s, b, h, q, kv: s + (q - kv), _unit_grad)


def bias(table):
    """Dynamic-bias feature request: score + bias[b, h, q, kv].

    `table[b, h, q, kv]` must support numpy advanced indexing and return
    bfloat16 bit patterns (a uint16 array, possibly with size-1 broadcast
    dims, or any object with that __getitem__).
    """
    return _with_grad(lambda s, b, h, q, kv: s + bf16_to_f64(table[b, h, q, kv]), _unit_grad)


# ---------------------------------------------------------------------------
# Attention forward (definition, dense, fp64)
# ---------------------------------------------------------------------------

def attention_rows(q, k, v, b: int, hq: int, rows, mask_mod=None, score_mod=None,
                   scale=None, check_rows_sum=True):
    """O and LSE for query rows `rows` of (b, hq).

    q: [B,Hq,Sq,D], k/v: [B,Hkv,Skv,D] bfloat16 bits.  Returns
    (O [len(rows), D] float64, LSE [len(rows)] float64, natural log).
    Steps follow the formula of paper review §2.1:
      1. S = (Q K^T) * scale, scale = 1/sqrt(D) unless given;
      2. M = mask_mod(b, hq, q_idx, kv_idx);
      3. S' = score_mod(S) where M holds, -inf elsewhere (Concepts, "When to use which?");
      4. softmax over kv of S', times V.
    """
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    group = Hq // Hkv
    hkv = hq // group
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rows = np.asarray(rows, dtype=np.int64)

    Q = _values(q[b, hq, rows])                     # [R, D]
    K = _values(k[b, hkv])                          # [Skv, D]
    V = _values(v[b, hkv])                          # [Skv, D]

    S = (Q @ K.T) * scale                           # step 1
    qi = rows[:, None]
    ki = np.arange(Skv, dtype=np.int64)[None, :]
    if mask_mod is None:
        M = np.ones(S.shape, dtype=bool)
    else:
        M = np.broadcast_to(np.asarray(mask_mod(b, hq, qi, ki), dtype=bool), S.shape)

    Sp = np.full(S.shape, NEG_INF)                  # step 3: -inf where masked
    if score_mod is None:
        Sp[M] = S[M]
    else:
        qb, kb = np.broadcast_arrays(qi, ki)
        Sp[M] = score_mod(S[M], b, hq, qb[M], kb[M])

    m = Sp.max(axis=1)                              # step 4
    O = np.zeros((rows.size, D))
    lse = np.full(rows.size, NEG_INF)
    live = m > NEG_INF
    if live.any():
        P = np.exp(Sp[live] - m[live, None])
        l = P.sum(axis=1)
        if check_rows_sum:
            assert np.allclose((P / l[:, None]).sum(axis=1), 1.0, rtol=0, atol=1e-12)
        O[live] = (P @ V) / l[:, None]
        lse[live] = m[live] + np.log(l)
    return O, lse


def attention(q, k, v, mask_mod=None, score_mod=None, scale=None, chunk=1024):
    """Full dense forward: O [B,Hq,Sq,D] float64 and LSE [B,Hq,Sq]."""
    B, Hq, Sq, D = q.shape
    O = np.zeros((B, Hq, Sq, D))
    L = np.full((B, Hq, Sq), NEG_INF)
    for b in range(B):
        for hq in range(Hq):
            for r0 in range(0, Sq, chunk):
                rows = np.arange(r0, min(Sq, r0 + chunk))
                O[b, hq, rows], L[b, hq, rows] = attention_rows(
                    q, k, v, b, hq, rows, mask_mod, score_mod, scale)
    return O, L


def decode(q, k_cache, v_cache, lengths, score_mod=None, scale=None, extra_mask=None, positions=None):
    """One query token per sequence against a KV cache (talk summary, Flex Decoding).

    q: [B,Hq,1,D]; caches: [B,Hkv,KV,D]; lengths: int [B]; positions: int [B]
    or None.  The query token of sequence b sits at position positions[b] (0
    when not given): that is the q_idx its mask_mod and score_mod see (the talk
    keeps the score_mod in decoding; Concepts "score_mod": ALiBi reads q_idx).
    The only mask is kv < lengths[b] (AND extra_mask if given).  The split-K +
    final reduction of the talk is an execution strategy that reaches this same
    value, so the oracle computes it directly.
    """
    pos = np.zeros(q.shape[0], dtype=np.int64) if positions is None else np.asarray(positions, dtype=np.int64)
    mask = kv_length(lengths)
    if extra_mask is not None:
        mask = and_masks(mask, extra_mask)

    def mask_at(b, h, qi, kv):       # row 0 of the one-token query is position pos[b]
        return mask(b, h, qi + pos[b], kv)

    mod_at = None
    if score_mod is not None:
        def mod_at(s, b, h, qi, kv):
            return score_mod(s, b, h, qi + pos[b], kv)
    return attention(q, k_cache, v_cache, mask_mod=mask_at, score_mod=mod_at, scale=scale)


# ---------------------------------------------------------------------------
# Attention backward (gradients of the definition above, dense, fp64)
# ---------------------------------------------------------------------------

def attention_backward(q, k, v, dout, mask_mod=None, score_mod=None, scale=None):
    """dQ, dK, dV of the forward definition for an upstream gradient dO.

    The pages name a backward pass and its transposed BlockMask view (Concepts
    "Key attributes": q_num_blocks / q_indices, "used in backward") but print
    no formulas, so this is the chain rule taken through the forward's steps
    one by one, for each (b, hq) with its KV head hkv:
      forward:  S = Q K^T * scale;  S' = mod(S) where kept, -inf elsewhere;
                P = softmax_kv(S');  O = P V
      backward: dV[hkv] += P^T dO
                dP = dO V^T
                dS' = P * (dP - rowsum(P * dP))        (softmax Jacobian)
                dS = dS' * mod'(S) where kept, 0 elsewhere
                dQ = scale * dS K;  dK[hkv] += scale * dS^T Q
    A row with every position masked has P = 0 and contributes nothing.
    Inputs are bfloat16 bits or float64 arrays; returns float64 arrays shaped
    like q, k, v.
    """
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dQ = np.zeros((B, Hq, Sq, D))
    dK = np.zeros((B, Hkv, Skv, D))
    dV = np.zeros((B, Hkv, Skv, D))
    qi = np.arange(Sq, dtype=np.int64)[:, None]
    ki = np.arange(Skv, dtype=np.int64)[None, :]
    for b in range(B):
        for hq in range(Hq):
            hkv = hq // (Hq // Hkv)
            Q, K, V = _values(q[b, hq]), _values(k[b, hkv]), _values(v[b, hkv])
            dO = _values(dout[b, hq])
            S = scale * (Q @ K.T)
            if mask_mod is None:
                M = np.ones(S.shape, dtype=bool)
            else:
                M = np.broadcast_to(np.asarray(mask_mod(b, hq, qi, ki), dtype=bool), S.shape)
            qb, kb = np.broadcast_arrays(qi, ki)
            Sp = np.full_like(S, NEG_INF)
            grad_mod = np.zeros(S.shape)
            if score_mod is None:
                Sp[M] = S[M]
                grad_mod[M] = 1.0
            else:
                kept = (S[M], b, hq, qb[M], kb[M])
                Sp[M] = score_mod(*kept)
                grad_mod[M] = score_mod.grad(*kept)
            m = Sp.max(axis=1)
            P = np.zeros(S.shape)
            live = m > NEG_INF
            E = np.exp(Sp[live] - m[live, None])
            P[live] = E / E.sum(axis=1, keepdims=True)
            dV[b, hkv] += P.T @ dO
            dP = dO @ V.T
            dSp = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dS = dSp * grad_mod
            dQ[b, hq] = scale * (dS @ K)
            dK[b, hkv] += scale * (dS.T @ Q)
    return dQ, dK, dV


def _kept_scores(q, k, b, hq, rows, kv_rows, mask_mod, score_mod, scale):
    """Mask, scaled scores S, S' = mod(S) (-inf where masked) and mod'(S) for a
    block of (query rows x key rows) of (b, hq), as in attention_backward."""
    Hq, Hkv = q.shape[1], k.shape[1]
    hkv = hq // (Hq // Hkv)
    Q, K = _values(q[b, hq, rows]), _values(k[b, hkv, kv_rows])
    S = scale * (Q @ K.T)
    qi, ki = np.asarray(rows)[:, None], np.asarray(kv_rows)[None, :]
    M = np.ones(S.shape, dtype=bool) if mask_mod is None else \
        np.broadcast_to(np.asarray(mask_mod(b, hq, qi, ki), dtype=bool), S.shape)
    qb, kb = np.broadcast_arrays(qi, ki)
    Sp, dmod = np.full_like(S, NEG_INF), np.zeros_like(S)
    if score_mod is None:
        Sp[M], dmod[M] = S[M], 1.0
    else:
        args = (S[M], b, hq, qb[M], kb[M])
        Sp[M], dmod[M] = score_mod(*args), score_mod.grad(*args)
    return Sp, dmod


def attention_backward_q_rows(q, k, v, dout, b, hq, rows, mask_mod=None, score_mod=None, scale=None):
    """dQ of query rows `rows` of (b, hq) alone: a row's dQ depends only on that
    row (its softmax, dP = dO V^T and Delta), so sampled rows of a large problem
    cost one row of work each.  Same steps as attention_backward."""
    D, Skv = q.shape[3], k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    hkv = hq // (q.shape[1] // k.shape[1])
    rows = np.asarray(rows, dtype=np.int64)
    Sp, dmod = _kept_scores(q, k, b, hq, rows, np.arange(Skv), mask_mod, score_mod, scale)
    m = Sp.max(axis=1)
    P = np.zeros_like(Sp)
    live = m > NEG_INF
    E = np.exp(Sp[live] - m[live, None])
    P[live] = E / E.sum(axis=1)[:, None]
    dP = _values(dout[b, hq, rows]) @ _values(v[b, hkv]).T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True)) * dmod
    return scale * (dS @ _values(k[b, hkv]))


def attention_backward_kv_rows(q, k, v, dout, b, hkv, kv_rows, mask_mod=None, score_mod=None, scale=None,
                               chunk=1024):
    """dK and dV of key rows `kv_rows` of (b, hkv), summed over the query heads of
    its group.  A key row's gradient needs P[q, kv] for every query row, i.e.
    every row's softmax normaliser, so each row's log-sum-exp is computed here
    first (attention_rows over all keys); then, per query head and row chunk,
    the same steps as attention_backward restricted to these key columns."""
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    kv_rows = np.asarray(kv_rows, dtype=np.int64)
    dK = np.zeros((kv_rows.size, D))
    dV = np.zeros((kv_rows.size, D))
    V = _values(v[b, hkv])
    for hq in range(hkv * (Hq // Hkv), (hkv + 1) * (Hq // Hkv)):
        for r0 in range(0, Sq, chunk):
            rows = np.arange(r0, min(Sq, r0 + chunk))
            O, lse = attention_rows(q, k, v, b, hq, rows, mask_mod, score_mod, scale, check_rows_sum=False)
            Sp, dmod = _kept_scores(q, k, b, hq, rows, kv_rows, mask_mod, score_mod, scale)
            live = lse > NEG_INF
            P = np.zeros_like(Sp)
            P[live] = np.exp(Sp[live] - lse[live, None])
            dO = _values(dout[b, hq, rows])
            dP = dO @ V[kv_rows].T
            delta = (dO * O).sum(axis=1, keepdims=True)    # rowsum(dO * O) = rowsum(P * dP) over all keys
            dS = P * (dP - delta) * dmod
            dV += P.T @ dO
            dK += scale * (dS.T @ _values(q[b, hq, rows]))
    return dK, dV


# ---------------------------------------------------------------------------
# BlockMask (Concepts "BlockMask Internals" / "Key attributes"; paper review §4.1-4.2)
# ---------------------------------------------------------------------------

EMPTY, PARTIAL, FULL = 0, 1, 2


def block_classes(mask_mod, Bm: int, Hm: int, Sq: int, Skv: int, block: int = 128):
    """int8 [Bm,Hm,NQ,NK]: EMPTY / PARTIAL / FULL per (block x block) tile.

    A tile is FULL when every in-range position attends, EMPTY when none
    does, PARTIAL otherwise; positions past Sq or Skv are not part of a tile.
    """
    NQ, NK = -(-Sq // block), -(-Skv // block)
    cls = np.zeros((Bm, Hm, NQ, NK), dtype=np.int8)
    kv_all = np.arange(Skv, dtype=np.int64)[None, :]
    for b in range(Bm):
        for h in range(Hm):
            for qb in range(NQ):
                q0, q1 = qb * block, min(Sq, (qb + 1) * block)
                qi = np.arange(q0, q1, dtype=np.int64)[:, None]
                M = np.broadcast_to(np.asarray(mask_mod(b, h, qi, kv_all), dtype=bool),
                                    (q1 - q0, Skv))
                for kb in range(NK):
                    k0, k1 = kb * block, min(Skv, (kb + 1) * block)
                    n = int(M[:, k0:k1].sum())
                    area = (q1 - q0) * (k1 - k0)
                    cls[b, h, qb, kb] = EMPTY if n == 0 else (FULL if n == area else PARTIAL)
    return cls


def _compact(sel: np.ndarray):
    """Ascending column indices of True entries per row, padded with 0."""
    lead, NK = sel.shape[:-1], sel.shape[-1]
    num = sel.sum(axis=-1).astype(np.int32)
    idx = np.zeros(sel.shape, dtype=np.int32)
    flat_sel = sel.reshape(-1, NK)
    flat_idx = idx.reshape(-1, NK)
    for r in range(flat_sel.shape[0]):
        cols = np.nonzero(flat_sel[r])[0]
        flat_idx[r, :cols.size] = cols
    return num.reshape(lead), idx


def block_mask(mask_mod, Bm: int, Hm: int, Sq: int, Skv: int, block: int = 128,
               separate_full: bool = True):
    """The BlockMask tensors of Concepts "Key attributes".

    separate_full=True (canonical): kv_* lists PARTIAL tiles only and full_*
    lists FULL tiles only.  separate_full=False: kv_* lists every non-empty
    tile and full_* the FULL ones among them.  q_* and full_q_* are the same
    lists seen per KV block (q blocks ascending, padded with 0, last dim NQ).
    """
    cls = block_classes(mask_mod, Bm, Hm, Sq, Skv, block)
    full = cls == FULL
    kv_sel = (cls == PARTIAL) if separate_full else (cls != EMPTY)
    kv_num, kv_idx = _compact(kv_sel)
    full_num, full_idx = _compact(full)
    # Transposed view (Concepts "Key attributes": q_num_blocks / q_indices, for
    # the backward): per KV block, the query blocks of the same lists, ascending.
    q_num, q_idx = _compact(np.swapaxes(kv_sel, -1, -2))
    full_q_num, full_q_idx = _compact(np.swapaxes(full, -1, -2))
    return {
        "kv_num_blocks": kv_num, "kv_indices": kv_idx,
        "full_kv_num_blocks": full_num, "full_kv_indices": full_idx,
        "q_num_blocks": q_num, "q_indices": q_idx,
        "full_q_num_blocks": full_q_num, "full_q_indices": full_q_idx,
        "classes": cls,
    }


def block_mask_ascii(cls2d: np.ndarray) -> str:
    """Concepts "Inspecting a BlockMask": full = '██', partial = '░░', empty = blank."""
    glyph = {FULL: "██", PARTIAL: "░░", EMPTY: "  "}
    return "\n".join("".join(glyph[int(c)] for c in row).rstrip() for row in cls2d)


def sparsity(cls: np.ndarray) -> float:
    """Concepts "Inspecting a BlockMask": percentage of tiles that are empty."""
    return 100.0 * float((cls == EMPTY).sum()) / float(cls.size)


def attended_count(mask_mod, B: int, H: int, Sq: int, Skv: int, chunk: int = 1024) -> int:
    """Number of (b, h, q, kv) positions the mask keeps: the attended work that
    attended FLOPs (4 D per position) are counted on.  mask_mod None keeps all."""
    if mask_mod is None:
        return B * H * Sq * Skv
    n = 0
    kv_all = np.arange(Skv, dtype=np.int64)[None, :]
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Sq, chunk):
                qi = np.arange(r0, min(Sq, r0 + chunk), dtype=np.int64)[:, None]
                n += int(np.broadcast_to(np.asarray(mask_mod(b, h, qi, kv_all), dtype=bool),
                                         (qi.shape[0], Skv)).sum())
    return n
