"""Pins for the fp64 oracle, against things other than itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
flipped sign, a wrong index, a transposed operand, the mod applied at the
wrong place) fails at least one of them; tests/test_oracle_mutations.py
plants such slips and checks they are caught.

Pins used:
  * brute force with scalar Python loops (math.exp / math.tanh) on tiny inputs;
  * torch's CPU scaled_dot_product_attention in float64 (a library routine)
    for boolean masks, additive biases and GQA;
  * closed forms: uniform V, causal row 0, sliding window 0, prefix limits,
    ALiBi / relative-position geometric series, LSE of equal scores, the
    value of tanh at ln 2;
  * BlockMask: brute-force per-position counting, closed-form tile counts for
    causal and sliding windows, the Concepts page's causal print (golden).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from block_sparse_attention_fa_amd import inputs as gen
from oracle import flex_oracle as fo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


# ---------------------------------------------------------------------------
# bf16 decoding
# ---------------------------------------------------------------------------

def test_bf16_decode_known_values():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x0001, 0x3FC0], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, math.inf, 2.0 ** -133, 1.5]
    got = fo.bf16_to_f64(bits)
    assert list(got) == want


def test_generator_rounding_is_nearest_even():
    # 1 + 2^-8 is exactly halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to even (1.0)
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9], dtype=np.float32)
    assert list(fo.bf16_to_f64(gen.f32_to_bf16_bits(x))) == [1.0, 1.0 + 2.0 ** -6, 1.0]


# ---------------------------------------------------------------------------
# Brute force (scalar loops) on tiny inputs
# ---------------------------------------------------------------------------

def _f(bits):
    """Scalar bf16 -> float via struct-free arithmetic on the bit fields."""
    bits = int(bits)
    sign = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return sign * m * 2.0 ** (-133)
    return sign * (1.0 + m / 128.0) * 2.0 ** (e - 127)


def brute_attention(q, k, v, mask, mod, scale):
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    O = np.zeros((B, Hq, Sq, D))
    L = np.full((B, Hq, Sq), -math.inf)
    for b in range(B):
        for h in range(Hq):
            hk = h * Hkv // Hq
            for i in range(Sq):
                scores = []
                for j in range(Skv):
                    if mask is not None and not mask(b, h, i, j):
                        scores.append(-math.inf)
                        continue
                    s = sum(_f(q[b, h, i, d]) * _f(k[b, hk, j, d]) for d in range(D)) * scale
                    scores.append(mod(s, b, h, i, j) if mod is not None else s)
                m = max(scores)
                if m == -math.inf:
                    continue
                w = [math.exp(s - m) for s in scores]
                tot = sum(w)
                for d in range(D):
                    O[b, h, i, d] = sum(w[j] * _f(v[b, hk, j, d]) for j in range(Skv)) / tot
                L[b, h, i] = m + math.log(tot)
    return O, L


def _tiny(seed, B=2, Hq=4, Hkv=2, Sq=7, Skv=9, D=8):
    return gen.qkv(seed, B, Hq, Hkv, Sq, Skv, D)


_DOC = np.array([[0, 0, 0, 1, 1, 2, 2, 2, 2], [0, 1, 1, 1, 1, 1, 2, 3, 3]], dtype=np.int32)
_LEN = np.array([5, 0], dtype=np.int32)
_BIAS = gen._normal_bf16([99, 16], (2, 4, 7, 9), 0.5)
_SLOPES = [0.5, 0.25, 0.125, 0.0625]

# name -> (builder of the oracle functor, scalar brute-force functor).  The oracle
# functors are built when a pin runs, so a pin exercised by the mutation tests
# sees the mutated oracle module.
MASKS = {
    "none": (lambda: None, None),
    "causal": (lambda: fo.causal(), lambda b, h, i, j: i >= j),
    "sliding_causal2": (lambda: fo.sliding_causal(2), lambda b, h, i, j: i >= j and i - j <= 2),
    # the window term alone keeps every later key (j > i): only i - j <= 2 is required
    "sliding_window2": (lambda: fo.sliding_window(2), lambda b, h, i, j: i - j <= 2),
    "document": (lambda: fo.document(_DOC), lambda b, h, i, j: _DOC[b, i] == _DOC[b, j]),
    "document_causal": (lambda: fo.document_causal(_DOC), lambda b, h, i, j: _DOC[b, i] == _DOC[b, j] and i >= j),
    "prefix_lm3": (lambda: fo.prefix_lm(3), lambda b, h, i, j: j < 3 or i >= j),
    "kv_len": (lambda: fo.kv_length(_LEN), lambda b, h, i, j: j < _LEN[b]),
}
MODS = {
    "none": (lambda: None, None),
    "alibi": (lambda: fo.alibi(_SLOPES), lambda s, b, h, i, j: s + _SLOPES[h] * (j - i)),
    "softcap": (lambda: fo.softcap(0.7), lambda s, b, h, i, j: 0.7 * math.tanh(s / 0.7)),
    "rel_pos": (lambda: fo.rel_pos(), lambda s, b, h, i, j: s + (i - j)),
    "bias": (lambda: fo.bias(_BIAS), lambda s, b, h, i, j: s + _f(_BIAS[b, h, i, j])),
}


@pytest.mark.parametrize("mname", list(MASKS))
@pytest.mark.parametrize("sname", list(MODS))
def test_oracle_matches_brute_force(mname, sname):
    q, k, v = _tiny(7)
    om, bm = MASKS[mname][0](), MASKS[mname][1]
    os_, bs = MODS[sname][0](), MODS[sname][1]
    scale = 1.0 / math.sqrt(8)
    O, L = fo.attention(q, k, v, om, os_)
    Ob, Lb = brute_attention(q, k, v, bm, bs, scale)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(L), np.isneginf(Lb))
    fin = np.isfinite(Lb)
    np.testing.assert_allclose(L[fin], Lb[fin], rtol=0, atol=1e-12)


def test_fully_masked_row_gives_zero_and_neg_inf_lse():
    q, k, v = _tiny(3)
    O, L = fo.attention(q, k, v, fo.kv_length(np.array([4, 0])))
    assert np.all(O[1] == 0.0) and np.all(np.isneginf(L[1]))
    assert np.all(np.isfinite(L[0]))


# ---------------------------------------------------------------------------
# torch SDPA (float64, CPU) as an independent library routine
# ---------------------------------------------------------------------------

def _t(bits):
    return torch.from_numpy(fo.bf16_to_f64(bits))


def _sdpa(q, k, v, attn_mask, Hq, Hkv):
    return torch.nn.functional.scaled_dot_product_attention(
        _t(q), _t(k), _t(v), attn_mask=attn_mask, enable_gqa=(Hq != Hkv)).numpy()


@pytest.mark.parametrize("D", [16, 64])
@pytest.mark.parametrize("case", ["causal", "sliding", "window", "document", "prefix", "none"])
def test_oracle_matches_sdpa_boolean_masks(D, case):
    B, Hq, Hkv, S = 2, 4, 2, 150
    q, k, v = gen.qkv(11, B, Hq, Hkv, S, S, D)
    docs = gen.document_ids(5, B, S, 20, 60)
    om = {"causal": fo.causal(), "sliding": fo.sliding_causal(17), "window": fo.sliding_window(17),
          "document": fo.document_causal(docs), "prefix": fo.prefix_lm(40), "none": None}[case]
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    dt = torch.from_numpy(docs)
    if case == "causal":
        tm = (i >= j)[None, None]
    elif case == "sliding":
        tm = ((i >= j) & (i - j <= 17))[None, None]
    elif case == "window":
        tm = (i - j <= 17)[None, None]
    elif case == "document":
        tm = ((dt[:, :, None] == dt[:, None, :]) & (i >= j)[None])[:, None]
    elif case == "prefix":
        tm = ((j < 40) | (i >= j))[None, None]
    else:
        tm = None
    O, _ = fo.attention(q, k, v, om, None)
    ref = _sdpa(q, k, v, tm, Hq, Hkv)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mod", ["alibi", "rel_pos", "bias"])
def test_oracle_matches_sdpa_additive_mods(mod):
    # SDPA adds attn_mask after scaling Q K^T, which is where the pages put the mod.
    B, Hq, Hkv, S, D = 2, 4, 1, 130, 32
    q, k, v = gen.qkv(12, B, Hq, Hkv, S, S, D)
    i = np.arange(S)[:, None].astype(np.float64)
    j = np.arange(S)[None, :].astype(np.float64)
    slopes = fo.default_alibi_slopes(Hq)
    bias_bits = gen._normal_bf16([12, 16], (B, Hq, S, S), 0.5)
    if mod == "alibi":
        add = np.broadcast_to(slopes[None, :, None, None] * (j - i), (B, Hq, S, S))
        sm = fo.alibi(slopes)
    elif mod == "rel_pos":
        add = np.broadcast_to(i - j, (B, Hq, S, S))
        sm = fo.rel_pos()
    else:
        add = fo.bf16_to_f64(bias_bits)
        sm = fo.bias(bias_bits)
    causal = (i >= j)
    fm = np.where(causal[None, None], add, -np.inf)
    O, _ = fo.attention(q, k, v, fo.causal(), sm)
    ref = _sdpa(q, k, v, torch.from_numpy(np.ascontiguousarray(fm)), Hq, Hkv)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-11)


def test_gqa_equals_mha_with_repeated_kv():
    B, Hq, Hkv, S, D = 1, 8, 2, 64, 16
    q, k, v = gen.qkv(13, B, Hq, Hkv, S, S, D)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    O1, L1 = fo.attention(q, k, v, fo.causal(), fo.alibi(fo.default_alibi_slopes(Hq)))
    O2, L2 = fo.attention(q, kr, vr, fo.causal(), fo.alibi(fo.default_alibi_slopes(Hq)))
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


def test_lse_matches_torch_logsumexp():
    B, H, S, D = 1, 2, 96, 16
    q, k, v = gen.qkv(14, B, H, H, S, S, D)
    _, L = fo.attention(q, k, v, fo.causal(), fo.softcap(5.0))
    Q, K = _t(q), _t(k)
    s = (Q @ K.transpose(-1, -2)) / math.sqrt(D)
    s = 5.0 * torch.tanh(s / 5.0)
    s = s.masked_fill(~torch.ones(S, S, dtype=torch.bool).tril(), -math.inf)
    np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def _const_rows(D, S, val_bits):
    return np.broadcast_to(val_bits[None, :], (S, D)).copy()


@pytest.mark.parametrize("mname", ["causal", "sliding_causal2", "document_causal", "prefix_lm3"])
@pytest.mark.parametrize("sname", ["none", "alibi", "softcap", "rel_pos", "bias"])
def test_uniform_v_gives_constant_output(mname, sname):
    q, k, v = _tiny(21)
    c = gen.f32_to_bf16_bits(np.linspace(-2, 3, 8).astype(np.float32))
    v = np.broadcast_to(c, v.shape).copy()
    O, _ = fo.attention(q, k, v, MASKS[mname][0](), MODS[sname][0]())
    np.testing.assert_allclose(O, np.broadcast_to(fo.bf16_to_f64(c), O.shape), rtol=0, atol=1e-12)


@pytest.mark.parametrize("sname", ["none", "alibi", "softcap", "rel_pos"])
def test_causal_row0_is_v0(sname):
    B, H, S, D = 2, 4, 40, 16
    q, k, v = gen.qkv(22, B, H, H, S, S, D)
    O, _ = fo.attention(q, k, v, fo.causal(), MODS[sname][0]() if sname != "alibi" else fo.alibi(_SLOPES))
    np.testing.assert_array_equal(O[:, :, 0], fo.bf16_to_f64(v[:, :, 0]))


def test_sliding_window_zero_is_identity_on_v():
    B, H, S, D = 1, 2, 50, 16
    q, k, v = gen.qkv(23, B, H, H, S, S, D)
    O, _ = fo.attention(q, k, v, fo.sliding_causal(0), None)
    np.testing.assert_array_equal(O, fo.bf16_to_f64(v))


def test_mask_limits():
    B, H, S, D = 1, 2, 45, 16
    q, k, v = gen.qkv(24, B, H, H, S, S, D)
    Oc, _ = fo.attention(q, k, v, fo.causal())
    np.testing.assert_array_equal(fo.attention(q, k, v, fo.sliding_causal(S - 1))[0], Oc)
    np.testing.assert_array_equal(fo.attention(q, k, v, fo.prefix_lm(0))[0], Oc)
    np.testing.assert_array_equal(fo.attention(q, k, v, fo.prefix_lm(S))[0],
                                  fo.attention(q, k, v, None)[0])


def test_document_mask_is_block_diagonal_causal():
    B, H, S, D = 1, 2, 60, 16
    q, k, v = gen.qkv(25, B, H, H, S, S, D)
    docs = gen.document_ids(25, B, S, 7, 25)
    O, _ = fo.attention(q, k, v, fo.document_causal(docs))
    for d in np.unique(docs[0]):
        idx = np.nonzero(docs[0] == d)[0]
        sl = slice(idx[0], idx[-1] + 1)
        Od, _ = fo.attention(q[:, :, sl], k[:, :, sl], v[:, :, sl], fo.causal())
        np.testing.assert_allclose(O[:, :, sl], Od, rtol=0, atol=1e-13)


def _geometric_mean_index(q, r):
    """Sum_{kv<=q} kv r^(q-kv) / Sum_{kv<=q} r^(q-kv), summed in closed form."""
    if q == 0:
        return 0.0
    s0 = (1 - r ** (q + 1)) / (1 - r)
    s1 = r * (1 - (q + 1) * r ** q + q * r ** (q + 1)) / (1 - r) ** 2
    return q - s1 / s0


def _index_valued_v(S, D):
    return np.broadcast_to(gen.f32_to_bf16_bits(np.arange(S, dtype=np.float32))[:, None], (S, D)).copy()


@pytest.mark.parametrize("H", [4, 8])
def test_alibi_geometric_closed_form(H):
    # Q = 0 makes every raw score 0, so the weights are exp(slope*(kv-q)) = r^(q-kv), r = e^-slope.
    S, D = 200, 8
    q = np.zeros((1, H, S, D), dtype=np.uint16)
    k = gen.qkv(26, 1, H, H, S, S, D)[1]
    v = np.broadcast_to(_index_valued_v(S, D), (1, H, S, D)).copy()
    slopes = fo.default_alibi_slopes(H)
    O, _ = fo.attention(q, k, v, fo.causal(), fo.alibi(slopes))
    for h in range(H):
        r = math.exp(-slopes[h])
        want = np.array([_geometric_mean_index(i, r) for i in range(S)])
        np.testing.assert_allclose(O[0, h, :, 0], want, rtol=1e-12, atol=1e-10)


def test_alibi_default_slopes_are_geometric():
    # For 8 heads the sequence is 1/2, 1/4, ..., 1/256.
    np.testing.assert_array_equal(fo.default_alibi_slopes(8), [2.0 ** -(i + 1) for i in range(8)])


def test_rel_pos_geometric_closed_form():
    # Q = 0: weights exp(q - kv) = r^(q-kv) with r = e (keys nearer the start weigh more).
    S, D = 30, 8
    q = np.zeros((1, 1, S, D), dtype=np.uint16)
    k = gen.qkv(27, 1, 1, 1, S, S, D)[1]
    v = _index_valued_v(S, D)[None, None]
    O, _ = fo.attention(q, k, v, fo.causal(), fo.rel_pos())
    want = np.array([_geometric_mean_index(i, math.e) for i in range(S)])
    np.testing.assert_allclose(O[0, 0, :, 0], want, rtol=1e-12, atol=1e-10)


def test_softcap_closed_form_and_limits():
    cap = 30.0
    sc = fo.softcap(cap)
    # tanh(ln 2) = (4 - 1) / (4 + 1) = 3/5
    assert abs(sc(np.array([cap * math.log(2.0)]), 0, 0, 0, 0)[0] - 0.6 * cap) < 1e-12
    assert abs(sc(np.array([-cap * math.log(2.0)]), 0, 0, 0, 0)[0] + 0.6 * cap) < 1e-12
    q, k, v = _tiny(28)
    O_big, _ = fo.attention(q, k, v, fo.causal(), fo.softcap(1e6))
    O_none, _ = fo.attention(q, k, v, fo.causal(), None)
    np.testing.assert_allclose(O_big, O_none, rtol=0, atol=1e-9)
    # cap -> 0 squashes every score to 0: the output is the plain mean of visible V rows
    O_tiny, _ = fo.attention(q, k, v, fo.causal(), fo.softcap(1e-12))
    V = fo.bf16_to_f64(v)
    for i in range(q.shape[2]):
        np.testing.assert_allclose(O_tiny[:, 0::2, i], V[:, :, :i + 1].mean(axis=2), atol=1e-9)


def test_equal_scores_lse_is_log_count():
    S, D = 77, 8
    q = np.zeros((1, 1, S, D), dtype=np.uint16)
    k, v = gen.qkv(29, 1, 1, 1, S, S, D)[1:]
    _, L = fo.attention(q, k, v, fo.causal())
    np.testing.assert_allclose(L[0, 0], np.log(np.arange(1, S + 1)), rtol=0, atol=1e-14)


def test_bias_equal_to_alibi_matches_alibi_functor():
    B, H, S, D = 1, 2, 24, 8
    q, k, v = gen.qkv(30, B, H, H, S, S, D)
    sl = [0.5, 0.25]  # slope * integer distance stays exact in bf16 for |kv-q| < 24
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    tab = gen.f32_to_bf16_bits(np.stack([s * (j - i) for s in sl]).astype(np.float32))[None]
    Oa, _ = fo.attention(q, k, v, fo.causal(), fo.alibi(sl))
    Ob, _ = fo.attention(q, k, v, fo.causal(), fo.bias(tab))
    np.testing.assert_allclose(Oa, Ob, rtol=0, atol=1e-14)
    zero = np.zeros((1, H, S, S), dtype=np.uint16)
    np.testing.assert_allclose(fo.attention(q, k, v, fo.causal(), fo.bias(zero))[0],
                               fo.attention(q, k, v, fo.causal(), None)[0], rtol=0, atol=1e-15)


def test_decode_equals_single_row_sdpa():
    B, Hq, Hkv, KV, D = 3, 8, 2, 300, 16
    q = gen.qkv(31, B, Hq, Hkv, 1, KV, D)[0]
    _, k, v = gen.qkv(32, B, Hkv, Hkv, 1, KV, D)
    lens = np.array([300, 129, 1], dtype=np.int32)
    O, _ = fo.decode(q, k, v, lens, fo.softcap(50.0))
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            Qv = fo.bf16_to_f64(q[b, h, 0])
            K = fo.bf16_to_f64(k[b, hk, :lens[b]])
            V = fo.bf16_to_f64(v[b, hk, :lens[b]])
            s = 50.0 * np.tanh((K @ Qv) / math.sqrt(D) / 50.0)
            w = np.exp(s - s.max())
            np.testing.assert_allclose(O[b, h, 0], (w @ V) / w.sum(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mod", ["alibi", "rel_pos"])
def test_decode_at_query_positions_matches_sdpa(mod):
    """A decode query at position p sees q_idx = p: ALiBi adds slope[h] (kv - p),
    the relative position (p - kv); torch SDPA with that additive mask."""
    B, Hq, Hkv, KV, D = 3, 4, 2, 200, 16
    q = gen.qkv(33, B, Hq, Hkv, 1, KV, D)[0]
    _, k, v = gen.qkv(34, B, Hkv, Hkv, 1, KV, D)
    lens = np.array([200, 77, 1], dtype=np.int32)
    pos = np.array([199, 500, 0], dtype=np.int64)     # a position need not be inside the cache
    slopes = fo.default_alibi_slopes(Hq)
    sm = fo.alibi(slopes) if mod == "alibi" else fo.rel_pos()
    O, L = fo.decode(q, k, v, lens, sm, positions=pos)
    kv = np.arange(KV, dtype=np.float64)
    for b in range(B):
        if mod == "alibi":
            add = slopes[:, None] * (kv[None, :] - pos[b])          # [Hq, KV]
        else:
            add = np.broadcast_to(pos[b] - kv[None, :], (Hq, KV))
        am = np.where(kv[None, :] < lens[b], add, -np.inf)[:, None, :]   # [Hq, 1, KV]
        ref = torch.nn.functional.scaled_dot_product_attention(
            _t(q[b:b + 1]), _t(k[b:b + 1]), _t(v[b:b + 1]), attn_mask=torch.from_numpy(am)[None],
            enable_gqa=True).numpy()
        np.testing.assert_allclose(O[b:b + 1], ref, rtol=0, atol=1e-12)
        # A position shifts every score of the row by the same amount, so O alone
        # cannot show it; the log-sum-exp does.
        hk = np.arange(Hq) // (Hq // Hkv)
        sc = (_t(q[b, :, 0])[:, None, :] * _t(k[b, hk])).sum(-1) / math.sqrt(D)   # [Hq, KV]
        lse = torch.logsumexp(sc + torch.from_numpy(am[:, 0, :]), dim=-1).numpy()
        np.testing.assert_allclose(L[b, :, 0], lse, rtol=0, atol=1e-12)


def test_decode_at_position_p_is_row_p_of_the_causal_forward():
    B, H, S, D, p = 2, 4, 90, 16, 61
    q, k, v = gen.qkv(35, B, H, H, S, S, D)
    sm = fo.alibi(fo.default_alibi_slopes(H))
    O, L = fo.attention(q, k, v, fo.causal(), sm)
    Od, Ld = fo.decode(q[:, :, p:p + 1], k, v, np.full(B, p + 1, dtype=np.int32), sm, positions=np.full(B, p))
    np.testing.assert_allclose(Od[:, :, 0], O[:, :, p], rtol=0, atol=1e-13)
    np.testing.assert_allclose(Ld[:, :, 0], L[:, :, p], rtol=0, atol=1e-12)
    # the same query at position 0: same output, LSE lower by slope[h] * p (softmax ignores a constant)
    O0, L0 = fo.decode(q[:, :, p:p + 1], k, v, np.full(B, p + 1, dtype=np.int32), sm)
    np.testing.assert_allclose(O0, Od, rtol=0, atol=1e-12)
    slopes = fo.default_alibi_slopes(H)[None, :, None]
    np.testing.assert_allclose(Ld, L0 - slopes * p, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# BlockMask
# ---------------------------------------------------------------------------

def _brute_classes(mask, Bm, Hm, Sq, Skv, bs):
    NQ, NK = -(-Sq // bs), -(-Skv // bs)
    out = np.zeros((Bm, Hm, NQ, NK), dtype=np.int8)
    for b in range(Bm):
        for h in range(Hm):
            for qb in range(NQ):
                for kb in range(NK):
                    yes = no = 0
                    for i in range(qb * bs, min(Sq, qb * bs + bs)):
                        for j in range(kb * bs, min(Skv, kb * bs + bs)):
                            if mask(b, h, i, j):
                                yes += 1
                            else:
                                no += 1
                    out[b, h, qb, kb] = 0 if yes == 0 else (2 if no == 0 else 1)
    return out


@pytest.mark.parametrize("Sq,Skv", [(37, 37), (37, 50), (50, 23), (1, 45)])
@pytest.mark.parametrize("mname", ["causal", "sliding_causal2", "document_causal", "prefix_lm3", "kv_len", "none"])
def test_block_classes_brute_force(Sq, Skv, mname):
    docs = gen.document_ids(41, 2, max(Sq, Skv), 3, 11)
    lens = np.array([17, 4], dtype=np.int32)
    om = {"causal": fo.causal(), "sliding_causal2": fo.sliding_causal(2),
          "document_causal": fo.document_causal(docs), "prefix_lm3": fo.prefix_lm(3),
          "kv_len": fo.kv_length(lens), "none": fo.no_mask()}[mname]
    bm = {"causal": lambda b, h, i, j: i >= j, "sliding_causal2": lambda b, h, i, j: i >= j and i - j <= 2,
          "document_causal": lambda b, h, i, j: docs[b, i] == docs[b, j] and i >= j,
          "prefix_lm3": lambda b, h, i, j: j < 3 or i >= j, "kv_len": lambda b, h, i, j: j < lens[b],
          "none": lambda b, h, i, j: True}[mname]
    got = fo.block_classes(om, 2, 1, Sq, Skv, block=8)
    np.testing.assert_array_equal(got, _brute_classes(bm, 2, 1, Sq, Skv, 8))


def test_block_mask_lists_from_classes():
    cls = fo.block_classes(fo.causal(), 1, 1, 37, 37, block=8)
    bm = fo.block_mask(fo.causal(), 1, 1, 37, 37, block=8)
    for qb in range(cls.shape[2]):
        part = [kb for kb in range(cls.shape[3]) if cls[0, 0, qb, kb] == 1]
        full = [kb for kb in range(cls.shape[3]) if cls[0, 0, qb, kb] == 2]
        assert bm["kv_num_blocks"][0, 0, qb] == len(part)
        assert list(bm["kv_indices"][0, 0, qb]) == part + [0] * (cls.shape[3] - len(part))
        assert bm["full_kv_num_blocks"][0, 0, qb] == len(full)
        assert list(bm["full_kv_indices"][0, 0, qb]) == full + [0] * (cls.shape[3] - len(full))
    for key in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices"):
        assert bm[key].dtype == np.int32


def test_golden_causal_256():
    g = json.load(open(os.path.join(GOLDEN, "causal_256_blockmask.json")))
    for mode, sep in (("separate_full", True), ("superset", False)):
        bm = fo.block_mask(fo.causal(), 1, 1, 256, 256, separate_full=sep)
        for key, want in g[mode].items():
            np.testing.assert_array_equal(bm[key], np.array(want, dtype=np.int32), err_msg=f"{mode}:{key}")


def test_golden_causal_2048_print():
    lines = [l.rstrip("\n") for l in open(os.path.join(GOLDEN, "causal_2048_blockmask.txt"), encoding="utf-8")
             if not l.startswith("#")]
    cls = fo.block_classes(fo.causal(), 1, 1, 2048, 2048)
    assert fo.block_mask_ascii(cls[0, 0]).split("\n") == lines


@pytest.mark.parametrize("n", [2, 5, 64])
def test_causal_tile_counts_closed_form(n):
    cls = fo.block_classes(fo.causal(), 1, 1, 128 * n, 128 * n)
    assert int((cls == 2).sum()) == n * (n - 1) // 2
    assert int((cls == 1).sum()) == n
    assert int((cls == 0).sum()) == n * (n - 1) // 2
    # work ratio of dense vs block-sparse causal approaches 2 (Concepts, "When to use which?")
    assert n * n / (n * (n + 1) / 2) == pytest.approx(2 * n / (n + 1))
    if n == 64:
        assert fo.sparsity(cls) == pytest.approx(100.0 * 2016 / 4096)


def test_sliding_window_tile_counts_closed_form():
    # Tile (qb, kb) with d = qb - kb covers q - kv in [128d - 127, 128d + 127].  With the window
    # 0 <= q - kv <= 1024 it is full iff 1 <= d <= 7, partial iff d in {0, 8}, empty otherwise.
    n = 128
    cls = fo.block_classes(fo.sliding_causal(1024), 1, 1, 128 * n, 128 * n)
    full = sum(n - d for d in range(1, 8))
    part = n + (n - 8)
    assert int((cls == 2).sum()) == full == 868
    assert int((cls == 1).sum()) == part == 248
    assert int((cls == 0).sum()) == n * n - full - part == 15268


def test_kv_length_tile_rule():
    lens = np.array([4096, 5000, 1, 32768, 128 * 37 + 5], dtype=np.int32)
    cls = fo.block_classes(fo.kv_length(lens), 5, 1, 1, 32768)
    for b, L in enumerate(lens):
        for kb in range(256):
            want = 2 if 128 * (kb + 1) <= L else (1 if 128 * kb < L else 0)
            assert cls[b, 0, 0, kb] == want


@pytest.mark.parametrize("chunk", [64, 1024])
def test_attended_count_closed_forms(chunk):
    """N_att, the number of attended (b, h, q, kv) positions, against closed forms:
    causal S(S+1)/2 per head, the sliding causal window min(q, W) + 1 per row, a
    document-causal mask sum L(L+1)/2 over its documents, the kv_len prefix
    Sq * len[b] per head; chunk sizes that do and do not divide S."""
    B, H, S, W = 2, 3, 300, 37
    assert fo.attended_count(fo.causal(), B, H, S, S, chunk) == B * H * S * (S + 1) // 2
    assert fo.attended_count(fo.sliding_causal(W), B, H, S, S, chunk) == \
        B * H * sum(min(q, W) + 1 for q in range(S))
    assert fo.attended_count(None, B, H, S, 170, chunk) == B * H * S * 170
    docs = gen.document_ids(41, B, S, 20, 90)
    want = H * sum(int(L) * (int(L) + 1) // 2 for b in range(B) for L in np.bincount(docs[b]))
    assert fo.attended_count(fo.document_causal(docs), B, H, S, S, chunk) == want
    lens = np.array([0, 123], dtype=np.int32)
    assert fo.attended_count(fo.kv_length(lens), B, H, 5, 200, chunk) == H * 5 * 123


@pytest.mark.parametrize("mname", ["sliding_window2", "prefix_lm3", "document"])
def test_attended_count_brute_force(mname):
    om, bm = MASKS[mname][0](), MASKS[mname][1]
    want = sum(1 for b in range(2) for h in range(4) for i in range(7) for j in range(9) if bm(b, h, i, j))
    assert fo.attended_count(om, 2, 4, 7, 9, chunk=3) == want


def test_blockmask_memory_ratio():
    # Paper review §4.1: one entry per 128x128 tile instead of per position -> 16384x fewer
    S = 8192
    cls = fo.block_classes(fo.causal(), 1, 1, S, S)
    assert (S * S) / cls.size == 16384


# ---------------------------------------------------------------------------
# Backward (attention_backward): finite differences, torch autograd, closed forms
# ---------------------------------------------------------------------------

def _loss(q, k, v, dO, om, sm, scale):
    O, _ = fo.attention(q, k, v, om, sm, scale=scale)
    return float((O * dO).sum())


@pytest.mark.parametrize("mname", ["causal", "sliding_causal2", "document_causal", "kv_len", "none"])
@pytest.mark.parametrize("sname", list(MODS))
def test_backward_matches_finite_differences(mname, sname):
    """Central differences of L = sum(O * dO) with respect to sampled entries of
    Q, K and V (float64 inputs, tiny GQA shapes), against the analytic gradients."""
    q, k, v = (fo.bf16_to_f64(x) for x in _tiny(7))
    om, sm = MASKS[mname][0](), MODS[sname][0]()
    scale = 1.0 / math.sqrt(8)
    rng = np.random.default_rng([21, len(mname), len(sname)])
    dO = rng.standard_normal(q.shape)
    grads = fo.attention_backward(q, k, v, dO, om, sm, scale)
    eps = 1e-6
    for x, g in zip((q, k, v), grads):
        for _ in range(8):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            x0 = x[idx]
            x[idx] = x0 + eps
            up = _loss(q, k, v, dO, om, sm, scale)
            x[idx] = x0 - eps
            dn = _loss(q, k, v, dO, om, sm, scale)
            x[idx] = x0
            np.testing.assert_allclose(g[idx], (up - dn) / (2 * eps), rtol=1e-5, atol=1e-8,
                                       err_msg=f"{mname}/{sname} at {idx}")


def _torch_grads(q, k, v, dO, fn):
    qt, kt, vt = (torch.from_numpy(fo.bf16_to_f64(x)).requires_grad_() for x in (q, k, v))
    out = fn(qt, kt, vt)
    out.backward(torch.from_numpy(dO))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("case", ["causal", "document", "alibi_causal", "bias_causal", "none"])
def test_backward_matches_torch_autograd_sdpa(case):
    """torch autograd through its CPU scaled_dot_product_attention (float64, GQA)."""
    B, Hq, Hkv, S, D = 2, 4, 2, 70, 16
    q, k, v = gen.qkv(31, B, Hq, Hkv, S, S, D)
    dO = np.random.default_rng(31).standard_normal((B, Hq, S, D))
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    docs = gen.document_ids(31, B, S, 10, 30)
    slopes = fo.default_alibi_slopes(Hq)
    bias_bits = gen._normal_bf16([31, 16], (B, Hq, S, S), 0.5)
    if case == "causal":
        om, sm, tm = fo.causal(), None, torch.from_numpy(i >= j)
    elif case == "document":
        om, sm = fo.document(docs), None
        tm = torch.from_numpy(docs[:, :, None] == docs[:, None, :])[:, None]
    elif case == "alibi_causal":
        om, sm = fo.causal(), fo.alibi(slopes)
        tm = torch.from_numpy(np.where((i >= j)[None], slopes[:, None, None] * (j - i), -np.inf))
    elif case == "bias_causal":
        om, sm = fo.causal(), fo.bias(bias_bits)
        tm = torch.from_numpy(np.where((i >= j)[None, None], fo.bf16_to_f64(bias_bits), -np.inf))
    else:
        om, sm, tm = None, None, None
    ref = _torch_grads(q, k, v, dO, lambda a, b_, c: torch.nn.functional.scaled_dot_product_attention(
        a, b_, c, attn_mask=tm, enable_gqa=True))
    got = fo.attention_backward(q, k, v, dO, om, sm)
    for name, g, r in zip("QKV", got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-11, err_msg=f"d{name} {case}")


def test_backward_softcap_matches_torch_autograd():
    """Softcap is no SDPA mask, so the reference is torch autograd through the
    forward written with torch ops (scale, cap*tanh(s/cap), causal -inf, softmax)."""
    B, Hq, Hkv, S, D, cap = 1, 2, 1, 50, 16, 0.8
    q, k, v = gen.qkv(33, B, Hq, Hkv, S, S, D)
    dO = np.random.default_rng(33).standard_normal((B, Hq, S, D))
    keep = torch.from_numpy(np.arange(S)[:, None] >= np.arange(S)[None, :])

    def fwd(a, b_, c):
        b_, c = b_.repeat_interleave(Hq // Hkv, dim=1), c.repeat_interleave(Hq // Hkv, dim=1)
        s = (a @ b_.transpose(-1, -2)) / math.sqrt(D)
        s = cap * torch.tanh(s / cap)
        return torch.softmax(s.masked_fill(~keep, -math.inf), dim=-1) @ c

    ref = _torch_grads(q, k, v, dO, fwd)
    got = fo.attention_backward(q, k, v, dO, fo.causal(), fo.softcap(cap))
    for name, g, r in zip("QKV", got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-11, err_msg=f"d{name} softcap")


def test_backward_closed_forms():
    """Uniform V: O does not depend on Q or K, so dQ = dK = 0 and dV sums
    P^T dO.  Causal row 0 attends one key: its dO flows to dV[0] unchanged."""
    B, Hq, Hkv, S, D = 1, 2, 1, 33, 8
    q, k, v = gen.qkv(35, B, Hq, Hkv, S, S, D)
    v[:] = v[:, :, :1, :]                                  # every V row equal
    dO = np.random.default_rng(35).standard_normal((B, Hq, S, D))
    dQ, dK, dV = fo.attention_backward(q, k, v, dO, fo.causal(), fo.alibi(fo.default_alibi_slopes(Hq)))
    np.testing.assert_allclose(dQ, 0.0, atol=1e-12)
    np.testing.assert_allclose(dK, 0.0, atol=1e-12)
    np.testing.assert_allclose(dV.sum(axis=2), dO.sum(axis=(1, 2))[:, None, :], rtol=0, atol=1e-11)
    dO0 = np.zeros_like(dO)
    dO0[:, :, 0] = dO[:, :, 0]
    _, _, dV0 = fo.attention_backward(q, k, v, dO0, fo.causal())
    np.testing.assert_allclose(dV0[:, 0, 0], dO[:, :, 0].sum(axis=1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV0[:, 0, 1:], 0.0, atol=1e-12)


def test_backward_gqa_equals_mha_summed_over_the_group():
    B, Hq, Hkv, S, D = 1, 4, 2, 40, 8
    q, k, v = gen.qkv(37, B, Hq, Hkv, S, S, D)
    dO = np.random.default_rng(37).standard_normal((B, Hq, S, D))
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    sm = fo.softcap(2.0)
    dQ1, dK1, dV1 = fo.attention_backward(q, k, v, dO, fo.causal(), sm)
    dQ2, dK2, dV2 = fo.attention_backward(q, kr, vr, dO, fo.causal(), sm)
    np.testing.assert_allclose(dQ1, dQ2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dK1, dK2.reshape(B, Hkv, Hq // Hkv, S, D).sum(axis=2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dV1, dV2.reshape(B, Hkv, Hq // Hkv, S, D).sum(axis=2), rtol=0, atol=1e-13)


def test_backward_fully_masked_row_contributes_nothing():
    q, k, v = _tiny(3)
    dO = np.random.default_rng(3).standard_normal(q.shape)
    dQ, dK, dV = fo.attention_backward(q, k, v, dO, fo.kv_length(np.array([4, 0])))
    assert np.all(dQ[1] == 0.0) and np.all(dK[1] == 0.0) and np.all(dV[1] == 0.0)
    assert np.all(np.isfinite(dQ)) and np.abs(dQ[0]).max() > 0


def test_transposed_block_lists():
    """q_* / full_q_* list, per KV block, the query blocks whose row lists hold it."""
    docs = gen.document_ids(43, 1, 300, 20, 90)
    for om in (fo.causal(), fo.sliding_causal(100), fo.document_causal(docs)):
        for sep in (True, False):
            bm = fo.block_mask(om, 1, 1, 300, 260, block=32, separate_full=sep)
            NQ, NK = bm["kv_num_blocks"].shape[-1], bm["q_num_blocks"].shape[-1]
            for kb in range(NK):
                rows = [qb for qb in range(NQ) if kb in bm["kv_indices"][0, 0, qb, :bm["kv_num_blocks"][0, 0, qb]]]
                full = [qb for qb in range(NQ)
                        if kb in bm["full_kv_indices"][0, 0, qb, :bm["full_kv_num_blocks"][0, 0, qb]]]
                assert bm["q_num_blocks"][0, 0, kb] == len(rows)
                assert list(bm["q_indices"][0, 0, kb]) == rows + [0] * (NQ - len(rows))
                assert bm["full_q_num_blocks"][0, 0, kb] == len(full)
                assert list(bm["full_q_indices"][0, 0, kb]) == full + [0] * (NQ - len(full))


def test_backward_row_and_column_samplers_match_the_full_backward():
    """The sampled-row helpers used at full sizes give the full backward's rows."""
    B, Hq, Hkv, S, D = 2, 4, 2, 90, 16
    q, k, v = gen.qkv(39, B, Hq, Hkv, S, S, D)
    dO = gen._normal_bf16([39, 30], (B, Hq, S, D), 1.0)
    docs = gen.document_ids(39, B, S, 10, 40)
    for om, sm in ((fo.causal(), fo.alibi(fo.default_alibi_slopes(Hq))), (fo.document_causal(docs), fo.softcap(1.5)),
                   (None, fo.rel_pos())):
        dQ, dK, dV = fo.attention_backward(q, k, v, dO, om, sm)
        rows = np.array([0, 5, 44, 89])
        for b, hq in ((0, 0), (1, 3)):
            np.testing.assert_allclose(fo.attention_backward_q_rows(q, k, v, dO, b, hq, rows, om, sm),
                                       dQ[b, hq, rows], rtol=0, atol=1e-12)
        for b, hkv in ((0, 1), (1, 0)):
            gk, gv = fo.attention_backward_kv_rows(q, k, v, dO, b, hkv, rows, om, sm, chunk=32)
            np.testing.assert_allclose(gk, dK[b, hkv, rows], rtol=0, atol=1e-12)
            np.testing.assert_allclose(gv, dV[b, hkv, rows], rtol=0, atol=1e-12)
