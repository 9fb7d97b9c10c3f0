"""Forward kernel vs the fp64 oracle, element by element, at sizes that span
several tiles and a ragged tail, for every mask_mod x score_mod, both head dims,
GQA, broadcast and per-batch BlockMasks, the superset list encoding and the
dense path.  Tolerance: max abs 2e-2 and mean abs 2e-3 (bf16 in, fp32 accumulate).
"""

import math

import numpy as np
import pytest

from block_sparse_attention_fa_amd import inputs as gen
from oracle import flex_oracle as fo
from tests import _cases as C

pytestmark = pytest.mark.gpu

BATCH_DEP = ("document", "document_causal", "kv_len")


def run_case(seed, mask, score, B, Hq, Hkv, Sq, Skv, D, separate_full=True, dense=False,
             per_head_mask=False, with_lse=True, order=None, **spec_kw):
    import torch
    from block_sparse_attention_fa_amd import fa
    print(f"[case] seed={seed} mask={mask} score={score} B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Skv={Skv} D={D} "
          f"sep={separate_full} dense={dense} order={order}", flush=True)
    q, k, v = gen.qkv(seed, B, Hq, Hkv, Sq, Skv, D)
    spec = C.make_spec(seed, mask, score, B, Hq, Sq, Skv, **spec_kw)
    qt, kt, vt = (gen.to_torch_bf16(x) for x in (q, k, v))
    bm = None
    if not dense:
        Bm = B if mask in BATCH_DEP else 1
        Hm = Hq if per_head_mask else 1
        bm = fa.fa_build_block_mask(C.gpu_mask(spec), Bm, Hm, Sq, Skv, separate_full=separate_full, order=order)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda") if with_lse else None
    out = fa.fa_forward(qt, kt, vt, block_mask=bm, score=C.gpu_score(spec), lse=lse)
    torch.cuda.synchronize()
    got = gen.bf16_bits_to_f32(gen.from_torch_bf16(out))
    O, L = fo.attention(q, k, v, None if dense else C.oracle_mask(spec), C.oracle_score(spec, Hq))
    C.compare(got, O, f"{mask}/{score}")
    if with_lse:
        C.compare_lse(lse.cpu().numpy(), L, f"{mask}/{score}")
    return got, O


def test_tiny_causal_workload():
    # B=1, H=2, S=256, D=64, causal, no score_mod (2x2 tiles)
    run_case(1, "causal", "none", 1, 2, 2, 256, 256, 64)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("score", C.SCORE_NAMES)
@pytest.mark.parametrize("mask", C.MASK_NAMES)
def test_mask_score_matrix(mask, score, D):
    run_case(10 + D, mask, score, 2, 4, 2, 300, 300, D)


@pytest.mark.parametrize("Sq,Skv", [(200, 333), (333, 200), (1, 257), (129, 129), (640, 640)])
@pytest.mark.parametrize("mask", ["causal", "sliding_causal", "prefix_lm", "kv_len", "none"])
def test_uneven_lengths(mask, Sq, Skv):
    run_case(20, mask, "alibi", 1, 2, 1, Sq, Skv, 128)


@pytest.mark.parametrize("mask", ["causal", "document_causal", "sliding_causal"])
def test_superset_encoding(mask):
    run_case(30, mask, "softcap", 2, 2, 2, 384, 384, 64, separate_full=False)


@pytest.mark.parametrize("mask", ["causal", "document_causal", "kv_len"])
def test_every_tile_listed_as_partial(mask):
    """The "no block skipping" encoding (every tile listed, the mask_mod applied to
    all of them) computes the same attention as the canonical BlockMask."""
    import torch
    from block_sparse_attention_fa_amd import fa
    B, H, S, D = 2, 2, 392, 128
    print(f"[case] every tile listed, mask={mask}", flush=True)
    q, k, v = gen.qkv(71, B, H, H, S, S, D)
    spec = C.make_spec(71, mask, "alibi", B, H, S, S)
    Bm = B if mask in BATCH_DEP else 1
    bm = fa.fa_build_block_mask(C.gpu_mask(spec), Bm, 1, S, S, separate_full=False).list_every_tile()
    torch.cuda.synchronize()
    assert int(bm.kv_num_blocks.min().item()) == bm.NK
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    out = fa.fa_forward(*(gen.to_torch_bf16(x) for x in (q, k, v)), block_mask=bm, score=C.gpu_score(spec), lse=lse)
    torch.cuda.synchronize()
    O, L = fo.attention(q, k, v, C.oracle_mask(spec), C.oracle_score(spec, H))
    C.compare(gen.bf16_bits_to_f32(gen.from_torch_bf16(out)), O, f"every tile {mask}")
    C.compare_lse(lse.cpu().numpy(), L, f"every tile {mask}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask,score,dense", [("none", "alibi", False), ("prefix_lm", "softcap", False),
                                              ("none", "rel_pos", True)])
def test_block_lists_longer_than_the_register_window(mask, score, dense, D):
    """Rows that list 157 tiles (prefix_lm with prefix 20000) or 258 (no mask, and
    the dense path, Skv = 33000 with a ragged last tile).  The forward keeps 64
    list entries in one register and slides that window along the row: here 2
    and 4 times."""
    run_case(80 + D, mask, score, 1, 2, 1, 256, 33000, D, dense=dense, prefix=20000)


@pytest.mark.parametrize("per_head_mask", [False, True])
@pytest.mark.parametrize("mask", ["document_causal", "document", "causal", "prefix_lm"])
def test_work_order_of_query_tiles(mask, per_head_mask):
    """With the BlockMask's q_order (B*Hq a multiple of 8: each XCD starts the
    heaviest query tiles of all its heads first) the forward matches the oracle
    and is bit-identical to the natural order, since the order only moves
    workgroups.  Ragged tiles, per-batch and per-head BlockMask rows."""
    got, _ = run_case(50, mask, "alibi", 2, 8, 2, 700, 700, 64, per_head_mask=per_head_mask, order=True)
    nat, _ = run_case(50, mask, "alibi", 2, 8, 2, 700, 700, 64, per_head_mask=per_head_mask, order=False)
    assert np.array_equal(got, nat)


def test_work_order_with_staged_bias_d128():
    got, _ = run_case(51, "document_causal", "bias", 1, 8, 8, 520, 520, 128, order=True)
    nat, _ = run_case(51, "document_causal", "bias", 1, 8, 8, 520, 520, 128, order=False)
    assert np.array_equal(got, nat)


@pytest.mark.parametrize("score", ["none", "alibi", "bias"])
def test_dense_without_blockmask(score):
    run_case(31, "none", score, 1, 4, 4, 250, 250, 128, dense=True)


def test_per_head_blockmask_and_gqa8():
    run_case(32, "causal", "rel_pos", 1, 8, 1, 260, 260, 128, per_head_mask=True)


def test_explicit_alibi_slopes_and_broadcast_bias():
    run_case(33, "causal", "alibi", 2, 4, 2, 270, 270, 64, explicit_slopes=True)
    run_case(34, "causal", "bias", 2, 4, 2, 270, 270, 64, bias_broadcast=True)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask,Sq,Skv", [("causal", 392, 392), ("none", 264, 392), ("document_causal", 256, 256),
                                         ("sliding_window", 392, 264)])
def test_bias_staged_through_lds(mask, Sq, Skv, D):
    # Skv a multiple of 8 and 16-byte aligned rows: the bias tile goes through
    # LDS (ragged query and key tiles included); the same result as the oracle.
    run_case(40 + D, mask, "bias", 2, 2, 1, Sq, Skv, D)
    run_case(41 + D, mask, "bias", 1, 2, 2, Sq, Skv, D, bias_broadcast=True)


@pytest.mark.parametrize("D", [64, 128])
def test_strided_views_and_custom_scale(D):
    """Q, K, V and O as [B,H,S,D] views of [B,S,H,D] buffers (the layout a fused
    projection produces), with a softmax scale other than 1/sqrt(D)."""
    import torch
    from block_sparse_attention_fa_amd import fa
    B, Hq, Hkv, S, scale = 2, 4, 2, 300, 0.05
    print(f"[case] strided views D={D} scale={scale}", flush=True)
    q, k, v = gen.qkv(61, B, Hq, Hkv, S, S, D)

    def bshd_view(x):  # same values, stored as [B,S,H,D]
        return gen.to_torch_bf16(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)

    qt, kt, vt = bshd_view(q), bshd_view(k), bshd_view(v)
    assert not qt.is_contiguous() and qt.stride(2) == Hq * D
    out = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    bm = fa.fa_build_block_mask(fa.MaskMod("causal"), 1, 1, S, S)
    fa.fa_forward(qt, kt, vt, block_mask=bm, score=fa.ScoreMod("alibi"), scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    got = gen.bf16_bits_to_f32(gen.from_torch_bf16(out))
    O, L = fo.attention(q, k, v, fo.causal(), fo.alibi(fo.default_alibi_slopes(Hq)), scale=scale)
    C.compare(got, O, "strided views")
    C.compare_lse(lse.cpu().numpy(), L, "strided views")


def test_fully_masked_rows_are_zero_with_neg_inf_lse():
    # kv_len = 0 for a batch row: every row of it is empty
    import torch
    from block_sparse_attention_fa_amd import fa
    B, H, S, D = 2, 2, 200, 64
    q, k, v = gen.qkv(35, B, H, H, S, S, D)
    lens = np.array([0, 150], dtype=np.int32)
    spec = {"mask": "kv_len", "lens": lens, "score": "none"}
    bm = fa.fa_build_block_mask(C.gpu_mask(spec), B, 1, S, S)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    out = fa.fa_forward(*(gen.to_torch_bf16(x) for x in (q, k, v)), block_mask=bm, lse=lse)
    torch.cuda.synchronize()
    o = gen.bf16_bits_to_f32(gen.from_torch_bf16(out))
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0].cpu().numpy()))
    O, _ = fo.attention(q, k, v, fo.kv_length(lens))
    C.compare(o, O, "kv_len rows")


def test_closed_forms_on_gpu():
    # uniform V -> constant output; causal row 0 -> V[0]; window 0 -> V
    import torch
    from block_sparse_attention_fa_amd import fa
    B, H, S, D = 1, 2, 384, 128
    q, k, v = gen.qkv(36, B, H, H, S, S, D)
    c = gen.f32_to_bf16_bits(np.linspace(-1, 1, D).astype(np.float32))
    vu = np.broadcast_to(c, v.shape).copy()
    bm = fa.fa_build_block_mask(fa.MaskMod("causal"), 1, 1, S, S)
    out = fa.fa_forward(gen.to_torch_bf16(q), gen.to_torch_bf16(k), gen.to_torch_bf16(vu), block_mask=bm,
                        score=fa.ScoreMod("alibi"))
    o = gen.bf16_bits_to_f32(gen.from_torch_bf16(out))
    assert np.abs(o - gen.bf16_bits_to_f32(c)).max() <= 2 ** -7
    out = fa.fa_forward(gen.to_torch_bf16(q), gen.to_torch_bf16(k), gen.to_torch_bf16(v), block_mask=bm)
    o = gen.from_torch_bf16(out)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    bm0 = fa.fa_build_block_mask(fa.MaskMod("sliding_causal", window=0), 1, 1, S, S)
    out = fa.fa_forward(gen.to_torch_bf16(q), gen.to_torch_bf16(k), gen.to_torch_bf16(v), block_mask=bm0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gen.from_torch_bf16(out), v)


def test_deterministic_repeat():
    import torch
    from block_sparse_attention_fa_amd import fa
    B, H, S, D = 1, 4, 1024, 128
    q, k, v = (gen.to_torch_bf16(x) for x in gen.qkv(37, B, H, H, S, S, D))
    bm = fa.fa_build_block_mask(fa.MaskMod("causal"), 1, 1, S, S)
    o1 = fa.fa_forward(q, k, v, block_mask=bm, score=fa.ScoreMod("softcap", softcap=30.0))
    o2 = fa.fa_forward(q, k, v, block_mask=bm, score=fa.ScoreMod("softcap", softcap=30.0))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_invalid_arguments_raise():
    import torch
    from block_sparse_attention_fa_amd import fa
    q = torch.zeros((1, 3, 128, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 128, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fa_forward(q, k, k)
    assert e.value.status == fa.FA_ERR_SHAPE
    q = torch.zeros((1, 2, 128, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fa_forward(q, q, q)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    bm = fa.fa_build_block_mask(fa.MaskMod("causal"), 1, 1, 256, 256)
    q = torch.zeros((1, 2, 200, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fa_forward(q, q, q, block_mask=bm)  # built for other lengths
    assert e.value.status == fa.FA_ERR_SHAPE


def _diagonal_scores(cap, S):
    """bf16 Q, K with one attended key per row (the diagonal) whose score is s_q, a
    dense grid over [-8 cap, 8 cap] plus points near 0: s_q = a_q + b_q with a_q, b_q
    bf16 (the residual of a_q), both multiplied by K = 1 in dims 0 and 1, so the
    fp32 product is exact.  Returns q, k bits [1,1,S,64] and s (fp64)."""
    grid = np.concatenate([np.linspace(-8 * cap, 8 * cap, S - 10),
                           [0.0, 1e-6, -1e-6, 1e-3, -1e-3, 0.1, -0.1, 1.0, -1.0, 2.5]])
    a = gen.f32_to_bf16_bits(grid.astype(np.float32))
    b = gen.f32_to_bf16_bits((grid - fo.bf16_to_f64(a)).astype(np.float32))
    s = fo.bf16_to_f64(a) + fo.bf16_to_f64(b)
    q = np.zeros((1, 1, S, 64), dtype=np.uint16)
    k = np.zeros((1, 1, S, 64), dtype=np.uint16)
    q[0, 0, :, 0], q[0, 0, :, 1] = a, b
    k[0, 0, :, 0] = k[0, 0, :, 1] = 0x3F80   # 1.0
    return q, k, s


def _tanh_bound(cap, ref):
    # a few fp32 roundings of cap * log2(e) * (1 - 2 / (1 + e^(2s/cap))) and of the LSE
    return cap * 2.0 ** -19 + np.abs(ref) * 2.0 ** -21


@pytest.mark.parametrize("cap", [30.0, 50.0, 1.0])
def test_device_softcap_tanh_error_bound(cap):
    """The device tanh of the softcap score_mod against fp64 tanh (paper review
    §2.1 table, softcapping; an approximate tanh is allowed).  With the sliding
    window 0 every row attends its diagonal key alone, so the forward's LSE is
    that key's modded score cap * tanh(s / cap); with a one-key cache the same
    holds for decode."""
    import torch
    from block_sparse_attention_fa_amd import fa
    S = 4096
    q, k, s = _diagonal_scores(cap, S)
    ref = cap * np.tanh(s / cap)
    v = gen.qkv(90, 1, 1, 1, 1, S, 64)[2]
    qt, kt, vt = (gen.to_torch_bf16(x) for x in (q, k, v))
    bm = fa.fa_build_block_mask(fa.MaskMod("sliding_causal", window=0), 1, 1, S, S)
    lse = torch.empty((1, 1, S), dtype=torch.float32, device="cuda")
    fa.fa_forward(qt, kt, vt, block_mask=bm, score=fa.ScoreMod("softcap", softcap=cap), scale=1.0, lse=lse)
    torch.cuda.synchronize()
    got = lse[0, 0].cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    print(f"[tanh fwd cap={cap}] max abs {err.max():.3e} at s={s[err.argmax()]:.4g}, "
          f"max err / bound {(err / _tanh_bound(cap, ref)).max():.3f}", flush=True)
    assert np.all(err <= _tanh_bound(cap, ref))
    # decode: sequence b holds one key, q_b . k = s_b
    qd = q[0, 0][:, None, None, :]                     # [S, 1, 1, 64]
    kd = np.zeros((S, 1, 128, 64), dtype=np.uint16)
    kd[:, 0, 0, :] = k[0, 0, 0]
    lens = torch.ones(S, dtype=torch.int32, device="cuda")
    bmd = fa.fa_build_block_mask(fa.MaskMod("kv_len", kv_len=lens), S, 1, 1, 128)
    lsed = torch.empty((S, 1, 1), dtype=torch.float32, device="cuda")
    fa.fa_decode(gen.to_torch_bf16(qd), gen.to_torch_bf16(kd), gen.to_torch_bf16(kd), block_mask=bmd,
                 score=fa.ScoreMod("softcap", softcap=cap), scale=1.0, lse=lsed)
    torch.cuda.synchronize()
    gd = lsed[:, 0, 0].cpu().numpy().astype(np.float64)
    errd = np.abs(gd - ref)
    print(f"[tanh decode cap={cap}] max abs {errd.max():.3e}, max err / bound "
          f"{(errd / _tanh_bound(cap, ref)).max():.3f}", flush=True)
    assert np.all(errd <= _tanh_bound(cap, ref))
