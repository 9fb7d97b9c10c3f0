"""Memory discipline of the kernels and the binding.

Guard regions: every output (O, LSE, the BlockMask tensors, dQ/dK/dV) and every
workspace is placed inside a larger buffer filled with a NaN bit pattern, on
ragged, strided and paged cases; after the call the bytes around each output
must be unchanged (no write outside it) and the output itself must hold no NaN
(every element written), and the values must still match the oracle.

Streams: calls made on a side stream give the results of the same calls on the
default stream, while the default stream reuses freed memory meanwhile.
"""

import ctypes

import numpy as np
import pytest

from block_sparse_attention_fa_amd import inputs as gen
from oracle import flex_oracle as fo
from tests import _cases as C

pytestmark = pytest.mark.gpu

NAN16 = np.uint16(0x7FC1)       # a bf16 quiet NaN with a payload
NAN32 = np.uint32(0x7FC00011)   # an fp32 quiet NaN with a payload
GUARD32 = -7777                  # int32 guard value
G = 64                           # guard elements on each side of a 1-d region


def _bf16_guarded(shape, pad_rows=16, pad_cols=32):
    """A bf16 view of `shape` [B,H,S,D] inside a NaN-filled [B,H,S+3p,D+2c] buffer."""
    import torch
    B, H, S, D = shape
    buf = torch.from_numpy(np.full((B, H, S + 3 * pad_rows, D + 2 * pad_cols), NAN16).view(np.int16)).cuda()
    buf = buf.view(torch.bfloat16)
    view = buf[:, :, pad_rows:pad_rows + S, pad_cols:pad_cols + D]
    inside = np.zeros(buf.shape, dtype=bool)
    inside[:, :, pad_rows:pad_rows + S, pad_cols:pad_cols + D] = True
    return buf, view, inside


def _check_bf16_guard(buf, inside, what):
    bits = buf.view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    assert np.all(bits[~inside] == NAN16), f"{what}: bytes outside the output were written"
    vals = gen.bf16_bits_to_f32(bits[inside])
    assert not np.any(np.isnan(vals)), f"{what}: part of the output was not written"


def _f32_guarded(n):
    import torch
    buf = torch.from_numpy(np.full(n + 2 * G, NAN32).view(np.float32)).cuda()
    return buf, buf[G:G + n]


def _check_f32_guard(buf, n, what, inner_written=True):
    bits = buf.cpu().numpy().view(np.uint32)
    assert np.all(bits[:G] == NAN32) and np.all(bits[G + n:] == NAN32), f"{what}: guard bytes written"
    if inner_written:
        assert not np.any(bits[G:G + n] == NAN32), f"{what}: part of the output was not written"


def _guarded_block_mask(mask, Bm, Hm, Sq, Skv, separate_full=True, transposed=False):
    """A BlockMask whose index tensors sit inside int32 guard buffers."""
    import torch
    from block_sparse_attention_fa_amd import fa
    bm = fa.BlockMask(mask, Bm, Hm, Sq, Skv, separate_full, "cuda", transposed)
    bufs = {}
    for name, t in bm.tensors().items():
        buf = torch.full((t.numel() + 2 * G,), GUARD32, dtype=torch.int32, device="cuda")
        view = buf[G:G + t.numel()].view(t.shape)
        setattr(bm, name, view)
        setattr(bm.c, name, view.data_ptr())
        bufs[name] = (buf, t.numel())
    fa._check(fa.lib().fa_build_block_mask(ctypes.byref(bm.c), Sq, Skv, None))
    return bm, bufs


def _check_int_guards(bufs, what):
    for name, (buf, n) in bufs.items():
        h = buf.cpu().numpy()
        assert np.all(h[:G] == GUARD32) and np.all(h[G + n:] == GUARD32), f"{what}: guard of {name} written"
        assert not np.any(h[G:G + n] == GUARD32), f"{what}: {name} not fully written"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask,score,Sq,Skv", [("causal", "alibi", 300, 300), ("sliding_window", "softcap", 200, 333),
                                               ("document_causal", "bias", 264, 264), ("kv_len", "rel_pos", 333, 200)])
def test_forward_writes_only_its_outputs(mask, score, Sq, Skv, D):
    import torch
    from block_sparse_attention_fa_amd import fa
    B, Hq, Hkv = 2, 4, 2
    print(f"[case] guarded forward mask={mask} score={score} Sq={Sq} Skv={Skv} D={D}", flush=True)
    q, k, v = gen.qkv(95, B, Hq, Hkv, Sq, Skv, D)
    spec = C.make_spec(95, mask, score, B, Hq, Sq, Skv)
    Bm = B if mask in ("document_causal", "kv_len") else 1
    bm, bufs = _guarded_block_mask(C.gpu_mask(spec), Bm, 1, Sq, Skv, transposed=True)
    obuf, out, inside = _bf16_guarded((B, Hq, Sq, D))
    lbuf, lse = _f32_guarded(B * Hq * Sq)
    fa.fa_forward(*(gen.to_torch_bf16(x) for x in (q, k, v)), block_mask=bm, score=C.gpu_score(spec),
                  out=out, lse=lse.view(B, Hq, Sq))
    torch.cuda.synchronize()
    _check_int_guards(bufs, "block mask")
    _check_bf16_guard(obuf, inside, "O")
    _check_f32_guard(lbuf, B * Hq * Sq, "LSE")
    ref = fo.block_mask(C.oracle_mask(spec), Bm, 1, Sq, Skv)
    for name, t in bm.tensors().items():
        np.testing.assert_array_equal(t.cpu().numpy(), ref[name], err_msg=name)
    O, L = fo.attention(q, k, v, C.oracle_mask(spec), C.oracle_score(spec, Hq))
    C.compare(gen.bf16_bits_to_f32(gen.from_torch_bf16(out)), O, "guarded forward")
    C.compare_lse(lse.view(B, Hq, Sq).cpu().numpy(), L, "guarded forward")


@pytest.mark.parametrize("paged", [False, True])
def test_decode_writes_only_its_outputs_and_workspace(paged):
    import torch
    from block_sparse_attention_fa_amd import fa
    B, Hq, Hkv, KV, D = 3, 8, 2, 1000, 128
    print(f"[case] guarded decode paged={paged}", flush=True)
    q = gen.qkv(96, B, Hq, Hkv, 1, KV, D)[0]
    _, k, v = gen.qkv(97, B, Hkv, Hkv, 1, KV, D)
    lens = np.array([1000, 0, 129], dtype=np.int32)
    bm = fa.fa_build_block_mask(fa.MaskMod("kv_len", kv_len=torch.from_numpy(lens).cuda()), B, 1, 1, KV)
    sc = fa.ScoreMod("softcap", softcap=50.0)
    kt, vt, table = gen.to_torch_bf16(k), gen.to_torch_bf16(v), None
    if paged:   # one page per logical block, in reverse order
        nkb = -(-KV // 128)
        pad = nkb * 128 - KV
        kp = torch.nn.functional.pad(kt, (0, 0, 0, pad)).view(B, Hkv, nkb, 128, D).permute(0, 2, 1, 3, 4)
        vp = torch.nn.functional.pad(vt, (0, 0, 0, pad)).view(B, Hkv, nkb, 128, D).permute(0, 2, 1, 3, 4)
        kt = kp.reshape(B * nkb, Hkv, 128, D).flip(0).contiguous()
        vt = vp.reshape(B * nkb, Hkv, 128, D).flip(0).contiguous()
        table = torch.from_numpy((B * nkb - 1 - np.arange(B * nkb)).reshape(B, nkb).astype(np.int32)).cuda()
    qt = gen.to_torch_bf16(q)
    n = fa.fa_decode_workspace_size(qt, kt, vt, bm, sc, page_table=table) // 4
    wbuf, ws = _f32_guarded(n)
    obuf, out, inside = _bf16_guarded((B, Hq, 1, D))
    lbuf, lse = _f32_guarded(B * Hq)
    fa.fa_decode(qt, kt, vt, block_mask=bm, score=sc, out=out, lse=lse.view(B, Hq, 1), workspace=ws,
                 page_table=table)
    torch.cuda.synchronize()
    _check_bf16_guard(obuf, inside, "decode O")
    _check_f32_guard(lbuf, B * Hq, "decode LSE")
    _check_f32_guard(wbuf, n, "decode workspace", inner_written=False)
    O, L = fo.decode(q, k, v, lens, fo.softcap(50.0))
    C.compare(gen.bf16_bits_to_f32(gen.from_torch_bf16(out)), O, "guarded decode")
    C.compare_lse(lse.view(B, Hq).cpu().numpy(), L[..., 0], "guarded decode")


def test_backward_writes_only_its_gradients_and_workspace():
    import torch
    from block_sparse_attention_fa_amd import fa
    B, Hq, Hkv, S, D = 1, 4, 2, 300, 128
    print("[case] guarded backward", flush=True)
    q, k, v = gen.qkv(98, B, Hq, Hkv, S, S, D)
    dO = gen._normal_bf16([98, 30], (B, Hq, S, D), 1.0)
    qt, kt, vt, dOt = (gen.to_torch_bf16(x) for x in (q, k, v, dO))
    bm = fa.fa_build_block_mask(fa.MaskMod("causal"), 1, 1, S, S, transposed=True)
    sc = fa.ScoreMod("alibi")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    out = fa.fa_forward(qt, kt, vt, block_mask=bm, score=sc, lse=lse)
    n = fa.fa_backward_workspace_size(qt, kt, vt, out, lse, bm, sc) // 4
    wbuf, ws = _f32_guarded(n)
    bq, dq, iq = _bf16_guarded((B, Hq, S, D))
    bk, dk, ik = _bf16_guarded((B, Hkv, S, D))
    bv, dv, iv = _bf16_guarded((B, Hkv, S, D))
    fa.fa_backward(qt, kt, vt, out, lse, dOt, block_mask=bm, score=sc, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    for buf, inside, what in ((bq, iq, "dQ"), (bk, ik, "dK"), (bv, iv, "dV")):
        _check_bf16_guard(buf, inside, what)
    _check_f32_guard(wbuf, n, "backward workspace", inner_written=False)
    refs = fo.attention_backward(q, k, v, dO, fo.causal(), fo.alibi(fo.default_alibi_slopes(Hq)))
    for t, r, what in zip((dq, dk, dv), refs, ("dQ", "dK", "dV")):
        C.compare_grad(gen.bf16_bits_to_f32(gen.from_torch_bf16(t)), r, "guarded " + what)


def test_side_stream_calls_match_default_stream():
    """fa_forward, fa_decode and fa_backward on a side stream, with the binding
    allocating their outputs and workspaces, while the default stream allocates
    and overwrites memory of the same sizes: the results equal the same calls
    on the default stream."""
    import torch
    from block_sparse_attention_fa_amd import fa
    B, Hq, Hkv, S, D = 2, 4, 2, 1000, 128
    print("[case] side stream", flush=True)
    q, k, v = (gen.to_torch_bf16(x) for x in gen.qkv(99, B, Hq, Hkv, S, S, D))
    dO = gen.to_torch_bf16(gen._normal_bf16([99, 30], (B, Hq, S, D), 1.0))
    lens = torch.tensor([1000, 517], dtype=torch.int32, device="cuda")
    sc = fa.ScoreMod("alibi")
    bm = fa.fa_build_block_mask(fa.MaskMod("causal"), 1, 1, S, S, transposed=True)
    bmd = fa.fa_build_block_mask(fa.MaskMod("kv_len", kv_len=lens), B, 1, 1, S)
    qd = q[:, :, :1].contiguous()

    def run(stream):
        # the test's own buffer lives on the stream that uses it, as the binding's do
        with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
            lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
        o = fa.fa_forward(q, k, v, block_mask=bm, score=sc, lse=lse, stream=stream)
        od = fa.fa_decode(qd, k, v, block_mask=bmd, score=sc, stream=stream)
        grads = fa.fa_backward(q, k, v, o, lse, dO, block_mask=bm, score=sc, stream=stream)
        return (o, od) + tuple(grads)

    ref = run(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = run(side)
    # meanwhile the default stream takes and overwrites freed memory of every size the calls used
    junk = [torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
            for n in (B * Hq * S, B * Hq * 64 * (D + 1), 2 * B * Hq * 1024, B * Hq * S * D // 2)]
    side.synchronize()
    torch.cuda.synchronize()
    for a, b, what in zip(ref, got, ("O", "decode O", "dQ", "dK", "dV")):
        assert torch.equal(a, b), f"{what} differs on the side stream"
    del junk
