"""fa_decode_noalloc, the decode entry point that allocates nothing (its split
partials live in the library's own per-GPU scratch), against fa_decode with a
caller workspace: the same kernels and plan, so the outputs must be identical.
Two calls in a row, the second with a smaller input, so a stale first call in
the shared scratch would show; and the size limit."""

import numpy as np
import pytest

from block_sparse_attention_fa_amd import inputs as gen
from oracle import flex_oracle as fo
from tests import _cases as C

pytestmark = pytest.mark.gpu


def _case(seed, B, Hq, Hkv, KV, D, lens, score, q_pos=None):
    import torch
    from block_sparse_attention_fa_amd import fa
    q = gen.qkv(seed, B, Hq, Hkv, 1, KV, D)[0]
    _, k, v = gen.qkv(seed + 1, B, Hkv, Hkv, 1, KV, D)
    lens = np.asarray(lens, dtype=np.int32)
    bm = fa.fa_build_block_mask(fa.MaskMod("kv_len", kv_len=torch.from_numpy(lens).cuda()), B, 1, 1, KV)
    qt, kt, vt = (gen.to_torch_bf16(x) for x in (q, k, v))
    qp = torch.from_numpy(np.asarray(q_pos, dtype=np.int32)).cuda() if q_pos is not None else None
    return q, k, v, lens, bm, qt, kt, vt, qp, score


def _run_both(case):
    import torch
    from block_sparse_attention_fa_amd import fa
    q, k, v, lens, bm, qt, kt, vt, qp, score = case
    B, Hq = q.shape[0], q.shape[1]
    lse_w = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
    lse_n = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
    out_w = fa.fa_decode(qt, kt, vt, block_mask=bm, score=score, lse=lse_w, q_pos=qp)
    out_n = torch.empty_like(qt)
    fa.fa_decode_noalloc(qt, kt, vt, block_mask=bm, score=score, out=out_n, lse=lse_n, q_pos=qp)
    torch.cuda.synchronize()
    return out_w, out_n, lse_w, lse_n


def test_noalloc_decode_equals_decode_twice_second_smaller():
    from block_sparse_attention_fa_amd import fa
    print("[case] fa_decode_noalloc: B8 Hq32 Hkv8 KV20000 softcap, then B3 Hq8 Hkv2 KV3000 alibi", flush=True)
    big = _case(61, 8, 32, 8, 20000, 128, [20000, 1, 7000, 12345, 0, 19999, 128, 4097],
                fa.ScoreMod("softcap", softcap=50.0))
    small = _case(63, 3, 8, 2, 3000, 64, [3000, 700, 129], fa.ScoreMod("alibi"), q_pos=[2999, 699, 5000])
    for case, what in ((big, "first call"), (small, "second call, smaller")):
        out_w, out_n, lse_w, lse_n = _run_both(case)
        assert torch_equal(out_w, out_n), f"{what}: outputs differ"
        assert torch_equal(lse_w, lse_n), f"{what}: LSEs differ"
        q, k, v, lens, _, _, _, _, qp, _ = case
        positions = None if qp is None else qp.cpu().numpy()
        sm = fo.softcap(50.0) if what == "first call" else fo.alibi(fo.default_alibi_slopes(q.shape[1]))
        O, L = fo.decode(q, k, v, lens, sm, positions=positions)
        C.compare(gen.bf16_bits_to_f32(gen.from_torch_bf16(out_n)), O, what)
        C.compare_lse(lse_n.cpu().numpy()[..., 0], L[..., 0], what)


def torch_equal(a, b):
    import torch
    return bool(torch.equal(a, b))


def test_noalloc_decode_rejects_work_beyond_its_scratch():
    import torch
    from block_sparse_attention_fa_amd import fa
    B, Hq, Hkv, KV, D = 64, 64, 8, 32768, 128          # 37 splits: 78 MB of partials
    q = torch.zeros((B, Hq, 1, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, Hkv, KV, D), dtype=torch.bfloat16, device="cuda")
    assert fa.fa_decode_workspace_size(q, kv, kv) > (32 << 20)
    with pytest.raises(fa.FAError) as e:
        fa.fa_decode_noalloc(q, kv, kv, out=torch.empty_like(q))
    assert e.value.status == fa.FA_ERR_WORKSPACE
