"""Split-KV decode vs the oracle, split-count invariance and decode == forward at Sq = 1."""

import numpy as np
import pytest

from block_sparse_attention_fa_amd import inputs as gen
from oracle import flex_oracle as fo
from tests import _cases as C

pytestmark = pytest.mark.gpu


def _decode(q, k, v, lens, score, num_splits=0, Bm=None, extra=None, order=None):
    import torch
    from block_sparse_attention_fa_amd import fa
    B, KV = k.shape[0], k.shape[2]
    bm = fa.fa_build_block_mask(fa.MaskMod("kv_len", kv_len=torch.from_numpy(lens).cuda()), B, 1, 1, KV, order=order)
    lse = torch.empty((B, q.shape[1], 1), dtype=torch.float32, device="cuda")
    out = fa.fa_decode(gen.to_torch_bf16(q), gen.to_torch_bf16(k), gen.to_torch_bf16(v), block_mask=bm,
                       score=score, num_splits=num_splits, lse=lse)
    torch.cuda.synchronize()
    return gen.bf16_bits_to_f32(gen.from_torch_bf16(out)), lse.cpu().numpy()


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("score", ["none", "softcap", "alibi", "bias"])
def test_decode_matches_oracle(G, D, score):
    from block_sparse_attention_fa_amd import fa
    print(f"[case] decode G={G} D={D} score={score}", flush=True)
    B, Hkv, KV = 3, 2, 1500
    Hq = G * Hkv
    q = gen.qkv(40 + G, B, Hq, Hkv, 1, KV, D)[0]
    _, k, v = gen.qkv(41 + G, B, Hkv, Hkv, 1, KV, D)
    lens = np.array([1500, 700, 129], dtype=np.int32)
    spec = C.make_spec(42, "kv_len", score, B, Hq, 1, KV, cap=50.0)
    spec["lens"] = lens
    got, lse = _decode(q, k, v, lens, C.gpu_score(spec))
    O, L = fo.decode(q, k, v, lens, C.oracle_score(spec, Hq))
    C.compare(got, O, f"decode G={G} D={D} {score}")
    C.compare_lse(lse[..., 0], L[..., 0], "decode")


def test_decode_row_order():
    """With the BlockMask's row order fa_decode starts the longest sequences first;
    output and LSE are bit-identical to the grid's own order, and match the oracle."""
    from block_sparse_attention_fa_amd import fa
    B, Hq, Hkv, KV, D = 6, 8, 2, 3000, 128
    q = gen.qkv(60, B, Hq, Hkv, 1, KV, D)[0]
    _, k, v = gen.qkv(61, B, Hkv, Hkv, 1, KV, D)
    lens = np.array([129, 3000, 1, 2048, 700, 2999], dtype=np.int32)
    sc = fa.ScoreMod("softcap", softcap=50.0)
    a, la = _decode(q, k, v, lens, sc, order=True)
    b, lb = _decode(q, k, v, lens, sc, order=False)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    O, L = fo.decode(q, k, v, lens, fo.softcap(50.0))
    C.compare(a, O, "decode with row order")
    C.compare_lse(la[..., 0], L[..., 0], "decode with row order")


def test_split_count_invariance_and_forward_equivalence():
    import torch
    from block_sparse_attention_fa_amd import fa
    B, Hq, Hkv, KV, D = 4, 8, 2, 5000, 128
    q = gen.qkv(50, B, Hq, Hkv, 1, KV, D)[0]
    _, k, v = gen.qkv(51, B, Hkv, Hkv, 1, KV, D)
    lens = np.array([5000, 1, 4097, 2500], dtype=np.int32)
    sc = fa.ScoreMod("softcap", softcap=50.0)
    outs = [_decode(q, k, v, lens, sc, n)[0] for n in (1, 3, 7, 40, 0)]
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2 ** -7  # one bf16 ulp at |O| < 1 at most
    O, _ = fo.decode(q, k, v, lens, fo.softcap(50.0))
    C.compare(outs[0], O, "decode splits")
    # fa_forward with Sq = 1 and the same BlockMask gives the same answer
    bm = fa.fa_build_block_mask(fa.MaskMod("kv_len", kv_len=torch.from_numpy(lens).cuda()), B, 1, 1, KV)
    of = fa.fa_forward(gen.to_torch_bf16(q), gen.to_torch_bf16(k), gen.to_torch_bf16(v), block_mask=bm, score=sc)
    torch.cuda.synchronize()
    C.compare(gen.bf16_bits_to_f32(gen.from_torch_bf16(of)), O, "forward Sq=1")


def test_decode_workspace_errors():
    import torch
    from block_sparse_attention_fa_amd import fa
    q = torch.zeros((1, 4, 1, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 1, 1024, 128), dtype=torch.bfloat16, device="cuda")
    n = fa.fa_decode_workspace_size(q, kv, kv)
    assert n > 0
    small = torch.empty(1, dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fa_decode(q, kv, kv, workspace=small)
    assert e.value.status == fa.FA_ERR_WORKSPACE
    q3 = torch.zeros((1, 3, 1, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fa_decode(q3, kv, kv)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED


def test_empty_sequence_strided_cache_and_scale():
    """A sequence with kv_len = 0 (every split empty: O = 0 and LSE = -inf), the
    caches as [B,H,KV,D] views of [B,KV,H,D] buffers, and a scale other than 1/sqrt(D)."""
    import torch
    from block_sparse_attention_fa_amd import fa
    B, Hq, Hkv, KV, D, scale = 3, 8, 2, 1300, 128, 0.07
    print(f"[case] decode empty sequence, strided caches, scale={scale}", flush=True)
    q = gen.qkv(55, B, Hq, Hkv, 1, KV, D)[0]
    _, k, v = gen.qkv(56, B, Hkv, Hkv, 1, KV, D)
    lens = np.array([900, 0, 1300], dtype=np.int32)

    def bshd_view(x):  # same values, stored as [B,KV,H,D]
        return gen.to_torch_bf16(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).permute(0, 2, 1, 3)

    kt, vt = bshd_view(k), bshd_view(v)
    assert not kt.is_contiguous()
    bm = fa.fa_build_block_mask(fa.MaskMod("kv_len", kv_len=torch.from_numpy(lens).cuda()), B, 1, 1, KV)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
    out = fa.fa_decode(gen.to_torch_bf16(q), kt, vt, block_mask=bm, score=fa.ScoreMod("softcap", softcap=50.0),
                       scale=scale, lse=lse)
    torch.cuda.synchronize()
    got = gen.bf16_bits_to_f32(gen.from_torch_bf16(out))
    gl = lse.cpu().numpy()
    O, L = fo.decode(q, k, v, lens, fo.softcap(50.0), scale=scale)
    C.compare(got, O, "decode strided")
    C.compare_lse(gl[..., 0], L[..., 0], "decode strided")
    assert np.all(got[1] == 0.0) and np.all(np.isneginf(gl[1]))


def _page_pools(k, v, lens, seed, share_first_page=False):
    """Scatter per-sequence caches [B,Hkv,KV,D] (bf16 bits) into shuffled page pools
    [P,Hkv,128,D] with a page table, the way a serving cache holds them: only the
    pages a sequence needs, in no particular order, with spare pages holding other
    data.  Returns the pools, the table and the logical caches the table
    describes (the oracle's input)."""
    B, Hkv, KV, D = k.shape
    nkb = -(-KV // 128)
    need = [-(-int(n) // 128) for n in lens]
    P = sum(need) + 3
    rng = np.random.default_rng([seed, 5])
    perm = rng.permutation(P)
    k_pool = gen._normal_bf16([seed, 6], (P, Hkv, 128, D), 1.0)   # spare pages: other finite data
    v_pool = gen._normal_bf16([seed, 7], (P, Hkv, 128, D), 1.0)
    table = np.full((B, nkb + 2), P + 1000, dtype=np.int32)       # entries past a sequence are never read
    i = 0
    for b in range(B):
        for j in range(need[b]):
            pg, rows = perm[i], min(128, KV - 128 * j)
            k_pool[pg, :, :rows] = k[b, :, 128 * j:128 * j + rows]
            v_pool[pg, :, :rows] = v[b, :, 128 * j:128 * j + rows]
            table[b, j] = pg
            i += 1
    if share_first_page:  # sequences 1.. reuse sequence 0's first page (a shared prompt prefix)
        table[1:, 0] = table[0, 0]
    k_log = np.zeros_like(k)
    v_log = np.zeros_like(v)
    for b in range(B):
        for j in range(need[b]):
            rows = min(128, KV - 128 * j)
            k_log[b, :, 128 * j:128 * j + rows] = k_pool[table[b, j], :, :rows]
            v_log[b, :, 128 * j:128 * j + rows] = v_pool[table[b, j], :, :rows]
    return k_pool, v_pool, table, k_log, v_log


@pytest.mark.parametrize("G,D,score", [(4, 128, "softcap"), (1, 64, "alibi"), (8, 128, "none")])
@pytest.mark.parametrize("share", [False, True])
def test_paged_decode(G, D, score, share):
    """Paged decode equals the oracle on the logical caches the page table
    describes, and equals contiguous decode on those caches bit for bit (same
    chunks, same arithmetic, only the row addresses differ)."""
    import torch
    from block_sparse_attention_fa_amd import fa
    print(f"[case] paged decode G={G} D={D} score={score} shared={share}", flush=True)
    B, Hkv, KV = 3, 2, 1500
    Hq = G * Hkv
    q = gen.qkv(80 + G, B, Hq, Hkv, 1, KV, D)[0]
    _, k, v = gen.qkv(81 + G, B, Hkv, Hkv, 1, KV, D)
    lens = np.array([1500, 700, 129], dtype=np.int32)
    k_pool, v_pool, table, k_log, v_log = _page_pools(k, v, lens, 90 + G, share)
    spec = C.make_spec(82, "kv_len", score, B, Hq, 1, KV, cap=50.0)
    spec["lens"] = lens
    sc = C.gpu_score(spec)
    bm = fa.fa_build_block_mask(fa.MaskMod("kv_len", kv_len=torch.from_numpy(lens).cuda()), B, 1, 1, KV)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
    qt = gen.to_torch_bf16(q)
    out = fa.fa_decode(qt, gen.to_torch_bf16(k_pool), gen.to_torch_bf16(v_pool), block_mask=bm, score=sc,
                       lse=lse, page_table=torch.from_numpy(table).cuda())
    lse_c = torch.empty_like(lse)
    out_c = fa.fa_decode(qt, gen.to_torch_bf16(k_log), gen.to_torch_bf16(v_log), block_mask=bm, score=sc, lse=lse_c)
    torch.cuda.synchronize()
    got = gen.bf16_bits_to_f32(gen.from_torch_bf16(out))
    O, L = fo.decode(q, k_log, v_log, lens, C.oracle_score(spec, Hq))
    C.compare(got, O, "paged decode")
    C.compare_lse(lse.cpu().numpy()[..., 0], L[..., 0], "paged decode")
    assert torch.equal(out, out_c) and torch.equal(lse, lse_c)


@pytest.mark.parametrize("score", ["alibi", "rel_pos", "softcap"])
def test_decode_at_query_positions(score):
    """The query of sequence b at position q_pos[b] (the newest token of its cache,
    or any other position): the score_mods see that q index, so ALiBi and the
    relative position shift every score of the row, which the LSE shows."""
    import torch
    from block_sparse_attention_fa_amd import fa
    B, Hq, Hkv, KV, D = 4, 8, 2, 1500, 128
    print(f"[case] decode at query positions, score={score}", flush=True)
    q = gen.qkv(57, B, Hq, Hkv, 1, KV, D)[0]
    _, k, v = gen.qkv(58, B, Hkv, Hkv, 1, KV, D)
    lens = np.array([1500, 700, 129, 1], dtype=np.int32)
    pos = np.array([1499, 699, 4000, 0], dtype=np.int32)
    spec = C.make_spec(59, "kv_len", score, B, Hq, 1, KV, cap=50.0)
    bm = fa.fa_build_block_mask(fa.MaskMod("kv_len", kv_len=torch.from_numpy(lens).cuda()), B, 1, 1, KV)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
    out = fa.fa_decode(gen.to_torch_bf16(q), gen.to_torch_bf16(k), gen.to_torch_bf16(v), block_mask=bm,
                       score=C.gpu_score(spec), lse=lse, q_pos=torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    O, L = fo.decode(q, k, v, lens, C.oracle_score(spec, Hq), positions=pos)
    C.compare(gen.bf16_bits_to_f32(gen.from_torch_bf16(out)), O, f"decode q_pos {score}")
    C.compare_lse(lse.cpu().numpy()[..., 0], L[..., 0], f"decode q_pos {score}")
