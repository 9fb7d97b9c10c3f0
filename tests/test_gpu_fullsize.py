"""Parity at the full workload sizes, through the same calls and launch
configuration that bench.py times (fa_build_block_mask + fa_forward, and
fa_decode with the automatic split plan).

For each forward workload every query row of two (b, h) pairs is compared
with the oracle (the whole [S, D] output of those heads, every q-tile and so
every list length), plus sampled rows of further heads: tile edges (rows
127/128/129), the first and last rows, document boundaries where the mask has
them, and seeded random rows.  Every one of the 1024 decode rows is compared.
Tolerance: max abs 2e-2 and mean abs 2e-3 over all compared elements; LSE
within 2e-3 + 1e-5 |LSE| (the fp32 row-sum bound).
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from block_sparse_attention_fa_amd import inputs as gen
from oracle import flex_oracle as fo
from tests import _cases as C

pytestmark = pytest.mark.gpu


def _sample_rows(seed, S, n_random, extra=()):
    rng = np.random.default_rng([seed, 99])
    rows = {0, 1, 127, 128, 129, S // 2, S - 129, S - 128, S - 1}
    rows |= {int(r) for r in extra}
    rows |= {int(r) for r in rng.integers(0, S, size=n_random)}
    return np.array(sorted(r for r in rows if 0 <= r < S), dtype=np.int64)


def _heads(seed, B, H, n):
    rng = np.random.default_rng([seed, 98])
    pairs = {(0, 0), (B - 1, H - 1)}
    while len(pairs) < min(n, B * H):
        pairs.add((int(rng.integers(0, B)), int(rng.integers(0, H))))
    return sorted(pairs)


def _check_rows(out, lse, q, k, v, checks, mask, score, what):
    """checks: list of ((b, h), rows).  Compares those rows of out / lse with the
    oracle, 1024 rows at a time; max and mean abs error over every compared element."""
    import torch
    torch.cuda.synchronize()
    n, err_sum, mx, lse_err = 0, 0.0, 0.0, 0.0
    for (b, h), rows in checks:
        for r0 in range(0, rows.size, 1024):
            rr = rows[r0:r0 + 1024]
            got = gen.bf16_bits_to_f32(gen.from_torch_bf16(out[b, h, torch.from_numpy(rr).to(out.device)]))
            O, L = fo.attention_rows(q, k, v, b, h, rr, mask, score)
            assert np.all(np.isfinite(got)), f"{what}: non-finite output at (b={b}, h={h})"
            e = np.abs(got.astype(np.float64) - O)
            n += e.size
            err_sum += float(e.sum())
            mx = max(mx, float(e.max()))
            lse_err = max(lse_err, C.compare_lse(lse[b, h].cpu().numpy()[rr], L, what))
    mean = err_sum / n
    print(f"[{what}] {sum(r.size for _, r in checks)} rows over {len(checks)} (b,h): max abs {mx:.3e}, "
          f"mean abs {mean:.3e}, lse abs {lse_err:.2e}", flush=True)
    assert mx <= C.TOL_MAX and mean <= C.TOL_MEAN, f"{what}: max abs {mx:.3e}, mean abs {mean:.3e}"


def _whole_and_sampled(seed, B, H, S, n_sampled_heads, rows):
    """Every row of (0, 0) and (B-1, H-1), and the sampled rows of other heads."""
    whole = [((0, 0), np.arange(S)), ((B - 1, H - 1), np.arange(S))]
    others = [bh for bh in _heads(seed, B, H, n_sampled_heads + 2) if bh not in ((0, 0), (B - 1, H - 1))]
    return whole + [(bh, rows) for bh in others]


def _forward(q, k, v, mask_mod, score_mod, Bm, S):
    import torch
    from block_sparse_attention_fa_amd import fa
    qt, kt, vt = (gen.to_torch_bf16(x) for x in (q, k, v))
    B, H = q.shape[0], q.shape[1]
    bm = fa.fa_build_block_mask(mask_mod, Bm, 1, S, S)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    out = fa.fa_forward(qt, kt, vt, block_mask=bm, score=score_mod, lse=lse)
    return out, lse


def test_causal_alibi_B4_H16_S8192_D128():
    from block_sparse_attention_fa_amd import fa
    B, H, S, D = 4, 16, 8192, 128
    print(f"[case] causal+alibi B{B} H{H} S{S} D{D}", flush=True)
    q, k, v = gen.qkv(2, B, H, H, S, S, D)
    out, lse = _forward(q, k, v, fa.MaskMod("causal"), fa.ScoreMod("alibi"), 1, S)
    _check_rows(out, lse, q, k, v, _whole_and_sampled(2, B, H, S, 4, _sample_rows(2, S, 24)),
                fo.causal(), fo.alibi(fo.default_alibi_slopes(H)), "causal+alibi 8192")


def test_sliding_causal_softcap_B2_H16_S16384_D128():
    from block_sparse_attention_fa_amd import fa
    B, H, S, D, W = 2, 16, 16384, 128, 1024
    print(f"[case] sliding_causal W{W} + softcap30 B{B} H{H} S{S} D{D}", flush=True)
    q, k, v = gen.qkv(3, B, H, H, S, S, D)
    out, lse = _forward(q, k, v, fa.MaskMod("sliding_causal", window=W),
                        fa.ScoreMod("softcap", softcap=30.0), 1, S)
    rows = _sample_rows(3, S, 24, extra=(W - 1, W, W + 1, 1151, 1152))
    _check_rows(out, lse, q, k, v, _whole_and_sampled(3, B, H, S, 4, rows),
                fo.sliding_causal(W), fo.softcap(30.0), "sliding+softcap 16384")


class _BiasTable:
    """bias[b, h, q, kv] (bf16 bits) of the checked heads, regenerated on the host
    from the seeded per-row-block streams of the input module."""

    def __init__(self, wid, heads, S):
        self.tab = {(b, h): gen.bias_slice(wid, b, h, S, S) for b, h in heads}

    def __getitem__(self, idx):
        b, h, q, kv = idx
        return self.tab[(int(b), int(h))][q, kv]


def _bias_on_gpu(wid, B, H, S):
    import torch
    t = torch.empty((B, H, S, S), dtype=torch.bfloat16, device="cuda")

    def fill(bh):
        b, h = divmod(bh, H)
        t[b, h].copy_(gen.to_torch_bf16(gen.bias_slice(wid, b, h, S, S, threads=1), device=None))

    with ThreadPoolExecutor(16) as ex:
        list(ex.map(fill, range(B * H)))
    return t


def test_document_causal_bias_B1_H32_S16384_D64():
    import torch
    from block_sparse_attention_fa_amd import fa
    B, H, S, D = 1, 32, 16384, 64
    print(f"[case] document_causal + bias[B,H,S,S] B{B} H{H} S{S} D{D}", flush=True)
    q, k, v = gen.qkv(4, B, H, H, S, S, D)
    docs = gen.document_ids(4, B, S)
    bias_t = _bias_on_gpu(4, B, H, S)
    mask = fa.MaskMod("document_causal", doc_ids=torch.from_numpy(docs).cuda())
    out, lse = _forward(q, k, v, mask, fa.ScoreMod("bias", bias=bias_t), B, S)
    del bias_t
    torch.cuda.empty_cache()
    starts = np.flatnonzero(np.diff(docs[0])) + 1          # first row of each later document
    rows = _sample_rows(4, S, 16, extra=np.concatenate([starts, starts - 1, starts + 1]))
    checks = _whole_and_sampled(4, B, H, S, 2, rows)
    _check_rows(out, lse, q, k, v, checks, fo.document_causal(docs),
                fo.bias(_BiasTable(4, [bh for bh, _ in checks], S)), "document+bias 16384")


def test_backward_causal_alibi_B4_H16_S8192_D128():
    """dQ on sampled query rows and dK, dV on sampled key rows of the forward
    workload, through fa_build_block_mask(transposed) + fa_forward + fa_backward."""
    import torch
    from block_sparse_attention_fa_amd import fa
    B, H, S, D = 4, 16, 8192, 128
    print(f"[case] backward causal+alibi B{B} H{H} S{S} D{D}", flush=True)
    q, k, v = gen.qkv(2, B, H, H, S, S, D)
    dO = gen._normal_bf16([2, 30], (B, H, S, D), 1.0)
    qt, kt, vt, dOt = (gen.to_torch_bf16(x) for x in (q, k, v, dO))
    bm = fa.fa_build_block_mask(fa.MaskMod("causal"), 1, 1, S, S, transposed=True)
    sc = fa.ScoreMod("alibi")
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    out = fa.fa_forward(qt, kt, vt, block_mask=bm, score=sc, lse=lse)
    dq, dk, dv = fa.fa_backward(qt, kt, vt, out, lse, dOt, block_mask=bm, score=sc)
    torch.cuda.synchronize()
    mask, score = fo.causal(), fo.alibi(fo.default_alibi_slopes(H))
    rows = _sample_rows(2, S, 12)
    got_q, ref_q = [], []
    for b, h in _heads(2, B, H, 3):
        got_q.append(gen.bf16_bits_to_f32(gen.from_torch_bf16(dq[b, h, torch.from_numpy(rows).cuda()])))
        ref_q.append(fo.attention_backward_q_rows(q, k, v, dO, b, h, rows, mask, score))
    C.compare_grad(np.concatenate(got_q), np.concatenate(ref_q), "dQ 8192 sampled rows")
    kv_rows = np.array(sorted({0, 127, 128, 4095, S - 129, S - 1} | set(np.random.default_rng([2, 97]).integers(0, S, 4).tolist())))
    got_k, got_v, ref_k, ref_v = [], [], [], []
    for b, h in ((0, 0), (B - 1, H - 1)):
        idx = torch.from_numpy(kv_rows).cuda()
        got_k.append(gen.bf16_bits_to_f32(gen.from_torch_bf16(dk[b, h, idx])))
        got_v.append(gen.bf16_bits_to_f32(gen.from_torch_bf16(dv[b, h, idx])))
        gk, gv = fo.attention_backward_kv_rows(q, k, v, dO, b, h, kv_rows, mask, score)
        ref_k.append(gk)
        ref_v.append(gv)
    C.compare_grad(np.concatenate(got_k), np.concatenate(ref_k), "dK 8192 sampled rows")
    C.compare_grad(np.concatenate(got_v), np.concatenate(ref_v), "dV 8192 sampled rows")


def test_decode_B32_Hq32_Hkv8_KV32768_softcap50():
    """Every one of the 32 x 32 decode rows against the oracle."""
    import torch
    from block_sparse_attention_fa_amd import fa
    B, Hq, Hkv, D, KV = 32, 32, 8, 128, 32768
    print(f"[case] decode B{B} Hq{Hq} Hkv{Hkv} KV{KV} D{D} softcap50 auto splits", flush=True)
    qd = gen.qkv(5, B, Hq, Hkv, 1, 1, D)[0]
    _, kc, vc = gen.qkv(105, B, Hkv, Hkv, 1, KV, D)
    lens = gen.kv_lengths(5, B, 4096, 32768)
    bm = fa.fa_build_block_mask(fa.MaskMod("kv_len", kv_len=torch.from_numpy(lens).cuda()), B, 1, 1, KV)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
    out = fa.fa_decode(gen.to_torch_bf16(qd), gen.to_torch_bf16(kc), gen.to_torch_bf16(vc), block_mask=bm,
                       score=fa.ScoreMod("softcap", softcap=50.0), lse=lse)
    torch.cuda.synchronize()
    got = gen.bf16_bits_to_f32(gen.from_torch_bf16(out)).astype(np.float64)
    gl = lse.cpu().numpy().astype(np.float64)
    O = np.zeros((B, Hq, 1, D))
    L = np.zeros((B, Hq, 1))
    for b in range(B):   # the caches of one sequence widened once, then every query head
        O[b:b + 1], L[b:b + 1] = fo.decode(qd[b:b + 1], fo.bf16_to_f64(kc[b:b + 1]), fo.bf16_to_f64(vc[b:b + 1]),
                                           lens[b:b + 1], fo.softcap(50.0))
    lse_err = C.compare_lse(gl[..., 0], L[..., 0], "decode")
    mx, mean = C.compare(got, O, "decode full")
    print(f"[decode full] {B * Hq} rows: max abs {mx:.3e}, mean abs {mean:.3e}, lse abs {lse_err:.2e}", flush=True)
