#!/usr/bin/env python3
"""Throughput of the block-sparse FlexAttention hot path on one MI355X.

One step = fa_build_block_mask + fa_forward on the causal + ALiBi workload
(B=4, H=16, S=8192, D=128, bf16 ~N(0,1); slopes 2^(-8(h+1)/16)); the reported
value is attended TFLOP/s (4*D per attended (b,h,q,kv) position).  The
split-KV decode (B=32, Hq=32, Hkv=8, D=128, KV cache 32768 with valid lengths
uniform in [4096, 32768], softcap 50) is timed in the same run and reported as
HBM GB/s.  Inputs are resident in HBM before timing starts.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 100]   (at least 30 untimed steps)
    python bench.py --ablation                              (block-skipping ablation, sparsity sweep)
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

FWD = dict(name="causal+alibi fwd B4 H16 S8192 D128 bf16", workload_id=2, B=4, H=16, S=8192, D=128)
DEC = dict(name="gqa4 split-kv decode B32 Hq32 Hkv8 D128 KV32768 softcap50 bf16", workload_id=5,
           B=32, Hq=32, Hkv=8, D=128, KV=32768, len_lo=4096, len_hi=32768, cap=50.0)

FWD_SOURCES = ["fwd_kernel.hpp", "mods.hpp", "fwd_causal.hip", "fa_internal.hpp"]
DEC_SOURCES = ["decode.hip", "mods.hpp", "fa_internal.hpp"]


def source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "block_sparse_attention_fa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(summary, files):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_sha = re.search(r"source_sha:\s*(\w+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_sha or not m_b or m_sha.group(1) != source_sha(files):
        return None
    return float(m_b.group(1))


def cpu_baseline(q, k, v, seconds):
    """The fp64 oracle on host cores, on (b, h, 1024-row) chunks of the forward
    workload taken from the last rows backwards until `seconds` have elapsed."""
    import numpy as np
    from oracle import flex_oracle as fo
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    B, H, S, D = FWD["B"], FWD["H"], FWD["S"], FWD["D"]
    mask, score = fo.causal(), fo.alibi(fo.default_alibi_slopes(H))
    chunks, flops = [], 0.0
    t0 = time.perf_counter()
    for b in range(B):
        for h in range(H):
            for r1 in range(S, 0, -1024):
                rows = np.arange(max(0, r1 - 1024), r1)
                fo.attention_rows(q, k, v, b, h, rows, mask, score)
                flops += 4.0 * D * float((rows + 1).sum())  # causal: row q attends q+1 keys
                chunks.append((b, h, int(rows[0])))
                if time.perf_counter() - t0 >= seconds:
                    break
            else:
                continue
            break
        else:
            continue
        break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(chunks)} chunks of 1024 query rows x all 8192 keys (fp64, dense) of the "
                      f"causal+ALiBi S=8192 workload, (b,h) in order from (0,0), rows from the end back; {dt:.1f} s; "
                      f"host cpu_count={os.cpu_count()}"}


def run_ablation(steps):
    """Block-skipping ablation and a sparsity sweep on the causal + ALiBi forward
    workload (B4 H16 S8192 D128): what skipping empty tiles and running full
    tiles without the mask_mod save, and how the time follows the fraction of
    non-empty tiles (sliding-window widths).  Each entry is the best of three
    timed runs of `steps` calls.  Prints one JSON line."""
    import torch
    from block_sparse_attention_fa_amd import fa
    from block_sparse_attention_fa_amd import inputs as gen
    fa.lib()
    B, H, S, D = FWD["B"], FWD["H"], FWD["S"], FWD["D"]
    q, k, v = gen.qkv(FWD["workload_id"], B, H, H, S, S, D)
    qt, kt, vt = (gen.to_torch_bf16(x) for x in (q, k, v))
    out = torch.empty_like(qt)
    score = fa.ScoreMod("alibi")

    def time_fwd(bm):
        for _ in range(3):
            fa.fa_forward(qt, kt, vt, block_mask=bm, score=score, out=out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fa.fa_forward(qt, kt, vt, block_mask=bm, score=score, out=out)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def entry(bm, n_att):
        ms = min(time_fwd(bm) for _ in range(3))
        cls = bm.classes() if bm.separate_full else None
        listed = int(bm.kv_num_blocks.sum().item()) + (int(bm.full_kv_num_blocks.sum().item()) if bm.separate_full else 0)
        e = {"ms": round(ms, 4), "attended_tflops": round(4.0 * D * n_att / (ms * 1e-3) / 1e12, 2),
             "tiles_visited": listed,
             "executed_tile_tflops": round(4.0 * D * 128 * 128 * listed * B * H / (ms * 1e-3) / 1e12, 2)}
        if cls is not None:
            e["tiles_partial"], e["tiles_full"] = int((cls == 1).sum()), int((cls == 2).sum())
        return e

    n_causal = B * H * S * (S + 1) // 2
    causal = fa.MaskMod("causal")
    warm = fa.fa_build_block_mask(causal, 1, 1, S, S)
    for _ in range(30):  # clocks and caches settle before the first timed mode
        fa.fa_forward(qt, kt, vt, block_mask=warm, score=score, out=out)
    modes = {
        "skip_empty__mask_on_partial_only": entry(fa.fa_build_block_mask(causal, 1, 1, S, S), n_causal),
        "skip_empty__mask_on_every_tile": entry(fa.fa_build_block_mask(causal, 1, 1, S, S, separate_full=False),
                                                n_causal),
        "no_skipping__mask_on_every_tile": entry(
            fa.fa_build_block_mask(causal, 1, 1, S, S, separate_full=False).list_every_tile(), n_causal),
    }
    sweep = []
    for W in (256, 1024, 2048, 4096, S - 1):
        bm = fa.fa_build_block_mask(fa.MaskMod("sliding_causal", window=W), 1, 1, S, S)
        n_att = B * H * (W * (W + 1) // 2 + (S - W) * (W + 1))   # row q attends min(q, W) + 1 keys
        e = entry(bm, n_att)
        e["window"] = W
        e["nonempty_tile_frac"] = round((e["tiles_partial"] + e["tiles_full"]) / float(bm.NQ * bm.NK), 4)
        sweep.append(e)
    print(json.dumps({"ablation": {"workload": FWD["name"], "steps": steps, "modes": modes,
                                   "sliding_causal_window_sweep": sweep}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--ablation", action="store_true",
                    help="only time the block-skipping ablation and the sliding-window sparsity sweep")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain fp16->bf16 copies of MIB MiB each (reads MIB MiB, writes "
                         "MIB MiB): the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU only: the library has no multi-GPU path "
                  "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if args.copy_calibration > 0:
        n = args.copy_calibration << 19  # 2-byte elements
        src = torch.zeros(n, dtype=torch.float16, device="cuda:0")
        dst = torch.empty(n, dtype=torch.bfloat16, device="cuda:0")
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"kernel": "fp16->bf16 elementwise copy", "launches": 5,
                                               "read_bytes_per_launch": 2 * n,
                                               "write_bytes_per_launch": 2 * n}}), flush=True)
        return
    if args.ablation:
        run_ablation(args.steps)
        return
    from block_sparse_attention_fa_amd import fa
    from block_sparse_attention_fa_amd import inputs as gen

    fa.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    dev = "cuda:0"

    # ---------------- forward workload ----------------
    B, H, S, D = FWD["B"], FWD["H"], FWD["S"], FWD["D"]
    print(f"[bench] generating {FWD['name']}", file=sys.stderr, flush=True)
    q, k, v = gen.qkv(FWD["workload_id"], B, H, H, S, S, D)
    qt, kt, vt = (gen.to_torch_bf16(x, dev) for x in (q, k, v))
    out = torch.empty_like(qt)
    mask, score = fa.MaskMod("causal"), fa.ScoreMod("alibi")
    bm = fa.BlockMask(mask, 1, 1, S, S, device=dev)
    stream = torch.cuda.current_stream()
    L = fa.lib()
    import ctypes
    args_c = fa._attn_args(qt, kt, vt, out, None, bm, score, 0.0, 0)
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def step(ev=None):
        fa._check(L.fa_build_block_mask(ctypes.byref(bm.c), S, S, sptr))
        if ev is not None:
            ev[0].record(stream)
        fa._check(L.fa_forward(ctypes.byref(args_c), sptr))
        if ev is not None:
            ev[1].record(stream)

    # At least 30 untimed steps: the GPU needs about that many calls (tens of ms of
    # continuous work) to reach its steady clock; with 3 the timed steps run
    # about 10% slower than in steady operation.
    fwd_settle = max(30, args.warmup)
    for _ in range(fwd_settle):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = (t1 - t0) * 1e3 / args.steps
    fwd_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps

    # block mask build alone
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        fa._check(L.fa_build_block_mask(ctypes.byref(bm.c), S, S, sptr))
    e1.record(stream)
    torch.cuda.synchronize()
    build_ms = e0.elapsed_time(e1) / 10
    cls = bm.classes()
    n_part, n_full = int((cls == 1).sum()), int((cls == 2).sum())

    n_att = B * H * S * (S + 1) // 2               # causal: row q attends q+1 keys
    att_flops = 4.0 * D * n_att
    exec_flops = 4.0 * D * 128 * 128 * (n_part + n_full) * B * H
    alg_bytes = 4 * B * H * S * D * 2               # Q, K, V, O once each
    fwd_tflops = att_flops / (fwd_ms * 1e-3) / 1e12
    value = att_flops / (step_ms * 1e-3) / 1e12
    traffic = read_traffic("fwd_causal_alibi_8192_traffic.md", FWD_SOURCES)

    result = {
        "metric": "fwd attended TFLOP/s & % bf16 MFMA peak; decode HBM GB/s (1 MI355X)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": fwd_settle, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": FWD["name"], "B": B, "H": H, "S": S, "D": D, "mask": "causal",
                   "score_mod": "alibi", "block": 128, "step": "fa_build_block_mask + fa_forward"},
        "fwd": {"kernel_ms": round(fwd_ms, 4), "attended_tflops": round(fwd_tflops, 2),
                "frac_bf16_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
                "executed_tile_tflops": round(exec_flops / (fwd_ms * 1e-3) / 1e12, 2),
                "tiles_partial": n_part, "tiles_full": n_full, "blockmask_build_ms": round(build_ms, 4),
                "sparsity_pct": round(100.0 * float((cls == 0).sum()) / cls.size, 3)},
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "algorithmic_bytes": alg_bytes,
                     "kernel": "fwd_kernel<128, MaskCausal, ScoreAlibi>"},
    }

    # ---------------- backward of the same workload ----------------
    if not args.no_backward:
        print("[bench] backward", file=sys.stderr, flush=True)
        bmt = fa.fa_build_block_mask(mask, 1, 1, S, S, device=dev, transposed=True)
        lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
        fa.fa_forward(qt, kt, vt, block_mask=bmt, score=score, out=out, lse=lse)
        dot = gen.to_torch_bf16(gen._normal_bf16([FWD["workload_id"], 30], (B, H, S, D)), dev)
        dq, dk, dv = torch.empty_like(qt), torch.empty_like(kt), torch.empty_like(vt)
        wsb = torch.empty(fa.fa_backward_workspace_size(qt, kt, vt, out, lse, bmt, score) // 4 + 4,
                          dtype=torch.float32, device=dev)

        def bwd():
            fa.fa_backward(qt, kt, vt, out, lse, dot, block_mask=bmt, score=score, dq=dq, dk=dk, dv=dv,
                           workspace=wsb)

        # ~4 ms per call; the clock keeps rising over the first 15-20 calls
        bwd_settle, bwd_steps = 30, 10
        for _ in range(bwd_settle):
            bwd()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(bwd_steps):
            bwd()
        e1.record(stream)
        torch.cuda.synchronize()
        bwd_ms = e0.elapsed_time(e1) / bwd_steps
        bwd_tflops = 10.0 * D * n_att / (bwd_ms * 1e-3) / 1e12
        result["backward"] = {
            "workload": "backward of " + FWD["name"], "ms": round(bwd_ms, 4),
            "attended_tflops": round(bwd_tflops, 2), "frac_bf16_peak": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
            "flops_per_attended_position": "10*D (S, dP, dV, dK, dQ products)",
            "kernels": "bwd_prep + bwd_dq_kernel + bwd_dkdv_kernel", "untimed_calls": bwd_settle,
            "timed_calls": bwd_steps}
        del dot, dq, dk, dv, wsb, lse
    del qt, kt, vt, out
    torch.cuda.empty_cache()

    # ---------------- decode workload ----------------
    if not args.no_decode:
        Bd, Hq, Hkv, Dd, KV = DEC["B"], DEC["Hq"], DEC["Hkv"], DEC["D"], DEC["KV"]
        print(f"[bench] generating {DEC['name']}", file=sys.stderr, flush=True)
        qd = gen.qkv(DEC["workload_id"], Bd, Hq, Hkv, 1, 1, Dd)[0]
        _, kc, vc = gen.qkv(DEC["workload_id"] + 100, Bd, Hkv, Hkv, 1, KV, Dd)
        lens = gen.kv_lengths(DEC["workload_id"], Bd, DEC["len_lo"], DEC["len_hi"])
        qdt = gen.to_torch_bf16(qd, dev)
        kct = gen.to_torch_bf16(kc, dev)
        del kc
        vct = gen.to_torch_bf16(vc, dev)
        del vc
        lens_t = torch.from_numpy(lens).to(dev)
        bmd = fa.fa_build_block_mask(fa.MaskMod("kv_len", kv_len=lens_t), Bd, 1, 1, KV, device=dev)
        od = torch.empty_like(qdt)
        sc = fa.ScoreMod("softcap", softcap=DEC["cap"])
        ws = torch.empty(fa.fa_decode_workspace_size(qdt, kct, vct, bmd, sc) // 4 + 1,
                         dtype=torch.float32, device=dev)
        dec_settle = max(30, args.warmup)
        for _ in range(dec_settle):  # settle clocks after the forward leg
            fa.fa_decode(qdt, kct, vct, block_mask=bmd, score=sc, out=od, workspace=ws)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.decode_steps):
            fa.fa_decode(qdt, kct, vct, block_mask=bmd, score=sc, out=od, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        dec_ms = e0.elapsed_time(e1) / args.decode_steps
        kv_bytes = int(lens.astype(np.int64).sum()) * Hkv * Dd * 2 * 2
        dec_bytes = kv_bytes + 2 * Bd * Hq * Dd * 2
        gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
        result["decode"] = {
            "workload": DEC["name"], "ms": round(dec_ms, 4), "GB/s": round(gbs, 1),
            "untimed_calls": dec_settle, "timed_calls": args.decode_steps,
            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": dec_bytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": read_traffic("decode_gqa4_kv32768_traffic.md", DEC_SOURCES),
                         "kernels": "decode_partial_kernel<128,4,ScoreSoftcap,false> + decode_merge_kernel<128>"}}
        # The same caches as a compact page pool (paper review §4.5): only the
        # 128-row pages each sequence needs, in shuffled order, reached through a
        # page table.  Same algorithmic bytes; the overhead is the indirection.
        NKb = KV // 128
        need = -(-lens.astype(np.int64) // 128)
        used = np.arange(NKb)[None, :] < need[:, None]                      # [B, NKb]
        n_pages = int(used.sum())
        perm = np.random.default_rng([DEC["workload_id"], 9]).permutation(n_pages)
        table = np.zeros((Bd, NKb), dtype=np.int32)
        table[used] = perm
        sel = torch.from_numpy(used).to(dev)
        perm_t = torch.from_numpy(perm).to(dev)
        pools = []
        for cache in (kct, vct):
            pages = cache.view(Bd, Hkv, NKb, 128, Dd).permute(0, 2, 1, 3, 4)[sel]  # [n_pages, Hkv, 128, D]
            pool = torch.empty_like(pages)
            pool[perm_t] = pages
            pools.append(pool)
            del pages
        del kct, vct
        table_t = torch.from_numpy(table).to(dev)
        odp = torch.empty_like(qdt)
        for _ in range(dec_settle):
            fa.fa_decode(qdt, pools[0], pools[1], block_mask=bmd, score=sc, out=odp, workspace=ws,
                         page_table=table_t)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.decode_steps):
            fa.fa_decode(qdt, pools[0], pools[1], block_mask=bmd, score=sc, out=odp, workspace=ws,
                         page_table=table_t)
        e1.record(stream)
        torch.cuda.synchronize()
        pg_ms = e0.elapsed_time(e1) / args.decode_steps
        result["decode"]["paged"] = {
            "pages": n_pages, "page_rows": 128, "pool_order": "shuffled", "ms": round(pg_ms, 4),
            "GB/s": round(dec_bytes / (pg_ms * 1e-3) / 1e9, 1), "overhead_pct": round(100.0 * (pg_ms / dec_ms - 1.0), 2),
            "same_output_as_contiguous": bool(torch.equal(od, odp))}
        del qdt, pools
        torch.cuda.empty_cache()

    # ---------------- CPU baseline (oracle) ----------------
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(q, k, v, args.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
