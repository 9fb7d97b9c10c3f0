#!/usr/bin/env python3
"""Throughput of the block-sparse FlexAttention hot path on one MI355X.

The timed step (`value`) is fa_build_block_mask + fa_forward on the causal +
ALiBi workload (B=4, H=16, S=8192, D=128, bf16 ~N(0,1); slopes 2^(-8(h+1)/16)),
reported as attended TFLOP/s (4*D per attended (b,h,q,kv) position).  The
other workloads are measured in the same run, each with its own roofline:

  causal_tiny      B1 H2 S256 D64 causal: launch latency (us)
  sliding_softcap  B2 H16 S16384 D128, causal AND window 1024, softcap 30: attended TFLOP/s (MFMA-bound)
  document_bias    B1 H32 S16384 D64, document AND causal, bias [1,32,S,S] bf16: HBM GB/s (bias-bound)
  decode           B32 Hq32 Hkv8 D128, KV 32768, lengths U[4096,32768], softcap 50: HBM GB/s
  backward         the backward of the timed workload: attended TFLOP/s (10*D per position)

plus measured peaks (a bf16 MFMA loop and a streaming copy, fa_probe_mfma /
fa_probe_copy) next to the published ones.  Inputs are resident in HBM before
any timing starts.  The legs run in the order above and the timed step runs
last, with exactly --warmup untimed steps before its --steps timed ones (the
earlier legs have brought the GPU to its steady clock by then).  Prints one
JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 10] [--legs a,b,...]
    python bench.py --ablation                 (block-skipping ablation, sparsity sweep)
    python bench.py --copy-calibration 1024    (counter calibration for rocprofv3 FETCH/WRITE_SIZE)
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published

FWD = dict(name="causal+alibi fwd B4 H16 S8192 D128 bf16", workload_id=2, B=4, H=16, S=8192, D=128)
TINY = dict(name="causal fwd B1 H2 S256 D64 bf16", workload_id=1, B=1, H=2, S=256, D=64)
SLIDE = dict(name="sliding1024+causal softcap30 fwd B2 H16 S16384 D128 bf16", workload_id=3, B=2, H=16,
             S=16384, D=128, W=1024, cap=30.0)
DOC = dict(name="document+causal bias[B,H,S,S] fwd B1 H32 S16384 D64 bf16", workload_id=4, B=1, H=32,
           S=16384, D=64)
DEC = dict(name="gqa4 split-kv decode B32 Hq32 Hkv8 D128 KV32768 softcap50 bf16", workload_id=5,
           B=32, Hq=32, Hkv=8, D=128, KV=32768, len_lo=4096, len_hi=32768, cap=50.0)
LEGS = ("peaks", "tiny", "sliding", "document", "decode", "backward", "main")

FWD_SOURCES = ["fwd_kernel.hpp", "mods.hpp", "fwd_causal.hip", "fa_internal.hpp"]
SLIDE_SOURCES = ["fwd_kernel.hpp", "mods.hpp", "fwd_sliding_causal.hip", "fa_internal.hpp"]
DOC_SOURCES = ["fwd_kernel.hpp", "mods.hpp", "fwd_document_causal.hip", "fa_internal.hpp"]
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


def roofline(bound, achieved, peak, unit, measured_peak, traffic, **extra):
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4),
         "measured_peak": round(measured_peak, 1) if measured_peak else None,
         "frac_measured_peak": round(achieved / measured_peak, 4) if measured_peak else None,
         "traffic": traffic}
    r.update(extra)
    return r


def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")} for i in threadpool_info()]
    except Exception:
        pass
    return model, blas


def cpu_baseline(q, k, v, seconds):
    """The fp64 oracle on host cores, on (b, h, 1024-row) chunks of the forward
    workload taken from the last rows backwards until `seconds` have elapsed."""
    import numpy as np
    from oracle import flex_oracle as fo
    model, blas = cpu_info()
    threads = max([b["threads"] or 1 for b in blas] or [os.cpu_count() or 1])
    B, H, S, D = FWD["B"], FWD["H"], FWD["S"], FWD["D"]
    mask, score = fo.causal(), fo.alibi(fo.default_alibi_slopes(H))
    chunks, flops = [], 0.0
    t0 = time.perf_counter()
    done = False
    for b in range(B):
        for h in range(H):
            for r1 in range(S, 0, -1024):
                rows = np.arange(max(0, r1 - 1024), r1)
                fo.attention_rows(q, k, v, b, h, rows, mask, score)
                flops += 4.0 * D * float((rows + 1).sum())  # causal: row q attends q+1 keys
                chunks.append((b, h, int(rows[0])))
                if time.perf_counter() - t0 >= seconds:
                    done = True
                    break
            if done:
                break
        if done:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(chunks)} chunks of 1024 query rows x all 8192 keys (fp64, dense) of the "
                      f"causal+ALiBi S=8192 workload, (b,h) in order from (0,0), rows from the end back; {dt:.1f} s",
            "cpu_model": model, "cpu_count": os.cpu_count(), "blas": blas}


def sample_power(fn, seconds=4.0):
    """Run fn back to back for `seconds` while `amd-smi metric -p -c` samples the
    board power and the graphics clocks (three samples, from the second second on).
    Returns {"socket_power_w": [...], "gfx_clk_mhz": [...]} or an error note."""
    import subprocess
    import threading
    import torch
    out = {"socket_power_w": [], "gfx_clk_mhz": []}

    def sampler():
        time.sleep(1.0)
        for _ in range(3):
            try:
                r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                                   timeout=10)
                d = json.loads(r.stdout)
                g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
                out["socket_power_w"].append(g["power"]["socket_power"]["value"])
                clk = [v["clk"]["value"] for k, v in g["clock"].items() if k.startswith("gfx_")]
                out["gfx_clk_mhz"].append(round(sum(clk) / len(clk)))
            except Exception as e:  # no amd-smi, or another JSON layout
                out["error"] = f"{type(e).__name__}: {e}"
                return
            time.sleep(0.5)

    th = threading.Thread(target=sampler)
    th.start()
    t0 = time.time()
    while time.time() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    th.join()
    return out


class Timer:
    """HIP events recorded on the launch stream around a batch of calls; with
    power=True each measurement is followed by sample_power on the same call."""

    def __init__(self, stream, power=False):
        import torch
        self.stream = stream
        self.power = power
        self.last_power = None
        self.last_stats = None
        self.e0 = torch.cuda.Event(enable_timing=True)
        self.e1 = torch.cuda.Event(enable_timing=True)

    def ms(self, fn, calls, untimed, per_call=False):
        """Mean ms per call over `calls` back-to-back calls after `untimed` ones.
        With per_call, an event is also recorded between calls, and the median
        and minimum per call go to self.last_stats."""
        import torch
        for _ in range(untimed):
            fn()
        torch.cuda.synchronize()
        if per_call:
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(calls + 1)]
            evs[0].record(self.stream)
            for i in range(calls):
                fn()
                evs[i + 1].record(self.stream)
            torch.cuda.synchronize()
            each = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(calls))
            total = evs[0].elapsed_time(evs[calls])
            self.last_stats = {"median_ms": round(each[calls // 2] if calls % 2 else
                                                  0.5 * (each[calls // 2 - 1] + each[calls // 2]), 4),
                               "min_ms": round(each[0], 4), "calls": calls}
        else:
            self.e0.record(self.stream)
            for _ in range(calls):
                fn()
            self.e1.record(self.stream)
            torch.cuda.synchronize()
            total = self.e0.elapsed_time(self.e1)
            self.last_stats = None
        if self.power:
            self.last_power = sample_power(fn)
        return total / calls


def leg_peaks(T, dev):
    import torch
    from block_sparse_attention_fa_amd import fa
    wgs, iters = 512, 4096              # 2 workgroups (8 waves) per CU: 2 waves per SIMD
    sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    flops = {}

    def mfma():
        flops["n"] = fa.fa_probe_mfma(wgs, iters, sink)

    mfma_ms = min(T.ms(mfma, 20, 30 if i == 0 else 2) for i in range(3))
    mfma_power = T.last_power

    def mfma_random():
        flops["r"] = fa.fa_probe_mfma(wgs, iters, sink, random_operands=True)

    rand_ms = min(T.ms(mfma_random, 20, 10 if i == 0 else 2) for i in range(3))
    rand_power = T.last_power
    n = 1 << 30
    src = torch.zeros(n // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    copy_ms = min(T.ms(lambda: fa.fa_probe_copy(src, dst), 20, 10 if i == 0 else 2) for i in range(3))
    copy_power = T.last_power
    del src, dst
    rsink = torch.empty(8192, dtype=torch.int32, device=dev)
    rsrc = torch.zeros(n, dtype=torch.bfloat16, device=dev)   # 2 GiB read per launch
    read_ms = min(T.ms(lambda: fa.fa_probe_read(rsrc, rsink), 20, 10 if i == 0 else 2) for i in range(3))
    del sink, rsrc, rsink
    return {"power": {"mfma_probe": mfma_power, "mfma_probe_random": rand_power, "copy_probe": copy_power,
                      "read_probe": T.last_power} if T.power else None,
            "mfma_bf16_tflops": round(flops["n"] / (mfma_ms * 1e-3) / 1e12, 1),
            "mfma_bf16_random_operands_tflops": round(flops["r"] / (rand_ms * 1e-3) / 1e12, 1),
            "mfma_probe": f"{wgs} workgroups x 4 waves x {iters} x 8 v_mfma_f32_32x32x16_bf16, best of 3 x 20 "
                          "launches; constant operands, and random bf16 operands alternating between two sets",
            "copy_gbs": round(2.0 * n / (copy_ms * 1e-3) / 1e9, 1),
            "copy_probe": "1 GiB read + 1 GiB written per launch, 16-byte non-temporal loads/stores, best of 3 x 20",
            "read_gbs": round(2.0 * n / (read_ms * 1e-3) / 1e9, 1),
            "read_probe": "2 GiB read per launch, 16-byte non-temporal loads, best of 3 x 20",
            "published": {"bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}}


def leg_tiny(T, dev):
    from block_sparse_attention_fa_amd import fa
    from block_sparse_attention_fa_amd import inputs as gen
    c = TINY
    q, k, v = (gen.to_torch_bf16(x, dev) for x in gen.qkv(c["workload_id"], c["B"], c["H"], c["H"], c["S"], c["S"], c["D"]))
    import ctypes
    bm = fa.fa_build_block_mask(fa.MaskMod("causal"), 1, 1, c["S"], c["S"], device=dev)
    out = q.new_empty(q.shape)
    a = fa._attn_args(q, k, v, out, None, bm, None, 0.0, 0)   # marshalled once: the loop is the C call
    sptr = ctypes.c_void_p(T.stream.cuda_stream)
    L = fa.lib()
    ms = T.ms(lambda: fa._check(L.fa_forward(ctypes.byref(a), sptr)), 200, 50)
    n_att = c["B"] * c["H"] * c["S"] * (c["S"] + 1) // 2
    return {"workload": c["name"], "latency_us": round(ms * 1e3, 2), "calls": 200,
            "note": "4 workgroups: bound by launch latency, no roofline claim; the time is per call "
                    "(fa_forward through ctypes + launch + kernel) from HIP events around 200 back-to-back calls",
            "attended_tflops": round(4.0 * c["D"] * n_att / (ms * 1e-3) / 1e12, 4), "roofline": None}


# Untimed calls before the sliding, document and decode legs are timed: each
# leg starts after seconds of host-side input generation with the GPU idle, and
# the clock needs tens of milliseconds of continuous work to settle.
LEG_UNTIMED = 100


def _fwd_leg(T, q, k, v, bm, score, calls, settle):
    out = q.new_empty(q.shape)
    from block_sparse_attention_fa_amd import fa
    return T.ms(lambda: fa.fa_forward(q, k, v, block_mask=bm, score=score, out=out), calls, settle, per_call=True), out


def leg_sliding(T, dev, peaks):
    from block_sparse_attention_fa_amd import fa
    from block_sparse_attention_fa_amd import inputs as gen
    c = SLIDE
    B, H, S, D, W = c["B"], c["H"], c["S"], c["D"], c["W"]
    q, k, v = (gen.to_torch_bf16(x, dev) for x in gen.qkv(c["workload_id"], B, H, H, S, S, D))
    bm = fa.fa_build_block_mask(fa.MaskMod("sliding_causal", window=W), 1, 1, S, S, device=dev)
    cls = bm.classes()
    ms, _ = _fwd_leg(T, q, k, v, bm, fa.ScoreMod("softcap", softcap=c["cap"]), 20, LEG_UNTIMED)
    n_att = B * H * (W * (W + 1) // 2 + (S - W) * (W + 1))   # row q attends min(q, W) + 1 keys
    flops = 4.0 * D * n_att
    tf = flops / (ms * 1e-3) / 1e12
    n_part, n_full = int((cls == 1).sum()), int((cls == 2).sum())
    return {"workload": c["name"], "kernel_ms": round(ms, 4), "per_call": T.last_stats, "untimed_calls": LEG_UNTIMED,
            "attended_tflops": round(tf, 2),
            "attended_flops": flops, "power": T.last_power if T.power else None,
            "tiles_partial": n_part, "tiles_full": n_full,
            "executed_tile_tflops": round(4.0 * D * 128 * 128 * (n_part + n_full) * B * H / (ms * 1e-3) / 1e12, 2),
            "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s", peaks.get("mfma_bf16_tflops"),
                                 read_traffic("fwd_sliding_softcap_16384_traffic.md", SLIDE_SOURCES),
                                 kernel="fwd_kernel<128, MaskAnd<MaskCausal, MaskWindow>, ScoreSoftcapBounded>",
                                 algorithmic_bytes=4 * B * H * S * D * 2)}


def leg_document(T, dev, peaks):
    import numpy as np
    import torch
    from concurrent.futures import ThreadPoolExecutor
    from block_sparse_attention_fa_amd import fa
    from block_sparse_attention_fa_amd import inputs as gen
    c = DOC
    B, H, S, D, wid = c["B"], c["H"], c["S"], c["D"], c["workload_id"]
    q, k, v = (gen.to_torch_bf16(x, dev) for x in gen.qkv(wid, B, H, H, S, S, D))
    docs = gen.document_ids(wid, B, S)
    bias = torch.empty((B, H, S, S), dtype=torch.bfloat16, device=dev)

    def fill(bh):
        b, h = divmod(bh, H)
        bias[b, h].copy_(gen.to_torch_bf16(gen.bias_slice(wid, b, h, S, S, threads=1), device=None))

    with ThreadPoolExecutor(min(16, os.cpu_count() or 4)) as ex:
        list(ex.map(fill, range(B * H)))
    mask = fa.MaskMod("document_causal", doc_ids=torch.from_numpy(docs).to(dev))
    bm = fa.fa_build_block_mask(mask, B, 1, S, S, device=dev)
    cls = bm.classes()
    ms, _ = _fwd_leg(T, q, k, v, bm, fa.ScoreMod("bias", bias=bias), 20, LEG_UNTIMED)
    doc_stats = T.last_stats
    lens = np.concatenate([np.bincount(docs[b]) for b in range(B)]).astype(np.int64)
    n_att = H * int((lens * (lens + 1) // 2).sum())          # document AND causal: L(L+1)/2 per document
    n_part, n_full = int((cls == 1).sum()), int((cls == 2).sum())
    qkvo = 4 * B * H * S * D * 2
    alg = qkvo + 2 * n_att                                   # + the bias at attended positions (bf16)
    gbs = alg / (ms * 1e-3) / 1e9
    tile_bias = 2 * 128 * 128 * (n_part + n_full) * H       # bias bytes of every visited tile
    del bias
    torch.cuda.empty_cache()
    return {"workload": c["name"], "kernel_ms": round(ms, 4), "per_call": doc_stats, "untimed_calls": LEG_UNTIMED,
            "documents": int(lens.size),
            "power": T.last_power if T.power else None,
            "attended_tflops": round(4.0 * D * n_att / (ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(4.0 * D * n_att / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "tiles_partial": n_part, "tiles_full": n_full, "algorithmic_bytes": alg,
            "block_granular_bytes": qkvo + tile_bias,
            "block_granular_gbs": round((qkvo + tile_bias) / (ms * 1e-3) / 1e9, 1),
            "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", peaks.get("read_gbs"),
                                 read_traffic("fwd_document_bias_16384_traffic.md", DOC_SOURCES),
                                 kernel="fwd_kernel<64, MaskAnd<MaskDocument, MaskCausal>, ScoreBiasTiled>",
                                 bytes_definition="Q, K, V read and O written once + the bf16 bias at attended positions")}


def leg_decode(T, dev, peaks, stream):
    import numpy as np
    import torch
    from block_sparse_attention_fa_amd import fa
    from block_sparse_attention_fa_amd import inputs as gen
    Bd, Hq, Hkv, Dd, KV = DEC["B"], DEC["Hq"], DEC["Hkv"], DEC["D"], DEC["KV"]
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
    ws = torch.empty(fa.fa_decode_workspace_size(qdt, kct, vct, bmd, sc) // 4 + 1, dtype=torch.float32, device=dev)
    calls, settle = 50, LEG_UNTIMED
    dec_ms = T.ms(lambda: fa.fa_decode(qdt, kct, vct, block_mask=bmd, score=sc, out=od, workspace=ws), calls, settle,
                  per_call=True)
    dec_stats = T.last_stats
    kv_bytes = int(lens.astype(np.int64).sum()) * Hkv * Dd * 2 * 2
    dec_bytes = kv_bytes + 2 * Bd * Hq * Dd * 2
    gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    res = {"workload": DEC["name"], "ms": round(dec_ms, 4), "per_call": dec_stats, "GB/s": round(gbs, 1),
           "power": T.last_power if T.power else None,
           "untimed_calls": settle, "timed_calls": calls, "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
           "algorithmic_bytes": dec_bytes,
           "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", peaks.get("read_gbs"),
                                read_traffic("decode_gqa4_kv32768_traffic.md", DEC_SOURCES),
                                kernels="decode_partial_kernel<128,4,ScoreSoftcap,false> + decode_merge_kernel<128>")}
    # The same caches as a compact page pool (paper review §4.5): only the
    # 128-row pages each sequence needs, in shuffled order, reached through a
    # page table.  Same algorithmic bytes; the overhead is the indirection.
    NKb = KV // 128
    need = -(-lens.astype(np.int64) // 128)
    used = np.arange(NKb)[None, :] < need[:, None]
    n_pages = int(used.sum())
    perm = np.random.default_rng([DEC["workload_id"], 9]).permutation(n_pages)
    table = np.zeros((Bd, NKb), dtype=np.int32)
    table[used] = perm
    sel = torch.from_numpy(used).to(dev)
    perm_t = torch.from_numpy(perm).to(dev)
    pools = []
    for cache in (kct, vct):
        pages = cache.view(Bd, Hkv, NKb, 128, Dd).permute(0, 2, 1, 3, 4)[sel]
        pool = torch.empty_like(pages)
        pool[perm_t] = pages
        pools.append(pool)
        del pages
    del kct, vct
    table_t = torch.from_numpy(table).to(dev)
    odp = torch.empty_like(qdt)
    pg_ms = T.ms(lambda: fa.fa_decode(qdt, pools[0], pools[1], block_mask=bmd, score=sc, out=odp, workspace=ws,
                                      page_table=table_t), calls, settle)
    res["paged"] = {"pages": n_pages, "page_rows": 128, "pool_order": "shuffled", "ms": round(pg_ms, 4),
                    "GB/s": round(dec_bytes / (pg_ms * 1e-3) / 1e9, 1),
                    "overhead_pct": round(100.0 * (pg_ms / dec_ms - 1.0), 2),
                    "same_output_as_contiguous": bool(torch.equal(od, odp))}
    del pools
    torch.cuda.empty_cache()
    return res


def leg_backward(T, dev, qt, kt, vt):
    import torch
    from block_sparse_attention_fa_amd import fa
    from block_sparse_attention_fa_amd import inputs as gen
    B, H, S, D = FWD["B"], FWD["H"], FWD["S"], FWD["D"]
    mask, score = fa.MaskMod("causal"), fa.ScoreMod("alibi")
    bmt = fa.fa_build_block_mask(mask, 1, 1, S, S, device=dev, transposed=True)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    out = fa.fa_forward(qt, kt, vt, block_mask=bmt, score=score, lse=lse)
    dot = gen.to_torch_bf16(gen._normal_bf16([FWD["workload_id"], 30], (B, H, S, D)), dev)
    dq, dk, dv = torch.empty_like(qt), torch.empty_like(kt), torch.empty_like(vt)
    wsb = torch.empty(fa.fa_backward_workspace_size(qt, kt, vt, out, lse, bmt, score) // 4 + 4,
                      dtype=torch.float32, device=dev)
    settle, calls = 30, 10
    ms = T.ms(lambda: fa.fa_backward(qt, kt, vt, out, lse, dot, block_mask=bmt, score=score, dq=dq, dk=dk, dv=dv,
                                     workspace=wsb), calls, settle, per_call=True)
    n_att = B * H * S * (S + 1) // 2
    tf = 10.0 * D * n_att / (ms * 1e-3) / 1e12
    return {"workload": "backward of " + FWD["name"], "ms": round(ms, 4), "per_call": T.last_stats,
            "attended_tflops": round(tf, 2),
            "power": T.last_power if T.power else None,
            "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "flops_per_attended_position": "10*D (S, dP, dV, dK, dQ products)",
            "kernels": "bwd_prep + bwd_dq_kernel + bwd_dkdv_kernel", "untimed_calls": settle, "timed_calls": calls}


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
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma-separated subset of " + ",".join(LEGS) + " (the timed step is 'main')")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--power", action="store_true",
                    help="after each leg's timing, loop its workload for 4 s and sample board power and "
                         "graphics clocks with amd-smi (reported under 'power')")
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
    legs = [x for x in args.legs.split(",") if x]
    bad = [x for x in legs if x not in LEGS]
    if bad:
        ap.error(f"unknown legs {bad}")

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
    stream = torch.cuda.current_stream()
    T = Timer(stream, power=args.power)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    extra = {}
    peaks = {}
    if "peaks" in legs:
        log("measured peaks (MFMA loop, streaming copy)")
        peaks = leg_peaks(T, dev)
        extra["peaks"] = peaks
    if "tiny" in legs:
        log(TINY["name"])
        extra["causal_tiny"] = leg_tiny(T, dev)
    if "sliding" in legs:
        log(SLIDE["name"])
        extra["sliding_softcap"] = leg_sliding(T, dev, peaks)
        torch.cuda.empty_cache()
    if "document" in legs:
        log(DOC["name"] + " (generating the 16 GiB bias)")
        extra["document_bias"] = leg_document(T, dev, peaks)
    if "decode" in legs:
        log(DEC["name"])
        extra["decode"] = leg_decode(T, dev, peaks, stream)

    # ---------------- the timed step: BlockMask build + forward, causal + ALiBi ----------------
    B, H, S, D = FWD["B"], FWD["H"], FWD["S"], FWD["D"]
    log(f"generating {FWD['name']}")
    q, k, v = gen.qkv(FWD["workload_id"], B, H, H, S, S, D)
    qt, kt, vt = (gen.to_torch_bf16(x, dev) for x in (q, k, v))
    if "backward" in legs:
        log("backward")
        extra["backward"] = leg_backward(T, dev, qt, kt, vt)
        torch.cuda.empty_cache()
    result = {}
    if "main" in legs:
        log("timed step")
        out = torch.empty_like(qt)
        mask, score = fa.MaskMod("causal"), fa.ScoreMod("alibi")
        bm = fa.BlockMask(mask, 1, 1, S, S, device=dev)
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

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        step_ms = (t1 - t0) * 1e3 / args.steps
        each = sorted(a.elapsed_time(b) for a, b in evs)
        fwd_ms = sum(each) / args.steps
        fwd_stats = {"median_ms": round(each[len(each) // 2] if len(each) % 2 else
                                        0.5 * (each[len(each) // 2 - 1] + each[len(each) // 2]), 4),
                     "min_ms": round(each[0], 4), "calls": len(each)}
        main_power = sample_power(step) if args.power else None
        build_ms = T.ms(lambda: fa._check(L.fa_build_block_mask(ctypes.byref(bm.c), S, S, sptr)), 10, 0)
        cls = bm.classes()
        n_part, n_full = int((cls == 1).sum()), int((cls == 2).sum())
        n_att = B * H * S * (S + 1) // 2               # causal: row q attends q+1 keys
        att_flops = 4.0 * D * n_att
        exec_flops = 4.0 * D * 128 * 128 * (n_part + n_full) * B * H
        alg_bytes = 4 * B * H * S * D * 2               # Q, K, V, O once each
        fwd_tflops = att_flops / (fwd_ms * 1e-3) / 1e12
        value = att_flops / (step_ms * 1e-3) / 1e12
        result = {
            "metric": "fwd attended TFLOP/s & % bf16 MFMA peak; decode HBM GB/s (1 MI355X)",
            "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": FWD["name"], "B": B, "H": H, "S": S, "D": D, "mask": "causal",
                       "score_mod": "alibi", "block": 128, "step": "fa_build_block_mask + fa_forward",
                       "legs_before_timed_step": [x for x in legs if x != "main"]},
            "fwd": {"kernel_ms": round(fwd_ms, 4), "per_call": fwd_stats, "attended_tflops": round(fwd_tflops, 2),
                    "power": main_power,
                    "frac_bf16_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
                    "executed_tile_tflops": round(exec_flops / (fwd_ms * 1e-3) / 1e12, 2),
                    "tiles_partial": n_part, "tiles_full": n_full, "blockmask_build_ms": round(build_ms, 4),
                    "sparsity_pct": round(100.0 * float((cls == 0).sum()) / cls.size, 3)},
            "roofline": roofline("mfma", fwd_tflops, PEAK_BF16_TFLOPS, "TFLOP/s", peaks.get("mfma_bf16_tflops"),
                                 read_traffic("fwd_causal_alibi_8192_traffic.md", FWD_SOURCES),
                                 algorithmic_bytes=alg_bytes, kernel="fwd_kernel<128, MaskCausal, ScoreAlibi>"),
        }
    result.update(extra)
    del qt, kt, vt
    torch.cuda.empty_cache()

    # ---------------- CPU baseline (oracle) ----------------
    if not args.no_cpu_baseline and "main" in legs:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(q, k, v, args.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
