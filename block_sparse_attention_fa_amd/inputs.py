"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module holds no attention arithmetic: it only draws random numbers,
encodes them as bfloat16 bit patterns and lays out integer structure
(document ids, per-sequence valid lengths).  Both the HIP path and the CPU
oracle receive exactly these arrays, so they see identical values.

Streams: every tensor comes from its own numpy ``Generator(PCG64)`` seeded
with ``default_rng([workload_id, stream, ...])``:

* stream 0 = Q, 1 = K, 2 = V, 3 = structure (document lengths / kv lengths);
* stream 16 = the dynamic bias, one generator per (b, h, 128-row block), so
  any row block of the ``[B, H, S, S]`` bias can be regenerated on its own
  without materialising the whole tensor on the host.

Normal samples are drawn in float32 and rounded to bfloat16 with
round-to-nearest-even in integer arithmetic.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_STRUCT, STREAM_BIAS = 0, 1, 2, 3, 16
BIAS_ROW_BLOCK = 128


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even) and return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(seed, shape, std=1.0) -> np.ndarray:
    g = np.random.default_rng(seed)
    x = g.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x).reshape(shape)


def _normal_bf16_per_head(seed, shape, threads=8) -> np.ndarray:
    """[B,H,S,D] ~N(0,1) bf16 bits; slice (b,h) comes from generator seed + [b, h]."""
    B, H = shape[0], shape[1]
    out = np.empty(shape, dtype=np.uint16)

    def fill(bh):
        b, h = divmod(bh, H)
        out[b, h] = _normal_bf16(list(seed) + [b, h], shape[2:])

    if threads > 1 and B * H > 1 and int(np.prod(shape)) >= (1 << 22):
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(B * H)))
    else:
        for bh in range(B * H):
            fill(bh)
    return out


def qkv(workload_id: int, B: int, Hq: int, Hkv: int, Sq: int, Skv: int, D: int):
    """Q [B,Hq,Sq,D], K and V [B,Hkv,Skv,D] as bf16 bits, ~N(0,1), one generator per (b, h)."""
    q = _normal_bf16_per_head([workload_id, STREAM_Q], (B, Hq, Sq, D))
    k = _normal_bf16_per_head([workload_id, STREAM_K], (B, Hkv, Skv, D))
    v = _normal_bf16_per_head([workload_id, STREAM_V], (B, Hkv, Skv, D))
    return q, k, v


def document_ids(workload_id: int, B: int, S: int, lo: int = 256, hi: int = 4096) -> np.ndarray:
    """int32 [B,S] document ids 0,1,2,... per batch row.

    Lengths are integer-uniform on [lo, hi] inclusive, drawn until S is
    filled; the last document is truncated so the total is exactly S.
    """
    g = np.random.default_rng([workload_id, STREAM_STRUCT])
    out = np.empty((B, S), dtype=np.int32)
    for b in range(B):
        pos, doc = 0, 0
        while pos < S:
            n = int(g.integers(lo, hi, endpoint=True))
            n = min(n, S - pos)
            out[b, pos:pos + n] = doc
            pos += n
            doc += 1
    return out


def kv_lengths(workload_id: int, B: int, lo: int, hi: int) -> np.ndarray:
    """int32 [B] valid KV lengths, integer-uniform on [lo, hi] inclusive."""
    g = np.random.default_rng([workload_id, STREAM_STRUCT])
    return g.integers(lo, hi, endpoint=True, size=B).astype(np.int32)


def bias_row_block(workload_id: int, b: int, h: int, qblk: int, Sq: int, Skv: int,
                   std: float = 0.5) -> np.ndarray:
    """Rows [128*qblk, min(Sq,128*(qblk+1))) of bias[b,h] as bf16 bits [rows, Skv]."""
    r0 = qblk * BIAS_ROW_BLOCK
    rows = min(Sq, r0 + BIAS_ROW_BLOCK) - r0
    return _normal_bf16([workload_id, STREAM_BIAS, b, h, qblk], (rows, Skv), std)


def bias_slice(workload_id: int, b: int, h: int, Sq: int, Skv: int, std: float = 0.5,
               threads: int = 8) -> np.ndarray:
    """The whole [Sq,Skv] bias slice for (b,h) as bf16 bits."""
    nblk = (Sq + BIAS_ROW_BLOCK - 1) // BIAS_ROW_BLOCK
    out = np.empty((Sq, Skv), dtype=np.uint16)

    def fill(i):
        r0 = i * BIAS_ROW_BLOCK
        blk = bias_row_block(workload_id, b, h, i, Sq, Skv, std)
        out[r0:r0 + blk.shape[0]] = blk

    if threads > 1 and nblk > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nblk)))
    else:
        for i in range(nblk):
            fill(i)
    return out


def bias_rows(workload_id: int, b: int, h: int, rows, Sq: int, Skv: int,
              std: float = 0.5) -> np.ndarray:
    """Selected bias rows of slice (b,h) as bf16 bits [len(rows), Skv]."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, Skv), dtype=np.uint16)
    cache = {}
    for i, r in enumerate(rows):
        blk = int(r) // BIAS_ROW_BLOCK
        if blk not in cache:
            cache[blk] = bias_row_block(workload_id, b, h, blk, Sq, Skv, std)
        out[i] = cache[blk][int(r) - blk * BIAS_ROW_BLOCK]
    return out


# --- device upload helpers (memory only) -----------------------------------

def to_torch_bf16(bits: np.ndarray, device="cuda"):
    """Upload bf16 bit patterns as a torch.bfloat16 tensor (no value change)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device) if device is not None else t


def from_torch_bf16(t) -> np.ndarray:
    """Download a torch.bfloat16 tensor as uint16 bit patterns."""
    import torch
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
