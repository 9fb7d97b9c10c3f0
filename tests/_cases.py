"""Helpers shared by the GPU parity tests: build the same mask/score on both sides.

The oracle side gets numpy functors from oracle/flex_oracle.py; the GPU side
gets MaskMod/ScoreMod descriptors pointing at device copies of the very same
seeded arrays.  No value ever flows from the GPU into an oracle input.
"""

import numpy as np

from block_sparse_attention_fa_amd import inputs as gen
from oracle import flex_oracle as fo

TOL_MAX = 2e-2   # max abs error, bf16 inputs with fp32 accumulation
TOL_MEAN = 2e-3  # mean abs error
# LSE (natural log, fp32).  Both kernels sum the fp32 exponentials of a row
# (the forward feeds bf16-rounded copies of them to the PV product), so the
# sum l of at most 32768 terms carries a relative error below (n - 1) 2^-24 <
# 2e-3 even in the worst case, and ln(l) an absolute one below that; fp32
# rounding of the scores and of m + ln(l) adds a few ulps of |LSE|.
LSE_TOL_ABS = 2e-3
LSE_TOL_REL = 1e-5

# Gradients (backward).  P and dS are rounded to bf16 for the MFMAs and the
# gradients are stored as bf16, so each element carries about 2^-9 relative
# error from each rounding; the bounds below are 2.5-4x what is measured
# (relative Frobenius 2.3e-3 to 3.8e-3, max abs <= 0.25 of its bound).
GRAD_TOL_REL_MAX = 2e-2   # max abs error <= 2e-2 * max|ref| + 2e-3
GRAD_TOL_ABS = 2e-3
GRAD_TOL_FRO = 1e-2       # ||got - ref|| / ||ref||


def compare_grad(got, ref, what=""):
    """Assert a bf16 gradient is within the bounds above of the fp64 oracle's."""
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    err = np.abs(got - ref)
    scale = float(np.abs(ref).max())
    fro = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    print(f"[{what}] max abs {err.max():.3e} (ref max {scale:.3e}), rel fro {fro:.3e}", flush=True)
    assert err.max() <= GRAD_TOL_REL_MAX * scale + GRAD_TOL_ABS, f"{what}: max abs {err.max():.3e}, ref max {scale:.3e}"
    assert fro <= GRAD_TOL_FRO or scale == 0.0, f"{what}: relative Frobenius error {fro:.3e}"
    return float(err.max()), fro


MASK_NAMES = ["none", "causal", "sliding_window", "sliding_causal", "document",
              "document_causal", "prefix_lm", "kv_len"]
SCORE_NAMES = ["none", "alibi", "softcap", "rel_pos", "bias"]


def oracle_mask(spec):
    k = spec["mask"]
    if k == "none":
        return None
    if k == "causal":
        return fo.causal()
    if k == "sliding_window":
        return fo.sliding_window(spec["window"])
    if k == "sliding_causal":
        return fo.sliding_causal(spec["window"])
    if k == "document":
        return fo.document(spec["docs"])
    if k == "document_causal":
        return fo.document_causal(spec["docs"])
    if k == "prefix_lm":
        return fo.prefix_lm(spec["prefix"])
    if k == "kv_len":
        return fo.kv_length(spec["lens"])
    raise KeyError(k)


def oracle_score(spec, Hq):
    k = spec.get("score", "none")
    if k == "none":
        return None
    if k == "alibi":
        return fo.alibi(spec["slopes"] if spec.get("slopes") is not None else fo.default_alibi_slopes(Hq))
    if k == "softcap":
        return fo.softcap(spec["cap"])
    if k == "rel_pos":
        return fo.rel_pos()
    if k == "bias":
        return fo.bias(spec["bias_table"])
    raise KeyError(k)


def gpu_mask(spec, device="cuda"):
    import torch
    from block_sparse_attention_fa_amd import fa
    docs = spec.get("docs")
    lens = spec.get("lens")
    return fa.MaskMod(spec["mask"], window=spec.get("window", 0), prefix_len=spec.get("prefix", 0),
                      doc_ids=torch.from_numpy(docs).to(device) if docs is not None else None,
                      kv_len=torch.from_numpy(lens).to(device) if lens is not None else None)


def gpu_score(spec, device="cuda"):
    import torch
    from block_sparse_attention_fa_amd import fa
    k = spec.get("score", "none")
    slopes = spec.get("slopes")
    bias = spec.get("bias_bits")
    return fa.ScoreMod(k, softcap=spec.get("cap", 0.0),
                       alibi_slopes=torch.tensor(slopes, dtype=torch.float32, device=device)
                       if slopes is not None else None,
                       bias=gen.to_torch_bf16(bias, device) if bias is not None else None)


def make_spec(seed, mask, score, B, Hq, Sq, Skv, window=None, prefix=None, cap=30.0,
              bias_broadcast=False, explicit_slopes=False):
    """A seeded mask/score specification with every array both sides need."""
    rng = np.random.default_rng([seed, 77])
    spec = {"mask": mask, "score": score}
    S = max(Sq, Skv)
    spec["window"] = window if window is not None else int(rng.integers(0, max(1, Skv // 2)))
    spec["prefix"] = prefix if prefix is not None else int(rng.integers(0, Skv + 1))
    spec["docs"] = gen.document_ids(seed, B, S, max(1, S // 10), max(2, S // 3)) if mask.startswith("document") else None
    spec["lens"] = (rng.integers(0, Skv + 1, size=B).astype(np.int32) if mask == "kv_len" else None)
    spec["cap"] = cap
    if score == "alibi" and explicit_slopes:
        spec["slopes"] = list(rng.uniform(0.01, 1.0, size=Hq))
    if score == "bias":
        shape = (1, 1, Sq, Skv) if bias_broadcast else (B, Hq, Sq, Skv)
        bits = gen._normal_bf16([seed, gen.STREAM_BIAS], shape, 0.5)
        spec["bias_bits"] = bits
        spec["bias_table"] = np.broadcast_to(bits, (B, Hq, Sq, Skv))
    return spec


def compare(out_f32, ref_f64, what=""):
    """Assert the bf16 GPU output is within the stated tolerance of the fp64 oracle."""
    err = np.abs(out_f32.astype(np.float64) - ref_f64)
    assert np.all(np.isfinite(out_f32)), f"{what}: non-finite output"
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= TOL_MAX and mean <= TOL_MEAN, f"{what}: max abs {mx:.3e}, mean abs {mean:.3e}"
    return mx, mean


def compare_lse(got, ref, what=""):
    """Assert GPU LSEs match the oracle: same -inf rows, finite ones within the bound above."""
    got = np.asarray(got, dtype=np.float64)
    np.testing.assert_array_equal(np.isneginf(got), np.isneginf(ref), err_msg=what)
    fin = np.isfinite(ref)
    if not fin.any():
        return 0.0
    err = np.abs(got[fin] - ref[fin])
    bound = LSE_TOL_ABS + LSE_TOL_REL * np.abs(ref[fin])
    assert np.all(err <= bound), f"{what}: LSE abs err {err.max():.3e}"
    return float(err.max())
