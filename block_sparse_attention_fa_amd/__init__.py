"""MI355X-native block-sparse FlexAttention forward / decode (HIP kernels behind a C ABI).

    from block_sparse_attention_fa_amd import fa
    bm = fa.fa_build_block_mask(fa.MaskMod("causal"), 1, 1, S, S)
    out = fa.fa_forward(q, k, v, block_mask=bm, score=fa.ScoreMod("alibi"))

`fa` loads libfa.so on first use and raises if it has not been built.
`inputs` holds the seeded synthetic input generators.
"""

__all__ = ["fa", "inputs"]


def __getattr__(name):
    if name in ("fa", "inputs"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
