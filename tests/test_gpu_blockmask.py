"""BlockMask builder on the GPU vs the oracle: bit-exact over the whole tensors,
row lists and their transposed (per-KV-block) view."""

import numpy as np
import pytest

from block_sparse_attention_fa_amd import inputs as gen
from oracle import flex_oracle as fo
from tests import _cases as C

pytestmark = pytest.mark.gpu
KEYS = ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices",
        "q_num_blocks", "q_indices", "full_q_num_blocks", "full_q_indices")


def _check_bitexact(spec, Bm, Hm, Sq, Skv, separate_full=True):
    """Every list, the transposed (per-KV-block) view included, equals the oracle's."""
    from block_sparse_attention_fa_amd import fa
    import torch
    bm = fa.fa_build_block_mask(C.gpu_mask(spec), Bm, Hm, Sq, Skv, separate_full=separate_full, transposed=True)
    torch.cuda.synchronize()
    mm = C.oracle_mask(spec) or fo.no_mask()
    ref = fo.block_mask(mm, Bm, Hm, Sq, Skv, separate_full=separate_full)
    for key in KEYS:
        got = getattr(bm, key).cpu().numpy()
        assert got.dtype == np.int32
        np.testing.assert_array_equal(got, ref[key], err_msg=f"{spec['mask']} {key} Sq={Sq} Skv={Skv}")
    return bm, ref


@pytest.mark.parametrize("mask", C.MASK_NAMES)
@pytest.mark.parametrize("Sq,Skv", [(256, 256), (300, 300), (1000, 1000), (129, 700), (700, 129), (1, 1000)])
@pytest.mark.parametrize("separate_full", [True, False])
def test_blockmask_bitexact_small(mask, Sq, Skv, separate_full):
    if mask.startswith("document") and Sq != Skv:
        pytest.skip("document masks share one id array for queries and keys")
    B = 2
    spec = C.make_spec(3, mask, "none", B, 1, Sq, Skv)
    Bm = B if mask in ("document", "document_causal", "kv_len") else 1
    _check_bitexact(spec, Bm, 1, Sq, Skv, separate_full)


def test_blockmask_workload_shapes():
    # causal 8192 (ALiBi workload), sliding 1024 at 16384, document-causal at 16384,
    # kv_len prefixes for 32 sequences of a 32768 cache
    _, r = _check_bitexact({"mask": "causal"}, 1, 1, 8192, 8192)
    assert fo.sparsity(r["classes"]) == pytest.approx(100.0 * 2016 / 4096)
    _, r = _check_bitexact({"mask": "sliding_causal", "window": 1024}, 1, 1, 16384, 16384)
    assert int((r["classes"] == 2).sum()) == 868 and int((r["classes"] == 1).sum()) == 248
    docs = gen.document_ids(4, 1, 16384)
    _check_bitexact({"mask": "document_causal", "docs": docs}, 1, 1, 16384, 16384)
    lens = gen.kv_lengths(5, 32, 4096, 32768)
    _check_bitexact({"mask": "kv_len", "lens": lens}, 32, 1, 1, 32768)


def test_blockmask_print_and_sparsity():
    from block_sparse_attention_fa_amd import fa
    import torch
    bm = fa.fa_build_block_mask(fa.MaskMod("causal"), 1, 1, 2048, 2048)
    torch.cuda.synchronize()
    cls = fo.block_classes(fo.causal(), 1, 1, 2048, 2048)
    assert bm.to_string() == fo.block_mask_ascii(cls[0, 0])
    assert bm.sparsity() == pytest.approx(fo.sparsity(cls))


def test_blockmask_rebuild_reuses_buffers():
    # a second build into the same tensors with another document layout (no recompilation)
    from block_sparse_attention_fa_amd import fa
    import torch
    S = 2048
    for seed in (1, 2, 3):
        docs = gen.document_ids(seed, 1, S, 100, 700)
        spec = {"mask": "document_causal", "docs": docs}
        _check_bitexact(spec, 1, 1, S, S)
