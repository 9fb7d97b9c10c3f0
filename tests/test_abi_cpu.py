"""The C ABI without a GPU: libfa.so loads, exports every function include/fa.h
declares, and host-side validation rejects bad arguments before any HIP call."""

import ctypes
import os
import re

import pytest

from block_sparse_attention_fa_amd import fa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fa.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(fa_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"fa_build_block_mask", "fa_forward", "fa_decode", "fa_decode_workspace_size",
            "fa_block_mask_dims", "fa_status_string", "fa_last_error", "fa_abi_version"} <= set(names)
    lib = ctypes.CDLL(fa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in fa.h but not exported"
    assert set(names) == set(fa.SIGNATURES), "binding signatures out of sync with fa.h"


def test_abi_version_and_status_strings():
    L = fa.lib()
    assert L.fa_abi_version() == 6
    for code, name in enumerate(["FA_OK", "FA_ERR_NULL", "FA_ERR_SHAPE", "FA_ERR_UNSUPPORTED",
                                 "FA_ERR_WORKSPACE", "FA_ERR_HIP"]):
        assert L.fa_status_string(code).decode() == name


def test_block_mask_dims():
    assert fa.fa_block_mask_dims(256, 256) == (2, 2)
    assert fa.fa_block_mask_dims(300, 1) == (3, 1)
    assert fa.fa_block_mask_dims(8192, 16384) == (64, 128)
    with pytest.raises(fa.FAError) as e:
        fa.fa_block_mask_dims(256, 256, 64, 64)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    with pytest.raises(fa.FAError) as e:
        fa.fa_block_mask_dims(0, 256)
    assert e.value.status == fa.FA_ERR_SHAPE


def _args(B=1, Hq=2, Hkv=2, Sq=256, Skv=256, D=64, ptr=0x10000):
    a = fa.AttnArgs()
    a.q = a.k = a.v = a.o = ptr
    for name, (H, S) in (("q_stride", (Hq, Sq)), ("k_stride", (Hkv, Skv)), ("v_stride", (Hkv, Skv)),
                         ("o_stride", (Hq, Sq))):
        st = getattr(a, name)
        st[0], st[1], st[2], st[3] = H * S * D, S * D, D, 1
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.D = B, Hq, Hkv, Sq, Skv, D
    return a


def _status(a, decode=False):
    L = fa.lib()
    if decode:
        n = ctypes.c_size_t()
        return L.fa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n))
    return L.fa_forward(ctypes.byref(a), None)


def test_forward_validation_codes():
    a = _args(); a.q = None
    assert _status(a) == fa.FA_ERR_NULL
    a = _args(Hq=3, Hkv=2)
    assert _status(a) == fa.FA_ERR_SHAPE
    a = _args(D=96)
    assert _status(a) == fa.FA_ERR_UNSUPPORTED
    a = _args(); a.q_stride[3] = 2
    assert _status(a) == fa.FA_ERR_UNSUPPORTED
    a = _args(); a.q = 0x10008  # not 16-byte aligned
    assert _status(a) == fa.FA_ERR_UNSUPPORTED
    a = _args(); a.score.kind = 9
    assert _status(a) == fa.FA_ERR_UNSUPPORTED
    a = _args(); a.score.kind = fa.SCORE_SOFTCAP; a.score.softcap = 0.0
    assert _status(a) == fa.FA_ERR_SHAPE
    a = _args(); a.score.kind = fa.SCORE_BIAS
    assert _status(a) == fa.FA_ERR_NULL
    a = _args(); a.B = 0
    assert _status(a) == fa.FA_ERR_SHAPE
    assert "sizes must be positive" in fa.lib().fa_last_error().decode()
    a = _args(); a.scale = -1.0
    assert _status(a) == fa.FA_ERR_SHAPE
    a = _args(); a.scale = 1e-30  # too small for the preloaded key-offset term
    assert _status(a) == fa.FA_ERR_SHAPE
    assert "scale" in fa.lib().fa_last_error().decode()
    # K/V rows are addressed with 32-bit offsets inside a 64-key sub-tile
    for name in ("k_stride", "v_stride"):
        a = _args(); getattr(a, name)[2] = 1 << 25
        assert _status(a) == fa.FA_ERR_UNSUPPORTED
        assert "row stride" in fa.lib().fa_last_error().decode()
        a = _args(); getattr(a, name)[2] = (1 << 25) - 8
        assert _status(a) != fa.FA_ERR_UNSUPPORTED


def _bm(Bm=1, Hm=1, NQ=2, NK=2, kind=fa.MASK_CAUSAL, Sq=256, Skv=256):
    b = fa.BlockMaskC()
    b.kv_num_blocks = b.kv_indices = b.full_kv_num_blocks = b.full_kv_indices = 0x10000
    b.Bm, b.Hm, b.NQ, b.NK = Bm, Hm, NQ, NK
    b.block_q = b.block_kv = 128
    b.separate_full = 1
    b.Sq, b.Skv = Sq, Skv
    b.mask.kind = kind
    return b


def test_blockmask_validation_codes():
    L = fa.lib()
    b = _bm(NQ=3)
    assert L.fa_build_block_mask(ctypes.byref(b), 256, 256, None) == fa.FA_ERR_SHAPE
    b = _bm(); b.block_q = 64
    assert L.fa_build_block_mask(ctypes.byref(b), 256, 256, None) == fa.FA_ERR_UNSUPPORTED
    b = _bm(kind=fa.MASK_DOCUMENT)
    assert L.fa_build_block_mask(ctypes.byref(b), 256, 256, None) == fa.FA_ERR_NULL
    b = _bm(kind=fa.MASK_SLIDING_CAUSAL); b.mask.window = -1
    assert L.fa_build_block_mask(ctypes.byref(b), 256, 256, None) == fa.FA_ERR_SHAPE
    b = _bm(kind=fa.MASK_KV_LEN)
    assert L.fa_build_block_mask(ctypes.byref(b), 256, 256, None) == fa.FA_ERR_NULL
    b = _bm(); b.kv_indices = None
    assert L.fa_build_block_mask(None, 256, 256, None) == fa.FA_ERR_NULL
    assert L.fa_build_block_mask(ctypes.byref(b), 256, 256, None) == fa.FA_ERR_NULL
    # the forward rejects a BlockMask built for other lengths, or with a bad broadcast
    a = _args(B=2); b = _bm(Sq=200)
    a.block_mask = ctypes.pointer(b)
    assert _status(a) == fa.FA_ERR_SHAPE
    a = _args(B=2); b = _bm(Bm=3)
    a.block_mask = ctypes.pointer(b)
    assert _status(a) == fa.FA_ERR_SHAPE
    a = _args(B=2); b = _bm(kind=fa.MASK_KV_LEN); b.mask.kv_len = 0x10000
    a.block_mask = ctypes.pointer(b)
    assert _status(a) == fa.FA_ERR_SHAPE  # batch-dependent mask with Bm = 1 < B
    a = _args(); b = _bm(kind=fa.MASK_DOCUMENT, Skv=300, NK=3); b.mask.doc_ids = 0x10000
    a.Skv = 300; a.block_mask = ctypes.pointer(b)
    assert _status(a) == fa.FA_ERR_SHAPE  # document masks need Sq == Skv


def test_decode_validation_and_workspace_size():
    a = _args(B=2, Hq=8, Hkv=2, Sq=1, Skv=5000, D=128)
    n = ctypes.c_size_t()
    assert fa.lib().fa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == fa.FA_OK
    # 40 kv tiles, B*Hkv = 4: the automatic plan shrinks chunks to one tile
    # (the grid stays below 4096 workgroups), so 40 splits.
    assert n.value == 40 * 2 * 8 * (128 + 1) * 4
    # explicit num_splits: chunk = clamp(ceil(40 / n), 1, 8) tiles, splits = ceil(40 / chunk)
    for ns, splits in ((7, 7), (3, 5), (40, 40), (100, 40), (1, 5)):
        a.num_splits = ns
        assert fa.lib().fa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == fa.FA_OK
        assert n.value == splits * 2 * 8 * (128 + 1) * 4, ns
    a.num_splits = 0
    a.B, a.Hkv, a.Hq, a.Skv = 32, 8, 32, 32768  # 256 tiles, 256 (b, kv head) pairs: 7-tile chunks
    assert fa.lib().fa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == fa.FA_OK
    assert n.value == 37 * 32 * 32 * (128 + 1) * 4
    a = _args(Sq=2)
    assert _status(a, decode=True) == fa.FA_ERR_SHAPE
    a = _args(Hq=6, Hkv=2, Sq=1)
    assert _status(a, decode=True) == fa.FA_ERR_UNSUPPORTED
    a = _args(Sq=1, Skv=512)
    assert fa.lib().fa_decode(ctypes.byref(a), None, 0, None) == fa.FA_ERR_WORKSPACE


def test_binding_rejects_mismatched_tensors():
    """The binding checks what the C ABI cannot see (it takes B, Hq, Sq, D from q
    and Hkv, Skv from k, and gets out/lse as bare pointers) before any call."""
    import torch
    bf = torch.bfloat16
    q = torch.zeros((2, 4, 64, 64), dtype=bf)
    k = torch.zeros((2, 2, 96, 64), dtype=bf)
    cases = [
        dict(q=q.float(), k=k, v=k),                                  # dtype
        dict(q=q[0], k=k, v=k),                                       # rank
        dict(q=q, k=torch.zeros((1, 2, 96, 64), dtype=bf), v=k),     # batch of k
        dict(q=q, k=torch.zeros((2, 2, 96, 128), dtype=bf), v=k),    # head dim of k
        dict(q=q, k=k, v=torch.zeros((2, 2, 80, 64), dtype=bf)),     # v differs from k
        dict(q=q, k=k, v=k, out=torch.zeros((2, 4, 63, 64), dtype=bf)),
        dict(q=q, k=k, v=k, lse=torch.zeros((2, 4, 64), dtype=torch.float64)),
        dict(q=q, k=k, v=k, lse=torch.zeros((2, 64, 4), dtype=torch.float32).transpose(1, 2)),
        dict(q=q, k=k, v=k),                                          # right shapes, host memory
    ]
    for c in cases:
        with pytest.raises(fa.FAError) as e:
            fa.fa_forward(c["q"], c["k"], c["v"], out=c.get("out"), lse=c.get("lse"))
        assert e.value.status == fa.FA_ERR_SHAPE, c


def test_paged_cache_validation():
    """A page table is for fa_decode only; its page count and row stride are checked on the host."""
    a = _args(Hq=4, Hkv=1, Sq=1, Skv=1000, D=128)
    a.page_table = 0x20000
    a.num_pages = 16
    a.page_table_stride = 8                       # ceil(1000 / 128) = 8
    assert _status(a) == fa.FA_ERR_UNSUPPORTED    # fa_forward
    n = ctypes.c_size_t()
    assert fa.lib().fa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == fa.FA_OK
    assert n.value > 0
    a.page_table_stride = 7
    assert _status(a, decode=True) == fa.FA_ERR_SHAPE
    a.page_table_stride = 8
    a.num_pages = 0
    assert _status(a, decode=True) == fa.FA_ERR_SHAPE


def test_transposed_view_is_all_or_nothing():
    """fa_build_block_mask fills the per-KV-block view only when all four buffers are given."""
    c = fa.BlockMaskC()
    c.kv_num_blocks = c.kv_indices = c.full_kv_num_blocks = c.full_kv_indices = 0x10000
    c.Bm = c.Hm = 1
    c.NQ = c.NK = 2
    c.block_q = c.block_kv = fa.FA_BLOCK
    c.separate_full = 1
    c.mask = fa.MaskMod("causal").desc()
    c.q_num_blocks = c.q_indices = 0x20000      # two of the four
    assert fa.lib().fa_build_block_mask(ctypes.byref(c), 256, 256, None) == fa.FA_ERR_NULL


def test_q_order_needs_nq_at_most_16384():
    """The work order of the query blocks is sorted in one workgroup's LDS, so
    fa_build_block_mask refuses it past 16384 query blocks (before any launch)."""
    S = 128 * 16385
    c = _bm(NQ=16385, NK=1, kind=fa.MASK_NONE, Sq=S, Skv=128)
    c.q_order = 0x30000
    assert fa.lib().fa_build_block_mask(ctypes.byref(c), S, 128, None) == fa.FA_ERR_UNSUPPORTED
    assert b"16384" in fa.lib().fa_last_error()


def test_kv_order_needs_the_transposed_view_and_nk_at_most_16384():
    """kv_order is sorted from the transposed view's counts: refused without that
    view, and past 16384 KV blocks (before any launch)."""
    c = _bm()
    c.kv_order = 0x30000
    assert fa.lib().fa_build_block_mask(ctypes.byref(c), 256, 256, None) == fa.FA_ERR_NULL
    S = 128 * 16385
    c = _bm(NQ=1, NK=16385, kind=fa.MASK_NONE, Sq=128, Skv=S)
    c.q_num_blocks = c.q_indices = c.full_q_num_blocks = c.full_q_indices = 0x20000
    c.kv_order = 0x30000
    assert fa.lib().fa_build_block_mask(ctypes.byref(c), 128, S, None) == fa.FA_ERR_UNSUPPORTED
    assert b"16384" in fa.lib().fa_last_error()


def test_row_order_needs_one_query_block_and_head_row():
    """row_order sorts batch rows of a one-query-block mask (decode): refused for
    NQ > 1 or Hm > 1 (before any launch)."""
    c = _bm(Bm=2, NQ=2, NK=2, kind=fa.MASK_NONE)
    c.row_order = 0x30000
    assert fa.lib().fa_build_block_mask(ctypes.byref(c), 256, 256, None) == fa.FA_ERR_SHAPE
    c = _bm(Bm=2, Hm=2, NQ=1, NK=2, kind=fa.MASK_NONE, Sq=1)
    c.row_order = 0x30000
    assert fa.lib().fa_build_block_mask(ctypes.byref(c), 1, 256, None) == fa.FA_ERR_SHAPE


def _rt_swizzle(D, r):
    # restated from rt_swizzle in block_sparse_attention_fa_amd/csrc/bwd_kernel.hpp
    return 4 * (r & 3) + ((r >> 2) & 3) if D == 128 else (((r >> 1) & 1) << 2) | ((r >> 2) & 3)


@pytest.mark.parametrize("D", [64, 128])
def test_backward_lds_swizzle_is_conflict_free(D):
    """The backward's tile swizzle: no LDS bank conflict for a row read (16 lanes,
    16 consecutive rows, one 16-byte chunk) nor for a transposed read (32 lanes,
    4 consecutive rows x 4 adjacent chunks), and one chunk per lane for all of a
    wave's DMA rows.  64 banks x 4 bytes: a 16-byte chunk covers one of 16 bank
    groups of a 256-byte bank row."""
    cpr = D // 8

    def group(r, c):
        return ((r * D * 2 + 16 * (c ^ _rt_swizzle(D, r))) % 256) // 16

    for r0 in range(0, 128, 16):
        for c in range(cpr):
            assert len({group(r0 + i, c) for i in range(16)}) == 16
    for r0 in range(0, 128, 4):
        for c0 in range(0, cpr, 4):
            assert len({group(r0 + i, c0 + j) for i in range(4) for j in range(4)}) == 16
    step = 16 if D == 128 else 32  # rows between the DMA loads of one lane
    for lrow in range(64):
        assert len({_rt_swizzle(D, lrow + step * i) for i in range(4)}) == 1


def test_backward_validation_codes():
    """fa_backward rejects bad arguments on the host, before any launch."""
    L = fa.lib()

    def grads(ptr=0x10000):
        g = fa.GradArgs()
        g.dout = g.dq = g.dk = g.dv = ptr
        for name in ("dout_stride", "dq_stride", "dk_stride", "dv_stride"):
            st = getattr(g, name)
            st[0], st[1], st[2], st[3] = 2 * 256 * 64, 256 * 64, 64, 1
        return g

    def bwd(a, g, ws=0x20000, nbytes=1 << 30):
        return L.fa_backward(ctypes.byref(a), None if g is None else ctypes.byref(g), ws, nbytes, None)

    a = _args(); a.lse = 0x30000
    n = ctypes.c_size_t()
    assert L.fa_backward_workspace_size(ctypes.byref(a), ctypes.byref(n)) == fa.FA_OK
    assert n.value == 2 * 4 * 1 * 2 * 256            # LSE and Delta, fp32, rows padded to 128
    assert bwd(a, None) == fa.FA_ERR_NULL
    a2 = _args()                                         # no LSE
    assert bwd(a2, grads()) == fa.FA_ERR_NULL
    assert "LSE" in L.fa_last_error().decode()
    g = grads(); g.dq = 0
    assert bwd(a, g) == fa.FA_ERR_NULL
    g = grads(); g.dk = 0x10008                          # not 16-byte aligned
    assert bwd(a, g) == fa.FA_ERR_UNSUPPORTED
    assert bwd(a, grads(), ws=0) == fa.FA_ERR_WORKSPACE
    assert bwd(a, grads(), nbytes=n.value - 4) == fa.FA_ERR_WORKSPACE
    assert bwd(a, grads(), ws=0x20008) == fa.FA_ERR_WORKSPACE
    bm = _bm()                                           # BlockMask without its transposed view
    a.block_mask = ctypes.pointer(bm)
    assert bwd(a, grads()) == fa.FA_ERR_NULL
    assert "transposed view" in L.fa_last_error().decode()


def test_binding_rejects_bad_mask_and_score_tensors():
    """doc_ids, kv_len, alibi_slopes and bias reach the kernels as bare pointers:
    the binding checks their dtype, length and device before any call (dtype and
    shape first, so these run without a GPU)."""
    import torch
    i32, bf = torch.int32, torch.bfloat16
    B, Hq, S = 2, 4, 300
    mask_cases = [
        fa.MaskMod("document_causal", doc_ids=torch.zeros((B, S), dtype=torch.int64)),   # int64 ids
        fa.MaskMod("document", doc_ids=torch.zeros((B, S - 1), dtype=i32)),               # too short
        fa.MaskMod("document", doc_ids=torch.zeros((S, B), dtype=i32).t()),              # strided tokens
        fa.MaskMod("document", doc_ids=None),
        fa.MaskMod("document", doc_ids=torch.zeros((B, S), dtype=i32)),                   # host memory
        fa.MaskMod("kv_len", kv_len=torch.full((B,), 7, dtype=torch.int64)),               # int64 lengths
        fa.MaskMod("kv_len", kv_len=torch.full((B - 1,), 7, dtype=i32)),                   # too few
        fa.MaskMod("kv_len", kv_len=torch.full((B,), 7, dtype=i32)),                       # host memory
    ]
    for m in mask_cases:
        with pytest.raises(fa.FAError) as e:
            fa.fa_build_block_mask(m, B, 1, S, S)
        assert e.value.status == fa.FA_ERR_SHAPE
    fa.MaskMod("causal").check(B, S, S)  # masks without tensors have nothing to check
    score_cases = [
        fa.ScoreMod("alibi", alibi_slopes=torch.ones(Hq, dtype=torch.float64)),
        fa.ScoreMod("alibi", alibi_slopes=torch.ones(Hq - 1)),
        fa.ScoreMod("alibi", alibi_slopes=torch.ones(Hq)),                                 # host memory
        fa.ScoreMod("bias", bias=torch.zeros((B, Hq, S, S), dtype=torch.float32)),         # fp32 bias
        fa.ScoreMod("bias", bias=torch.zeros((Hq, S, S), dtype=bf)),                       # 3-d
        fa.ScoreMod("bias", bias=torch.zeros((B, Hq, S, S - 8), dtype=bf)),                # too few keys
        fa.ScoreMod("bias", bias=torch.zeros((B, 2, S, S), dtype=bf)),                     # 2 of 4 heads
        fa.ScoreMod("bias", bias=torch.zeros((1, 1, S, S), dtype=bf)),                     # host memory
        fa.ScoreMod("bias"),
    ]
    for sm in score_cases:
        with pytest.raises(fa.FAError) as e:
            sm.check(B, Hq, S, S)
        assert e.value.status == fa.FA_ERR_SHAPE
    fa.ScoreMod("alibi").check(B, Hq, S, S)  # default slopes: nothing to check


def test_decode_accepts_only_position_free_masks_and_forward_rejects_q_pos():
    """The decode BlockMask has one query row built at q index 0, so fa_decode
    takes only the masks that do not look at the query position (none, kv_len);
    q_pos belongs to fa_decode alone."""
    n = ctypes.c_size_t()
    for kind in range(fa.MASK_KV_LEN + 1):
        a = _args(B=1, Hq=2, Hkv=2, Sq=1, Skv=512, D=128)
        b = _bm(kind=kind, Sq=1, Skv=512, NQ=1, NK=4)
        b.mask.kv_len = b.mask.doc_ids = 0x10000
        if kind in (fa.MASK_DOCUMENT, fa.MASK_DOCUMENT_CAUSAL):
            continue  # already rejected for Sq != Skv
        a.block_mask = ctypes.pointer(b)
        st = fa.lib().fa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n))
        want = fa.FA_OK if kind in (fa.MASK_NONE, fa.MASK_KV_LEN) else fa.FA_ERR_UNSUPPORTED
        assert st == want, (kind, st)
        if st != fa.FA_OK:
            assert "query" in fa.lib().fa_last_error().decode()
    a = _args(Sq=1)
    a.q_pos = 0x10000
    assert fa.lib().fa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == fa.FA_OK
    assert _status(a) == fa.FA_ERR_UNSUPPORTED  # fa_forward


def test_probe_validation_codes():
    L = fa.lib()
    f = ctypes.c_double()
    assert L.fa_probe_mfma(1, 1, 0, None, ctypes.byref(f), None) == fa.FA_ERR_NULL
    assert L.fa_probe_mfma(0, 1, 0, 0x10000, ctypes.byref(f), None) == fa.FA_ERR_SHAPE
    assert L.fa_probe_mfma(1, 0, 1, 0x10000, ctypes.byref(f), None) == fa.FA_ERR_SHAPE
    assert L.fa_probe_copy(None, 0x10000, 16, None) == fa.FA_ERR_NULL
    assert L.fa_probe_copy(0x10000, 0x20000, 0, None) == fa.FA_ERR_SHAPE
    assert L.fa_probe_copy(0x10000, 0x20000, 24, None) == fa.FA_ERR_SHAPE
    assert L.fa_probe_copy(0x10008, 0x20000, 32, None) == fa.FA_ERR_UNSUPPORTED
    assert L.fa_probe_read(None, 16, 0x20000, 1, None) == fa.FA_ERR_NULL
    assert L.fa_probe_read(0x10000, 24, 0x20000, 1, None) == fa.FA_ERR_SHAPE
    assert L.fa_probe_read(0x10008, 32, 0x20000, 1, None) == fa.FA_ERR_UNSUPPORTED
    assert L.fa_probe_read(0x10000, 1 << 30, 0x20000, 8191, None) == fa.FA_ERR_SHAPE   # needs 8192 sink words


def test_noalloc_decode_size_limit_is_checked_on_the_host():
    """fa_decode_noalloc rejects a decode whose workspace would exceed the library's
    scratch (FA_DECODE_SCRATCH_BYTES = 32 MiB) before any HIP call."""
    a = _args(B=64, Hq=64, Hkv=8, Sq=1, Skv=32768, D=128)
    n = ctypes.c_size_t()
    assert fa.lib().fa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == fa.FA_OK
    assert n.value > (32 << 20)
    assert fa.lib().fa_decode_noalloc(ctypes.byref(a), None) == fa.FA_ERR_WORKSPACE
    assert "scratch" in fa.lib().fa_last_error().decode()
    a = _args(Sq=2)
    assert fa.lib().fa_decode_noalloc(ctypes.byref(a), None) == fa.FA_ERR_SHAPE


def test_binding_structs_match_the_c_layout(tmp_path):
    """Every ctypes struct of the binding has the size and field offsets the C
    compiler gives the matching struct of include/fa.h (a mismatch would pass
    wrong values through the ABI without any error)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    pairs = [("fa_mask_desc", fa.MaskDesc), ("fa_score_desc", fa.ScoreDesc), ("fa_block_mask", fa.BlockMaskC),
             ("fa_attn_args", fa.AttnArgs), ("fa_grad_args", fa.GradArgs)]
    lines = ['#include <stdio.h>', '#include "fa.h"', "int main(void) {"]
    for cname, py in pairs:
        lines.append(f'  printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([cc, "-std=c99", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        c, f, v = line.split()
        got[(c, f)] = int(v)
    for cname, py in pairs:
        assert got[(cname, "sizeof")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, f"{cname}.{fname}"
