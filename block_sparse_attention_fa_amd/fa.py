"""Thin ctypes binding of libfa.so (include/fa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch supplies device memory and the current
stream.  The functions keep the C names:

    fa_block_mask_dims, fa_build_block_mask, fa_forward,
    fa_decode_workspace_size, fa_decode, fa_decode_noalloc,
    fa_backward_workspace_size, fa_backward, fa_probe_mfma, fa_probe_copy

plus small helpers to describe mask_mods / score_mods and to inspect a
BlockMask (ASCII print and sparsity, as on the attention-gym "Concepts"
page, "Inspecting a BlockMask").
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

# --- enums (include/fa.h) ----------------------------------------------------
FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(6)
FA_BLOCK = 128
ABI_VERSION = 6          # the layout of the structs below (include/fa.h FA_ABI_VERSION)
MAX_ORDER_NQ = 16384     # largest NQ (NK) for which fa_build_block_mask can write q_order (kv_order)

MASK_NONE, MASK_CAUSAL, MASK_SLIDING_WINDOW, MASK_SLIDING_CAUSAL = 0, 1, 2, 3
MASK_DOCUMENT, MASK_DOCUMENT_CAUSAL, MASK_PREFIX_LM, MASK_KV_LEN = 4, 5, 6, 7
SCORE_NONE, SCORE_ALIBI, SCORE_SOFTCAP, SCORE_REL_POS, SCORE_BIAS = 0, 1, 2, 3, 4

MASK_KINDS = {"none": MASK_NONE, "causal": MASK_CAUSAL, "sliding_window": MASK_SLIDING_WINDOW,
              "sliding_causal": MASK_SLIDING_CAUSAL, "document": MASK_DOCUMENT,
              "document_causal": MASK_DOCUMENT_CAUSAL, "prefix_lm": MASK_PREFIX_LM, "kv_len": MASK_KV_LEN}
SCORE_KINDS = {"none": SCORE_NONE, "alibi": SCORE_ALIBI, "softcap": SCORE_SOFTCAP,
               "rel_pos": SCORE_REL_POS, "bias": SCORE_BIAS}


class MaskDesc(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("window", c_int32), ("prefix_len", c_int32), ("reserved0", c_int32),
                ("doc_ids", c_void_p), ("doc_stride_b", c_int64), ("kv_len", c_void_p)]


class ScoreDesc(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("softcap", c_float), ("alibi_slopes", c_void_p),
                ("bias", c_void_p), ("bias_stride", c_int64 * 4)]


class BlockMaskC(ctypes.Structure):
    _fields_ = [("kv_num_blocks", c_void_p), ("kv_indices", c_void_p),
                ("full_kv_num_blocks", c_void_p), ("full_kv_indices", c_void_p),
                ("Bm", c_int32), ("Hm", c_int32), ("NQ", c_int32), ("NK", c_int32),
                ("block_q", c_int32), ("block_kv", c_int32), ("separate_full", c_int32),
                ("Sq", c_int32), ("Skv", c_int32), ("mask", MaskDesc),
                ("q_num_blocks", c_void_p), ("q_indices", c_void_p),
                ("full_q_num_blocks", c_void_p), ("full_q_indices", c_void_p),
                ("q_order", c_void_p), ("kv_order", c_void_p), ("row_order", c_void_p)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("o", c_void_p), ("lse", c_void_p),
                ("q_stride", c_int64 * 4), ("k_stride", c_int64 * 4), ("v_stride", c_int64 * 4),
                ("o_stride", c_int64 * 4),
                ("B", c_int32), ("Hq", c_int32), ("Hkv", c_int32), ("Sq", c_int32), ("Skv", c_int32),
                ("D", c_int32), ("scale", c_float), ("block_mask", POINTER(BlockMaskC)),
                ("score", ScoreDesc), ("num_splits", c_int32),
                ("page_table", c_void_p), ("page_table_stride", c_int64), ("num_pages", c_int32),
                ("q_pos", c_void_p)]


class GradArgs(ctypes.Structure):
    _fields_ = [("dout", c_void_p), ("dout_stride", c_int64 * 4),
                ("dq", c_void_p), ("dk", c_void_p), ("dv", c_void_p),
                ("dq_stride", c_int64 * 4), ("dk_stride", c_int64 * 4), ("dv_stride", c_int64 * 4)]


# symbol -> (restype, argtypes)
SIGNATURES = {
    "fa_abi_version": (c_int32, []),
    "fa_status_string": (c_char_p, [c_int32]),
    "fa_last_error": (c_char_p, []),
    "fa_block_mask_dims": (c_int32, [c_int32, c_int32, c_int32, c_int32, POINTER(c_int32), POINTER(c_int32)]),
    "fa_build_block_mask": (c_int32, [POINTER(BlockMaskC), c_int32, c_int32, c_void_p]),
    "fa_forward": (c_int32, [POINTER(AttnArgs), c_void_p]),
    "fa_decode_workspace_size": (c_int32, [POINTER(AttnArgs), POINTER(c_size_t)]),
    "fa_decode": (c_int32, [POINTER(AttnArgs), c_void_p, c_size_t, c_void_p]),
    "fa_decode_noalloc": (c_int32, [POINTER(AttnArgs), c_void_p]),
    "fa_backward_workspace_size": (c_int32, [POINTER(AttnArgs), POINTER(c_size_t)]),
    "fa_backward": (c_int32, [POINTER(AttnArgs), POINTER(GradArgs), c_void_p, c_size_t, c_void_p]),
    "fa_probe_mfma": (c_int32, [c_int32, c_int32, c_int32, c_void_p, POINTER(ctypes.c_double), c_void_p]),
    "fa_probe_copy": (c_int32, [c_void_p, c_void_p, c_size_t, c_void_p]),
    "fa_probe_read": (c_int32, [c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]),
}


class FAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def lib():
    """The loaded libfa.so.  Raises if it has not been built: there is no fallback path.

    torch is imported first: its HIP runtime must be the one libfa.so binds to
    (loaded the other way round, the process would hold two HIP runtimes and
    the library's launches would not see torch's streams)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_sparse_attention_fa_amd._build`")
        import torch  # noqa: F401  (see above)
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        if l.fa_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI version {l.fa_abi_version()}, this binding needs "
                              f"{ABI_VERSION}: rebuild it")
        _lib = l
    return _lib


def _check(status: int):
    if status != FA_OK:
        L = lib()
        raise FAError(status, f"{L.fa_status_string(status).decode()}: {L.fa_last_error().decode()}")


def _torch_stream(stream):
    """The stream a call runs on as a torch stream object: the current stream for
    None, a torch stream as given, or a raw hipStream_t handle wrapped."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if hasattr(stream, "cuda_stream"):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _stream(stream):
    return c_void_p(_torch_stream(stream).cuda_stream)


def _on(stream):
    """Context in which the binding allocates what a call writes (outputs it
    creates, workspaces): the call's own stream, so the caching allocator never
    hands that memory to other work while the call's kernels still use it."""
    import torch
    return torch.cuda.stream(_torch_stream(stream))


def _need(cond, msg):
    if not cond:
        raise FAError(FA_ERR_SHAPE, msg)


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


# --- descriptors ---------------------------------------------------------------

class MaskMod:
    """A mask_mod kind with its runtime parameters (tensors stay referenced here)."""

    def __init__(self, kind="none", window=0, prefix_len=0, doc_ids=None, kv_len=None):
        self.kind = MASK_KINDS[kind] if isinstance(kind, str) else int(kind)
        self.window, self.prefix_len = int(window), int(prefix_len)
        self.doc_ids, self.kv_len = doc_ids, kv_len

    def check(self, B, Sq, Skv):
        """What the C ABI cannot see behind the raw pointers: dtype, layout, length
        and device of doc_ids ([S] or [1 or >= B, S] int32, unit stride along
        tokens, S >= max(Sq, Skv)) and kv_len ([>= B] int32, contiguous).
        Checks run dtype and shape first, device last.  Raises FAError(FA_ERR_SHAPE)."""
        import torch
        if self.kind in (MASK_DOCUMENT, MASK_DOCUMENT_CAUSAL):
            d = self.doc_ids
            _need(d is not None, "a document mask needs doc_ids")
            _need(d.dtype == torch.int32, f"doc_ids must be torch.int32 (got {d.dtype})")
            _need(d.dim() in (1, 2) and d.stride(-1) == 1, "doc_ids must be [S] or [B, S] with unit stride along S")
            _need(d.shape[-1] >= max(Sq, Skv), f"doc_ids has {d.shape[-1]} tokens, the call needs {max(Sq, Skv)}")
            _need(d.dim() == 1 or d.shape[0] == 1 or d.shape[0] >= B,
                  f"doc_ids has {d.shape[0]} batch rows, the call has B={B}")
            _need(d.is_cuda, "doc_ids must be on the GPU")
        if self.kind == MASK_KV_LEN:
            t = self.kv_len
            _need(t is not None, "a kv_len mask needs kv_len")
            _need(t.dtype == torch.int32, f"kv_len must be torch.int32 (got {t.dtype})")
            _need(t.dim() == 1 and t.stride(0) == 1, "kv_len must be a contiguous 1-d tensor")
            _need(t.shape[0] >= B, f"kv_len has {t.shape[0]} entries, the call has B={B}")
            _need(t.is_cuda, "kv_len must be on the GPU")

    def desc(self) -> MaskDesc:
        d = MaskDesc()
        d.kind, d.window, d.prefix_len = self.kind, self.window, self.prefix_len
        if self.doc_ids is not None:
            d.doc_ids = self.doc_ids.data_ptr()
            d.doc_stride_b = self.doc_ids.stride(0) if self.doc_ids.dim() == 2 and self.doc_ids.shape[0] > 1 else 0
        if self.kv_len is not None:
            d.kv_len = self.kv_len.data_ptr()
        return d


class ScoreMod:
    """A score_mod kind with its runtime parameters."""

    def __init__(self, kind="none", softcap=0.0, alibi_slopes=None, bias=None):
        self.kind = SCORE_KINDS[kind] if isinstance(kind, str) else int(kind)
        self.softcap, self.alibi_slopes, self.bias = float(softcap), alibi_slopes, bias

    def check(self, B, Hq, Sq, Skv):
        """What the C ABI cannot see: alibi_slopes must be a contiguous float32
        tensor of >= Hq entries; bias a 4-d bfloat16 tensor whose dims are each 1
        (broadcast) or at least (B, Hq, Sq, Skv), unit stride along keys.  Checks
        run dtype and shape first, device last.  Raises FAError(FA_ERR_SHAPE)."""
        import torch
        if self.kind == SCORE_ALIBI and self.alibi_slopes is not None:
            t = self.alibi_slopes
            _need(t.dtype == torch.float32, f"alibi_slopes must be torch.float32 (got {t.dtype})")
            _need(t.dim() == 1 and t.stride(0) == 1, "alibi_slopes must be a contiguous 1-d tensor")
            _need(t.shape[0] >= Hq, f"alibi_slopes has {t.shape[0]} entries, the call has Hq={Hq}")
            _need(t.is_cuda, "alibi_slopes must be on the GPU")
        if self.kind == SCORE_BIAS:
            t = self.bias
            _need(t is not None, "a bias score needs a bias tensor")
            _need(t.dtype == torch.bfloat16, f"bias must be torch.bfloat16 (got {t.dtype})")
            _need(t.dim() == 4 and t.stride(3) == 1, "bias must be 4-d [B, H, Sq, Skv] with unit stride along keys")
            for i, (n, want) in enumerate(zip(t.shape, (B, Hq, Sq, Skv))):
                _need(n == 1 or n >= want, f"bias dim {i} has size {n}, the call needs 1 or >= {want}")
            _need(t.is_cuda, "bias must be on the GPU")

    def desc(self) -> ScoreDesc:
        d = ScoreDesc()
        d.kind, d.softcap = self.kind, self.softcap
        if self.alibi_slopes is not None:
            d.alibi_slopes = self.alibi_slopes.data_ptr()
        if self.bias is not None:
            d.bias = self.bias.data_ptr()
            for i, s in enumerate(self.bias.stride()):
                d.bias_stride[i] = s if (self.bias.shape[i] > 1 or i == 3) else 0
        return d


class BlockMask:
    """Device BlockMask: the four int32 tensors of the Concepts page's "Key attributes"."""

    def __init__(self, mask: MaskMod, Bm, Hm, Sq, Skv, separate_full=True, device="cuda", transposed=False,
                 order=None):
        import torch
        NQ, NK = fa_block_mask_dims(Sq, Skv)
        self.mask = mask
        self.Bm, self.Hm, self.NQ, self.NK, self.Sq, self.Skv = Bm, Hm, NQ, NK, Sq, Skv
        self.separate_full = bool(separate_full)
        z = dict(dtype=torch.int32, device=device)
        self.kv_num_blocks = torch.empty((Bm, Hm, NQ), **z)
        self.kv_indices = torch.empty((Bm, Hm, NQ, NK), **z)
        self.full_kv_num_blocks = torch.empty((Bm, Hm, NQ), **z)
        self.full_kv_indices = torch.empty((Bm, Hm, NQ, NK), **z)
        self.c = BlockMaskC()
        c = self.c
        c.kv_num_blocks, c.kv_indices = self.kv_num_blocks.data_ptr(), self.kv_indices.data_ptr()
        c.full_kv_num_blocks, c.full_kv_indices = self.full_kv_num_blocks.data_ptr(), self.full_kv_indices.data_ptr()
        c.Bm, c.Hm, c.NQ, c.NK = Bm, Hm, NQ, NK
        c.block_q = c.block_kv = FA_BLOCK
        c.separate_full = 1 if separate_full else 0
        c.mask = mask.desc()
        # transposed view (q_num_blocks / q_indices, for the backward), built on request
        self.transposed = bool(transposed)
        if self.transposed:
            self.q_num_blocks = torch.empty((Bm, Hm, NK), **z)
            self.q_indices = torch.empty((Bm, Hm, NK, NQ), **z)
            self.full_q_num_blocks = torch.empty((Bm, Hm, NK), **z)
            self.full_q_indices = torch.empty((Bm, Hm, NK, NQ), **z)
            c.q_num_blocks, c.q_indices = self.q_num_blocks.data_ptr(), self.q_indices.data_ptr()
            c.full_q_num_blocks, c.full_q_indices = self.full_q_num_blocks.data_ptr(), self.full_q_indices.data_ptr()
        # work order of the query blocks (heaviest first), which the forward
        # follows when it starts its workgroups.  By default only for document
        # masks, whose work per query tile follows the position inside the
        # document; the causal, window and prefix masks already have the
        # heaviest tiles last, which the forward starts first without it.
        # Decode masks (one query block, several batch rows) get the order of
        # their rows instead: fa_decode starts the longest sequences first.
        if order is None:
            order = mask.kind in (MASK_DOCUMENT, MASK_DOCUMENT_CAUSAL) or (NQ == 1 and Hm == 1 and Bm > 1)
        self.q_order = None
        if order and NQ <= MAX_ORDER_NQ:
            self.q_order = torch.empty((Bm, Hm, NQ), **z)
            c.q_order = self.q_order.data_ptr()
        # the same for the KV blocks (the backward's dK/dV pass), from the transposed view
        self.kv_order = None
        if order and self.transposed and NK <= MAX_ORDER_NQ:
            self.kv_order = torch.empty((Bm, Hm, NK), **z)
            c.kv_order = self.kv_order.data_ptr()
        self.row_order = None
        if order and NQ == 1 and Hm == 1 and 1 < Bm <= MAX_ORDER_NQ:
            self.row_order = torch.empty((Bm,), **z)
            c.row_order = self.row_order.data_ptr()

    def list_every_tile(self):
        """Re-encode as "no block skipping": every tile of every row is listed as
        partial (superset encoding), so the forward visits all of them and applies
        the mask_mod everywhere, the way masking through a score_mod would.  Only
        for measuring what block sparsity and mask-free full tiles save."""
        import torch
        self.kv_num_blocks.fill_(self.NK)
        self.kv_indices.copy_(torch.arange(self.NK, dtype=torch.int32, device=self.kv_indices.device)
                              .expand_as(self.kv_indices))
        self.separate_full = False
        self.c.separate_full = 0
        if self.transposed:
            self.q_num_blocks.fill_(self.NQ)
            self.q_indices.copy_(torch.arange(self.NQ, dtype=torch.int32, device=self.q_indices.device)
                                 .expand_as(self.q_indices))
        return self

    def tensors(self):
        t = {"kv_num_blocks": self.kv_num_blocks, "kv_indices": self.kv_indices,
             "full_kv_num_blocks": self.full_kv_num_blocks, "full_kv_indices": self.full_kv_indices}
        if self.transposed:
            t.update({"q_num_blocks": self.q_num_blocks, "q_indices": self.q_indices,
                      "full_q_num_blocks": self.full_q_num_blocks, "full_q_indices": self.full_q_indices})
        return t

    def classes(self):
        """int8 [Bm,Hm,NQ,NK] on the host: 0 empty, 1 partial, 2 full (decoded from the lists)."""
        import numpy as np
        kn = self.kv_num_blocks.cpu().numpy()
        ki = self.kv_indices.cpu().numpy()
        fn = self.full_kv_num_blocks.cpu().numpy()
        fi = self.full_kv_indices.cpu().numpy()
        cls = np.zeros((self.Bm, self.Hm, self.NQ, self.NK), dtype=np.int8)
        for idx in np.ndindex(self.Bm, self.Hm, self.NQ):
            cls[idx][ki[idx][:kn[idx]]] = 1
            cls[idx][fi[idx][:fn[idx]]] = 2
        return cls

    def sparsity(self) -> float:
        """Percentage of tiles that are empty (Concepts, "Inspecting a BlockMask")."""
        cls = self.classes()
        return 100.0 * float((cls == 0).sum()) / float(cls.size)

    def to_string(self, b=0, h=0) -> str:
        """ASCII picture: full '██', partial '░░', empty blank."""
        glyph = {2: "██", 1: "░░", 0: "  "}
        return "\n".join("".join(glyph[int(x)] for x in row).rstrip() for row in self.classes()[b, h])

    __str__ = to_string


# --- entry points (same names as the C ABI) ---------------------------------------

def fa_block_mask_dims(Sq, Skv, block_q=FA_BLOCK, block_kv=FA_BLOCK):
    nq, nk = c_int32(), c_int32()
    _check(lib().fa_block_mask_dims(Sq, Skv, block_q, block_kv, ctypes.byref(nq), ctypes.byref(nk)))
    return nq.value, nk.value


def fa_build_block_mask(mask: MaskMod, Bm, Hm, Sq, Skv, separate_full=True, device="cuda", stream=None,
                        transposed=False, order=None):
    """Allocate a BlockMask and build it on the device (asynchronously on `stream`);
    transposed=True also builds the per-KV-block view the backward needs, and
    order=True the heaviest-first work orders of the query blocks (q_order)
    and, with the transposed view, of the KV blocks (kv_order), and for masks of
    one query block the order of the batch rows (row_order); None: for document
    masks and for masks of one query block over several rows (decode)."""
    mask.check(Bm, Sq, Skv)
    with _on(stream):
        bm = BlockMask(mask, Bm, Hm, Sq, Skv, separate_full, device, transposed, order)
    _check(lib().fa_build_block_mask(ctypes.byref(bm.c), Sq, Skv, _stream(stream)))
    return bm


def _check_tensors(q, k, v, out, lse, paged=False):
    """What the C ABI cannot see from pointers and strides: dtypes, devices, and
    the dims it takes from q and k alone (k's B and D, v's shape, out, lse).
    With a paged cache, k and v are page pools [num_pages, Hkv, FA_BLOCK, D]."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise FAError(FA_ERR_SHAPE, f"{name} must be a 4-d torch.bfloat16 tensor")
    if paged:
        if k.shape[2] != FA_BLOCK or k.shape[3] != q.shape[3] or tuple(v.shape) != tuple(k.shape):
            raise FAError(FA_ERR_SHAPE, f"page pools k {tuple(k.shape)} / v {tuple(v.shape)} must both be "
                                        f"[num_pages, Hkv, {FA_BLOCK}, D={q.shape[3]}]")
    elif k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3] or tuple(v.shape) != tuple(k.shape):
        raise FAError(FA_ERR_SHAPE, f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    if tuple(out.shape) != tuple(q.shape):
        raise FAError(FA_ERR_SHAPE, f"out has shape {tuple(out.shape)}, q has {tuple(q.shape)}")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != tuple(q.shape[:3])):
        raise FAError(FA_ERR_SHAPE, "lse must be a contiguous torch.float32 [B, Hq, Sq] tensor")
    if not all(t.is_cuda for t in (q, k, v, out) + ((lse,) if lse is not None else ())):
        raise FAError(FA_ERR_SHAPE, "every tensor must be on the GPU")


def _attn_args(q, k, v, out, lse, block_mask, score, scale, num_splits, page_table=None):
    import torch
    _check_tensors(q, k, v, out, lse, paged=page_table is not None)
    a = AttnArgs()
    a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", out)):
        arr = getattr(a, name)
        for i, s in enumerate(t.stride()):
            arr[i] = s
    a.B, a.Hq, a.Sq, a.D = q.shape
    a.Hkv, a.Skv = k.shape[1], k.shape[2]
    if page_table is not None:
        if page_table.dtype != torch.int32 or page_table.dim() != 2 or not page_table.is_cuda \
                or page_table.stride(1) != 1 or page_table.shape[0] < q.shape[0]:
            raise FAError(FA_ERR_SHAPE, "page_table must be a torch.int32 [B, blocks] GPU tensor with unit "
                                        "stride along blocks")
        # logical capacity: the BlockMask's KV length, else every block of the table
        a.Skv = block_mask.Skv if block_mask is not None else page_table.shape[1] * FA_BLOCK
        a.page_table = page_table.data_ptr()
        a.page_table_stride = page_table.stride(0)
        a.num_pages = k.shape[0]
    a.scale = float(scale)
    if block_mask is not None:
        block_mask.mask.check(a.B, a.Sq, a.Skv)
    score = score or ScoreMod()
    score.check(a.B, a.Hq, a.Sq, a.Skv)
    a.block_mask = ctypes.pointer(block_mask.c) if block_mask is not None else None
    a.score = score.desc()
    a.num_splits = int(num_splits)
    return a


def fa_forward(q, k, v, block_mask: BlockMask | None = None, score: ScoreMod | None = None,
               scale=0.0, out=None, lse=None, stream=None):
    """O = softmax(mod(Q K^T * scale)) V for bf16 Q [B,Hq,Sq,D], K/V [B,Hkv,Skv,D]."""
    import torch
    if out is None:
        _check_tensors(q, k, v, q, lse)  # before touching the device
        with _on(stream):
            out = torch.empty_like(q)
    a = _attn_args(q, k, v, out, lse, block_mask, score, scale, 0)
    _check(lib().fa_forward(ctypes.byref(a), _stream(stream)))
    return out


def fa_decode_workspace_size(q, k, v, block_mask=None, score=None, num_splits=0, page_table=None):
    a = _attn_args(q, k, v, q, None, block_mask, score, 0.0, num_splits, page_table)
    n = c_size_t()
    _check(lib().fa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    return n.value


def _decode_args(q, k_cache, v_cache, block_mask, score, scale, num_splits, out, lse, stream, page_table, q_pos):
    import torch
    if q_pos is not None:
        _need(q_pos.dtype == torch.int32 and q_pos.dim() == 1 and q_pos.stride(0) == 1,
              "q_pos must be a contiguous 1-d torch.int32 tensor")
        _need(q_pos.shape[0] >= q.shape[0], f"q_pos has {q_pos.shape[0]} entries, the call has B={q.shape[0]}")
        _need(q_pos.is_cuda, "q_pos must be on the GPU")
    if out is None:
        _check_tensors(q, k_cache, v_cache, q, lse, paged=page_table is not None)  # before touching the device
        with _on(stream):
            out = torch.empty_like(q)
    a = _attn_args(q, k_cache, v_cache, out, lse, block_mask, score, scale, num_splits, page_table)
    a.q_pos = q_pos.data_ptr() if q_pos is not None else None
    return a, out


def fa_decode(q, k_cache, v_cache, block_mask: BlockMask | None = None, score: ScoreMod | None = None,
              scale=0.0, num_splits=0, out=None, lse=None, workspace=None, stream=None, page_table=None,
              q_pos=None):
    """Split-KV decode: q [B,Hq,1,D] against caches [B,Hkv,KV,D], or, with an int32
    page_table [B, blocks], against page pools [num_pages, Hkv, 128, D] where
    logical block j of sequence b is page page_table[b, j].  q_pos (int32 [B],
    optional) is each query token's position, the q index the score_mods see
    (0 when not given); pass kv_len - 1 for the newest token of a causal cache."""
    import torch
    a, out = _decode_args(q, k_cache, v_cache, block_mask, score, scale, num_splits, out, lse, stream,
                          page_table, q_pos)
    n = c_size_t()
    _check(lib().fa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(1, n.value // 4), dtype=torch.float32, device=q.device)
    _check(lib().fa_decode(ctypes.byref(a), c_void_p(workspace.data_ptr()),
                           workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def fa_decode_noalloc(q, k_cache, v_cache, block_mask: BlockMask | None = None, score: ScoreMod | None = None,
                      scale=0.0, num_splits=0, out=None, lse=None, stream=None, page_table=None, q_pos=None):
    """fa_decode with the library's own scratch instead of a workspace: the C call
    allocates nothing (pass `out` to keep this wrapper from allocating either).
    Calls on one GPU share the scratch and must not overlap."""
    a, out = _decode_args(q, k_cache, v_cache, block_mask, score, scale, num_splits, out, lse, stream,
                          page_table, q_pos)
    _check(lib().fa_decode_noalloc(ctypes.byref(a), _stream(stream)))
    return out


def fa_backward_workspace_size(q, k, v, out, lse, block_mask=None, score=None):
    a = _attn_args(q, k, v, out, lse, block_mask, score, 0.0, 0)
    n = c_size_t()
    _check(lib().fa_backward_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    return n.value


def fa_backward(q, k, v, out, lse, dout, block_mask: BlockMask | None = None, score: ScoreMod | None = None,
                scale=0.0, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """dQ, dK, dV of fa_forward(q, k, v, ...) for the upstream gradient dout.

    out and lse are what fa_forward returned for the same arguments; a
    BlockMask must have been built with transposed=True.  Returns (dq, dk, dv)."""
    import torch
    if block_mask is not None and not block_mask.transposed:
        raise FAError(FA_ERR_NULL, "the backward needs a BlockMask built with transposed=True")
    if lse is None:
        raise FAError(FA_ERR_NULL, "the backward needs the forward's lse")
    _check_tensors(q, k, v, out, lse)  # before touching the device
    with _on(stream):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dout", dout, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != tuple(ref.shape) or not t.is_cuda:
            raise FAError(FA_ERR_SHAPE, f"{name} must be a torch.bfloat16 GPU tensor shaped {tuple(ref.shape)}")
    a = _attn_args(q, k, v, out, lse, block_mask, score, scale, 0)
    g = GradArgs()
    g.dout, g.dq, g.dk, g.dv = dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    for name, t in (("dout_stride", dout), ("dq_stride", dq), ("dk_stride", dk), ("dv_stride", dv)):
        arr = getattr(g, name)
        for i, st in enumerate(t.stride()):
            arr[i] = st
    n = c_size_t()
    _check(lib().fa_backward_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(4, n.value // 4), dtype=torch.float32, device=q.device)
    _check(lib().fa_backward(ctypes.byref(a), ctypes.byref(g), c_void_p(workspace.data_ptr()),
                             workspace.numel() * workspace.element_size(), _stream(stream)))
    return dq, dk, dv


# --- measurement probes ------------------------------------------------------------

def fa_probe_mfma(workgroups, iterations, sink, random_operands=False, stream=None):
    """Launch the bf16 MFMA loop (include/fa.h); returns its flop count.
    sink: float32 GPU tensor of >= workgroups * 256 elements."""
    import torch
    _need(sink.dtype == torch.float32 and sink.is_cuda and sink.numel() >= workgroups * 256,
          "sink must be a float32 GPU tensor of >= workgroups * 256 elements")
    flops = ctypes.c_double()
    _check(lib().fa_probe_mfma(int(workgroups), int(iterations), 1 if random_operands else 0,
                               c_void_p(sink.data_ptr()), ctypes.byref(flops), _stream(stream)))
    return flops.value


def fa_probe_copy(src, dst, stream=None):
    """Streaming copy of src's bytes into dst (GPU tensors of equal byte size)."""
    n = src.numel() * src.element_size()
    _need(src.is_cuda and dst.is_cuda and dst.numel() * dst.element_size() == n and src.is_contiguous()
          and dst.is_contiguous(), "src and dst must be contiguous GPU tensors of the same byte size")
    _check(lib().fa_probe_copy(c_void_p(src.data_ptr()), c_void_p(dst.data_ptr()), n, _stream(stream)))


def fa_probe_read(src, sink, stream=None):
    """Read-only stream over src's bytes (a contiguous GPU tensor); sink: int32 GPU
    tensor of >= min(8192, ceil(bytes / 16384)) elements."""
    n = src.numel() * src.element_size()
    _need(src.is_cuda and src.is_contiguous() and sink.is_cuda and sink.element_size() == 4,
          "src must be a contiguous GPU tensor and sink a 4-byte GPU tensor")
    _check(lib().fa_probe_read(c_void_p(src.data_ptr()), n, c_void_p(sink.data_ptr()), sink.numel(), _stream(stream)))
