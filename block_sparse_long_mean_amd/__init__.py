"""Python binding of libbsa (block-sparse attention for MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libbsa.so, called through its C ABI (include/bsa.h).  PyTorch
supplies device memory (outputs and workspaces) and the current stream.
There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "lib",
    "BsaError",
    "sparse_attn_prefill",
    "select_blocks",
    "sparse_attn_decode",
    "sparse_attn_decode_noalloc",
    "block_summary",
    "sparse_attn_backward",
    "backward_workspace_bytes",
    "prefill_workspace_bytes",
    "decode_workspace_bytes",
    "timer_enable",
    "timer_reset",
    "timer_report",
    "version",
    "build_digest",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

BSA_OK, BSA_ERR_INVALID_ARG, BSA_ERR_UNSUPPORTED, BSA_ERR_WORKSPACE, BSA_ERR_HIP = range(5)
BSA_DTYPE_F32, BSA_DTYPE_BF16 = 0, 1
BSA_GATE_PER_HEAD, BSA_GATE_PER_GROUP = 0, 1
MAX_TOPK = 64

_STATUS = {1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "HIP error"}

I64x3 = ctypes.c_int64 * 3
I64x2 = ctypes.c_int64 * 2
VP = ctypes.c_void_p


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Lq", ctypes.c_int32), ("Lk", ctypes.c_int32),
        ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("q", VP), ("q_stride", I64x3),
        ("k", VP), ("k_stride", I64x3),
        ("v", VP), ("v_stride", I64x3),
        ("o", VP), ("o_stride", I64x3),
        ("block", ctypes.c_int32), ("topk", ctypes.c_int32), ("causal", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
        ("index_q", VP), ("iq_stride", I64x3),
        ("index_k", VP), ("ik_stride", I64x3),
        ("Di", ctypes.c_int32),
        ("doc_ids_q", VP), ("doc_ids_k", VP),
        ("rope_theta", ctypes.c_float), ("scale", ctypes.c_float),
        ("pooled", VP),
        ("sel_out", VP),
        ("lse_out", VP),
        ("chunk_tokens", ctypes.c_int32),
        ("chunks_per_pass", ctypes.c_int32),
        ("pooled_hi", VP), ("pooled_lo", VP),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Lc", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("q", VP), ("q_stride", I64x2),
        ("kcache", VP), ("k_stride", I64x3),
        ("vcache", VP), ("v_stride", I64x3),
        ("pooled", VP), ("p_stride", I64x3),
        ("pooled_dtype", ctypes.c_int32),
        ("cache_lens", VP),
        ("block", ctypes.c_int32), ("topk", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("o", VP), ("o_stride", I64x2),
        ("sel_out", VP),
        ("lse_out", VP),
        ("block_table", VP),
        ("table_w", ctypes.c_int32), ("num_pages", ctypes.c_int32),
    ]


class SummaryArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("L", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32), ("block", ctypes.c_int32),
        ("k", VP), ("k_stride", I64x3),
        ("doc_ids", VP),
        ("rope_theta", ctypes.c_float),
        ("pooled", VP),
        ("pooled_dtype", ctypes.c_int32),
        ("k_rot", VP),
        ("pos_out", VP),
        ("plane_hi", VP), ("plane_lo", VP),
    ]


class BackwardArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Lq", ctypes.c_int32), ("Lk", ctypes.c_int32),
        ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("q", VP), ("q_stride", I64x3),
        ("k", VP), ("k_stride", I64x3),
        ("v", VP), ("v_stride", I64x3),
        ("o", VP), ("o_stride", I64x3),
        ("dout", VP), ("do_stride", I64x3),
        ("lse", VP),
        ("sel", VP),
        ("sel_w", ctypes.c_int32),
        ("block", ctypes.c_int32), ("causal", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dq", VP), ("dk", VP), ("dv", VP),
    ]


class BsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libbsa {_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded libbsa.so.  Raises if it has not been built, or if it was built
    from sources other than the tree's (its embedded digest differs)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_long_mean_amd.build`")
        from . import build as _build

        L = ctypes.CDLL(LIB_PATH)
        try:
            fn = L.bsa_build_digest
        except AttributeError:
            raise ImportError(f"{LIB_PATH} predates its sources (no build digest): rebuild it with "
                              f"`python -m block_sparse_long_mean_amd.build`") from None
        fn.argtypes = []
        fn.restype = ctypes.c_char_p
        built, tree = fn().decode(), _build.source_digest()
        if built != tree:
            raise ImportError(f"{LIB_PATH} was built from other sources (library {built}, tree {tree}): rebuild it "
                              f"with `python -m block_sparse_long_mean_amd.build`")
        L.bsa_prefill_workspace_bytes.argtypes = [ctypes.POINTER(PrefillArgs)]
        L.bsa_prefill_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_sparse_attn_prefill.argtypes = [ctypes.POINTER(PrefillArgs), VP, ctypes.c_size_t, VP]
        L.bsa_sparse_attn_prefill.restype = ctypes.c_int32
        L.bsa_select_blocks.argtypes = [ctypes.POINTER(PrefillArgs), VP, ctypes.c_size_t, VP]
        L.bsa_select_blocks.restype = ctypes.c_int32
        L.bsa_sparse_attn_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), VP]
        L.bsa_sparse_attn_decode_noalloc.restype = ctypes.c_int32
        L.bsa_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeArgs)]
        L.bsa_decode_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_sparse_attn_decode.argtypes = [ctypes.POINTER(DecodeArgs), VP, ctypes.c_size_t, VP]
        L.bsa_sparse_attn_decode.restype = ctypes.c_int32
        L.bsa_summary_workspace_bytes.argtypes = [ctypes.POINTER(SummaryArgs)]
        L.bsa_summary_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_block_summary.argtypes = [ctypes.POINTER(SummaryArgs), VP, ctypes.c_size_t, VP]
        L.bsa_block_summary.restype = ctypes.c_int32
        L.bsa_backward_workspace_bytes.argtypes = [ctypes.POINTER(BackwardArgs)]
        L.bsa_backward_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_sparse_attn_backward.argtypes = [ctypes.POINTER(BackwardArgs), VP, ctypes.c_size_t, VP]
        L.bsa_sparse_attn_backward.restype = ctypes.c_int32
        L.bsa_last_error.argtypes = []
        L.bsa_last_error.restype = ctypes.c_char_p
        L.bsa_version.argtypes = []
        L.bsa_version.restype = ctypes.c_int32
        L.bsa_timer_enable.argtypes = [ctypes.c_int32]
        L.bsa_timer_enable.restype = None
        L.bsa_timer_reset.argtypes = []
        L.bsa_timer_reset.restype = None
        L.bsa_timer_report.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        L.bsa_timer_report.restype = ctypes.c_int32
        _lib = L
    return _lib


def _check(st: int):
    if st != BSA_OK:
        raise BsaError(st, lib().bsa_last_error().decode())


def version() -> int:
    return lib().bsa_version()


def build_digest() -> str:
    """Digest of the sources the loaded library was built from."""
    return lib().bsa_build_digest().decode()


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BSA_DTYPE_BF16
    if t.dtype == torch.float32:
        return BSA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _strides(t, n):
    if t.stride(-1) != 1:
        raise ValueError("the innermost dimension must be contiguous")
    return tuple(int(s) for s in t.stride()[:n])


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(nbytes: int, device, workspace=None):
    torch = _torch()
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _gpu(t):
    """Where outputs and workspaces go: the tensor's GPU, or the current GPU when the tensor lives in
    (pinned) host memory."""
    if t.is_cuda:
        return t.device
    torch = _torch()
    return torch.device("cuda", torch.cuda.current_device())


def _doc(d, B, L, device):
    if d is None:
        return None
    torch = _torch()
    d = d.to(device=device, dtype=torch.int32)
    if d.dim() == 1:
        d = d.unsqueeze(0).expand(B, L)
    return d.contiguous()


def _prefill_args(q, k, v, o, *, block, topk, causal, gate, index_q, index_k, doc_ids_q, doc_ids_k,
                  rope_theta, scale, pooled, sel, lse, chunk_tokens=0, chunks_per_pass=0):
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    a = PrefillArgs()
    a.dtype = _dtype_code(q)
    a.B, a.Lq, a.Lk, a.Hq, a.Hkv, a.D = B, Lq, Lk, Hq, Hkv, D
    a.q, a.q_stride = _ptr(q), I64x3(*_strides(q, 3))
    a.k, a.k_stride = _ptr(k), I64x3(*_strides(k, 3))
    if v is not None:
        a.v, a.v_stride = _ptr(v), I64x3(*_strides(v, 3))
    if o is not None:
        a.o, a.o_stride = _ptr(o), I64x3(*_strides(o, 3))
    a.block, a.topk, a.causal = int(block), int(topk), int(bool(causal))
    a.gate_mode = BSA_GATE_PER_GROUP if gate == "group" else BSA_GATE_PER_HEAD
    if index_q is not None:
        a.index_q, a.iq_stride = _ptr(index_q), I64x3(*_strides(index_q, 3))
        a.index_k, a.ik_stride = _ptr(index_k), I64x3(*_strides(index_k, 3))
        a.Di = index_q.shape[-1]
    a.doc_ids_q = _ptr(doc_ids_q)
    a.doc_ids_k = _ptr(doc_ids_k)
    a.rope_theta = float(rope_theta)
    a.scale = 0.0 if scale is None else float(scale)
    if isinstance(pooled, (tuple, list)):
        # the gate's bf16 planes (hi, lo), each [B, Hkv, Nb, Dg]
        a.pooled_hi, a.pooled_lo = _ptr(pooled[0]), _ptr(pooled[1])
    else:
        a.pooled = _ptr(pooled)
    a.sel_out = _ptr(sel)
    a.lse_out = _ptr(lse)
    a.chunk_tokens = int(chunk_tokens)
    a.chunks_per_pass = int(chunks_per_pass)
    return a


# --------------------------------------------------------------------------
# public calls
# --------------------------------------------------------------------------

def prefill_workspace_bytes(q, k, *, block, topk, causal=True, gate="head", index_q=None, index_k=None,
                            doc_ids_q=None, doc_ids_k=None, pooled=None, chunk_tokens: int = 0,
                            chunks_per_pass: int = 0) -> int:
    dq = _doc(doc_ids_q, q.shape[0], q.shape[1], _gpu(q))
    dk = _doc(doc_ids_k, k.shape[0], k.shape[1], _gpu(k))
    a = _prefill_args(q, k, k, q, block=block, topk=topk, causal=causal, gate=gate, index_q=index_q,
                      index_k=index_k, doc_ids_q=dq, doc_ids_k=dk, rope_theta=10000.0, scale=None,
                      pooled=pooled, sel=None, lse=None, chunk_tokens=chunk_tokens,
                      chunks_per_pass=chunks_per_pass)
    n = lib().bsa_prefill_workspace_bytes(ctypes.byref(a))
    if n == 0:
        raise BsaError(BSA_ERR_INVALID_ARG, lib().bsa_last_error().decode())
    return int(n)


def sparse_attn_prefill(q, k, v, block: int, topk: int, causal: bool = True, doc_ids=None, *, gate: str = "head",
                        index_q=None, index_k=None, doc_ids_q=None, doc_ids_k=None, rope_theta: float = 10000.0,
                        scale: float | None = None, pooled=None, return_sel: bool = False,
                        return_lse: bool = False, out=None, workspace=None, stream=None, chunk_tokens: int = 0,
                        chunks_per_pass: int = 0, sel_out=None):
    """Block-sparse attention prefill (see include/bsa.h for the semantics).

    q [B, Lq, Hq, D], k/v [B, Lk, Hkv, D] device tensors (bf16 or fp32).
    `doc_ids` sets both doc_ids_q and doc_ids_k.  Returns o, or a tuple
    (o, sel[, lse]) when return_sel / return_lse are set.  sel_out: optional
    int32 [B, Hs, Lq, topk + causal] contiguous buffer that receives the
    selection (implies return_sel).
    """
    torch = _torch()
    if doc_ids is not None:
        doc_ids_q = doc_ids if doc_ids_q is None else doc_ids_q
        doc_ids_k = doc_ids if doc_ids_k is None else doc_ids_k
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    o = out if out is not None else torch.empty(q.shape, dtype=q.dtype, device=_gpu(q))
    hs = Hkv if gate == "group" else Hq
    sel_shape = (B, hs, Lq, topk + (1 if causal else 0))
    if sel_out is not None:
        if tuple(sel_out.shape) != sel_shape or sel_out.dtype != torch.int32 or not sel_out.is_contiguous():
            raise BsaError(BSA_ERR_INVALID_ARG, f"sel_out must be contiguous int32 {list(sel_shape)}")
        sel, return_sel = sel_out, True
    else:
        sel = torch.empty(sel_shape, dtype=torch.int32, device=_gpu(q)) if return_sel else None
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=_gpu(q)) if return_lse else None
    dq = _doc(doc_ids_q, B, Lq, _gpu(q))
    dk = _doc(doc_ids_k, B, Lk, _gpu(k))
    a = _prefill_args(q, k, v, o, block=block, topk=topk, causal=causal, gate=gate, index_q=index_q, index_k=index_k,
                      doc_ids_q=dq, doc_ids_k=dk, rope_theta=rope_theta, scale=scale, pooled=pooled, sel=sel, lse=lse,
                      chunk_tokens=chunk_tokens, chunks_per_pass=chunks_per_pass)
    n = lib().bsa_prefill_workspace_bytes(ctypes.byref(a))
    if n == 0:
        raise BsaError(BSA_ERR_INVALID_ARG, lib().bsa_last_error().decode())
    ws = _workspace(n, _gpu(q), workspace)
    _check(lib().bsa_sparse_attn_prefill(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(n), _stream(stream)))
    res = [o]
    if return_sel:
        res.append(sel)
    if return_lse:
        res.append(lse)
    return res[0] if len(res) == 1 else tuple(res)


def select_blocks(q, k, block: int, topk: int, causal: bool = True, *, gate: str = "head", index_q=None,
                  index_k=None, doc_ids_q=None, doc_ids_k=None, rope_theta: float = 10000.0, pooled=None,
                  workspace=None, stream=None):
    """Gate + top-k only: returns sel [B, Hs, Lq, topk + causal] int32."""
    torch = _torch()
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    hs = Hkv if gate == "group" else Hq
    sel = torch.empty((B, hs, Lq, topk + (1 if causal else 0)), dtype=torch.int32, device=_gpu(q))
    dq = _doc(doc_ids_q, B, Lq, _gpu(q))
    dk = _doc(doc_ids_k, B, Lk, _gpu(k))
    a = _prefill_args(q, k, None, None, block=block, topk=topk, causal=causal, gate=gate, index_q=index_q,
                      index_k=index_k, doc_ids_q=dq, doc_ids_k=dk, rope_theta=rope_theta, scale=None, pooled=pooled,
                      sel=sel, lse=None)
    # workspace query for the full call is an upper bound of the gate-only need
    a_full = _prefill_args(q, k, k, q, block=block, topk=topk, causal=causal, gate=gate, index_q=index_q,
                           index_k=index_k, doc_ids_q=dq, doc_ids_k=dk, rope_theta=rope_theta, scale=None,
                           pooled=pooled, sel=sel, lse=None)
    n = lib().bsa_prefill_workspace_bytes(ctypes.byref(a_full))
    if n == 0:
        raise BsaError(BSA_ERR_INVALID_ARG, lib().bsa_last_error().decode())
    ws = _workspace(n, _gpu(q), workspace)
    _check(lib().bsa_select_blocks(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(n), _stream(stream)))
    return sel


def _decode_args(q, kcache, vcache, pooled, o, *, block, topk, gate, cache_lens, scale, sel, lse, block_table=None):
    B, Hq, D = q.shape
    Lc, Hkv = kcache.shape[1], kcache.shape[2]
    a = DecodeArgs()
    if block_table is not None:
        # paged caches [pages, block, Hkv, D]; the logical capacity is one block per routing key
        Lc = pooled.shape[1] * int(block)
        a.block_table = _ptr(block_table)
        a.table_w, a.num_pages = block_table.shape[1], kcache.shape[0]
    a.dtype = _dtype_code(q)
    a.B, a.Lc, a.Hq, a.Hkv, a.D = B, Lc, Hq, Hkv, D
    a.q, a.q_stride = _ptr(q), I64x2(*_strides(q, 2))
    a.kcache, a.k_stride = _ptr(kcache), I64x3(*_strides(kcache, 3))
    a.vcache, a.v_stride = _ptr(vcache), I64x3(*_strides(vcache, 3))
    a.pooled, a.p_stride = _ptr(pooled), I64x3(*_strides(pooled, 3))
    a.pooled_dtype = _dtype_code(pooled)
    a.cache_lens = _ptr(cache_lens)
    a.block, a.topk = int(block), int(topk)
    a.gate_mode = BSA_GATE_PER_GROUP if gate == "group" else BSA_GATE_PER_HEAD
    a.scale = 0.0 if scale is None else float(scale)
    if o is not None:
        a.o, a.o_stride = _ptr(o), I64x2(*_strides(o, 2))
    a.sel_out = _ptr(sel)
    a.lse_out = _ptr(lse)
    return a


def decode_workspace_bytes(q, kcache, vcache, pooled, *, block, topk, gate="head", block_table=None) -> int:
    a = _decode_args(q, kcache, vcache, pooled, q, block=block, topk=topk, gate=gate, cache_lens=None, scale=None,
                     sel=None, lse=None, block_table=block_table)
    n = lib().bsa_decode_workspace_bytes(ctypes.byref(a))
    if n == 0:
        raise BsaError(BSA_ERR_INVALID_ARG, lib().bsa_last_error().decode())
    return int(n)


def sparse_attn_decode(q, kcache, vcache, pooled, topk: int, block: int, *, gate: str = "head", cache_lens=None,
                       scale: float | None = None, return_sel: bool = False, return_lse: bool = False, out=None,
                       workspace=None, stream=None, block_table=None):
    """One decode step: q [B, Hq, D], caches [B, Lc, Hkv, D], pooled [B, Nb, Hkv, D].

    With block_table (int32 [B, >= Nb] on the device) the caches are pages [P, block, Hkv, D]
    (any strides) and block j of sequence b is page block_table[b, j]."""
    torch = _torch()
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
            raise BsaError(BSA_ERR_INVALID_ARG, "block_table must be int32 [B, table_w] with unit inner stride")
        if block_table.stride(0) != block_table.shape[1]:
            block_table = block_table.contiguous()
    B, Hq, D = q.shape
    Hkv = kcache.shape[2]
    o = out if out is not None else torch.empty(q.shape, dtype=q.dtype, device=_gpu(q))
    hs = Hkv if gate == "group" else Hq
    sel = torch.empty((B, hs, topk + 1), dtype=torch.int32, device=_gpu(q)) if return_sel else None
    lse = torch.empty((B, Hq), dtype=torch.float32, device=_gpu(q)) if return_lse else None
    if cache_lens is not None:
        cache_lens = cache_lens.to(device=_gpu(q), dtype=torch.int32).contiguous()
    a = _decode_args(q, kcache, vcache, pooled, o, block=block, topk=topk, gate=gate, cache_lens=cache_lens,
                     scale=scale, sel=sel, lse=lse, block_table=block_table)
    n = lib().bsa_decode_workspace_bytes(ctypes.byref(a))
    if n == 0:
        raise BsaError(BSA_ERR_INVALID_ARG, lib().bsa_last_error().decode())
    ws = _workspace(n, _gpu(q), workspace)
    _check(lib().bsa_sparse_attn_decode(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(n), _stream(stream)))
    res = [o]
    if return_sel:
        res.append(sel)
    if return_lse:
        res.append(lse)
    return res[0] if len(res) == 1 else tuple(res)


NOALLOC_MAX_BYTES = 64 << 20  # BSA_DECODE_NOALLOC_MAX_BYTES


def sparse_attn_decode_noalloc(q, kcache, vcache, pooled, topk: int, block: int, *, out, gate: str = "head",
                               cache_lens=None, scale: float | None = None, sel_out=None, lse_out=None,
                               stream=None, block_table=None):
    """sparse_attn_decode through bsa_sparse_attn_decode_noalloc: the library's own per-GPU
    scratch array is the workspace, so the call allocates nothing.  The caller passes every
    output (out, and optionally sel_out [B, Hs, topk + 1] int32 and lse_out [B, Hq] fp32) and
    every input already in the right dtype and on the device (cache_lens int32, block_table
    int32 [B, table_w] contiguous).  Returns out."""
    a = _decode_args(q, kcache, vcache, pooled, out, block=block, topk=topk, gate=gate, cache_lens=cache_lens,
                     scale=scale, sel=sel_out, lse=lse_out, block_table=block_table)
    _check(lib().bsa_sparse_attn_decode_noalloc(ctypes.byref(a), _stream(stream)))
    return out


def block_summary(k, block: int, doc_ids=None, *, rope_theta: float = 10000.0, out_dtype=None,
                  return_k_rot: bool = False, return_pos: bool = False, return_planes: bool = False, stream=None):
    """Mean-pooled block summaries [B, Nb, H, D] (after document-wise RoPE when doc_ids is given).

    return_planes adds the summaries split into the prefill gate's bf16 planes, a tuple
    (hi, lo) of [B, H, Nb, D] tensors: pass it as sparse_attn_prefill's `pooled`."""
    torch = _torch()
    B, L, H, D = k.shape
    nb = -(-L // block)
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    pooled = torch.empty((B, nb, H, D), dtype=out_dtype, device=_gpu(k))
    d = _doc(doc_ids, B, L, _gpu(k))
    k_rot = torch.empty((B, L, H, D), dtype=k.dtype, device=_gpu(k)) if return_k_rot else None
    pos = torch.empty((B, L), dtype=torch.int32, device=_gpu(k)) if return_pos else None
    planes = None
    if return_planes:
        planes = tuple(torch.empty((B, H, nb, D), dtype=torch.bfloat16, device=_gpu(k)) for _ in range(2))
    a = SummaryArgs()
    a.dtype = _dtype_code(k)
    a.B, a.L, a.H, a.D, a.block = B, L, H, D, int(block)
    a.k, a.k_stride = _ptr(k), I64x3(*_strides(k, 3))
    a.doc_ids = _ptr(d)
    a.rope_theta = float(rope_theta)
    a.pooled = _ptr(pooled)
    a.pooled_dtype = _dtype_code(pooled)
    a.k_rot = _ptr(k_rot)
    a.pos_out = _ptr(pos)
    if planes is not None:
        a.plane_hi, a.plane_lo = _ptr(planes[0]), _ptr(planes[1])
    n = lib().bsa_summary_workspace_bytes(ctypes.byref(a))
    if n == 0:
        raise BsaError(BSA_ERR_INVALID_ARG, lib().bsa_last_error().decode())
    ws = _workspace(n, _gpu(k))
    _check(lib().bsa_block_summary(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(n), _stream(stream)))
    res = [pooled]
    if return_k_rot:
        res.append(k_rot)
    if return_pos:
        res.append(pos)
    if return_planes:
        res.append(planes)
    return res[0] if len(res) == 1 else tuple(res)


def _backward_args(q, k, v, o, lse, sel, dout, dq, dk, dv, *, block, causal, gate, scale):
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    a = BackwardArgs()
    a.dtype = _dtype_code(q)
    a.B, a.Lq, a.Lk, a.Hq, a.Hkv, a.D = B, Lq, Lk, Hq, Hkv, D
    a.q, a.q_stride = _ptr(q), I64x3(*_strides(q, 3))
    a.k, a.k_stride = _ptr(k), I64x3(*_strides(k, 3))
    a.v, a.v_stride = _ptr(v), I64x3(*_strides(v, 3))
    a.o, a.o_stride = _ptr(o), I64x3(*_strides(o, 3))
    a.dout, a.do_stride = _ptr(dout), I64x3(*_strides(dout, 3))
    a.lse, a.sel, a.sel_w = _ptr(lse), _ptr(sel), int(sel.shape[-1])
    a.block, a.causal = int(block), int(bool(causal))
    a.gate_mode = BSA_GATE_PER_GROUP if gate == "group" else BSA_GATE_PER_HEAD
    a.scale = 0.0 if scale is None else float(scale)
    a.dq, a.dk, a.dv = _ptr(dq), _ptr(dk), _ptr(dv)
    return a


def backward_workspace_bytes(q, k, sel, *, block, causal, gate="head") -> int:
    # only sizes are read by the query; any non-null pointer stands in for lse
    a = _backward_args(q, k, k, q, q, sel, q, q, k, k, block=block, causal=causal, gate=gate, scale=None)
    n = lib().bsa_backward_workspace_bytes(ctypes.byref(a))
    if n == 0:
        raise BsaError(BSA_ERR_INVALID_ARG, lib().bsa_last_error().decode())
    return int(n)


def sparse_attn_backward(q, k, v, o, lse, sel, dout, block: int, causal: bool, *, gate: str = "head",
                         scale: float | None = None, out=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv), fp32, of the prefill's output through its fixed selection.

    q, k, v: the attended bf16 tensors; o, lse, sel: the forward call's outputs (o, lse [B, Hq, Lq],
    sel [B, Hs, Lq, topk + causal]); dout: dL/do.  out: optional (dq, dk, dv) fp32 contiguous."""
    torch = _torch()
    dev = _gpu(q)
    if out is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
        dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
        dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    else:
        dq, dk, dv = out
    for t in (dq, dk, dv):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise BsaError(BSA_ERR_INVALID_ARG, "dq, dk and dv must be contiguous float32")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or sel.dtype != torch.int32 or not sel.is_contiguous():
        raise BsaError(BSA_ERR_INVALID_ARG, "lse must be contiguous float32 and sel contiguous int32")
    a = _backward_args(q, k, v, o, lse, sel, dout, dq, dk, dv, block=block, causal=causal, gate=gate, scale=scale)
    n = lib().bsa_backward_workspace_bytes(ctypes.byref(a))
    if n == 0:
        raise BsaError(BSA_ERR_INVALID_ARG, lib().bsa_last_error().decode())
    ws = _workspace(n, dev, workspace)
    _check(lib().bsa_sparse_attn_backward(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(n),
                                          _stream(stream)))
    return dq, dk, dv


def timer_enable(level=1):
    """0/False: off; 1/True: every launch, the attention passes as one "attn" phase; 2: every launch."""
    lib().bsa_timer_enable(int(level))


def timer_reset():
    lib().bsa_timer_reset()


def timer_report(kernel: str):
    """(total milliseconds, launch count) of `kernel` since the last reset."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().bsa_timer_report(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
