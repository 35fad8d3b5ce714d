"""The C-ABI library: it loads, exports every symbol include/bsa.h declares,
and rejects bad arguments with the documented status codes before anything
is enqueued (host-only checks; no kernel runs here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


@pytest.fixture(scope="module")
def m():
    import block_sparse_long_mean_amd as m
    from block_sparse_long_mean_amd import build

    if not build.is_current():
        build.build()  # missing, or built from other sources: this CPU-side check builds it
    m.lib()
    return m


def test_library_matches_its_sources(m):
    """The library carries the digest of the sources it was built from, and the
    binding refuses one whose digest differs from the tree's."""
    from block_sparse_long_mean_amd import build

    assert m.build_digest() == build.source_digest()
    assert re.fullmatch(r"[0-9a-f]{16}", m.build_digest())
    saved, real = m._lib, build.source_digest
    try:
        m._lib = None
        build.source_digest = lambda: "0" * 16
        with pytest.raises(ImportError, match="built from other sources"):
            m.lib()
    finally:
        build.source_digest = real
        m._lib = saved


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(m):
    names = declared_functions()
    assert len(names) >= 12, names
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (bsa_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(m.lib(), n)
    # nothing but the C ABI is exported under the bsa_ prefix
    assert exported == set(names), exported - set(names)


def test_version(m):
    assert m.version() >= 100


def _args(m, **kw):
    a = m.PrefillArgs()
    a.dtype = m.BSA_DTYPE_BF16
    a.B, a.Lq, a.Lk, a.Hq, a.Hkv, a.D = 1, 256, 256, 4, 2, 128
    buf = ctypes.create_string_buffer(1 << 16)
    base = (ctypes.addressof(buf) + 255) & ~255
    a.q = a.k = a.v = a.o = base
    a.q_stride = m.I64x3(256 * 4 * 128, 4 * 128, 128)
    a.k_stride = a.v_stride = m.I64x3(256 * 2 * 128, 2 * 128, 128)
    a.o_stride = a.q_stride
    a.block, a.topk, a.causal, a.gate_mode = 64, 2, 1, 0
    for key, val in kw.items():
        setattr(a, key, val)
    return a, buf


@pytest.mark.parametrize("field,value,status", [
    ("B", 0, 1), ("Lq", 0, 1), ("Lk", 0, 1), ("Hkv", 0, 1), ("Hq", 3, 1), ("D", 96, 2), ("block", 0, 1), ("topk", -1, 1), ("topk", 65, 2),
    ("causal", 2, 1), ("gate_mode", 7, 1), ("dtype", 5, 1), ("chunk_tokens", -1, 1),
    ("chunks_per_pass", -2, 1),
])
def test_prefill_rejects_bad_arguments(m, field, value, status):
    a, _buf = _args(m, **{field: value})
    assert m.lib().bsa_prefill_workspace_bytes(ctypes.byref(a)) == 0
    st = m.lib().bsa_sparse_attn_prefill(ctypes.byref(a), None, 0, None)
    assert st == status, (st, m.lib().bsa_last_error())
    assert m.lib().bsa_last_error()


def test_prefill_rejects_2_31_query_rows(m):
    """B * Hq * Lq (in whole query chunks) must stay below 2^31: 64 query heads over 2^25 tokens
    reach it.  Per-group gating keeps the selection entries (one row per kv head) under their own
    bound, and a large block keeps the bucket count small, so this is the bound that applies."""
    L = 1 << 25
    a, _buf = _args(m, Lq=L, Lk=L, Hq=64, Hkv=8, block=1 << 20, topk=2, gate_mode=1)
    a.q_stride = m.I64x3(L * 64 * 128, 64 * 128, 128)
    a.k_stride = a.v_stride = m.I64x3(L * 8 * 128, 8 * 128, 128)
    a.o_stride = a.q_stride
    assert m.lib().bsa_prefill_workspace_bytes(ctypes.byref(a)) == 0
    assert m.lib().bsa_sparse_attn_prefill(ctypes.byref(a), None, 0, None) == m.BSA_ERR_UNSUPPORTED
    assert b"query rows" in m.lib().bsa_last_error()
    a.Hq = 32  # half the rows: planned
    a.q_stride = a.o_stride = m.I64x3(L * 32 * 128, 32 * 128, 128)
    assert m.lib().bsa_prefill_workspace_bytes(ctypes.byref(a)) > 0


def test_prefill_short_workspace(m):
    a, _buf = _args(m)
    need = m.lib().bsa_prefill_workspace_bytes(ctypes.byref(a))
    assert need > 0
    assert m.lib().bsa_sparse_attn_prefill(ctypes.byref(a), None, 0, None) == m.BSA_ERR_WORKSPACE
    assert m.lib().bsa_sparse_attn_prefill(ctypes.byref(a), ctypes.c_void_p(256), need - 1, None) == m.BSA_ERR_WORKSPACE
    # misaligned workspace
    assert m.lib().bsa_sparse_attn_prefill(ctypes.byref(a), ctypes.c_void_p(257), need + 512, None) == m.BSA_ERR_WORKSPACE


def test_prefill_misaligned_and_null(m):
    a, _buf = _args(m)
    a.q = a.q + 2
    assert m.lib().bsa_sparse_attn_prefill(ctypes.byref(a), None, 0, None) == m.BSA_ERR_INVALID_ARG
    a, _buf = _args(m)
    a.v = None
    assert m.lib().bsa_sparse_attn_prefill(ctypes.byref(a), None, 0, None) == m.BSA_ERR_INVALID_ARG
    a, _buf = _args(m, Lq=300)  # causal needs Lq <= Lk
    assert m.lib().bsa_sparse_attn_prefill(ctypes.byref(a), None, 0, None) == m.BSA_ERR_INVALID_ARG
    assert m.lib().bsa_select_blocks(ctypes.byref(_args(m)[0]), None, 0, None) == m.BSA_ERR_INVALID_ARG  # no sel_out


def test_prefill_gate_planes_validation(m):
    """The summaries as the gate's bf16 planes: both planes or neither, not
    together with fp32 `pooled`, bf16 inputs only, 16-byte aligned."""
    a, buf = _args(m)
    base = a.q
    a.pooled_hi = base
    assert m.lib().bsa_prefill_workspace_bytes(ctypes.byref(a)) == 0  # lo missing
    assert m.lib().bsa_sparse_attn_prefill(ctypes.byref(a), None, 0, None) == m.BSA_ERR_INVALID_ARG
    a.pooled_lo = base
    assert m.lib().bsa_prefill_workspace_bytes(ctypes.byref(a)) > 0
    a.pooled = base
    assert m.lib().bsa_prefill_workspace_bytes(ctypes.byref(a)) == 0  # both forms
    a.pooled = None
    a.pooled_lo = base + 2
    assert m.lib().bsa_prefill_workspace_bytes(ctypes.byref(a)) == 0  # misaligned
    a, buf2 = _args(m, dtype=m.BSA_DTYPE_F32)
    a.pooled_hi = a.pooled_lo = a.q
    assert m.lib().bsa_sparse_attn_prefill(ctypes.byref(a), None, 0, None) == m.BSA_ERR_UNSUPPORTED
    s = m.SummaryArgs()
    s.dtype, s.B, s.L, s.H, s.D, s.block = m.BSA_DTYPE_BF16, 1, 100, 2, 128, 64
    s.k = s.pooled = base
    s.k_stride = m.I64x3(100 * 2 * 128, 2 * 128, 128)
    s.pooled_dtype = m.BSA_DTYPE_F32
    s.plane_hi = base
    assert m.lib().bsa_summary_workspace_bytes(ctypes.byref(s)) == 0  # plane_lo missing
    s.plane_lo = base
    assert m.lib().bsa_summary_workspace_bytes(ctypes.byref(s)) > 0


def test_decode_and_summary_validation(m):
    d = m.DecodeArgs()
    d.dtype = m.BSA_DTYPE_F32
    d.B, d.Lc, d.Hq, d.Hkv, d.D = 1, 1024, 4, 2, 128
    assert m.lib().bsa_sparse_attn_decode(ctypes.byref(d), None, 0, None) == m.BSA_ERR_UNSUPPORTED
    d.dtype = m.BSA_DTYPE_BF16
    assert m.lib().bsa_sparse_attn_decode(ctypes.byref(d), None, 0, None) == m.BSA_ERR_INVALID_ARG  # null tensors
    s = m.SummaryArgs()
    s.dtype, s.B, s.L, s.H, s.D, s.block = m.BSA_DTYPE_BF16, 1, 100, 2, 128, 0
    assert m.lib().bsa_block_summary(ctypes.byref(s), None, 0, None) == m.BSA_ERR_INVALID_ARG


def test_decode_block_table_validation(m):
    """Paged caches: the table must cover every logical block and name at least one page."""
    buf = ctypes.create_string_buffer(1 << 12)
    base = (ctypes.addressof(buf) + 255) & ~255  # never dereferenced: only the workspace query runs
    d = m.DecodeArgs()
    d.dtype, d.pooled_dtype = m.BSA_DTYPE_BF16, m.BSA_DTYPE_BF16
    d.B, d.Lc, d.Hq, d.Hkv, d.D, d.block, d.topk = 2, 1000, 8, 2, 128, 64, 4
    d.q = d.kcache = d.vcache = d.pooled = d.o = base
    d.q_stride = m.I64x2(8 * 128, 128)
    d.k_stride = d.v_stride = m.I64x3(64 * 2 * 128, 2 * 128, 128)  # (page, token, head)
    d.p_stride = m.I64x3(16 * 2 * 128, 2 * 128, 128)
    d.o_stride = m.I64x2(8 * 128, 128)
    contiguous = m.lib().bsa_decode_workspace_bytes(ctypes.byref(d))
    assert contiguous > 0
    d.block_table, d.table_w, d.num_pages = base, 16, 40
    assert m.lib().bsa_decode_workspace_bytes(ctypes.byref(d)) == contiguous
    d.table_w = 15  # ceil(1000 / 64) = 16 logical blocks
    assert m.lib().bsa_decode_workspace_bytes(ctypes.byref(d)) == 0
    assert b"table_w" in m.lib().bsa_last_error()
    d.table_w, d.num_pages = 16, 0
    assert m.lib().bsa_decode_workspace_bytes(ctypes.byref(d)) == 0
    assert b"num_pages" in m.lib().bsa_last_error()
    d.num_pages, d.block_table = 40, base + 2
    assert m.lib().bsa_decode_workspace_bytes(ctypes.byref(d)) == 0


def test_backward_validation_and_workspace(m):
    """The backward entry point validates before anything else and sizes its workspace from the
    shapes alone."""
    buf = ctypes.create_string_buffer(1 << 12)
    base = (ctypes.addressof(buf) + 255) & ~255  # never dereferenced: only validation and the query run
    a = m.BackwardArgs()
    a.dtype = m.BSA_DTYPE_BF16
    a.B, a.Lq, a.Lk, a.Hq, a.Hkv, a.D = 1, 512, 512, 8, 2, 128
    for f in ("q", "k", "v", "o", "dout", "lse", "sel", "dq", "dk", "dv"):
        setattr(a, f, base)
    a.q_stride = a.o_stride = a.do_stride = m.I64x3(512 * 8 * 128, 8 * 128, 128)
    a.k_stride = a.v_stride = m.I64x3(512 * 2 * 128, 2 * 128, 128)
    a.sel_w, a.block, a.causal, a.gate_mode = 4, 64, 1, m.BSA_GATE_PER_HEAD
    n = m.lib().bsa_backward_workspace_bytes(ctypes.byref(a))
    assert n > 0
    assert m.lib().bsa_sparse_attn_backward(ctypes.byref(a), None, 0, None) == m.BSA_ERR_WORKSPACE
    a.gate_mode = m.BSA_GATE_PER_GROUP
    assert 0 < m.lib().bsa_backward_workspace_bytes(ctypes.byref(a)) < n  # one selection row per group
    for field, value, status in (("dtype", m.BSA_DTYPE_F32, m.BSA_ERR_UNSUPPORTED), ("D", 96, m.BSA_ERR_UNSUPPORTED),
                                 ("sel_w", 66, m.BSA_ERR_INVALID_ARG), ("causal", 2, m.BSA_ERR_INVALID_ARG),
                                 ("dout", None, m.BSA_ERR_INVALID_ARG), ("Lk", 100, m.BSA_ERR_INVALID_ARG)):
        old = getattr(a, field)
        setattr(a, field, value)
        assert m.lib().bsa_backward_workspace_bytes(ctypes.byref(a)) == 0
        assert m.lib().bsa_sparse_attn_backward(ctypes.byref(a), None, 0, None) == status, field
        setattr(a, field, old)


def test_timer_report_unknown_kernel_is_empty(m):
    m.timer_reset()
    assert m.timer_report("no_such_kernel") == (0.0, 0)


def test_query_chunks_bound_the_workspace(m):
    """Passes over chunks of query tokens keep only one pass's partial outputs."""
    a, _buf = _args(m, Lq=4096, Lk=4096)
    full = m.lib().bsa_prefill_workspace_bytes(ctypes.byref(a))
    a.chunk_tokens, a.chunks_per_pass = 512, 1
    chunked = m.lib().bsa_prefill_workspace_bytes(ctypes.byref(a))
    a.chunks_per_pass = 3
    three = m.lib().bsa_prefill_workspace_bytes(ctypes.byref(a))
    a.chunk_tokens, a.chunks_per_pass = 100000, 1  # more than Lq: one pass per (b, kv head)
    capped = m.lib().bsa_prefill_workspace_bytes(ctypes.byref(a))
    a.chunk_tokens, a.chunks_per_pass = 512, 0  # every chunk in one pass
    single = m.lib().bsa_prefill_workspace_bytes(ctypes.byref(a))
    assert 0 < chunked < three < capped <= full <= single, (chunked, three, capped, full, single)
