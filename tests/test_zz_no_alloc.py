"""The decode entry point that allocates nothing (bsa_sparse_attn_decode_noalloc),
against the decode entry point with a caller's workspace: two calls in a row,
the second on a smaller input (the shared scratch array still holds the first
call's contents), both bitwise equal to the workspace call and checked against
the oracle; and a request above the scratch size is rejected before anything
is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from bsa_testutil import assert_close, check_selection, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    import block_sparse_long_mean_amd as m

    m.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


CASES = [
    # (B, Hq, Hkv, Lc, D, block, topk, gate, lens, seed): the second is smaller in every dimension
    (2, 8, 2, 5000, 128, 128, 8, "head", [5000, 3333], 70),
    (1, 4, 1, 700, 64, 32, 4, "group", [611], 71),
]


def test_noalloc_decode_matches_workspace_decode(bsa):
    for B, Hq, Hkv, Lc, D, block, topk, gate, lens, seed in CASES:
        print(f"case no-alloc decode B{B} H{Hq}/{Hkv} Lc{Lc} D{D} block{block} topk{topk} {gate}", flush=True)
        q = synth.host_tensor((B, Hq, D), 1.0, seed, synth.TID["q"], "bf16")
        k = synth.host_tensor((B, Lc, Hkv, D), 1.0, seed, synth.TID["k"], "bf16")
        v = synth.host_tensor((B, Lc, Hkv, D), 1.0, seed, synth.TID["v"], "bf16")
        pooled = torch.from_numpy(oracle.block_pool(k, block)).to(torch.bfloat16)
        lens_np = np.array(lens, dtype=np.int32)
        qd, kd, vd, pd, ld = q.cuda(), k.cuda(), v.cuda(), pooled.cuda(), torch.from_numpy(lens_np).cuda()
        assert bsa.decode_workspace_bytes(qd, kd, vd, pd, block=block, topk=topk, gate=gate) <= bsa.NOALLOC_MAX_BYTES
        o1, s1, l1 = bsa.sparse_attn_decode(qd, kd, vd, pd, topk, block, gate=gate, cache_lens=ld, return_sel=True,
                                            return_lse=True)
        hs = Hkv if gate == "group" else Hq
        o2 = torch.empty_like(qd)
        s2 = torch.empty((B, hs, topk + 1), dtype=torch.int32, device="cuda")
        l2 = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        bsa.sparse_attn_decode_noalloc(qd, kd, vd, pd, topk, block, out=o2, gate=gate, cache_lens=ld, sel_out=s2,
                                       lse_out=l2)
        torch.cuda.synchronize()
        assert torch.equal(s1, s2)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)
        ref = oracle.decode(q, k, v, pooled, block=block, topk=topk, gate=gate, cache_lens=lens_np,
                            return_scores=True)
        nb = pooled.shape[1]
        scores = np.full((B, hs, 1, nb), np.nan)
        for (b, h), sc in ref["scores"].items():
            scores[b, h, 0, : len(sc)] = sc
        gsel = s2.cpu().numpy()[:, :, None]
        if check_selection(gsel, ref["sel"][:, :, None], scores, topk, True):
            ref = oracle.decode(q, k, v, pooled, block=block, topk=topk, gate=gate, cache_lens=lens_np,
                                force_sel=gsel[:, :, 0])
        assert_close(to_np(o2), ref["o"], 1e-2, 1e-2, bf16_storage=True)
        assert_close(to_np(l2), ref["lse"], 5e-3, None, what="lse")


def test_noalloc_decode_rejects_a_workspace_above_the_limit(bsa):
    """64 sequences over 1,048,576-token caches need more workspace than the scratch array
    holds: the call fails validation with BSA_ERR_WORKSPACE and enqueues nothing (the tensors
    named are small; no kernel could read past them because none is launched)."""
    t = torch.zeros(1 << 16, dtype=torch.bfloat16, device="cuda")
    a = bsa.DecodeArgs()
    a.dtype = bsa.BSA_DTYPE_BF16
    a.B, a.Lc, a.Hq, a.Hkv, a.D = 64, 1 << 20, 32, 8, 128
    a.q = a.kcache = a.vcache = a.pooled = a.o = t.data_ptr()
    a.q_stride = bsa.I64x2(32 * 128, 128)
    a.k_stride = a.v_stride = bsa.I64x3((1 << 20) * 8 * 128, 8 * 128, 128)
    a.p_stride = bsa.I64x3(8192 * 8 * 128, 8 * 128, 128)
    a.o_stride = bsa.I64x2(32 * 128, 128)
    a.pooled_dtype = bsa.BSA_DTYPE_BF16
    a.block, a.topk, a.gate_mode = 128, 32, bsa.BSA_GATE_PER_HEAD
    assert bsa.lib().bsa_decode_workspace_bytes(ctypes.byref(a)) > bsa.NOALLOC_MAX_BYTES
    st = bsa.lib().bsa_sparse_attn_decode_noalloc(ctypes.byref(a), None)
    assert st == bsa.BSA_ERR_WORKSPACE
    assert b"no-allocation limit" in bsa.lib().bsa_last_error()
