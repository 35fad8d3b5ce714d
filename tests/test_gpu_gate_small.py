"""The gate's path for small candidate sets, on the device, against the oracle.

When every selection row has at most 64 candidate blocks, k <= 4 and the
gate is per head (MoBA-style gating over a few dozen blocks), the library
stages the block summaries once per workgroup and lets each wave walk several
tiles of rows.  These cases take that path with both head dims, causal and
not, exact bf16 and rotated (fp32) gate queries, a ragged row count, more
than one tile per wave, and a requested top-k above the number of blocks.
Selections must match the oracle's except inside the 1e-4 tie window (or
exactly where stated); outputs within max-abs 1e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from bsa_testutil import assert_close, check_selection, ref_with_gpu_sel, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    import block_sparse_long_mean_amd as m

    m.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _say(msg):
    print(msg, flush=True)


CASES = {
    # name: (B, Lq, Lk, Hq, Hkv, D, block, topk, causal, doc_mean, token step)
    "noncausal_nb64_k4_ragged": (2, 777, 4096, 8, 2, 128, 64, 4, False, None, 1),
    "causal_k1_d64": (1, 2500, 2500, 4, 1, 64, 40, 1, True, None, 1),
    "doc_rope_noncausal_k4": (1, 128, 4000, 8, 2, 128, 64, 4, False, 300.0, 1),
    "causal_two_tiles_per_wave": (1, 4096, 4096, 64, 2, 64, 128, 2, True, None, 5),
}


@pytest.mark.parametrize("name", list(CASES))
def test_small_gate_matches_oracle(bsa, name):
    B, Lq, Lk, Hq, Hkv, D, block, topk, causal, doc_mean, step = CASES[name]
    _say(f"case small gate {name}: B{B} Lq{Lq} Lk{Lk} H{Hq}/{Hkv} D{D} block{block} topk{topk} causal{causal} "
         f"doc={doc_mean}")
    seed = 70
    sigma = D ** -0.5
    q = synth.host_tensor((B, Lq, Hq, D), sigma, seed, synth.TID["q"], "bf16")
    k = synth.host_tensor((B, Lk, Hkv, D), sigma, seed, synth.TID["k"], "bf16")
    v = synth.host_tensor((B, Lk, Hkv, D), 1.0, seed, synth.TID["v"], "bf16")
    dq = dk = None
    if doc_mean:
        dk = np.stack([synth.random_doc_ids(Lk, doc_mean, seed + b) for b in range(B)])
        dq = np.zeros((B, Lq), dtype=np.int32)
    o, sel, lse = bsa.sparse_attn_prefill(
        q.cuda(), k.cuda(), v.cuda(), block, topk, causal,
        doc_ids_q=None if dq is None else torch.from_numpy(dq).cuda(),
        doc_ids_k=None if dk is None else torch.from_numpy(dk).cuda(), return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    _say("  gpu done")
    toks = list(range(0, Lq, step)) if step > 1 else None

    def run_oracle(tokens=None, force_sel=None, scores=False):
        return oracle.prefill(q, k, v, block=block, topk=topk, causal=causal, doc_ids_q=dq, doc_ids_k=dk,
                              tokens=tokens, force_sel=force_sel, return_scores=scores)

    ref = run_oracle(tokens=toks, scores=True)
    gsel = sel.cpu().numpy()
    glse = to_np(lse)
    go = to_np(o)
    if toks is not None:
        gsel, glse, go = gsel[:, :, toks], glse[:, :, toks], go[:, toks]
    diff = check_selection(gsel, ref["sel"], ref["scores"], topk, causal)
    _say(f"  selection rows {gsel.shape[0] * gsel.shape[1] * gsel.shape[2]}, near-tie differences {len(diff)}")
    ref = ref_with_gpu_sel(ref, diff, gsel, run_oracle, tokens=toks)
    assert_close(go, ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(glse, ref["lse"], 5e-3, None, what="lse")


@pytest.mark.parametrize("topk", [4, 6])
def test_small_gate_topk_above_block_count(bsa, topk):
    """Causal, 256 tokens in 4 blocks of 64: every earlier block is chosen and every later slot of
    each selection row reads -1, with the selection buffer and the workspace starting out as zeros."""
    B, L, Hq, Hkv, D, block = 1, 256, 8, 2, 128, 64
    _say(f"case small gate, top-k above the block count: topk{topk} L256 block64")
    seed = 71
    q = synth.host_tensor((B, L, Hq, D), 1.0, seed, synth.TID["q"], "bf16")
    k = synth.host_tensor((B, L, Hkv, D), 1.0, seed, synth.TID["k"], "bf16")
    v = synth.host_tensor((B, L, Hkv, D), 1.0, seed, synth.TID["v"], "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    sel_out = torch.zeros((B, Hq, L, topk + 1), dtype=torch.int32, device="cuda")
    ws = torch.zeros(bsa.prefill_workspace_bytes(qd, kd, block=block, topk=topk, causal=True),
                     dtype=torch.uint8, device="cuda")
    o, sel, lse = bsa.sparse_attn_prefill(qd, kd, vd, block, topk, True, sel_out=sel_out, workspace=ws,
                                          return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.prefill(q, k, v, block=block, topk=topk, causal=True)
    assert np.array_equal(sel.cpu().numpy(), ref["sel"])
    assert_close(to_np(o), ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(to_np(lse), ref["lse"], 5e-3, None, what="lse")
