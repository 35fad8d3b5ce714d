"""Exact ties in the gate, on the device: the lower block index wins.

The pages state no tie rule; the library's contract (include/bsa.h) is that
equal gate scores go to the lower block index.  Random N(0,1) inputs never
produce an exact tie, so these cases build them: every input is a coarse
dyadic value (a multiple of 1/4 in [-3/4, 3/4]) and the key blocks repeat
with a short period.  Block means, gate scores and group sums are then exact
in every arithmetic the library and the oracle use, so equal blocks score
exactly alike on both sides, and with the period shorter than k, equal scores
straddle the k-th place in most rows.  Selections are compared with the
oracle's strictly (array equality, no tie window), and outputs as usual.

Covered: the per-head and per-group prefill gate with one, three and four
16-key register lists, and with a small k over a single chunk of candidates
(taken by repeated group maxima); a long candidate list split over workgroups and
merged (non-causal, a few queries over a long key sequence); the fp32 gate;
the decode selection per head and per group, including its 4-buffer
variant.  Also the regression case of a requested top-k above the number of
blocks (every slot of the selection row written).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from bsa_testutil import assert_close, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    import block_sparse_long_mean_amd as m

    m.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _say(msg):
    print(msg, flush=True)


def _tie_rows(scores, sel, causal):
    """Rows whose k-th and (k+1)-th oracle scores are exactly equal."""
    n = 0
    B, Hs, T, W = sel.shape
    for b in range(B):
        for hs in range(Hs):
            for ti in range(T):
                s = scores[b, hs, ti]
                cand = np.nonzero(~np.isnan(s))[0]
                k = int((sel[b, hs, ti] >= 0).sum()) - (1 if causal else 0)
                if 0 < k < len(cand):
                    srt = np.sort(s[cand])[::-1]
                    n += int(srt[k - 1] == srt[k])
    return n


PREFILL_CASES = {
    # name: (dtype, B, Lq, Lk, Hq, Hkv, D, block, topk, causal, gate, Di, period)
    "head_causal_k6": ("bf16", 1, 2048, 2048, 4, 2, 128, 64, 6, True, "head", None, 4),
    "group_index_k16": ("bf16", 1, 2560, 2560, 16, 2, 128, 64, 16, True, "group", 64, 5),
    "head_causal_k40_d64": ("bf16", 1, 4096, 4096, 4, 2, 64, 64, 40, True, "head", None, 8),
    "head_noncausal_split_k20": ("bf16", 1, 64, 16384, 8, 2, 128, 16, 20, False, "head", None, 7),
    "group_noncausal_split_k64": ("bf16", 1, 32, 32768, 8, 2, 64, 16, 64, False, "group", None, 9),
    "f32_head_causal_k3": ("f32", 1, 1024, 1024, 2, 1, 64, 64, 3, True, "head", None, 2),
    # at most 64 candidate blocks and k <= 4: the repeated-maximum path
    "head_causal_k3_one_chunk": ("bf16", 1, 4096, 4096, 4, 2, 128, 64, 3, True, "head", None, 2),
    "group_causal_k4_one_chunk": ("bf16", 1, 2048, 2048, 8, 2, 64, 64, 4, True, "group", None, 3),
}


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_prefill_ties_lowest_index(bsa, name):
    dtype, B, Lq, Lk, Hq, Hkv, D, block, topk, causal, gate, Di, period = PREFILL_CASES[name]
    _say(f"case ties {name}: {dtype} B{B} Lq{Lq} Lk{Lk} H{Hq}/{Hkv} D{D} block{block} topk{topk} "
         f"causal{causal} {gate} Di={Di} period{period}")
    seed = 60
    q = synth.dyadic_host((B, Lq, Hq, D), seed, synth.TID["q"], dtype)
    k = synth.repeat_blocks(synth.dyadic_host((B, Lk, Hkv, D), seed, synth.TID["k"], dtype), block, period)
    v = synth.host_tensor((B, Lk, Hkv, D), 1.0, seed, synth.TID["v"], dtype)
    iq = ik = None
    if Di:
        iq = synth.dyadic_host((B, Lq, Hq, Di), seed, synth.TID["index_q"], dtype)
        ik = synth.repeat_blocks(synth.dyadic_host((B, Lk, Hkv, Di), seed, synth.TID["index_k"], dtype), block,
                                 period)
    dev = lambda x: None if x is None else x.cuda()
    o, sel, lse = bsa.sparse_attn_prefill(dev(q), dev(k), dev(v), block, topk, causal, gate=gate, index_q=dev(iq),
                                          index_k=dev(ik), return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    _say("  gpu done")
    ref = oracle.prefill(q, k, v, block=block, topk=topk, causal=causal, gate=gate, index_q=iq, index_k=ik,
                         return_scores=True)
    gsel = sel.cpu().numpy()
    ties = _tie_rows(ref["scores"], ref["sel"], causal)
    rows = gsel.shape[0] * gsel.shape[1] * gsel.shape[2]
    _say(f"  selection rows {rows}, rows with an exact tie at the k-th place {ties}")
    assert ties > rows // 4, "the inputs should tie at the k-th place in many rows"
    bad = np.nonzero(np.any(gsel != ref["sel"], axis=-1))
    assert bad[0].size == 0, (f"{bad[0].size} rows differ, first {tuple(int(x[0]) for x in bad)}: "
                              f"gpu {gsel[tuple(x[0] for x in bad)]} oracle {ref['sel'][tuple(x[0] for x in bad)]}")
    if dtype == "f32":
        assert_close(to_np(o), ref["o"], 1e-5, None)
    else:
        assert_close(to_np(o), ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(to_np(lse), ref["lse"], 5e-3 if dtype == "bf16" else 1e-5, None, what="lse")


@pytest.mark.parametrize("gate,topk", [("head", 32), ("group", 32), ("head", 48), ("group", 60)])
def test_decode_ties_lowest_index(bsa, gate, topk):
    """Routing keys with rows repeating every 6 blocks; the decode's selection (its threshold
    filter, buffer compaction and the pairwise merge of its waves' shares) against the oracle,
    strictly; ragged cache lengths."""
    B, Hq, Hkv, Lc, D, block, period = 2, 8, 2, 4096, 128, 32, 6
    nb = Lc // block
    _say(f"case decode ties gate={gate} topk{topk} B2 H8/2 Lc4096 block32 period{period}")
    seed = 61
    q = synth.dyadic_host((B, Hq, D), seed, synth.TID["q"], "bf16")
    pooled = synth.repeat_blocks(synth.dyadic_host((B, nb, Hkv, D), seed, synth.TID["pooled"], "bf16"), 1, period)
    k = synth.host_tensor((B, Lc, Hkv, D), 1.0, seed, synth.TID["k"], "bf16")
    v = synth.host_tensor((B, Lc, Hkv, D), 1.0, seed, synth.TID["v"], "bf16")
    lens = np.array([Lc, 2001], dtype=np.int32)
    o, sel, lse = bsa.sparse_attn_decode(q.cuda(), k.cuda(), v.cuda(), pooled.cuda(), topk, block, gate=gate,
                                         cache_lens=torch.from_numpy(lens).cuda(), return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.decode(q, k, v, pooled, block=block, topk=topk, gate=gate, cache_lens=lens, return_scores=True)
    gsel = sel.cpu().numpy()
    assert np.array_equal(gsel, ref["sel"]), (gsel, ref["sel"])
    ties = 0
    for (b, hs), s in ref["scores"].items():
        kk = min(topk, len(s))
        if 0 < kk < len(s):
            srt = np.sort(s)[::-1]
            ties += int(srt[kk - 1] == srt[kk])
    _say(f"  rows {len(ref['scores'])}, exact ties at the k-th place {ties}")
    assert ties >= len(ref["scores"]) // 2
    assert_close(to_np(o), ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(to_np(lse), ref["lse"], 5e-3, None, what="lse")


@pytest.mark.parametrize("gate", ["head", "group"])
@pytest.mark.parametrize("topk", [32, 64])
def test_topk_above_block_count(bsa, gate, topk):
    """Causal, 1024 tokens in 16 blocks of 64, top-k 32 or 64: every earlier block is chosen,
    and every slot of each selection row past the chosen and forced blocks must read -1.  The
    selection buffer and the workspace start out holding block 0 / zeros, so a slot left
    unwritten would show up in the selection and, through the attention, in the output."""
    B, L, Hq, Hkv, D, block = 1, 1024, 4, 2, 128, 64
    _say(f"case top-k above the block count: gate={gate} topk{topk} L1024 block64")
    seed = 62
    q = synth.host_tensor((B, L, Hq, D), 1.0, seed, synth.TID["q"], "bf16")
    k = synth.host_tensor((B, L, Hkv, D), 1.0, seed, synth.TID["k"], "bf16")
    v = synth.host_tensor((B, L, Hkv, D), 1.0, seed, synth.TID["v"], "bf16")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    hs = Hkv if gate == "group" else Hq
    sel_out = torch.zeros((B, hs, L, topk + 1), dtype=torch.int32, device="cuda")
    ws = torch.zeros(bsa.prefill_workspace_bytes(qd, kd, block=block, topk=topk, causal=True, gate=gate),
                     dtype=torch.uint8, device="cuda")
    o, sel, lse = bsa.sparse_attn_prefill(qd, kd, vd, block, topk, True, gate=gate, sel_out=sel_out, workspace=ws,
                                          return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.prefill(q, k, v, block=block, topk=topk, causal=True, gate=gate)
    assert np.array_equal(sel.cpu().numpy(), ref["sel"])
    assert_close(to_np(o), ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(to_np(lse), ref["lse"], 5e-3, None, what="lse")
