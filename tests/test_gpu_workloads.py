"""Parity at the full sizes of the five workloads.

Inputs are the seeded device draws of `synth` at the real shapes; the library
runs the whole call (in the benchmark's launch configuration where one is
timed), and the float64 oracle evaluates sampled outputs one by one: sampled
query tokens with every head for prefill, every (sequence, head) for decode,
sampled blocks for the summaries.  The oracle reads back only the slices it
needs.  Sampled tokens always include the first and last positions and block
edges.  Selections must match except inside the 1e-4 tie window; outputs
within max-abs 1e-2 on top of bf16 output rounding.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from bsa_testutil import HostSlices, RowView, assert_close, check_selection, ref_with_gpu_sel, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

SEED = 0
T = synth.TID


@pytest.fixture(scope="module")
def bsa():
    import block_sparse_long_mean_amd as m

    m.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _say(msg):
    print(msg, flush=True)


def _sample_tokens(L, block, n_random, seed, extra=()):
    rng = np.random.default_rng(seed)
    fixed = {0, 1, block - 1, block, block + 1, 2 * block - 1, L // 2, L - block - 1, L - block, L - 2, L - 1, *extra}
    fixed = {t for t in fixed if 0 <= t < L}
    rand = set(int(x) for x in rng.choice(L, size=n_random, replace=False))
    return sorted(fixed | rand)


def _check_prefill_rows(o, sel, lse, toks, run_oracle, topk, causal):
    """Compare sampled rows of a full GPU prefill with the oracle."""
    ref = run_oracle(tokens=toks, scores=True)
    tix = torch.tensor(toks, dtype=torch.long, device=o.device)
    gsel = sel.index_select(2, tix).cpu().numpy()
    diff = check_selection(gsel, ref["sel"], ref["scores"], topk, causal)
    _say(f"  sampled tokens {len(toks)}, selection rows {gsel.shape[1] * gsel.shape[2]}, near-tie differences {len(diff)}")
    ref = ref_with_gpu_sel(ref, diff, gsel, run_oracle, tokens=toks)
    got_o = to_np(o.index_select(1, tix))
    got_lse = to_np(lse.index_select(2, tix))
    assert_close(got_o, ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(got_lse, ref["lse"], 5e-3, None, what="lse")


def test_moba_prefill_32k_fullsize(bsa):
    """MoBA-style: B1, 32/8 heads, L32768, D128, block 512, top-3 + own block per query head, causal,
    bf16 N(0,1)/sqrt(128)."""
    B, L, Hq, Hkv, D, block, topk, sigma = 1, 32768, 32, 8, 128, 512, 3, 128 ** -0.5
    _say("case MoBA prefill B1 L32768 H32/8 D128 block512 topk3 causal per-head")
    q = synth.device_tensor((B, L, Hq, D), sigma, SEED, T["q"], "bf16")
    k = synth.device_tensor((B, L, Hkv, D), sigma, SEED, T["k"], "bf16")
    v = synth.device_tensor((B, L, Hkv, D), sigma, SEED, T["v"], "bf16")
    o, sel, lse = bsa.sparse_attn_prefill(q, k, v, block, topk, True, return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    _say("  gpu done")
    toks = _sample_tokens(L, block, 40, 100, extra=(3 * block - 1, 3 * block, 4 * block))
    qh = q[:, toks].cpu()
    kh, vh = k.cpu(), v.cpu()
    pooled = oracle.block_pool(kh, block)

    def run_oracle(tokens, force_sel=None, scores=False):
        return oracle.prefill(RowView(qh, toks, L), kh, vh, block=block, topk=topk, causal=True, pooled=pooled,
                              tokens=tokens, force_sel=force_sel, return_scores=scores)

    _check_prefill_rows(o, sel, lse, toks, run_oracle, topk, True)


def test_moba_backward_32k_fullsize(bsa):
    """The MoBA-style 32K backward in the benchmark's launch configuration (caller-provided gradient
    buffers and workspace), through the forward's own selection.  Sampled: dq of 40 tokens with
    every head (first / last tokens and block edges included), and dk, dv of every key of two
    whole blocks, (kv head 0, block 63) and (kv head 5, block 40), for which the oracle sums the
    contributions of every row that chose them.  Bound: 1e-2 of the largest reference gradient
    of each compared set."""
    B, L, Hq, Hkv, D, block, topk, sigma = 1, 32768, 32, 8, 128, 512, 3, 128 ** -0.5
    G = Hq // Hkv
    _say("case MoBA backward B1 L32768 H32/8 D128 block512 topk3 causal per-head")
    q = synth.device_tensor((B, L, Hq, D), sigma, SEED, T["q"], "bf16")
    k = synth.device_tensor((B, L, Hkv, D), sigma, SEED, T["k"], "bf16")
    v = synth.device_tensor((B, L, Hkv, D), sigma, SEED, T["v"], "bf16")
    g = synth.device_tensor((B, L, Hq, D), 1.0, SEED, T["dout"], "bf16")
    o, sel, lse = bsa.sparse_attn_prefill(q, k, v, block, topk, True, return_sel=True, return_lse=True)
    grads = tuple(torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in (q, k, v))
    ws = torch.empty(bsa.backward_workspace_bytes(q, k, sel, block=block, causal=True), dtype=torch.uint8,
                     device="cuda")
    dq, dk, dv = bsa.sparse_attn_backward(q, k, v, o, lse, sel, g, block, True, out=grads, workspace=ws)
    torch.cuda.synchronize()
    _say("  gpu done")
    qh, kh, vh, gh = q.cpu(), k.cpu(), v.cpu(), g.cpu()
    sh = sel.cpu().numpy()
    toks = _sample_tokens(L, block, 30, 101, extra=(block - 1, block, 40 * block + 7))
    rows = [(0, t, h) for t in toks for h in range(Hq)]
    ref = oracle.prefill_backward(qh, kh, vh, gh, sh, block=block, causal=True, rows=rows)
    ti = torch.tensor(toks)
    assert_close(to_np(dq[0].index_select(0, ti.cuda())), ref["dq"][0, toks],
                 1e-2 * float(np.abs(ref["dq"][0, toks]).max()), None, what="dq")
    for hk, j in ((0, 63), (5, 40)):
        chose = np.nonzero((sh[0, hk * G:(hk + 1) * G] == j).any(axis=-1))  # (head in group, token)
        rows = [(0, int(t), hk * G + int(hh)) for hh, t in zip(*chose)]
        _say(f"  block ({hk}, {j}): {len(rows)} rows chose it")
        ref = oracle.prefill_backward(qh, kh, vh, gh, sh, block=block, causal=True, rows=rows)
        a, e = j * block, (j + 1) * block
        for nm, got in (("dk", dk), ("dv", dv)):
            r = ref[nm][0, a:e, hk]
            assert_close(to_np(got[0, a:e, hk]), r, 1e-2 * float(np.abs(r).max()), None, what=nm)


def test_index_branch_prefill_128k_fullsize(bsa):
    """MiniMax-style 128K: B1, 64/8 heads, D128, block 64, index q/k of dim 64, scores summed per group,
    top-16 + own block, causal, bf16 N(0,1) -- the benchmark's prefill, in its launch configuration
    (caller-provided output and workspace)."""
    B, L, Hq, Hkv, D, Di, block, topk = 1, 131072, 64, 8, 128, 64, 64, 16
    _say("case index-branch prefill B1 L131072 H64/8 D128 Di64 block64 topk16 causal group")
    q = synth.device_tensor((B, L, Hq, D), 1.0, SEED, T["q"], "bf16")
    k = synth.device_tensor((B, L, Hkv, D), 1.0, SEED, T["k"], "bf16")
    v = synth.device_tensor((B, L, Hkv, D), 1.0, SEED, T["v"], "bf16")
    iq = synth.device_tensor((B, L, Hq, Di), 1.0, SEED, T["index_q"], "bf16")
    ik = synth.device_tensor((B, L, Hkv, Di), 1.0, SEED, T["index_k"], "bf16")
    kw = dict(gate="group", index_q=iq, index_k=ik)
    o_bench = torch.empty_like(q)
    ws = torch.empty(bsa.prefill_workspace_bytes(q, k, block=block, topk=topk, causal=True, **kw),
                     dtype=torch.uint8, device="cuda")
    bsa.sparse_attn_prefill(q, k, v, block, topk, True, out=o_bench, workspace=ws, **kw)
    o, sel, lse = bsa.sparse_attn_prefill(q, k, v, block, topk, True, return_sel=True, return_lse=True, **kw)
    torch.cuda.synchronize()
    _say("  gpu done")
    # asking for the selection and lse changes nothing in the output
    assert torch.equal(o.view(torch.int16), o_bench.view(torch.int16))
    del o_bench, ws
    toks = _sample_tokens(L, block, 24, 101, extra=(16 * block - 1, 16 * block, 17 * block))
    qh, iqh = q[:, toks].cpu(), iq[:, toks].cpu()
    kh, vh, ikh = k.cpu(), v.cpu(), ik.cpu()
    pooled = oracle.block_pool(ikh, block)

    def run_oracle(tokens, force_sel=None, scores=False):
        return oracle.prefill(RowView(qh, toks, L), kh, vh, block=block, topk=topk, causal=True, gate="group",
                              index_q=RowView(iqh, toks, L), index_k=ikh, pooled=pooled, tokens=tokens,
                              force_sel=force_sel, return_scores=scores)

    _check_prefill_rows(o, sel, lse, toks, run_oracle, topk, True)


def _decode_check(bsa, q, kc, vc, pooled, topk, block, lens, table=None, gate="head"):
    o, sel, lse = bsa.sparse_attn_decode(q, kc, vc, pooled, topk, block, gate=gate, return_sel=True, return_lse=True,
                                         cache_lens=None if lens is None else torch.from_numpy(lens).cuda(),
                                         block_table=None if table is None else torch.from_numpy(table).cuda())
    torch.cuda.synchronize()
    _say("  gpu done")
    ph = pooled.cpu()
    qh = q.cpu()
    kv = (HostSlices(kc), HostSlices(vc))
    if table is not None:
        Lc = pooled.shape[1] * block
        kv = (oracle.PagedCache(kv[0], table, block, Lc), oracle.PagedCache(kv[1], table, block, Lc))
    ref = oracle.decode(qh, *kv, ph, block=block, topk=topk, gate=gate, cache_lens=lens, return_scores=True)
    B, Hs = ref["sel"].shape[:2]
    nb = pooled.shape[1]
    scores = np.full((B, Hs, 1, nb), np.nan)
    for (b, hs), s in ref["scores"].items():
        scores[b, hs, 0, : len(s)] = s
    gsel = sel.cpu().numpy()[:, :, None]
    diff = check_selection(gsel, ref["sel"][:, :, None], scores, topk, True)
    _say(f"  decode rows {B * Hs}, near-tie differences {len(diff)}")
    if diff:
        ref = oracle.decode(qh, *kv, ph, block=block, topk=topk, gate=gate, cache_lens=lens, force_sel=gsel[:, :, 0])
    assert_close(to_np(o), ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(to_np(lse), ref["lse"], 5e-3, None, what="lse")


def test_decode_1m_cache_fullsize(bsa):
    """Long-context decode: 16 sequences x 1 token over 1,048,576-token caches, 32/8 heads, D128,
    block 128 (8192 routing keys per sequence and KV head), top-32 + own block per query head, bf16
    N(0,1).  The routing keys are a seeded input of the mean-pooled keys' scale (N(0,1)/sqrt(128));
    the library's own block summary of these caches is checked in the next test.  Every
    (sequence, head) is compared; full caches (the benchmark's call), then ragged lengths down to
    a single token."""
    B, Lc, Hq, Hkv, D, block, topk = 16, 1 << 20, 32, 8, 128, 128, 32
    nb = Lc // block
    _say("case decode B16 Lc1048576 H32/8 D128 block128 topk32 (68.7 GB of cache)")
    q = synth.device_tensor((B, Hq, D), 1.0, SEED + 1, T["q"], "bf16")
    # head-major caches as the benchmark stores them, seen as [B, Lc, Hkv, D]
    kc = synth.device_tensor((B, Hkv, Lc, D), 1.0, SEED + 1, T["k"], "bf16").transpose(1, 2)
    vc = synth.device_tensor((B, Hkv, Lc, D), 1.0, SEED + 1, T["v"], "bf16").transpose(1, 2)
    pooled = synth.device_tensor((B, nb, Hkv, D), 128 ** -0.5, SEED + 1, T["pooled"], "bf16")
    _decode_check(bsa, q, kc, vc, pooled, topk, block, None)
    lens = np.array([1, 2, 127, 128, 129, 256, 257, 33 * 128, 33 * 128 + 1, 500_000, 777_777,
                     Lc - 129, Lc - 128, Lc - 1, Lc, 4097], dtype=np.int32)
    _say("case decode ragged lengths " + ",".join(str(int(x)) for x in lens))
    _decode_check(bsa, q, kc, vc, pooled, topk, block, lens)


def test_paged_decode_1m_cache_fullsize(bsa):
    """The long-context decode over a paged cache: the 16 sequences' 1,048,576-token caches cut
    into 128-token pages (head-major inside a page), stored in a seeded random order, one table
    row of 8192 pages per sequence; every (sequence, head) is compared, full and ragged lengths,
    then with per-group gating (the group's scores summed; one block list per kv head)."""
    B, Lc, Hq, Hkv, D, block, topk = 16, 1 << 20, 32, 8, 128, 128, 32
    nb = Lc // block
    P = B * nb
    _say("case paged decode B16 Lc1048576 H32/8 D128 block128 topk32, 131072 shuffled pages")
    q = synth.device_tensor((B, Hq, D), 1.0, SEED + 3, T["q"], "bf16")
    kp = synth.device_tensor((P, Hkv, block, D), 1.0, SEED + 3, T["k"], "bf16").transpose(1, 2)
    vp = synth.device_tensor((P, Hkv, block, D), 1.0, SEED + 3, T["v"], "bf16").transpose(1, 2)
    pooled = synth.device_tensor((B, nb, Hkv, D), 128 ** -0.5, SEED + 3, T["pooled"], "bf16")
    table = np.random.default_rng(SEED + 3).permutation(P).astype(np.int32).reshape(B, nb)
    _decode_check(bsa, q, kp, vp, pooled, topk, block, None, table)
    lens = np.array([1, 2, 127, 128, 129, 256, 257, 33 * 128, 33 * 128 + 1, 500_000, 777_777,
                     Lc - 129, Lc - 128, Lc - 1, Lc, 4097], dtype=np.int32)
    _say("case paged decode ragged lengths")
    _decode_check(bsa, q, kp, vp, pooled, topk, block, lens, table)
    _say("case paged decode, per-group gating")
    _decode_check(bsa, q, kp, vp, pooled, topk, block, None, table, gate="group")


def _check_summary_blocks(got, k, block, blocks, pos=None, bf16_out=False, atol=2e-6):
    """Compare summaries of sampled blocks with the oracle's means of the same tokens."""
    L = k.shape[1]
    ks = HostSlices(k)
    worst = 0.0
    for j in blocks:
        a, e = j * block, min(L, (j + 1) * block)
        kk = ks[:, a:e]
        pp = None if pos is None else pos[:, a:e]
        ref = oracle.block_pool(kk, block, pos=pp)[:, 0]
        g = got[:, j].float().cpu().numpy().astype(np.float64)
        bound = atol + (np.abs(ref) * 2.0 ** -8 if bf16_out else 0.0)
        err = np.abs(g - ref) - bound
        worst = max(worst, float(err.max()))
        assert np.all(err <= 0.0), f"block {j}: summary off by {float((np.abs(g - ref)).max()):.3e}"
    return worst


def test_block_summary_1m_cache_fullsize(bsa):
    """The routing keys of the decode caches (head-major, as the benchmark stores them): bf16 block
    means of 16 x 1,048,576 keys, block 128, sampled blocks of every sequence against the oracle."""
    B, Lc, Hkv, D, block = 16, 1 << 20, 8, 128, 128
    _say("case block_summary B16 L1048576 H8 D128 block128 bf16 out")
    kc = synth.device_tensor((B, Hkv, Lc, D), 1.0, SEED + 1, T["k"], "bf16").transpose(1, 2)
    pooled = bsa.block_summary(kc, block, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    nb = Lc // block
    rng = np.random.default_rng(102)
    blocks = sorted({0, 1, nb // 2, nb - 2, nb - 1} | set(int(x) for x in rng.choice(nb, 27, replace=False)))
    _check_summary_blocks(pooled, kc, block, blocks, bf16_out=True, atol=1e-7)


def _memory_bank():
    lengths = synth.doc_lengths(10_000_000, 2000, 5000.0, 0.8, SEED)
    return synth.doc_ids_from_lengths(lengths)[None]  # [1, 10M]


def test_memory_bank_10m_fullsize(bsa):
    """MSA-style memory bank: 10M tokens in 2000 lognormal documents (mean 5000, log-sigma 0.8),
    document-wise RoPE on q and k, block 64 (156,250 blocks), a 512-token query chunk that is its
    own document, 32/8 heads, D128, top-64 per query head, non-causal, bf16 N(0,1).  The routing
    keys are a seeded fp32 input of the pooled keys' scale (N(0,1)/8), as a memory's stored keys
    would be; the library's own summary of this memory is checked in the next test."""
    B, Lk, Lq, Hq, Hkv, D, block, topk = 1, 10_000_000, 512, 32, 8, 128, 64, 64
    nb = Lk // block
    _say("case memory bank Lk10M docs2000 Lq512 H32/8 D128 block64 topk64 non-causal doc-RoPE")
    ids_k = _memory_bank()
    ids_q = np.zeros((B, Lq), dtype=np.int32)
    q = synth.device_tensor((B, Lq, Hq, D), 1.0, SEED, T["q"], "bf16")
    k = synth.device_tensor((B, Lk, Hkv, D), 1.0, SEED, T["k"], "bf16")
    v = synth.device_tensor((B, Lk, Hkv, D), 1.0, SEED, T["v"], "bf16")
    pooled = synth.device_tensor((B, nb, Hkv, D), 0.125, SEED, T["pooled"], "f32")
    o, sel, lse = bsa.sparse_attn_prefill(q, k, v, block, topk, False, doc_ids_q=torch.from_numpy(ids_q).cuda(),
                                          doc_ids_k=torch.from_numpy(ids_k).cuda(), pooled=pooled,
                                          return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    _say("  gpu done")
    toks = [0, 1, 63, 64, 255, 510, 511] + [int(x) for x in np.random.default_rng(103).choice(512, 3, replace=False)]
    toks = sorted(set(toks))
    qh = q[:, toks].cpu()
    ph = pooled.cpu()
    ks, vs = HostSlices(k), HostSlices(v)

    def run_oracle(tokens, force_sel=None, scores=False):
        return oracle.prefill(RowView(qh, toks, Lq), ks, vs, block=block, topk=topk, causal=False,
                              doc_ids_q=ids_q, doc_ids_k=ids_k, pooled=ph, tokens=tokens, force_sel=force_sel,
                              return_scores=scores)

    _check_prefill_rows(o, sel, lse, toks, run_oracle, topk, False)


def test_block_summary_memory_bank_fullsize(bsa):
    """Summaries of the 10M-token memory with document-wise RoPE (fp32 out), sampled blocks
    including blocks that straddle a document start, against the oracle."""
    B, Lk, Hkv, D, block = 1, 10_000_000, 8, 128, 64
    _say("case block_summary memory bank L10M H8 D128 block64 doc-RoPE fp32 out")
    ids = _memory_bank()
    k = synth.device_tensor((B, Lk, Hkv, D), 1.0, SEED, T["k"], "bf16")
    pooled = bsa.block_summary(k, block, doc_ids=torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    pos = oracle.doc_positions(ids)
    nb = Lk // block
    starts = np.nonzero(np.diff(ids[0]))[0] + 1
    straddle = sorted({int(s) // block for s in starts if s % block})[:: 97][:12]
    longest = int(np.argmax(np.diff(np.r_[0, starts, Lk])))  # deepest positions of the memory
    end_of_longest = int(np.r_[starts, Lk][longest]) - 1
    rng = np.random.default_rng(104)
    blocks = sorted({0, nb - 1, end_of_longest // block, *straddle} | set(int(x) for x in rng.choice(nb, 16, replace=False)))
    _check_summary_blocks(pooled, k, block, blocks, pos=pos, atol=2e-6)
