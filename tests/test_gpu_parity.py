"""Parity of the HIP library (through its C ABI) against the float64 oracle.

Every case is seeded and synthetic; sizes span several tiles and a ragged
tail.  Selections must match exactly except inside the 1e-4 tie window;
outputs within max-abs 1e-2 (bf16) or 1e-5 (fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from bsa_testutil import assert_close, bf16_half_ulp, check_selection, ref_with_gpu_sel, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    import block_sparse_long_mean_amd as m

    m.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _say(msg):
    print(msg, flush=True)


def run_prefill_case(bsa, *, dtype, B, Lq, Lk, Hq, Hkv, D, block, topk, causal, gate="head", sigma=1.0, seed=0,
                     Di=None, doc_mean=None, atol, rel, lse_atol, chunk_tokens=0, chunks_per_pass=0):
    name = (f"prefill dtype={dtype} B{B} Lq{Lq} Lk{Lk} H{Hq}/{Hkv} D{D} block{block} topk{topk} causal{causal} "
            f"gate={gate} Di={Di} doc={doc_mean} seed{seed} chunk{chunk_tokens} per_pass{chunks_per_pass}")
    _say("case " + name)
    q = synth.host_tensor((B, Lq, Hq, D), sigma, seed, synth.TID["q"], dtype)
    k = synth.host_tensor((B, Lk, Hkv, D), sigma, seed, synth.TID["k"], dtype)
    v = synth.host_tensor((B, Lk, Hkv, D), sigma, seed, synth.TID["v"], dtype)
    iq = ik = None
    if Di:
        iq = synth.host_tensor((B, Lq, Hq, Di), sigma, seed, synth.TID["index_q"], dtype)
        ik = synth.host_tensor((B, Lk, Hkv, Di), sigma, seed, synth.TID["index_k"], dtype)
    dq = dk = None
    if doc_mean:
        dk = np.stack([synth.random_doc_ids(Lk, doc_mean, seed + b) for b in range(B)])
        dq = np.zeros((B, Lq), dtype=np.int32)  # the query chunk is one document
    dev = lambda x: None if x is None else x.cuda()
    o, sel, lse = bsa.sparse_attn_prefill(
        dev(q), dev(k), dev(v), block, topk, causal, gate=gate, index_q=dev(iq), index_k=dev(ik),
        doc_ids_q=None if dq is None else torch.from_numpy(dq).cuda(),
        doc_ids_k=None if dk is None else torch.from_numpy(dk).cuda(),
        return_sel=True, return_lse=True, chunk_tokens=chunk_tokens, chunks_per_pass=chunks_per_pass)
    torch.cuda.synchronize()
    _say("  gpu done")
    if chunk_tokens or chunks_per_pass:
        # the attention schedule changes nothing in the results
        o1, sel1, lse1 = bsa.sparse_attn_prefill(
            dev(q), dev(k), dev(v), block, topk, causal, gate=gate, index_q=dev(iq), index_k=dev(ik),
            doc_ids_q=None if dq is None else torch.from_numpy(dq).cuda(),
            doc_ids_k=None if dk is None else torch.from_numpy(dk).cuda(),
            return_sel=True, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(sel, sel1)
        assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o, o1.view(torch.int16) if o1.dtype == torch.bfloat16 else o1)
        assert torch.equal(lse, lse1)
        _say("  chunked == default schedule, bitwise")

    def run_oracle(tokens=None, force_sel=None, scores=False):
        return oracle.prefill(q, k, v, block=block, topk=topk, causal=causal, gate=gate, index_q=iq, index_k=ik,
                              doc_ids_q=dq, doc_ids_k=dk, tokens=tokens, force_sel=force_sel,
                              return_scores=scores)

    ref = run_oracle(scores=True)
    gsel = sel.cpu().numpy()
    diff = check_selection(gsel, ref["sel"], ref["scores"], topk, causal)
    _say(f"  selection rows {gsel.shape[0] * gsel.shape[1] * gsel.shape[2]}, near-tie differences {len(diff)}")
    ref = ref_with_gpu_sel(ref, diff, gsel, run_oracle)
    st = assert_close(to_np(o), ref["o"], atol, rel, bf16_storage=(dtype == "bf16"))
    assert_close(to_np(lse), ref["lse"], lse_atol, None, what="lse")
    return st


def test_tiny_fp32_causal(bsa):
    """1 head, L2048, D64, block 128, top-3 + own block, fp32 N(0,1), seed 0."""
    run_prefill_case(bsa, dtype="f32", B=1, Lq=2048, Lk=2048, Hq=1, Hkv=1, D=64, block=128, topk=3, causal=True,
                     seed=0, atol=1e-5, rel=None, lse_atol=1e-5)


def test_fp32_group_ragged(bsa):
    run_prefill_case(bsa, dtype="f32", B=2, Lq=333, Lk=333, Hq=4, Hkv=2, D=128, block=48, topk=2, causal=True,
                     gate="group", seed=1, atol=1e-5, rel=None, lse_atol=1e-5)


def test_fp32_doc_rope_memory(bsa):
    """fp32 inputs with document-wise RoPE: a 64-token query chunk over 4000 keys of short
    documents, non-causal, top-4 per head (the fp32 rotation tables and summaries)."""
    run_prefill_case(bsa, dtype="f32", B=1, Lq=64, Lk=4000, Hq=4, Hkv=2, D=64, block=64, topk=4, causal=False,
                     seed=6, doc_mean=300.0, atol=1e-5, rel=None, lse_atol=1e-5)


def test_bf16_per_head_moba_like(bsa):
    """GQA 8/2, D128, block 256, top-3 + own block, N(0,1)/sqrt(128), ragged length."""
    run_prefill_case(bsa, dtype="bf16", B=1, Lq=3000, Lk=3000, Hq=8, Hkv=2, D=128, block=256, topk=3, causal=True,
                     sigma=128 ** -0.5, seed=2, atol=1e-2, rel=1e-2, lse_atol=5e-3)


def test_bf16_index_branch_group(bsa):
    """Index q/k of dim 64 per head, scores summed over the group, block 64, top-16 + own."""
    run_prefill_case(bsa, dtype="bf16", B=1, Lq=2085, Lk=2085, Hq=16, Hkv=2, D=128, block=64, topk=16, causal=True,
                     gate="group", Di=64, seed=3, atol=1e-2, rel=1e-2, lse_atol=5e-3)


def test_bf16_d64_batch_offset_queries(bsa):
    """B=2, Lq < Lk (queries at the end), D64, block 32."""
    run_prefill_case(bsa, dtype="bf16", B=2, Lq=200, Lk=1500, Hq=4, Hkv=4, D=64, block=32, topk=5, causal=True,
                     seed=4, atol=1e-2, rel=1e-2, lse_atol=5e-3)


def test_bf16_memory_doc_rope_noncausal(bsa):
    """MSA-style: a memory of short documents with document-wise RoPE, one query chunk, non-causal top-16."""
    run_prefill_case(bsa, dtype="bf16", B=1, Lq=128, Lk=20000, Hq=8, Hkv=2, D=128, block=64, topk=16, causal=False,
                     seed=5, doc_mean=400.0, atol=1e-2, rel=1e-2, lse_atol=5e-3)


def test_bf16_memory_topk64_global_buckets(bsa):
    """Non-causal top-64 over a 600K-token memory of documents with document-wise RoPE: more blocks
    per KV head (9375) than the bucket histogram keeps on chip, and a 64-entry top-k."""
    run_prefill_case(bsa, dtype="bf16", B=1, Lq=64, Lk=600000, Hq=8, Hkv=2, D=128, block=64, topk=64, causal=False,
                     seed=13, doc_mean=3000.0, atol=1e-2, rel=1e-2, lse_atol=5e-3)


@pytest.mark.parametrize("case", ["head_l3000_c512_p1", "group_l2085_c256_all", "offset_b2_c64_p3", "memory_c32_p1"])
def test_bf16_query_chunks(bsa, case):
    """Attention over chunks of query tokens (a ragged last chunk), in passes of one chunk, of
    three chunks (a ragged last pass) or of all chunks: same results as the default schedule,
    and the oracle's."""
    kw = dict(dtype="bf16", atol=1e-2, rel=1e-2, lse_atol=5e-3)
    if case == "head_l3000_c512_p1":
        run_prefill_case(bsa, B=1, Lq=3000, Lk=3000, Hq=8, Hkv=2, D=128, block=256, topk=3, causal=True,
                         sigma=128 ** -0.5, seed=15, chunk_tokens=512, chunks_per_pass=1, **kw)
    elif case == "group_l2085_c256_all":
        run_prefill_case(bsa, B=1, Lq=2085, Lk=2085, Hq=16, Hkv=2, D=128, block=64, topk=16, causal=True,
                         gate="group", Di=64, seed=16, chunk_tokens=256, **kw)
    elif case == "offset_b2_c64_p3":
        run_prefill_case(bsa, B=2, Lq=200, Lk=1500, Hq=4, Hkv=4, D=64, block=32, topk=5, causal=True,
                         seed=17, chunk_tokens=64, chunks_per_pass=3, **kw)
    else:
        run_prefill_case(bsa, B=1, Lq=128, Lk=20000, Hq=8, Hkv=2, D=128, block=64, topk=16, causal=False,
                         seed=18, doc_mean=400.0, chunk_tokens=32, chunks_per_pass=1, **kw)


@pytest.mark.parametrize("case", ["group_d64_causal_offset", "head_block128_causal", "group_d64_passes"])
def test_bf16_sparse_buckets(bsa, case):
    """A few query tokens over a long key sequence: a handful of rows per selected block, so the
    gather takes its sparse-bucket kernel (keys streamed from HBM, causal mask inside the query's
    own block, blocks longer than one 64-key pass, query chunks in passes of three)."""
    kw = dict(dtype="bf16", atol=1e-2, rel=1e-2, lse_atol=5e-3)
    if case == "group_d64_causal_offset":
        run_prefill_case(bsa, B=2, Lq=48, Lk=40000, Hq=8, Hkv=2, D=64, block=64, topk=6, causal=True,
                         gate="group", seed=21, **kw)
    elif case == "group_d64_passes":
        run_prefill_case(bsa, B=2, Lq=48, Lk=40000, Hq=8, Hkv=2, D=64, block=64, topk=6, causal=True,
                         gate="group", seed=23, chunk_tokens=16, chunks_per_pass=3, **kw)
    else:
        run_prefill_case(bsa, B=1, Lq=40, Lk=50000, Hq=4, Hkv=4, D=128, block=128, topk=5, causal=True,
                         sigma=128 ** -0.5, seed=22, **kw)


def test_bf16_topk_zero_and_full(bsa):
    run_prefill_case(bsa, dtype="bf16", B=1, Lq=700, Lk=700, Hq=2, Hkv=1, D=128, block=64, topk=0, causal=True,
                     seed=6, atol=1e-2, rel=1e-2, lse_atol=5e-3)
    run_prefill_case(bsa, dtype="bf16", B=1, Lq=700, Lk=700, Hq=2, Hkv=1, D=128, block=64, topk=11, causal=True,
                     seed=7, atol=1e-2, rel=1e-2, lse_atol=5e-3)


def test_dense_switch_matches_torch_sdpa(bsa):
    """top-k covering every block is full causal attention (MoBA's full/sparse switch)."""
    B, L, H, D = 1, 1024, 4, 128
    q = synth.host_tensor((B, L, H, D), 1.0, 8, 0, "bf16").cuda()
    k = synth.host_tensor((B, L, H, D), 1.0, 8, 1, "bf16").cuda()
    v = synth.host_tensor((B, L, H, D), 1.0, 8, 2, "bf16").cuda()
    _say("case dense switch L1024 block64 topk16")
    o = bsa.sparse_attn_prefill(q, k, v, 64, 16, True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.float().transpose(1, 2), k.float().transpose(1, 2), v.float().transpose(1, 2), is_causal=True).transpose(1, 2)
    assert_close(o.float().cpu().numpy(), ref.cpu().numpy(), 1e-2, 1e-2, bf16_storage=True)


def test_block_summary_with_doc_rope(bsa):
    B, L, H, D, block = 2, 3000, 2, 128, 64
    _say("case block_summary doc-rope B2 L3000 H2 D128 block64")
    k = synth.host_tensor((B, L, H, D), 1.0, 9, 1, "bf16")
    ids = np.stack([synth.random_doc_ids(L, 300.0, 9 + b) for b in range(B)])
    pooled, k_rot, pos = bsa.block_summary(k.cuda(), block, doc_ids=torch.from_numpy(ids).cuda(),
                                           return_k_rot=True, return_pos=True)
    torch.cuda.synchronize()
    pos_ref = oracle.doc_positions(ids)
    assert np.array_equal(pos.cpu().numpy(), pos_ref)
    rot_ref = oracle.rope_rotate_half(k, pos_ref)
    got = k_rot.float().cpu().numpy().astype(np.float64)
    # bf16 storage: within half an ulp of the float64 value (plus fp32 rotation error)
    assert np.all(np.abs(got - rot_ref) <= np.abs(rot_ref) * 2.0 ** -8 + 1e-6)
    pool_ref = oracle.block_pool(k, block, pos=pos_ref)
    assert_close(pooled.cpu().numpy(), pool_ref, 2e-6, None, what="pooled")
    # plain summary, bf16 output: nearest-even rounding of the fp32 mean
    p16 = bsa.block_summary(k.cuda(), block, out_dtype=torch.bfloat16)
    ref = oracle.block_pool(k, block)
    got = p16.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-7)


@pytest.mark.parametrize("block,D,L,dtype", [(1, 128, 300, "bf16"), (40, 64, 1000, "bf16"), (100, 128, 1950, "bf16"),
                                             (64, 64, 2000, "bf16"), (40, 64, 1000, "f32"), (100, 128, 1950, "f32")])
def test_block_summary_doc_rope_block_sizes(bsa, block, D, L, dtype):
    """Rotation tables of sub-blocks that leave some of the four table-building waves without
    tokens (blocks of 1 and 40), two sub-blocks per block (100 = 64 + 36), a ragged last block,
    and half-width frequency lanes (D 64), for bf16 and fp32 keys; short documents so that many
    blocks restart a document inside them."""
    B, H = 2, 2
    _say(f"case block_summary doc-rope block{block} D{D} L{L} {dtype}")
    k = synth.host_tensor((B, L, H, D), 1.0, 31, 1, dtype)
    ids = np.stack([synth.random_doc_ids(L, 90.0, 31 + b) for b in range(B)])
    pooled, k_rot, pos = bsa.block_summary(k.cuda(), block, doc_ids=torch.from_numpy(ids).cuda(),
                                           return_k_rot=True, return_pos=True)
    torch.cuda.synchronize()
    pos_ref = oracle.doc_positions(ids)
    assert np.array_equal(pos.cpu().numpy(), pos_ref)
    rot_ref = oracle.rope_rotate_half(k, pos_ref)
    got = k_rot.float().cpu().numpy().astype(np.float64)
    if dtype == "bf16":  # bf16 storage: within half an ulp of the float64 value (plus fp32 rotation error)
        assert np.all(np.abs(got - rot_ref) <= np.abs(rot_ref) * 2.0 ** -8 + 1e-6)
    else:  # fp32 (cos, sin) and fp32 products: a few fp32 ulps of the pair's magnitude
        assert np.all(np.abs(got - rot_ref) <= 1e-5)
    pool_ref = oracle.block_pool(k, block, pos=pos_ref)
    assert_close(pooled.cpu().numpy(), pool_ref, 2e-6, None, what="pooled")


@pytest.mark.parametrize("gate", ["head", "group"])
def test_decode_ragged_lengths(bsa, gate):
    B, Hq, Hkv, Lc, D, block, topk = 3, 8, 2, 5000, 128, 128, 8
    _say(f"case decode gate={gate} B3 H8/2 Lc5000 block128 topk8")
    q = synth.host_tensor((B, Hq, D), 1.0, 10, 0, "bf16")
    k = synth.host_tensor((B, Lc, Hkv, D), 1.0, 10, 1, "bf16")
    v = synth.host_tensor((B, Lc, Hkv, D), 1.0, 10, 2, "bf16")
    lens = np.array([5000, 3333, 129], dtype=np.int32)
    pooled = torch.from_numpy(oracle.block_pool(k, block)).to(torch.bfloat16)  # caller's routing keys
    o, sel, lse = bsa.sparse_attn_decode(q.cuda(), k.cuda(), v.cuda(), pooled.cuda(), topk, block, gate=gate,
                                         cache_lens=torch.from_numpy(lens).cuda(), return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.decode(q, k, v, pooled, block=block, topk=topk, gate=gate, cache_lens=lens, return_scores=True)
    Hs = Hkv if gate == "group" else Hq
    nb = pooled.shape[1]
    scores = np.full((B, Hs, 1, nb), np.nan)
    for (b, hs), s in ref["scores"].items():
        scores[b, hs, 0, : len(s)] = s
    gsel = sel.cpu().numpy()[:, :, None]
    diff = check_selection(gsel, ref["sel"][:, :, None], scores, topk, True)
    if diff:
        ref = oracle.decode(q, k, v, pooled, block=block, topk=topk, gate=gate, cache_lens=lens, force_sel=gsel[:, :, 0])
    assert_close(to_np(o), ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(to_np(lse), ref["lse"], 5e-3, None, what="lse")


@pytest.mark.parametrize("topk", [32, 48])
def test_decode_three_share_lists(bsa, topk):
    """4375 candidate blocks, so that each head's candidates fall in three shares: their lists
    hold 96 keys at top-32 (merged in one sort) and 144 at top-48 (merged list by list)."""
    B, Hq, Hkv, Lc, D, block = 2, 4, 1, 70000, 64, 16
    _say(f"case decode three shares B2 H4/1 Lc70000 D64 block16 topk{topk}")
    q = synth.host_tensor((B, Hq, D), 1.0, 21, 0, "bf16")
    k = synth.host_tensor((B, Lc, Hkv, D), 1.0, 21, 1, "bf16")
    v = synth.host_tensor((B, Lc, Hkv, D), 1.0, 21, 2, "bf16")
    lens = np.array([70000, 50001], dtype=np.int32)
    pooled = torch.from_numpy(oracle.block_pool(k, block)).to(torch.bfloat16)
    o, sel, lse = bsa.sparse_attn_decode(q.cuda(), k.cuda(), v.cuda(), pooled.cuda(), topk, block,
                                         cache_lens=torch.from_numpy(lens).cuda(), return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.decode(q, k, v, pooled, block=block, topk=topk, cache_lens=lens, return_scores=True)
    nb = pooled.shape[1]
    scores = np.full((B, Hq, 1, nb), np.nan)
    for (b, hs), s in ref["scores"].items():
        scores[b, hs, 0, : len(s)] = s
    gsel = sel.cpu().numpy()[:, :, None]
    diff = check_selection(gsel, ref["sel"][:, :, None], scores, topk, True)
    if diff:
        ref = oracle.decode(q, k, v, pooled, block=block, topk=topk, cache_lens=lens, force_sel=gsel[:, :, 0])
    assert_close(to_np(o), ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(to_np(lse), ref["lse"], 5e-3, None, what="lse")


def test_decode_topk60_group_of_8(bsa):
    """Eight query heads per KV head with top-60 each: 488 (head, block) pairs per group to unite."""
    B, Hq, Hkv, Lc, D, block, topk = 2, 16, 2, 20000, 128, 64, 60
    _say(f"case decode B2 H16/2 Lc20000 block64 topk60")
    q = synth.host_tensor((B, Hq, D), 1.0, 14, 0, "bf16")
    k = synth.host_tensor((B, Lc, Hkv, D), 1.0, 14, 1, "bf16")
    v = synth.host_tensor((B, Lc, Hkv, D), 1.0, 14, 2, "bf16")
    lens = np.array([20000, 12345], dtype=np.int32)
    pooled = torch.from_numpy(oracle.block_pool(k, block)).float()
    o, sel, lse = bsa.sparse_attn_decode(q.cuda(), k.cuda(), v.cuda(), pooled.cuda(), topk, block,
                                         cache_lens=torch.from_numpy(lens).cuda(), return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.decode(q, k, v, pooled, block=block, topk=topk, cache_lens=lens, return_scores=True)
    nb = pooled.shape[1]
    scores = np.full((B, Hq, 1, nb), np.nan)
    for (b, hs), s in ref["scores"].items():
        scores[b, hs, 0, : len(s)] = s
    gsel = sel.cpu().numpy()[:, :, None]
    diff = check_selection(gsel, ref["sel"][:, :, None], scores, topk, True)
    if diff:
        ref = oracle.decode(q, k, v, pooled, block=block, topk=topk, cache_lens=lens, force_sel=gsel[:, :, 0])
    assert_close(to_np(o), ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(to_np(lse), ref["lse"], 5e-3, None, what="lse")


def test_prerotated_keys_equal_internal_rotation(bsa):
    """A memory stored with its keys already rotated (the block summary's k_rot output) gives the
    same attention as rotating them inside the call."""
    B, Lq, Lk, Hq, Hkv, D, block, topk = 1, 96, 9000, 8, 2, 128, 64, 8
    _say("case pre-rotated keys vs in-call doc-RoPE")
    q = synth.host_tensor((B, Lq, Hq, D), 1.0, 19, 0, "bf16").cuda()
    k = synth.host_tensor((B, Lk, Hkv, D), 1.0, 19, 1, "bf16").cuda()
    v = synth.host_tensor((B, Lk, Hkv, D), 1.0, 19, 2, "bf16").cuda()
    dk = torch.from_numpy(synth.random_doc_ids(Lk, 700.0, 19)[None]).cuda()
    dq = torch.zeros((B, Lq), dtype=torch.int32, device="cuda")
    pooled, k_rot = bsa.block_summary(k, block, doc_ids=dk, return_k_rot=True)
    o1, s1 = bsa.sparse_attn_prefill(q, k, v, block, topk, False, doc_ids_q=dq, doc_ids_k=dk, pooled=pooled,
                                     return_sel=True)
    o2, s2 = bsa.sparse_attn_prefill(q, k_rot, v, block, topk, False, doc_ids_q=dq, pooled=pooled, return_sel=True)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("case", ["memory_split_candidates", "causal_group", "causal_head", "causal_head_small"])
def test_gate_planes_equal_fp32_summaries(bsa, case):
    """Summaries handed to the prefill as the gate's bf16 planes (written by the block summary) give
    the same selection and the same output, bit for bit, as the fp32 summaries they split; and the
    planes are that split: hi = bf16(s), lo = bf16(s - hi), round to nearest even."""
    causal = case != "memory_split_candidates"
    gate = "group" if case == "causal_group" else "head"
    if case == "causal_head_small":
        # at most 46 candidates and k = 3: the gate's small-candidate path stages either form
        B, Lq, Lk, Hq, Hkv, D, block, topk = 1, 3000, 3000, 8, 2, 128, 64, 3
    elif causal:
        B, Lq, Lk, Hq, Hkv, D, block, topk = 1, 3000, 3000, 8, 2, 128, 64, 6
    else:  # a few queries over a long memory: the candidates split over workgroups, then merged
        B, Lq, Lk, Hq, Hkv, D, block, topk = 1, 128, 200000, 8, 2, 128, 64, 16
    _say(f"case gate planes {case}: Lq{Lq} Lk{Lk} H{Hq}/{Hkv} block{block} topk{topk} {gate}")
    q = synth.host_tensor((B, Lq, Hq, D), 1.0, 23, 0, "bf16").cuda()
    k = synth.host_tensor((B, Lk, Hkv, D), 1.0, 23, 1, "bf16").cuda()
    v = synth.host_tensor((B, Lk, Hkv, D), 1.0, 23, 2, "bf16").cuda()
    kw = {}
    if causal:
        pooled, planes = bsa.block_summary(k, block, return_planes=True)
        k_att = k
    else:
        dk = torch.from_numpy(synth.random_doc_ids(Lk, 700.0, 23)[None]).cuda()
        kw["doc_ids_q"] = torch.zeros((B, Lq), dtype=torch.int32, device="cuda")
        pooled, k_att, planes = bsa.block_summary(k, block, doc_ids=dk, return_k_rot=True, return_planes=True)
    hi = pooled.to(torch.bfloat16)
    lo = (pooled - hi.float()).to(torch.bfloat16)
    assert torch.equal(planes[0].view(torch.int16), hi.permute(0, 2, 1, 3).contiguous().view(torch.int16))
    assert torch.equal(planes[1].view(torch.int16), lo.permute(0, 2, 1, 3).contiguous().view(torch.int16))
    o1, s1 = bsa.sparse_attn_prefill(q, k_att, v, block, topk, causal, gate=gate, pooled=pooled, return_sel=True, **kw)
    o2, s2 = bsa.sparse_attn_prefill(q, k_att, v, block, topk, causal, gate=gate, pooled=planes, return_sel=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_decode_head_major_cache(bsa):
    """Caches stored head-major ([B, Hkv, Lc, D]) and passed as strided [B, Lc, Hkv, D] views."""
    B, Hq, Hkv, Lc, D, block, topk = 2, 8, 2, 3000, 128, 128, 6
    _say("case decode head-major caches B2 H8/2 Lc3000 block128 topk6")
    q = synth.host_tensor((B, Hq, D), 1.0, 20, 0, "bf16")
    k = synth.host_tensor((B, Lc, Hkv, D), 1.0, 20, 1, "bf16")
    v = synth.host_tensor((B, Lc, Hkv, D), 1.0, 20, 2, "bf16")
    kd = k.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    vd = v.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    assert not kd.is_contiguous()
    lens = np.array([3000, 1777], dtype=np.int32)
    pooled = bsa.block_summary(kd, block, out_dtype=torch.bfloat16)  # checked against the oracle below
    ref_pool = oracle.block_pool(k, block)
    got_pool = pooled.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_pool - ref_pool) <= np.abs(ref_pool) * 2.0 ** -8 + 1e-7)
    ph = torch.from_numpy(ref_pool).to(torch.bfloat16)  # the oracle's own routing keys, rounded like the input
    o, sel, lse = bsa.sparse_attn_decode(q.cuda(), kd, vd, ph.cuda(), topk, block,
                                         cache_lens=torch.from_numpy(lens).cuda(), return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.decode(q, k, v, ph, block=block, topk=topk, cache_lens=lens, return_scores=True)
    nb = ph.shape[1]
    scores = np.full((B, Hq, 1, nb), np.nan)
    for (b, hs), sc in ref["scores"].items():
        scores[b, hs, 0, : len(sc)] = sc
    gsel = sel.cpu().numpy()[:, :, None]
    diff = check_selection(gsel, ref["sel"][:, :, None], scores, topk, True)
    if diff:
        ref = oracle.decode(q, k, v, ph, block=block, topk=topk, cache_lens=lens, force_sel=gsel[:, :, 0])
    assert_close(to_np(o), ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(to_np(lse), ref["lse"], 5e-3, None, what="lse")


@pytest.mark.parametrize("gate,layout,D", [("head", "token", 128), ("group", "head", 64), ("head", "head", 64)])
def test_decode_paged_cache(bsa, gate, layout, D):
    """Paged caches: 32-token pages drawn at random (with repeats) from a pool with spare pages, so
    sequences share pages and the pages of one sequence are out of order; pages stored token-major
    ([P, block, Hkv, D]) or head-major ([P, Hkv, block, D] passed as a strided view).  Checked
    against the oracle over the paged view, and bitwise against the contiguous call on the logical
    caches gathered on the host."""
    B, Hq, Hkv, block, nb, topk = 3, 8, 2, 32, 40, 6
    P = B * nb + 5
    Lc = nb * block
    _say(f"case paged decode gate={gate} layout={layout} D{D} B3 H8/2 pages{P} block32 topk6")
    q = synth.host_tensor((B, Hq, D), 1.0, 33, 0, "bf16")
    kp = synth.host_tensor((P, block, Hkv, D), 1.0, 33, 1, "bf16")
    vp = synth.host_tensor((P, block, Hkv, D), 1.0, 33, 2, "bf16")
    table = np.random.default_rng(33).integers(0, P, size=(B, nb)).astype(np.int32)
    lens = np.array([Lc, 700, 33], dtype=np.int32)
    # logical caches by plain indexing (host), their routing keys from the oracle
    k_log = kp[torch.from_numpy(table).long()].reshape(B, Lc, Hkv, D)
    v_log = vp[torch.from_numpy(table).long()].reshape(B, Lc, Hkv, D)
    pooled = torch.from_numpy(oracle.block_pool(k_log, block)).to(torch.bfloat16)
    if layout == "head":
        kd = kp.transpose(1, 2).contiguous().cuda().transpose(1, 2)
        vd = vp.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    else:
        kd, vd = kp.cuda(), vp.cuda()
    tab = torch.from_numpy(table).cuda()
    cl = torch.from_numpy(lens).cuda()
    o, sel, lse = bsa.sparse_attn_decode(q.cuda(), kd, vd, pooled.cuda(), topk, block, gate=gate, cache_lens=cl,
                                         block_table=tab, return_sel=True, return_lse=True)
    o2, sel2, lse2 = bsa.sparse_attn_decode(q.cuda(), k_log.cuda(), v_log.cuda(), pooled.cuda(), topk, block,
                                            gate=gate, cache_lens=cl, return_sel=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse, lse2)
    kv = (oracle.PagedCache(kp, table, block, Lc), oracle.PagedCache(vp, table, block, Lc))
    ref = oracle.decode(q, *kv, pooled, block=block, topk=topk, gate=gate, cache_lens=lens, return_scores=True)
    Hs = Hkv if gate == "group" else Hq
    scores = np.full((B, Hs, 1, nb), np.nan)
    for (b, hs), sc in ref["scores"].items():
        scores[b, hs, 0, : len(sc)] = sc
    gsel = sel.cpu().numpy()[:, :, None]
    diff = check_selection(gsel, ref["sel"][:, :, None], scores, topk, True)
    if diff:
        ref = oracle.decode(q, *kv, pooled, block=block, topk=topk, gate=gate, cache_lens=lens,
                            force_sel=gsel[:, :, 0])
    assert_close(to_np(o), ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(to_np(lse), ref["lse"], 5e-3, None, what="lse")


def _pinned(t):
    """A copy of a host tensor in pinned (page-locked, device-mapped) host memory."""
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


def test_host_tier_decode(bsa):
    """Host content tier: the caches stay in pinned host RAM (the kernels read the chosen blocks over
    the host link), the routing keys in GPU memory.  The library's routing keys summarised from the
    host caches equal the device-resident ones bitwise and the oracle's within bf16 rounding; the
    decode from host caches (contiguous and paged) is bitwise equal to the device-resident call, and
    its selection and output match the oracle's on the oracle's own routing keys."""
    B, Hq, Hkv, Lc, D, block, topk = 2, 8, 2, 3000, 128, 128, 6
    _say("case host-tier decode B2 H8/2 Lc3000 block128 topk6")
    q = synth.host_tensor((B, Hq, D), 1.0, 34, 0, "bf16")
    k = synth.host_tensor((B, Lc, Hkv, D), 1.0, 34, 1, "bf16")
    v = synth.host_tensor((B, Lc, Hkv, D), 1.0, 34, 2, "bf16")
    kh, vh = _pinned(k), _pinned(v)
    lens_np = np.array([3000, 1777], dtype=np.int32)
    lens = torch.from_numpy(lens_np).cuda()
    p_dev = bsa.block_summary(k.cuda(), block, out_dtype=torch.bfloat16)
    p_host = bsa.block_summary(kh, block, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(p_dev.view(torch.int16), p_host.view(torch.int16))
    ref_pool = oracle.block_pool(k, block)
    got_pool = p_host.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_pool - ref_pool) <= bf16_half_ulp(ref_pool) + 1e-7)
    # the oracle's own routing keys, rounded to bf16 like a stored input, drive both sides
    ph = torch.from_numpy(ref_pool).to(torch.bfloat16)
    qd, pd = q.cuda(), ph.cuda()
    o1, s1, l1 = bsa.sparse_attn_decode(qd, k.cuda(), v.cuda(), pd, topk, block, cache_lens=lens,
                                        return_sel=True, return_lse=True)
    o2, s2, l2 = bsa.sparse_attn_decode(qd, kh, vh, pd, topk, block, cache_lens=lens,
                                        return_sel=True, return_lse=True)
    # the same caches as host pages of 128 tokens, in order
    nb = -(-Lc // block)
    Lp = nb * block
    kp = torch.zeros((B * nb, block, Hkv, D), dtype=torch.bfloat16, pin_memory=True)
    vp = torch.zeros((B * nb, block, Hkv, D), dtype=torch.bfloat16, pin_memory=True)
    kp.view(B, Lp, Hkv, D)[:, :Lc] = k
    vp.view(B, Lp, Hkv, D)[:, :Lc] = v
    table = torch.arange(B * nb, dtype=torch.int32).reshape(B, nb).cuda()
    o3 = bsa.sparse_attn_decode(qd, kp, vp, pd, topk, block, cache_lens=lens, block_table=table)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(l1, l2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    ref = oracle.decode(q, k, v, ph, block=block, topk=topk, cache_lens=lens_np, return_scores=True)
    nbk = ph.shape[1]
    scores = np.full((B, Hq, 1, nbk), np.nan)
    for (b, hs), sc in ref["scores"].items():
        scores[b, hs, 0, : len(sc)] = sc
    gsel = s2.cpu().numpy()[:, :, None]
    diff = check_selection(gsel, ref["sel"][:, :, None], scores, topk, True)
    if diff:
        ref = oracle.decode(q, k, v, ph, block=block, topk=topk, cache_lens=lens_np, force_sel=gsel[:, :, 0])
    assert_close(to_np(o2), ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(to_np(l2), ref["lse"], 5e-3, None, what="lse")


@pytest.mark.parametrize("case", ["memory_prerotated", "causal_gather"])
def test_host_tier_prefill(bsa, case):
    """Host content tier for prefill: keys and values in pinned host RAM.  The memory-bank flow (keys
    stored rotated with their routing keys in GPU memory, a query chunk of its own document,
    non-causal) and a causal prefill whose attention runs on the LDS-staged gather; both bitwise
    equal to the device-resident call, and checked against the oracle (every query of the memory
    case; sampled queries with every head of the causal case)."""
    if case == "memory_prerotated":
        B, Lq, Lk, Hq, Hkv, D, block, topk, causal = 1, 96, 20000, 8, 2, 128, 64, 16, False
    else:
        B, Lq, Lk, Hq, Hkv, D, block, topk, causal = 1, 3000, 3000, 8, 2, 128, 128, 4, True
    _say(f"case host-tier prefill {case} Lq{Lq} Lk{Lk} H8/2 block{block} topk{topk}")
    qh_ = synth.host_tensor((B, Lq, Hq, D), 1.0, 35, 0, "bf16")
    q = qh_.cuda()
    k = synth.host_tensor((B, Lk, Hkv, D), 1.0, 35, 1, "bf16")
    v = synth.host_tensor((B, Lk, Hkv, D), 1.0, 35, 2, "bf16")
    kw = {}
    okw = {}
    if case == "memory_prerotated":
        ids = synth.random_doc_ids(Lk, 700.0, 35)[None]
        dk = torch.from_numpy(ids).cuda()
        # the oracle's routing keys (document-wise RoPE, then block means), fp32 as the gate takes them
        pos = oracle.doc_positions(ids)
        pool_ref = oracle.block_pool(k, block, pos=pos)
        pooled = torch.from_numpy(pool_ref).float().cuda()
        _, k_rot = bsa.block_summary(k.cuda(), block, doc_ids=dk, return_k_rot=True)
        kd = k_rot
        dq_ids = np.zeros((B, Lq), dtype=np.int32)
        kw = dict(doc_ids_q=torch.from_numpy(dq_ids).cuda(), pooled=pooled)
        okw = dict(doc_ids_q=dq_ids, doc_ids_k=ids, pooled=pooled.cpu())
        toks = None
    else:
        kd = k.cuda()
        toks = sorted({0, 1, 127, 128, 129, 1500, 2998, 2999} |
                      set(int(x) for x in np.random.default_rng(35).choice(Lq, 24, replace=False)))
    kh, vh = _pinned(kd.cpu()), _pinned(v)
    o1, s1, l1 = bsa.sparse_attn_prefill(q, kd, v.cuda(), block, topk, causal, return_sel=True, return_lse=True, **kw)
    o2, s2, l2 = bsa.sparse_attn_prefill(q, kh, vh, block, topk, causal, return_sel=True, return_lse=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)

    # the oracle rotates the original keys itself (memory case) and reads the host copies' contents
    def run_oracle(tokens=None, force_sel=None, scores=False):
        return oracle.prefill(qh_, k, v, block=block, topk=topk, causal=causal, tokens=tokens, force_sel=force_sel,
                              return_scores=scores, **okw)

    ref = run_oracle(tokens=toks, scores=True)
    gsel = s2.cpu().numpy() if toks is None else s2.cpu().numpy()[:, :, toks]
    diff = check_selection(gsel, ref["sel"], ref["scores"], topk, causal)
    _say(f"  selection rows {gsel.shape[1] * gsel.shape[2]}, near-tie differences {len(diff)}")
    ref = ref_with_gpu_sel(ref, diff, gsel, run_oracle, tokens=toks)
    go = to_np(o2) if toks is None else to_np(o2)[:, toks]
    gl = to_np(l2) if toks is None else to_np(l2)[:, :, toks]
    assert_close(go, ref["o"], 1e-2, 1e-2, bf16_storage=True)
    assert_close(gl, ref["lse"], 5e-3, None, what="lse")


def test_pageable_host_memory_rejected(bsa):
    """Pageable host memory cannot be read by a kernel: the call fails validation and enqueues
    nothing.  (The block table names no page, so even a launch would read no cache row.)"""
    B, Hq, Hkv, D, block, topk, nb = 1, 4, 1, 128, 64, 2, 4
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((nb, block, Hkv, D), dtype=torch.bfloat16)  # ordinary (pageable) host memory
    vc = torch.zeros((nb, block, Hkv, D), dtype=torch.bfloat16, device="cuda")
    pooled = torch.zeros((B, nb, Hkv, D), dtype=torch.bfloat16, device="cuda")
    table = torch.full((B, nb), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(bsa.BsaError) as e:
        bsa.sparse_attn_decode(q, kc, vc, pooled, topk, block, block_table=table)
    assert e.value.status == bsa.BSA_ERR_INVALID_ARG
    assert "pinned host memory" in str(e.value)


def test_deterministic_bitwise(bsa):
    B, L, Hq, Hkv, D = 1, 4096, 8, 2, 128
    _say("case determinism L4096 H8/2 block128 topk4")
    q = synth.host_tensor((B, L, Hq, D), 1.0, 11, 0, "bf16").cuda()
    k = synth.host_tensor((B, L, Hkv, D), 1.0, 11, 1, "bf16").cuda()
    v = synth.host_tensor((B, L, Hkv, D), 1.0, 11, 2, "bf16").cuda()
    a, sa = bsa.sparse_attn_prefill(q, k, v, 128, 4, True, return_sel=True)
    b, sb = bsa.sparse_attn_prefill(q, k, v, 128, 4, True, return_sel=True)
    torch.cuda.synchronize()
    assert torch.equal(sa, sb)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_select_blocks_matches_prefill_selection(bsa):
    B, L, Hq, Hkv, D = 1, 2048, 4, 2, 128
    _say("case select_blocks vs prefill")
    q = synth.host_tensor((B, L, Hq, D), 1.0, 12, 0, "bf16").cuda()
    k = synth.host_tensor((B, L, Hkv, D), 1.0, 12, 1, "bf16").cuda()
    v = synth.host_tensor((B, L, Hkv, D), 1.0, 12, 2, "bf16").cuda()
    _, s1 = bsa.sparse_attn_prefill(q, k, v, 64, 8, True, return_sel=True)
    s2 = bsa.select_blocks(q, k, 64, 8, True)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)


# --------------------------------------------------------------------------
# backward through the fixed selection
# --------------------------------------------------------------------------

BWD_CASES = {
    # name: (B, Lq, Lk, Hq, Hkv, D, block, topk, causal, gate)
    "head_causal_two_chunks": (1, 2500, 2500, 8, 2, 128, 64, 3, True, "head"),
    "group_causal_offset_d64": (2, 300, 500, 8, 2, 64, 32, 4, True, "group"),
    "head_noncausal_memory": (1, 40, 2000, 8, 2, 128, 64, 8, False, "head"),
    "group_block200_ragged": (1, 450, 450, 4, 1, 128, 200, 1, True, "group"),
}


@pytest.mark.parametrize("name", list(BWD_CASES))
def test_backward_matches_oracle(bsa, name):
    """Gradients through the GPU forward's own selection, element by element against the float64
    oracle on that selection.  Bound: 1e-2 of the largest reference gradient -- the kernel forms
    g . o from the bf16-rounded forward output (2^-9 relative) where the oracle uses the exact o;
    fp32 accumulation adds ~1e-6.  Also: a second call is bitwise identical."""
    B, Lq, Lk, Hq, Hkv, D, block, topk, causal, gate = BWD_CASES[name]
    _say(f"case backward {name}: B{B} Lq{Lq} Lk{Lk} H{Hq}/{Hkv} D{D} block{block} topk{topk} causal{causal} {gate}")
    q = synth.host_tensor((B, Lq, Hq, D), 1.0, 50, 0, "bf16")
    k = synth.host_tensor((B, Lk, Hkv, D), 1.0, 50, 1, "bf16")
    v = synth.host_tensor((B, Lk, Hkv, D), 1.0, 50, 2, "bf16")
    g = synth.host_tensor((B, Lq, Hq, D), 1.0, 50, 3, "bf16")
    qd, kd, vd, gd = q.cuda(), k.cuda(), v.cuda(), g.cuda()
    o, sel, lse = bsa.sparse_attn_prefill(qd, kd, vd, block, topk, causal, gate=gate, return_sel=True,
                                          return_lse=True)
    dq, dk, dv = bsa.sparse_attn_backward(qd, kd, vd, o, lse, sel, gd, block, causal, gate=gate)
    dq2, dk2, dv2 = bsa.sparse_attn_backward(qd, kd, vd, o, lse, sel, gd, block, causal, gate=gate)
    torch.cuda.synchronize()
    for a_, b_ in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a_.view(torch.int32), b_.view(torch.int32))
    ref = oracle.prefill_backward(q, k, v, g, sel.cpu().numpy(), block=block, causal=causal, gate=gate)
    for nm, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        r = ref[nm]
        top = float(np.abs(r).max())
        assert_close(to_np(got), r, 1e-2 * top, None, what=nm)
