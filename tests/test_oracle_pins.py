"""Pins of the float64 oracle against things other than itself.

Each test ties one oracle step to an independent fact: a library routine
(torch's scaled_dot_product_attention in float64), a closed form, brute-force
enumeration with exact rational arithmetic, a hand-derived example, or an
invariant of the mathematics.  They are chosen so that a dropped term, a wrong
sign or index, or a transposed operand in the oracle fails at least one.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    """float64 CPU library attention; q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D] (GQA by repeat)."""
    G = q.shape[2] // k.shape[2]
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))
    kt = torch.from_numpy(np.ascontiguousarray(np.repeat(k, G, axis=2).transpose(0, 2, 1, 3)))
    vt = torch.from_numpy(np.ascontiguousarray(np.repeat(v, G, axis=2).transpose(0, 2, 1, 3)))
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal, scale=scale)
    return o.numpy().transpose(0, 2, 1, 3)


def _rand(shape, seed, tid, sigma=1.0):
    return synth.normal_host(shape, sigma, seed, tid).astype(np.float64)


# --------------------------------------------------------------------------
# attention step
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("block", [1, 3, 8, 64])
def test_full_topk_is_dense_attention(causal, block):
    """top-k covering every block reproduces dense attention (MoBA's full/sparse switch)."""
    B, L, Hq, Hkv, D = 2, 40, 4, 2, 16
    q, k, v = _rand((B, L, Hq, D), 1, 0), _rand((B, L, Hkv, D), 1, 1), _rand((B, L, Hkv, D), 1, 2)
    nb = -(-L // block)
    r = oracle.prefill(q, k, v, block=block, topk=nb, causal=causal)
    ref = _sdpa(q, k, v, causal=causal)
    np.testing.assert_allclose(r["o"], ref, rtol=0, atol=1e-12)


def test_dense_causal_with_offset_queries():
    """Lq < Lk: query i sits at key position Lk-Lq+i (bottom-right causal alignment)."""
    B, Lq, Lk, H, D = 1, 7, 29, 2, 8
    q, k, v = _rand((B, Lq, H, D), 2, 0), _rand((B, Lk, H, D), 2, 1), _rand((B, Lk, H, D), 2, 2)
    r = oracle.prefill(q, k, v, block=4, topk=100, causal=True)
    mask = np.zeros((Lq, Lk), dtype=bool)
    for i in range(Lq):
        mask[i, : Lk - Lq + i + 1] = True
    np.testing.assert_allclose(r["o"], _sdpa(q, k, v, mask=mask), rtol=0, atol=1e-12)


@pytest.mark.parametrize("gate", ["head", "group"])
@pytest.mark.parametrize("causal", [True, False])
def test_sparse_attention_equals_masked_dense(gate, causal):
    """Given the selection, the output is dense attention restricted to the chosen keys.

    The mask is built from the selected block ids (plus the causal mask) and fed
    to the library routine; one softmax spans all selected blocks.
    """
    B, L, Hq, Hkv, D, block, topk = 1, 48, 4, 2, 8, 5, 3
    q, k, v = _rand((B, L, Hq, D), 3, 0), _rand((B, L, Hkv, D), 3, 1), _rand((B, L, Hkv, D), 3, 2)
    r = oracle.prefill(q, k, v, block=block, topk=topk, causal=causal, gate=gate)
    G = Hq // Hkv
    mask = np.zeros((B, Hq, L, L), dtype=bool)
    for h in range(Hq):
        hs = h // G if gate == "group" else h
        for t in range(L):
            for j in r["sel"][0, hs, t]:
                if j < 0:
                    continue
                for u in range(j * block, min(L, (j + 1) * block)):
                    if not causal or u <= t:
                        mask[0, h, t, u] = True
    ref = _sdpa(q, k, v, mask=mask)
    np.testing.assert_allclose(r["o"], ref, rtol=0, atol=1e-12)
    # the selection really is sparse here
    assert (r["sel"] >= 0).sum(-1).max() <= topk + causal


def test_weights_sum_to_one_and_convex_hull():
    B, L, H, D = 1, 64, 2, 8
    q, k = _rand((B, L, H, D), 4, 0), _rand((B, L, H, D), 4, 1)
    c = np.full((B, L, H, D), 0.375)
    r = oracle.prefill(q, k, c, block=8, topk=2, causal=True)
    np.testing.assert_allclose(r["o"], 0.375, rtol=0, atol=1e-14)  # sum of weights is 1
    v = _rand((B, L, H, D), 4, 2)
    r = oracle.prefill(q, k, v, block=8, topk=2, causal=True)
    for h in range(H):
        for t in range(L):
            keys = []
            for j in r["sel"][0, h, t]:
                if j >= 0:
                    keys += [u for u in range(j * 8, (j + 1) * 8) if u <= t]
            lo, hi = v[0, keys, h].min(0), v[0, keys, h].max(0)
            assert np.all(r["o"][0, t, h] >= lo - 1e-12) and np.all(r["o"][0, t, h] <= hi + 1e-12)


def test_single_token_blocks_attend_only_self():
    """block=1, topk=0, causal: the forced own block is the token itself, so o = v."""
    B, L, H, D = 1, 17, 2, 4
    q, k, v = _rand((B, L, H, D), 5, 0), _rand((B, L, H, D), 5, 1), _rand((B, L, H, D), 5, 2)
    r = oracle.prefill(q, k, v, block=1, topk=0, causal=True)
    np.testing.assert_allclose(r["o"], v, rtol=0, atol=0)
    np.testing.assert_allclose(r["lse"], np.einsum("bthd,bthd->bht", q, k) / 2.0, atol=1e-14)


def test_attend_closed_form_two_keys():
    """Two keys with logits a, b: o = (e^a v1 + e^b v2)/(e^a + e^b), lse = log(e^a + e^b)."""
    q = np.array([1.0, 2.0])
    K = np.array([[0.5, 0.0], [0.0, 1.0]])  # logits 0.5, 2.0 at scale 1
    V = np.array([[1.0, 0.0], [0.0, 1.0]])
    o, lse = oracle.attend(q, K, V, 1.0)
    a, b = 0.5, 2.0
    np.testing.assert_allclose(o, [math.exp(a) / (math.exp(a) + math.exp(b)), math.exp(b) / (math.exp(a) + math.exp(b))], atol=1e-15)
    assert abs(lse - math.log(math.exp(a) + math.exp(b))) < 1e-14
    o, lse = oracle.attend(q, np.zeros((0, 2)), np.zeros((0, 2)), 1.0)
    assert lse == -math.inf and np.all(o == 0)


# --------------------------------------------------------------------------
# selection: brute force with exact rationals
# --------------------------------------------------------------------------

def _brute_select(scores, n_cand, topk):
    best = None
    kk = min(topk, n_cand)
    for comb in itertools.combinations(range(n_cand), kk):
        s = sum((scores[j] for j in comb), Fraction(0))
        key = (s, tuple(-j for j in comb))  # larger sum, then lexicographically lowest
        if best is None or key > best[0]:
            best = (key, comb)
    return list(best[1]) if best else []


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("block", [1, 2, 4, 8])
def test_selection_brute_force(seed, block):
    rng = np.random.default_rng(seed)
    L, D = 32, 4
    topk = int(rng.integers(1, 4))
    # small integers, with duplicated blocks to force exact ties
    k = rng.integers(-2, 3, size=(1, L, 1, D)).astype(np.float64)
    if L // block >= 4:
        k[0, block:2 * block] = k[0, 0:block]
        k[0, 3 * block:4 * block] = k[0, 2 * block:3 * block]
    q = rng.integers(-2, 3, size=(1, L, 1, D)).astype(np.float64)
    v = rng.standard_normal((1, L, 1, D))
    r = oracle.prefill(q, k, v, block=block, topk=topk, causal=True)
    nb = L // block
    pooled = [[Fraction(int(sum(k[0, j * block + i, 0, d] for i in range(block))), block) for d in range(D)] for j in range(nb)]
    for t in range(L):
        cur = t // block
        sc = [sum(Fraction(int(q[0, t, 0, d])) * pooled[j][d] for d in range(D)) for j in range(nb)]
        want = _brute_select(sc, cur, topk) + [cur]
        got = [int(x) for x in r["sel"][0, 0, t] if x >= 0]
        assert got == want, (t, got, want)


def test_selection_invariant_to_positive_query_scale():
    B, L, H, D = 1, 96, 2, 8
    q, k, v = _rand((B, L, H, D), 6, 0), _rand((B, L, H, D), 6, 1), _rand((B, L, H, D), 6, 2)
    a = oracle.prefill(q, k, v, block=8, topk=3, causal=True)
    b = oracle.prefill(q * 4.0, k, v, block=8, topk=3, causal=True)
    assert np.array_equal(a["sel"], b["sel"])


def test_fewer_candidates_than_k_takes_all():
    B, L, H, D = 1, 40, 1, 4
    q, k, v = _rand((B, L, H, D), 7, 0), _rand((B, L, H, D), 7, 1), _rand((B, L, H, D), 7, 2)
    r = oracle.prefill(q, k, v, block=8, topk=10, causal=True)
    for t in range(L):
        cur = t // 8
        assert [int(x) for x in r["sel"][0, 0, t] if x >= 0] == list(range(cur + 1))


def test_noncausal_block_permutation_equivariance():
    B, L, H, D, block = 1, 64, 2, 8, 8
    q, k, v = _rand((B, 16, H, D), 8, 0), _rand((B, L, H, D), 8, 1), _rand((B, L, H, D), 8, 2)
    perm = np.array([5, 2, 7, 0, 1, 6, 3, 4])
    tok = np.concatenate([np.arange(p * block, (p + 1) * block) for p in perm])
    a = oracle.prefill(q, k, v, block=block, topk=3, causal=False)
    b = oracle.prefill(q, k[:, tok], v[:, tok], block=block, topk=3, causal=False)
    np.testing.assert_allclose(a["o"], b["o"], atol=1e-12)
    inv = np.argsort(perm)  # new block position of old block p is inv[p]
    for h in range(H):
        for t in range(16):
            old = [int(x) for x in a["sel"][0, h, t]]
            new = sorted(int(inv[j]) for j in old)
            assert new == [int(x) for x in b["sel"][0, h, t]]


# --------------------------------------------------------------------------
# gate per group
# --------------------------------------------------------------------------

def test_group_gate_scores_are_sums_of_head_scores():
    B, L, Hq, Hkv, D = 1, 48, 6, 2, 8
    q, k, v = _rand((B, L, Hq, D), 9, 0), _rand((B, L, Hkv, D), 9, 1), _rand((B, L, Hkv, D), 9, 2)
    rh = oracle.prefill(q, k, v, block=6, topk=2, causal=True, gate="head", return_scores=True)
    rg = oracle.prefill(q, k, v, block=6, topk=2, causal=True, gate="group", return_scores=True)
    G = Hq // Hkv
    for g in range(Hkv):
        s = rh["scores"][0, g * G:(g + 1) * G].sum(0)
        np.testing.assert_allclose(rg["scores"][0, g], s, atol=1e-12, equal_nan=True)


def test_group_of_one_equals_per_head():
    B, L, H, D = 1, 48, 3, 8
    q, k, v = _rand((B, L, H, D), 10, 0), _rand((B, L, H, D), 10, 1), _rand((B, L, H, D), 10, 2)
    a = oracle.prefill(q, k, v, block=6, topk=2, causal=True, gate="head")
    b = oracle.prefill(q, k, v, block=6, topk=2, causal=True, gate="group")
    assert np.array_equal(a["sel"], b["sel"])
    np.testing.assert_allclose(a["o"], b["o"], atol=0)


def test_index_branch_tensors_drive_only_the_gate():
    """Separate index q/k change the selection but attention still uses q/k/v."""
    B, L, Hq, Hkv, D, Di = 1, 64, 4, 2, 8, 4
    q, k, v = _rand((B, L, Hq, D), 11, 0), _rand((B, L, Hkv, D), 11, 1), _rand((B, L, Hkv, D), 11, 2)
    iq, ik = _rand((B, L, Hq, Di), 11, 3), _rand((B, L, Hkv, Di), 11, 4)
    r = oracle.prefill(q, k, v, block=8, topk=2, causal=True, gate="group", index_q=iq, index_k=ik, return_scores=True)
    pooled = oracle.block_pool(ik, 8)
    t = 50
    for g in range(Hkv):
        want = pooled[0, :6, g] @ iq[0, t, g * 2:(g + 1) * 2].sum(0)
        np.testing.assert_allclose(r["scores"][0, g, t, :6], want, atol=1e-12)
    # and the attention is the masked dense attention of q/k/v over that selection
    mask = np.zeros((B, Hq, L, L), dtype=bool)
    for h in range(Hq):
        for tt in range(L):
            for j in r["sel"][0, h // 2, tt]:
                if j >= 0:
                    mask[0, h, tt, j * 8:min(L, j * 8 + 8)] = True
            mask[0, h, tt, tt + 1:] = False
    np.testing.assert_allclose(r["o"], _sdpa(q, k, v, mask=mask), atol=1e-12)


# --------------------------------------------------------------------------
# pooling
# --------------------------------------------------------------------------

def test_pool_block_one_is_identity_and_sum_is_preserved():
    k = _rand((2, 37, 3, 5), 12, 1)
    np.testing.assert_array_equal(oracle.block_pool(k, 1), k)
    for block in (4, 5, 37, 64):
        p = oracle.block_pool(k, block, chunk_blocks=2)
        nb = p.shape[1]
        n = np.array([min(block, 37 - j * block) for j in range(nb)], dtype=np.float64)
        np.testing.assert_allclose((p * n[None, :, None, None]).sum(1), k.sum(1), atol=1e-12)


def test_pool_hand_example():
    k = np.array([1.0, 3.0, 4.0, 8.0, 5.0]).reshape(1, 5, 1, 1)
    np.testing.assert_array_equal(oracle.block_pool(k, 2)[0, :, 0, 0], [2.0, 6.0, 5.0])


# --------------------------------------------------------------------------
# positions and RoPE
# --------------------------------------------------------------------------

def test_doc_positions_hand_and_loop():
    d = np.array([[7, 7, 7, 3, 3, 9, 7, 7]])
    assert oracle.doc_positions(d).tolist() == [[0, 1, 2, 0, 1, 0, 0, 1]]
    ids = synth.random_doc_ids(500, 13.0, seed=3)
    pos = oracle.doc_positions(ids)
    run = 0
    for t in range(500):
        run = 0 if t == 0 or ids[t] != ids[t - 1] else run + 1
        assert pos[t] == run


def test_rope_matches_complex_rotation_and_invariants():
    rng = np.random.default_rng(0)
    L, H, D = 12, 2, 16
    x = rng.standard_normal((L, H, D))
    pos = rng.integers(0, 5000, size=L)
    y = oracle.rope_rotate_half(x, pos)
    half = D // 2
    # complex form: (x_i + i x_{i+D/2}) * exp(i * pos * theta^(-2i/D))
    w = np.exp(1j * np.outer(pos, 10000.0 ** (-np.arange(half) * 2.0 / D)))
    z = (x[..., :half] + 1j * x[..., half:]) * w[:, None, :]
    np.testing.assert_allclose(y[..., :half], z.real, atol=1e-12)
    np.testing.assert_allclose(y[..., half:], z.imag, atol=1e-12)
    # position 0 is the identity, pair norms are kept
    np.testing.assert_array_equal(oracle.rope_rotate_half(x, np.zeros(L, int)), x)
    np.testing.assert_allclose(y[..., :half] ** 2 + y[..., half:] ** 2, x[..., :half] ** 2 + x[..., half:] ** 2, atol=1e-12)
    # pair 0 turns by exactly `pos` radians
    e = np.zeros((1, 1, D))
    e[..., 0] = 1.0
    r = oracle.rope_rotate_half(e, np.array([1]))
    assert abs(r[0, 0, 0] - math.cos(1.0)) < 1e-15 and abs(r[0, 0, half] - math.sin(1.0)) < 1e-15


def test_rope_relative_position_property():
    rng = np.random.default_rng(1)
    D = 8
    a, b = rng.standard_normal(D), rng.standard_normal(D)
    vals = []
    for m, n in [(10, 3), (107, 100), (7, 0), (5007, 5000)]:
        ra = oracle.rope_rotate_half(a.reshape(1, 1, D), np.array([m]))[0, 0]
        rb = oracle.rope_rotate_half(b.reshape(1, 1, D), np.array([n]))[0, 0]
        vals.append(ra @ rb)
    np.testing.assert_allclose(vals, vals[0], atol=1e-9)


def test_doc_rope_restart_equals_document_alone():
    """A document later in the memory is rotated exactly as if it stood alone at position 0."""
    rng = np.random.default_rng(2)
    L, H, D = 30, 2, 8
    k = rng.standard_normal((1, L, H, D))
    ids = np.array([[0] * 11 + [1] * 19])
    pos = oracle.doc_positions(ids)
    whole = oracle.rope_rotate_half(k, pos)
    alone = oracle.rope_rotate_half(k[:, 11:], np.arange(19)[None])
    np.testing.assert_allclose(whole[:, 11:], alone, atol=1e-14)
    # and one document is plain RoPE at 0..L-1
    np.testing.assert_allclose(oracle.rope_rotate_half(k, oracle.doc_positions(np.zeros((1, L), int))),
                               oracle.rope_rotate_half(k, np.arange(L)[None]), atol=0)


def test_doc_rope_prefill_uses_rotated_q_and_k():
    """With doc ids the whole pipeline equals the pipeline on pre-rotated inputs."""
    B, L, Hq, Hkv, D = 1, 40, 2, 1, 8
    q, k, v = _rand((B, L, Hq, D), 13, 0), _rand((B, L, Hkv, D), 13, 1), _rand((B, L, Hkv, D), 13, 2)
    ids = synth.random_doc_ids(L, 9.0, seed=13)[None]
    pos = oracle.doc_positions(ids)
    a = oracle.prefill(q, k, v, block=4, topk=2, causal=False, doc_ids_q=ids, doc_ids_k=ids)
    b = oracle.prefill(oracle.rope_rotate_half(q, pos), oracle.rope_rotate_half(k, pos), v, block=4, topk=2, causal=False)
    assert np.array_equal(a["sel"], b["sel"])
    np.testing.assert_allclose(a["o"], b["o"], atol=1e-12)


# --------------------------------------------------------------------------
# decode and prefill agree
# --------------------------------------------------------------------------

@pytest.mark.parametrize("gate", ["head", "group"])
def test_decode_equals_last_prefill_row(gate):
    B, L, Hq, Hkv, D, block = 2, 77, 4, 2, 8, 8
    q, k, v = _rand((B, L, Hq, D), 14, 0), _rand((B, L, Hkv, D), 14, 1), _rand((B, L, Hkv, D), 14, 2)
    pf = oracle.prefill(q, k, v, block=block, topk=3, causal=True, gate=gate)
    pooled = oracle.block_pool(k, block)
    dc = oracle.decode(q[:, -1], k, v, pooled, block=block, topk=3, gate=gate)
    np.testing.assert_allclose(dc["o"], pf["o"][:, -1], atol=1e-12)
    np.testing.assert_array_equal(dc["sel"], pf["sel"][:, :, -1])
    # shorter cache lengths: decode over the first n tokens = prefill on the prefix
    lens = np.array([50, 33])
    dc2 = oracle.decode(np.stack([q[0, 49], q[1, 32]]), k, v, pooled, block=block, topk=3, gate=gate, cache_lens=lens)
    for b, n in enumerate(lens):
        p2 = oracle.prefill(q[b:b + 1, :n], k[b:b + 1, :n], v[b:b + 1, :n], block=block, topk=3, causal=True, gate=gate)
        np.testing.assert_allclose(dc2["o"][b], p2["o"][0, -1], atol=1e-12)


def _paged_from_contiguous(cache, block, perm, spare):
    """Pages of `cache` [B, Lc, Hkv, D] (Lc a multiple of block) stored at shuffled page slots
    perm[b * Nb + j] among Nb * B + spare pages (spare slots hold unrelated values), plus the
    table that maps logical blocks back to them -- built with plain array indexing."""
    B, Lc, Hkv, D = cache.shape
    nb = Lc // block
    blocks = cache.reshape(B * nb, block, Hkv, D)
    pages = np.full((B * nb + spare, block, Hkv, D), 7.5)
    pages[perm] = blocks
    return pages, perm.reshape(B, nb)


@pytest.mark.parametrize("gate", ["head", "group"])
def test_paged_decode_equals_contiguous(gate):
    """Token t of sequence b lives in row t mod block of page table[b, t div block]: decode over the
    shuffled pages equals decode over the contiguous cache, for identity and shuffled tables."""
    B, Lc, Hq, Hkv, D, block = 3, 48, 4, 2, 8, 8
    q = _rand((B, Hq, D), 31, 0)
    k, v = _rand((B, Lc, Hkv, D), 31, 1), _rand((B, Lc, Hkv, D), 31, 2)
    pooled = oracle.block_pool(k, block)
    lens = np.array([48, 21, 1])
    ref = oracle.decode(q, k, v, pooled, block=block, topk=2, gate=gate, cache_lens=lens)
    nb = Lc // block
    rng = np.random.default_rng(5)
    for perm in (np.arange(B * nb), rng.permutation(B * nb + 4)[: B * nb]):
        kp, table = _paged_from_contiguous(k, block, perm, 4)
        vp, _ = _paged_from_contiguous(v, block, perm, 4)
        got = oracle.decode(q, oracle.PagedCache(kp, table, block, Lc), oracle.PagedCache(vp, table, block, Lc),
                            pooled, block=block, topk=2, gate=gate, cache_lens=lens)
        np.testing.assert_array_equal(got["sel"], ref["sel"])
        np.testing.assert_array_equal(got["o"], ref["o"])
        np.testing.assert_array_equal(got["lse"], ref["lse"])


def test_paged_cache_slices_cross_pages():
    """Every slice [b, a:e, h] of the paged view equals the contiguous cache's, including slices
    that start or end inside a page and span several pages."""
    B, Lc, Hkv, D, block = 2, 30, 2, 3, 4
    Lp = -(-Lc // block) * block
    cache = _rand((B, Lp, Hkv, D), 32, 1)
    perm = np.random.default_rng(6).permutation(B * Lp // block)
    pages, table = _paged_from_contiguous(cache, block, perm, 0)
    view = oracle.PagedCache(pages, table, block, Lc)
    assert view.shape == (B, Lc, Hkv, D)
    for b in range(B):
        for h in range(Hkv):
            for a in range(Lc + 1):
                for e in range(a, Lc + 1):
                    np.testing.assert_array_equal(view[b, a:e, h], cache[b, a:e, h])


# --------------------------------------------------------------------------
# gradients through a fixed selection
# --------------------------------------------------------------------------

@pytest.mark.parametrize("gate,causal", [("head", True), ("group", True), ("head", False)])
def test_backward_matches_finite_differences(gate, causal):
    """Central differences of L = sum(dO * O), with O from the forward oracle on the same fixed
    selection, agree with every analytic gradient element."""
    B, Lq, Lk, Hq, Hkv, D, block = 1, 7, 10, 4, 2, 3, 4
    q, k, v = _rand((B, Lq, Hq, D), 40, 0), _rand((B, Lk, Hkv, D), 40, 1), _rand((B, Lk, Hkv, D), 40, 2)
    g = _rand((B, Lq, Hq, D), 40, 3)
    sel = oracle.prefill(q, k, v, block=block, topk=1, causal=causal, gate=gate)["sel"]
    grads = oracle.prefill_backward(q, k, v, g, sel, block=block, causal=causal, gate=gate)

    def loss(qq, kk, vv):
        o = oracle.prefill(qq, kk, vv, block=block, topk=1, causal=causal, gate=gate, force_sel=sel)["o"]
        return float((o * g).sum())

    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            args = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
            argm = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
            num[i] = (loss(*args) - loss(*argm)) / (2 * h)
        np.testing.assert_allclose(grads[name], num, atol=1e-7, rtol=1e-6, err_msg=name)


def test_backward_dense_equals_torch_autograd():
    """With every block selected, the gradients are those of dense causal attention (offset
    queries, GQA): torch float64 autograd through scaled_dot_product_attention."""
    B, Lq, Lk, Hq, Hkv, D, block = 2, 9, 13, 4, 2, 8, 4
    q, k, v = _rand((B, Lq, Hq, D), 41, 0), _rand((B, Lk, Hkv, D), 41, 1), _rand((B, Lk, Hkv, D), 41, 2)
    g = _rand((B, Lq, Hq, D), 41, 3)
    nb = -(-Lk // block)
    sel = oracle.prefill(q, k, v, block=block, topk=nb, causal=True)["sel"]
    ours = oracle.prefill_backward(q, k, v, g, sel, block=block, causal=True)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    G = Hq // Hkv
    kk = tk.repeat_interleave(G, dim=2).transpose(1, 2)
    vv = tv.repeat_interleave(G, dim=2).transpose(1, 2)
    mask = torch.arange(Lk)[None, :] <= (Lk - Lq + torch.arange(Lq))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(tq.transpose(1, 2), kk, vv, attn_mask=mask)
    (o.transpose(1, 2) * torch.from_numpy(g)).sum().backward()
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(ours[name], t.grad.numpy(), atol=1e-12, rtol=1e-10, err_msg=name)


def test_backward_sum_rules():
    """Each row's softmax weights sum to one, so summed over all keys dv equals the summed output
    gradients of the heads that read them, and dk sums to zero (each row's ds sums to zero)."""
    B, L, Hq, Hkv, D, block = 2, 40, 6, 2, 5, 8
    q, k, v = _rand((B, L, Hq, D), 42, 0), _rand((B, L, Hkv, D), 42, 1), _rand((B, L, Hkv, D), 42, 2)
    g = _rand((B, L, Hq, D), 42, 3)
    sel = oracle.prefill(q, k, v, block=block, topk=2, causal=True, gate="group")["sel"]
    r = oracle.prefill_backward(q, k, v, g, sel, block=block, causal=True, gate="group")
    G = Hq // Hkv
    for hk in range(Hkv):
        np.testing.assert_allclose(r["dv"][:, :, hk].sum(axis=1), g[:, :, hk * G:(hk + 1) * G].sum(axis=(1, 2)),
                                   atol=1e-12)
        np.testing.assert_allclose(r["dk"][:, :, hk].sum(axis=1), 0.0, atol=1e-12)


# --------------------------------------------------------------------------
# hand-derived golden cases
# --------------------------------------------------------------------------

def _golden():
    with open(GOLDEN) as f:
        return {c["name"]: c for c in json.load(f)["cases"]}


def test_golden_causal_head_tie():
    c = _golden()["causal_head_tie"]
    q = np.array(c["q"], float).reshape(1, 8, 1, 2)
    k = np.array(c["k"], float).reshape(1, 8, 1, 2)
    v = np.array(c["v"], float).reshape(1, 8, 1, 2)
    r = oracle.prefill(q, k, v, block=c["block"], topk=c["topk"], causal=True, scale=c["scale"])
    assert r["sel"].tolist() == c["expected_sel"]
    env = {"E": math.e, "log": math.log}
    o0 = [eval(e, {}, env) for e in c["expected_o0_expr"]]
    lse = [eval(e, {}, env) for e in c["expected_lse_expr"]]
    np.testing.assert_allclose(r["o"][0, :, 0, 0], o0, atol=1e-14)
    np.testing.assert_allclose(r["o"][0, :, 0, 1], 1.0, atol=1e-15)
    np.testing.assert_allclose(r["lse"][0, 0], lse, atol=1e-14)


def test_golden_noncausal_group_vs_head():
    c = _golden()["noncausal_group_vs_head"]
    L = c["L"]
    q = np.tile(np.array(c["q_heads"], float)[None, None], (1, L, 1, 1))
    k = np.array(c["k"], float).reshape(1, L, 1, 2)
    v = np.array(c["v"], float).reshape(1, L, 1, 2)
    rg = oracle.prefill(q, k, v, block=2, topk=1, causal=False, gate="group", scale=1.0)
    rh = oracle.prefill(q, k, v, block=2, topk=1, causal=False, gate="head", scale=1.0)
    assert (rg["sel"][0, 0, :, 0] == c["expected_group_sel"][0]).all()
    for t in range(L):
        np.testing.assert_allclose(rg["o"][0, t], c["expected_group_o"], atol=1e-14)
        np.testing.assert_allclose(rh["o"][0, t], c["expected_head_o"], atol=1e-14)
        assert [int(rh["sel"][0, h, t, 0]) for h in range(2)] == c["expected_head_sel"]
