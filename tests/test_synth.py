"""Seeded input generator: determinism and the document-length recipe."""
import numpy as np

import synth


def test_host_draws_are_seeded_and_independent():
    a = synth.normal_host((4, 5), 1.0, 0, 0)
    b = synth.normal_host((4, 5), 1.0, 0, 0)
    c = synth.normal_host((4, 5), 1.0, 0, 1)
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_bf16_rounding_is_nearest_even():
    import torch

    t = synth.host_tensor((1000,), 1.0, 0, 0, "bf16")
    f = torch.from_numpy(synth.normal_host((1000,), 1.0, 0, 0))
    err = (t.float() - f).abs() / f.abs().clamp_min(1e-30)
    assert float(err.max()) <= 2.0 ** -8  # half an ulp of an 8-bit significand


def test_doc_lengths_recipe():
    n = synth.doc_lengths(10_000_000, 2000, 5000.0, 0.8, seed=0)
    assert n.sum() == 10_000_000 and n.min() >= 1 and len(n) == 2000
    # lognormal with log-sigma 0.8: the spread of log-lengths is close to 0.8
    assert abs(np.log(n).std() - 0.8) < 0.05
    ids = synth.doc_ids_from_lengths(n)
    assert ids.shape == (10_000_000,) and ids[0] == 0 and ids[-1] == 1999
    assert np.array_equal(n, synth.doc_lengths(10_000_000, 2000, 5000.0, 0.8, seed=0))


def test_repeated_dyadic_blocks_tie_exactly():
    """The premise of the device tie tests: with coarse dyadic keys whose
    blocks repeat, the oracle's block means and gate scores of equal blocks
    are exactly equal, per head and summed per group, and the top-k takes the
    lower index of a tie."""
    import oracle

    block, period = 16, 3
    k = synth.repeat_blocks(synth.dyadic_host((1, 160, 2, 64), 5, 1, "bf16"), block, period)
    q = synth.dyadic_host((1, 4, 64), 5, 0, "bf16")
    pooled = oracle.block_pool(k, block)  # [1, 10, 2, 64]
    for j in range(period, 10):
        assert np.array_equal(pooled[0, j], pooled[0, j % period])
    for per_group in (False, True):
        g = oracle.gate_query(q[0, :2], per_group)[0]
        s = pooled[0, :, 0, :] @ g
        for j in range(period, 10):
            assert s[j] == s[j % period]
        best = int(np.argmax(s[:period]))
        # top-2 of a score held by blocks best, best+3, best+6, best+9: the two lowest
        assert oracle.select_topk(s, 10, 2) == [best, best + period]
