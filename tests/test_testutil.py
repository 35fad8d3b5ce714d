"""The comparison helpers the GPU tests rely on, pinned on the CPU: the bf16
half-ulp against torch's own round-to-nearest, and the output bound's two
regimes."""
import numpy as np
import torch

from bsa_testutil import bf16_half_ulp, bf16_output_bound, check_selection


def test_half_ulp_values():
    # |x| in [2^k, 2^(k+1)) has ulp 2^(k-7): half of it is 2^(k-8)
    for x, k in ((1.0, 0), (1.9999, 0), (2.0, 1), (3.64, 1), (3.99, 1), (4.0, 2), (0.3, -2), (-5.5, 2)):
        assert bf16_half_ulp(x) == 2.0 ** (k - 8), x
    assert bf16_half_ulp(3.64) == 2.0 ** -7  # 7.8e-3


def test_half_ulp_bounds_torch_rounding():
    """Rounding to bf16 never moves a value by more than half an ulp, and the
    value halfway between two neighbours moves by exactly that much."""
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 1.0, 3.0, 100.0)])
    r = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    x32 = x.astype(np.float32).astype(np.float64)
    assert np.all(np.abs(r - x32) <= bf16_half_ulp(x32))
    # midpoints between consecutive bf16 values in [2, 4): ulp 2^-6, error exactly 2^-7
    base = 2.0 + np.arange(0, 64) * 2.0 ** -6
    mid = base + 2.0 ** -7
    rm = torch.from_numpy(mid.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.all(np.abs(rm - mid) == bf16_half_ulp(mid))


def test_output_bound_regimes():
    atol = 1e-2
    # every |o| < 4: the plain bound
    for o in (0.0, 0.5, 2.0, 3.64, 3.999):
        assert bf16_output_bound(o, atol) == atol
    # |o| in [4, 8): half an ulp (2^-6) plus the room the plain bound leaves below 4
    assert np.isclose(bf16_output_bound(4.5, atol), 2.0 ** -6 + atol - 2.0 ** -7)
    assert bf16_output_bound(-6.0, atol) > atol


def test_check_selection_rejects_a_wrong_tie_order():
    """Two blocks with exactly equal scores: the lower index wins, and a
    selection holding the higher one is a failure (no tie window applies
    to equal scores... the window admits both, so the strict comparison used
    by the tie tests is exact equality)."""
    scores = np.array([[[[1.0, 2.0, 2.0, 0.5]]]])
    ora = np.array([[[[1, -1]]]])  # top-1 non-causal: blocks 1 and 2 tie, 1 wins
    gpu_ok = ora.copy()
    assert check_selection(gpu_ok, ora, scores, 1, False) == []
    gpu_bad = np.array([[[[2, -1]]]])
    # the tie window accepts either member of an exact tie ...
    assert check_selection(gpu_bad, ora, scores, 1, False) == [(0, 0, 0)]
    # ... which is why the device tie tests compare selections with np.array_equal
    assert not np.array_equal(gpu_bad, ora)
