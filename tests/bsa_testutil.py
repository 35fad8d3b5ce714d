"""Helpers for comparing the HIP library with the float64 oracle.

Selection rule: the chosen block set must equal the oracle's, except where the
k-th and (k+1)-th best gate scores lie within a relative 1e-4 of each other.
Then the GPU set passes if it has the oracle's size, holds the forced block,
holds every block scoring above tau + delta, and no block scoring below
tau - delta (tau = the oracle's k-th best score, delta = 1e-4 * max(|s_k|,
|s_k+1|)); that row's output is compared with the oracle's exact attention on
the GPU's own set.

Output rule: max-abs error <= 1e-2 for bf16 inputs and <= 1e-5 for fp32
inputs.  A bf16 output is itself rounded to nearest, which alone moves a
value by up to half a bf16 ulp: 2^(k-8) for |o| in [2^k, 2^(k+1)), i.e.
7.8e-3 below |o| = 4 and 1.56e-2 in [4, 8), more than the 1e-2 itself.  The
bound is therefore the plain 1e-2 wherever that rounding leaves the
computation at least 1e-2 - 2^-7 = 2.19e-3 of room (every |o| < 4), and
half an ulp plus that same 2.19e-3 above (bf16_output_bound).  The plain
max-abs error, the relative error (max-abs / max |o_ref|), the RMS error and
the largest |o_ref| are printed for every case.
"""
from __future__ import annotations

import math

import numpy as np

TIE_REL = 1e-4


def valid_set(row):
    return sorted(int(x) for x in row if x >= 0)


def check_selection(gpu_sel, ora_sel, ora_scores, topk, causal, cur_of=None, rel=TIE_REL):
    """Compare [B, Hs, T, W] selections. Returns list of (b, hs, ti) rows that
    differ within the tie window (callers re-evaluate those rows)."""
    gpu_sel = np.asarray(gpu_sel)
    ora_sel = np.asarray(ora_sel)
    assert gpu_sel.shape == ora_sel.shape, (gpu_sel.shape, ora_sel.shape)
    diff_rows = []
    B, Hs, T, W = gpu_sel.shape
    neq = np.any(gpu_sel != ora_sel, axis=-1)
    for b, hs, ti in zip(*np.nonzero(neq)):
        g = valid_set(gpu_sel[b, hs, ti])
        o = valid_set(ora_sel[b, hs, ti])
        if g == o:
            # same set, different order/padding: the layout is part of the contract
            raise AssertionError(f"row {(b, hs, ti)}: same set, different layout {gpu_sel[b, hs, ti]} vs {ora_sel[b, hs, ti]}")
        cur = None
        if causal:
            cur = o[-1]
            assert g and g[-1] == cur, f"row {(b, hs, ti)}: forced block missing {g} vs {o}"
        gg = [j for j in g if j != cur]
        og = [j for j in o if j != cur]
        assert len(gg) == len(og), f"row {(b, hs, ti)}: sizes differ {g} vs {o}"
        s = np.asarray(ora_scores[b, hs, ti], dtype=np.float64)
        cand = np.nonzero(~np.isnan(s))[0]
        order = sorted(cand, key=lambda j: (-s[j], j))
        k = len(og)
        tau = s[order[k - 1]]
        nxt = s[order[k]] if k < len(order) else tau
        delta = rel * max(abs(tau), abs(nxt))
        must = {int(j) for j in cand if s[j] > tau + delta}
        forbid = {int(j) for j in cand if s[j] < tau - delta}
        assert all(not np.isnan(s[j]) for j in gg), f"row {(b, hs, ti)}: non-candidate chosen {gg}"
        assert must <= set(gg), f"row {(b, hs, ti)}: missing clear winners {sorted(must - set(gg))}; gpu {g} oracle {o}"
        assert not (forbid & set(gg)), f"row {(b, hs, ti)}: chose clear losers {sorted(forbid & set(gg))}; gpu {g} oracle {o}"
        diff_rows.append((int(b), int(hs), int(ti)))
    return diff_rows


def err_stats(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    e = np.abs(got - ref)
    mx = float(e.max()) if e.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    rms = float(np.sqrt((e ** 2).mean())) if e.size else 0.0
    return {"max_abs": mx, "rel": mx / scale if scale > 0 else mx, "rms": rms, "ref_max": scale}


def bf16_half_ulp(x):
    """Half a bf16 unit in the last place at each |x|: 2^(k-8) for |x| in
    [2^k, 2^(k+1)) (8 significant bits), the largest error of rounding a
    real value of that magnitude to bf16 by nearest; 2^-134 (half the
    smallest subnormal) at 0 and below the normal range."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(a)  # a = f * 2^e, f in [0.5, 1): k = e - 1
    h = np.ldexp(1.0, e - 9)
    return np.where(a >= 2.0 ** -126, h, 2.0 ** -134)


def bf16_output_bound(ref, atol):
    """Element-wise bound for a bf16 output: room = atol - 2^-7 is what atol
    leaves the computation below |o| = 4 (where half an ulp is at most
    2^-7); the bound is the plain atol wherever half an ulp of ref is at most
    atol - room, and half an ulp plus room where it is larger."""
    room = atol - 2.0 ** -7  # 2.19e-3 for atol = 1e-2
    return np.maximum(atol, bf16_half_ulp(ref) + room)


def assert_close(got, ref, atol, rel=None, what="o", bf16_storage=False):
    st = err_stats(got, ref)
    msg = f"{what}: max_abs={st['max_abs']:.3e} rel={st['rel']:.3e} rms={st['rms']:.3e} |ref|max={st['ref_max']:.3e}"
    print(msg)
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    bound = bf16_output_bound(r, atol) if bf16_storage else atol
    worst = float(np.max(np.abs(g - r) - bound)) if g.size else -1.0
    assert worst <= 0.0, msg + f" (exceeds bound by {worst:.3e})"
    if rel is not None:
        assert st["rel"] <= rel, msg
    return st


def to_np(t):
    import torch

    return t.detach().to("cpu", torch.float64).numpy() if t.dtype.is_floating_point else t.detach().cpu().numpy()


def ln2():
    return math.log(2.0)


class RowView:
    """Sampled query rows presented to the oracle at their true positions.

    rows: CPU tensor [B, T, ...] holding the rows of `toks` (in that order) of a
    [B, L, ...] tensor; only [b, t] indexing with t in `toks` is supported.
    """

    def __init__(self, rows, toks, L):
        self.rows = rows
        self.index = {int(t): i for i, t in enumerate(toks)}
        self.shape = (rows.shape[0], L) + tuple(rows.shape[2:])

    def __getitem__(self, key):
        b, t = key
        return self.rows[b, self.index[int(t)]]


class HostSlices:
    """A device tensor presented to the oracle as host copies of the slices it
    asks for (the oracle reads only the blocks it needs from a large cache)."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, key):
        import torch

        if not isinstance(key, tuple):
            key = (key,)
        key = tuple(k.to(self.t.device) if isinstance(k, torch.Tensor) else k for k in key)
        return self.t[key].cpu()


def ref_with_gpu_sel(ref, diff_rows, gpu_sel, run_oracle, tokens=None):
    """Recompute the oracle outputs of the evaluated tokens whose selection
    legitimately differs (near-ties), on the GPU's own selection.

    ref: oracle prefill result over evaluated tokens (index ti); diff_rows:
    (b, hs, ti) from check_selection; gpu_sel [B, Hs, T, W] for the same
    evaluated tokens; tokens[ti] = the query index of evaluated token ti
    (default ti itself); run_oracle(tokens=..., force_sel=...) reruns the oracle.
    """
    if not diff_rows:
        return ref
    tis = sorted({ti for (_, _, ti) in diff_rows})
    toks = [int(tokens[ti]) if tokens is not None else ti for ti in tis]
    fs = np.asarray(gpu_sel)[:, :, tis]
    r2 = run_oracle(tokens=toks, force_sel=fs)
    o = ref["o"].copy()
    lse = ref["lse"].copy()
    for i, ti in enumerate(tis):
        o[:, ti] = r2["o"][:, i]
        lse[:, :, ti] = r2["lse"][:, :, i]
    return {"o": o, "lse": lse}
