"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and rounds them to the storage dtype; it
holds none of the attention method's arithmetic, and neither the oracle nor
the HIP library imports it.

Host draws use NumPy's PCG64.  Large device tensors are filled chunk by chunk
with torch's device generator seeded per (seed, tensor id, chunk), so a
tensor's contents do not depend on what else was generated before it.

Tensor ids (fixed so that every consumer regenerates the same data):
q=0, k=1, v=2, index_q=3, index_k=4, doc lengths=5, pooled=6.
"""
from __future__ import annotations

import hashlib

import numpy as np

TID = {"q": 0, "k": 1, "v": 2, "index_q": 3, "index_k": 4, "doc_lengths": 5, "pooled": 6, "dout": 7}

CHUNK = 1 << 24  # elements per device chunk


def _seed(seed: int, tensor_id: int, chunk: int = 0) -> int:
    h = hashlib.sha256(f"{seed}:{tensor_id}:{chunk}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def normal_host(shape, sigma: float, seed: int, tensor_id: int) -> np.ndarray:
    """float32 N(0, sigma^2) drawn on the host (PCG64)."""
    rng = np.random.Generator(np.random.PCG64(_seed(seed, tensor_id)))
    return (rng.standard_normal(size=tuple(shape), dtype=np.float64) * sigma).astype(np.float32)


def host_tensor(shape, sigma: float, seed: int, tensor_id: int, dtype: str):
    """CPU torch tensor of N(0, sigma^2) values in `dtype` ("f32" or "bf16").

    bf16 values are the float32 draws rounded to nearest-even by torch.
    """
    import torch

    x = torch.from_numpy(normal_host(shape, sigma, seed, tensor_id))
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def device_tensor(shape, sigma: float, seed: int, tensor_id: int, dtype: str, device="cuda"):
    """Device tensor of N(0, sigma^2) values, generated in fixed-size chunks.

    Each chunk of CHUNK elements (in row-major order) has its own generator
    seeded from (seed, tensor_id, chunk index).
    """
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.empty(tuple(shape), dtype=tdt, device=device)
    flat = out.view(-1)
    n = flat.numel()
    g = torch.Generator(device=device)
    for c, a in enumerate(range(0, n, CHUNK)):
        e = min(n, a + CHUNK)
        g.manual_seed(_seed(seed, tensor_id, c))
        tmp = torch.randn(e - a, generator=g, device=device, dtype=torch.float32)
        tmp.mul_(sigma)
        flat[a:e].copy_(tmp)
        del tmp
    return out


def dyadic_host(shape, seed: int, tensor_id: int, dtype: str, levels: int = 3, step: float = 0.25):
    """CPU torch tensor of coarse values: uniform integers in [-levels, levels]
    times `step` (a power of two), exact in bf16 and fp32.  Sums and products
    of a few hundred such values stay exact in fp32 and fp64, so two blocks
    holding the same keys score exactly alike in any arithmetic."""
    import torch

    rng = np.random.Generator(np.random.PCG64(_seed(seed, tensor_id)))
    x = rng.integers(-levels, levels + 1, size=tuple(shape)).astype(np.float32) * np.float32(step)
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def repeat_blocks(x, block: int, period: int, axis: int = 1):
    """Copy of `x` whose block j (tokens [j*block, (j+1)*block) along `axis`)
    holds the tokens of block j mod period: blocks repeat with the given
    period, so equal blocks (and equal block summaries) recur.  A short last
    block takes the first tokens of its source block."""
    y = x.clone()
    L = x.shape[axis]
    nb = -(-L // block)
    for j in range(period, nb):
        a, e = j * block, min(L, (j + 1) * block)
        src = (j % period) * block
        y.narrow(axis, a, e - a).copy_(x.narrow(axis, src, e - a))
    return y


def doc_lengths(total: int, n_docs: int, mean: float, sigma_log: float, seed: int) -> np.ndarray:
    """Lognormal document lengths rescaled to sum to exactly `total`.

    sigma_log is the log-space sigma; the log-space mu is chosen so that the
    lognormal's mean is `mean` (mu = ln(mean) - sigma^2/2).  The draws are
    rounded to integers >= 1 and rescaled to the exact total by the
    largest-remainder method.
    """
    rng = np.random.Generator(np.random.PCG64(_seed(seed, TID["doc_lengths"])))
    mu = np.log(mean) - 0.5 * sigma_log * sigma_log
    raw = rng.lognormal(mu, sigma_log, size=n_docs)
    raw = np.maximum(raw, 1.0)
    want = raw / raw.sum() * total
    base = np.maximum(np.floor(want).astype(np.int64), 1)
    short = total - int(base.sum())
    if short > 0:
        order = np.argsort(-(want - np.floor(want)), kind="stable")
        base[order[:short]] += 1
    elif short < 0:
        order = np.argsort(-base, kind="stable")
        i = 0
        while short < 0:
            j = order[i % n_docs]
            if base[j] > 1:
                base[j] -= 1
                short += 1
            i += 1
    assert int(base.sum()) == total and base.min() >= 1
    return base


def doc_ids_from_lengths(lengths) -> np.ndarray:
    """int32 [sum(lengths)]: document index of every token."""
    lengths = np.asarray(lengths, dtype=np.int64)
    return np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)


def random_doc_ids(L: int, mean_len: float, seed: int, tensor_id: int = TID["doc_lengths"]) -> np.ndarray:
    """int32 [L] document ids with geometric-ish random lengths (small tests)."""
    rng = np.random.Generator(np.random.PCG64(_seed(seed, tensor_id)))
    ids = np.empty(L, dtype=np.int32)
    d, t = 0, 0
    while t < L:
        n = int(max(1, rng.exponential(mean_len)))
        ids[t:t + n] = d
        t += n
        d += 1
    return ids
