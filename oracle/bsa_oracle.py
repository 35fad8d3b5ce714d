"""Plain float64 CPU oracle for block-sparse attention with a top-k block gate.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library and imports
nothing from it.

What it computes, step by step, and where each step comes from:

* Per-document positions and document-wise RoPE -- "100 Millionen Token:
  Gedaechtnis oder Trugbild?" (aitalk.it), section "Das Gehirn mit zwei
  Geschwindigkeiten": the position counter restarts at zero at the start of
  every document so that a model trained on short texts sees only short
  positions.
* Per-block key summaries ("routing keys") -- same page and section: light,
  heavily compressed keys are what the router scores.  The pages do not say
  how they are formed; the reading used here is the arithmetic mean of the
  keys of each block (a short last block averages over the tokens it has).
* The gate -- MoBA repo card (ross.abutalabs.com/products/moba.json), field
  card.what_it_is: an MoE-style top-k gate picks KV blocks per query; and
  "MiniMax released MSA ..." (news.hamidun.com), section "How MSA Works": an
  index branch picks the top-k blocks per query and per GQA group.  Reading:
  the score of block j is the plain dot product of the (index) query with the
  block summary; for per-group gating the scores of the group's query heads
  are added.
* Masking and ties (the pages are silent): in causal mode blocks after the
  query's own block are never candidates, the query's own block is always
  attended and is not counted in k; ties go to the lower block index.
* The attention -- "MiniMax released MSA ...", sections "How MSA Works" and
  "Why Long Context is Hard to Scale": exact, un-approximated softmax
  attention over the union of the selected blocks' tokens (one softmax over
  all of them), with the token-level causal mask inside the query's own
  block.  MoBA's card (card.what_it_is) adds that top-k covering every block
  is full attention.

* Paged caches (PagedCache): a storage mapping only, defined in its
  docstring; decode over it is decode over the logical cache it stands for.
* Gradients (attend_grad, prefill_backward): the plain derivative of the
  exact attention above with the block selection held fixed -- the method is
  trained end to end (MoBA card, card.what_it_is; "MSA: Memory Sparse
  Attention", "Key Points"), and a top-k choice has no gradient, so the
  gradient flows through the chosen keys only.

Every array is widened to float64 before any arithmetic; nothing is rounded
in between.  Inputs may be NumPy arrays or CPU torch tensors (bfloat16 is
widened exactly).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "f64",
    "doc_positions",
    "rope_rotate_half",
    "block_pool",
    "gate_query",
    "current_block",
    "select_topk",
    "attend",
    "prefill",
    "decode",
    "PagedCache",
    "attend_grad",
    "prefill_backward",
]


def f64(x) -> np.ndarray:
    """Widen a NumPy array or a CPU torch tensor to a float64 NumPy array."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64, copy=False)
    try:  # torch tensor (kept optional: the oracle itself needs only NumPy)
        import torch

        if isinstance(x, torch.Tensor):
            if x.device.type != "cpu":
                raise ValueError("oracle inputs must live on the host")
            return x.detach().to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _int(x) -> np.ndarray:
    if isinstance(x, np.ndarray):
        return x.astype(np.int64, copy=False)
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().cpu().to(torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.int64)


# ---------------------------------------------------------------------------
# positions and document-wise RoPE
# ---------------------------------------------------------------------------

def doc_positions(doc_ids) -> np.ndarray:
    """Position of every token inside its own document.

    Document-wise RoPE ("100 Millionen Token ...", section "Das Gehirn mit
    zwei Geschwindigkeiten") restarts the position counter at 0 at each
    document start.  Reading: a document is a maximal run of equal
    consecutive ids, so pos[t] = t - (first index of t's run).

    doc_ids: [..., L] integers.  Returns int64 of the same shape.
    """
    d = _int(doc_ids)
    L = d.shape[-1]
    t = np.arange(L, dtype=np.int64)
    starts = np.zeros(d.shape, dtype=np.int64)
    if L:
        is_start = np.ones(d.shape, dtype=bool)
        is_start[..., 1:] = d[..., 1:] != d[..., :-1]
        # start of t's run = the largest run start <= t (a running maximum)
        starts = np.maximum.accumulate(np.where(is_start, t, 0), axis=-1)
    return t - starts


def rope_rotate_half(x, pos, theta: float = 10000.0) -> np.ndarray:
    """Rotary position embedding with the rotate-half pairing (i, i + D/2).

    The pages fix only that positions restart per document; the rotation
    form is the standard one (reading): for i < D/2, with w_i = theta^(-2i/D)
    and angle a = pos * w_i,
        x'_i       = x_i cos a - x_{i+D/2} sin a
        x'_{i+D/2} = x_i sin a + x_{i+D/2} cos a.

    x: [..., L, H, D]; pos: [..., L].  Float64 throughout.
    """
    x = f64(x)
    D = x.shape[-1]
    if D % 2:
        raise ValueError("RoPE needs an even head dimension")
    half = D // 2
    omega = theta ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    ang = _int(pos).astype(np.float64)[..., :, None] * omega  # [..., L, half]
    c = np.cos(ang)[..., :, None, :]
    s = np.sin(ang)[..., :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


# ---------------------------------------------------------------------------
# block summaries
# ---------------------------------------------------------------------------

def block_pool(k, block: int, chunk_blocks: int = 4096, pos=None, theta: float = 10000.0) -> np.ndarray:
    """Mean of the keys of each block (the routing-key reading).

    k: [..., L, H, D].  Returns [..., ceil(L/block), H, D] float64.  Block j
    covers tokens [j*block, min((j+1)*block, L)).  When `pos` ([..., L]) is
    given, each key is first rotated by document-wise RoPE at its own
    position.  Works through the key sequence `chunk_blocks` blocks at a time
    so that a large bfloat16 memory never has to be widened whole.
    """
    if block < 1:
        raise ValueError("block must be >= 1")
    L = k.shape[-3]
    nb = (L + block - 1) // block
    out = np.empty(tuple(k.shape[:-3]) + (nb,) + tuple(k.shape[-2:]), dtype=np.float64)
    for j0 in range(0, nb, chunk_blocks):
        j1 = min(nb, j0 + chunk_blocks)
        t0, t1 = j0 * block, min(L, j1 * block)
        kk = f64(k[..., t0:t1, :, :])
        if pos is not None:
            kk = rope_rotate_half(kk, _int(pos)[..., t0:t1], theta)
        for j in range(j0, j1):
            a, b = j * block - t0, min(L, (j + 1) * block) - t0
            out[..., j, :, :] = kk[..., a:b, :, :].mean(axis=-3)
    return out


# ---------------------------------------------------------------------------
# gate
# ---------------------------------------------------------------------------

def gate_query(q_heads, per_group: bool) -> np.ndarray:
    """Query that scores the block summaries.

    q_heads: [..., G, Dg] -- the (index) query vectors of one GQA group.
    Per head, every head scores with its own vector (returned unchanged).
    Per group ("MiniMax released MSA ...", section "How MSA Works": selection
    per GQA group; reading: the group's scores are the sum of its heads'
    scores), the score sum_h q_h . s equals (sum_h q_h) . s, so the group's
    query is the sum of its heads' vectors.
    """
    q = f64(q_heads)
    return q.sum(axis=-2, keepdims=True) if per_group else q


def current_block(qpos_abs: int, block: int) -> int:
    """Index of the block holding absolute position `qpos_abs`."""
    return qpos_abs // block


def select_topk(scores, n_cand: int, topk: int) -> list[int]:
    """Top-k of candidates 0..n_cand-1 by (score descending, index ascending).

    Keeps min(topk, n_cand) blocks and returns their indices ascending.  The
    tie rule (lower index wins) is a reading: the pages do not state one.
    """
    s = f64(scores)[:n_cand]
    idx = np.arange(n_cand)
    order = np.lexsort((idx, -s))  # primary key: -score; secondary: index
    return sorted(int(j) for j in order[: max(0, min(topk, n_cand))])


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def attend(q_row, keys, values, scale: float):
    """Exact softmax attention of one query over an explicit key set.

    q_row: [D]; keys, values: [n, D].  Returns (o [D], lse) with
    lse = log(sum_u exp(scale * q . k_u)) (natural log).  An empty key set
    gives o = 0 and lse = -inf.
    """
    q = f64(q_row)
    K = f64(keys)
    V = f64(values)
    if K.shape[0] == 0:
        return np.zeros(V.shape[-1] if V.ndim == 2 else q.shape[-1]), -math.inf
    z = (K @ q) * scale
    m = z.max()
    w = np.exp(z - m)
    tot = w.sum()
    return (w @ V) / tot, m + math.log(tot)


def _block_tokens(j: int, block: int, L: int):
    return j * block, min(L, (j + 1) * block)


def _rows(x, b: int, idx: np.ndarray, hk: int) -> np.ndarray:
    """x[b, idx, hk] widened to float64 (x: NumPy array or CPU torch tensor)."""
    if isinstance(x, np.ndarray):
        return f64(x[b, idx, hk])
    import torch

    return f64(x[b, torch.from_numpy(idx), hk])


def prefill(
    q,
    k,
    v,
    *,
    block: int,
    topk: int,
    causal: bool,
    gate: str = "head",
    index_q=None,
    index_k=None,
    doc_ids_q=None,
    doc_ids_k=None,
    theta: float = 10000.0,
    scale: float | None = None,
    pooled=None,
    tokens=None,
    return_scores: bool = False,
    force_sel=None,
):
    """Block-sparse attention prefill, evaluated row by row.

    q: [B, Lq, Hq, D]; k, v: [B, Lk, Hkv, D]; Hq = G * Hkv (GQA).
    gate: "head" -> one selection per query head (MoBA card); "group" -> one
      selection per GQA group with the heads' scores summed (MiniMax page).
    index_q [B, Lq, Hq, Di] / index_k [B, Lk, Hkv, Di]: optional separate
      index-branch tensors (MiniMax page, "How MSA Works"); when absent the
      gate scores with q and the (rotated) keys.
    doc_ids_q / doc_ids_k [B, Lq] / [B, Lk]: when given, q / k are rotated by
      document-wise RoPE at their per-document positions before use.
    causal: query i sits at absolute position Lk - Lq + i; its own block is
      forced, later blocks are excluded, and keys after the query inside its
      own block are masked.
    pooled: optional precomputed block summaries [B, Nb, Hkv, Dg].
    tokens: optional list of query indices to evaluate (all by default).
    force_sel: optional [B, Hs, T, w] block lists (-1 padded) that replace
      the gate's choice for the evaluated tokens -- used to evaluate the exact
      attention on another implementation's selection when two selections
      differ only by near-tied gate scores.

    Returns a dict with
      o    [B, T, Hq, D]       outputs for the evaluated tokens,
      lse  [B, Hq, T]          natural-log softmax normaliser,
      sel  [B, Hs, T, topk+c]  chosen blocks ascending (gate-chosen first,
                               then the forced block when causal), -1 padded,
      scores (optional) [B, Hs, T, Nb] gate scores (NaN where not a candidate),
      tokens               the evaluated query indices.
    """
    B, Lq, Hq, D = q.shape
    Bk, Lk, Hkv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    per_group = gate == "group"
    if gate not in ("head", "group"):
        raise ValueError("gate must be 'head' or 'group'")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nb = (Lk + block - 1) // block
    Hs = Hkv if per_group else Hq
    tok = list(range(Lq)) if tokens is None else [int(t) for t in tokens]
    T = len(tok)
    width = topk + (1 if causal else 0)

    pos_q = doc_positions(doc_ids_q) if doc_ids_q is not None else None
    pos_k = doc_positions(doc_ids_k) if doc_ids_k is not None else None

    # block summaries (routing keys)
    if pooled is None:
        src = index_k if index_k is not None else k
        rot = pos_k if (index_k is None and pos_k is not None) else None
        pooled = block_pool(src, block, pos=rot, theta=theta)
    pooled = f64(pooled)

    o = np.zeros((B, T, Hq, D))
    lse = np.full((B, Hq, T), -math.inf)
    sel = np.full((B, Hs, T, width), -1, dtype=np.int64)
    scores_out = np.full((B, Hs, T, nb), np.nan) if return_scores else None

    for b in range(B):
        for ti, t in enumerate(tok):
            qt = f64(q[b, t])  # [Hq, D]
            if pos_q is not None:
                qt = rope_rotate_half(qt[None], pos_q[b, t:t + 1], theta)[0]
            if index_q is not None:
                gq = f64(index_q[b, t])  # [Hq, Di]
            else:
                gq = qt
            qabs = Lk - Lq + t
            cur = current_block(qabs, block) if causal else None
            n_cand = cur if causal else nb
            # keys of the forced block, up to the query itself
            chosen_by_head = {}
            for hs in range(Hs):
                hk = hs if per_group else hs // G
                if per_group:
                    gvec = gate_query(gq[hk * G:(hk + 1) * G], True)[0]
                else:
                    gvec = gq[hs]
                s = pooled[b, :n_cand, hk, :] @ gvec if n_cand > 0 else np.zeros(0)
                if return_scores and n_cand > 0:
                    scores_out[b, hs, ti, :n_cand] = s
                ch = select_topk(s, n_cand, topk)
                row = ch + ([cur] if causal else [])
                if force_sel is not None:
                    row = [int(x) for x in np.asarray(force_sel)[b, hs, ti] if x >= 0]
                sel[b, hs, ti, : len(row)] = row
                chosen_by_head[hs] = row
            for h in range(Hq):
                hk = h // G
                hs = hk if per_group else h
                blocks = chosen_by_head[hs]
                idx = []
                for j in blocks:
                    a, e = _block_tokens(j, block, Lk)
                    if causal and j == cur:
                        e = min(e, qabs + 1)
                    idx.extend(range(a, e))
                idx = np.asarray(idx, dtype=np.int64)
                if idx.size:
                    kk = _rows(k, b, idx, hk)
                    if pos_k is not None:
                        kk = rope_rotate_half(kk[:, None, :], pos_k[b, idx], theta)[:, 0, :]
                    vv = _rows(v, b, idx, hk)
                else:
                    kk = np.zeros((0, D))
                    vv = np.zeros((0, D))
                o[b, ti, h], lse[b, h, ti] = attend(qt[h], kk, vv, scale)
    out = {"o": o, "lse": lse, "sel": sel, "tokens": tok}
    if return_scores:
        out["scores"] = scores_out
    return out


def decode(
    q,
    kcache,
    vcache,
    pooled,
    *,
    block: int,
    topk: int,
    gate: str = "head",
    cache_lens=None,
    scale: float | None = None,
    pairs=None,
    return_scores: bool = False,
    force_sel=None,
):
    """One decode step per sequence over a cached KV sequence.

    q: [B, Hq, D]; kcache, vcache: [B, Lc, Hkv, D]; pooled: [B, Nb, Hkv, D]
    (block summaries supplied by the caller, routing keys kept in fast memory
    per "100 Millionen Token ...", section "Das Gehirn mit zwei
    Geschwindigkeiten").  cache_lens [B] (default Lc for all): the new token
    is already in the cache at position n-1, so its block cur = (n-1)//block
    is forced, candidates are blocks 0..cur-1, and keys 0..n-1 of the forced
    block are attended.  pairs: optional list of (b, h) query rows to
    evaluate (default all).  force_sel [B, Hs, w] (optional) replaces the
    gate's choice, as in prefill.  kcache/vcache only need to support slicing
    [b, a:e, hk] -- a caller may pass an object that fetches slices lazily.

    Returns dict: o [B, Hq, D] (rows not evaluated stay 0), lse [B, Hq],
    sel [B, Hs, topk + 1] (-1 padded), optional scores {(b, hs): array}.
    """
    B, Hq, D = q.shape
    Lc = kcache.shape[1]
    Hkv = kcache.shape[2]
    G = Hq // Hkv
    per_group = gate == "group"
    Hs = Hkv if per_group else Hq
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lens = [Lc] * B if cache_lens is None else [int(x) for x in _int(cache_lens)]
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(Hq)]
    o = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -math.inf)
    sel = np.full((B, Hs, topk + 1), -1, dtype=np.int64)
    scores = {}
    done_sel = {}
    for b, h in pairs:
        n = lens[b]
        hk = h // G
        hs = hk if per_group else h
        cur = (n - 1) // block
        if (b, hs) not in done_sel:
            qg = f64(q[b, hk * G:(hk + 1) * G]) if per_group else f64(q[b, h])[None]
            gvec = gate_query(qg, per_group)[0]
            pk = f64(pooled[b, :cur, hk, :])
            s = pk @ gvec if cur > 0 else np.zeros(0)
            ch = select_topk(s, cur, topk)
            row = ch + [cur]
            if force_sel is not None:
                row = [int(x) for x in np.asarray(force_sel)[b, hs] if x >= 0]
            sel[b, hs, : len(row)] = row
            done_sel[(b, hs)] = row
            if return_scores:
                scores[(b, hs)] = s
        blocks = done_sel[(b, hs)]
        ks, vs = [], []
        for j in blocks:
            a, e = j * block, min(n, (j + 1) * block)
            ks.append(f64(kcache[b, a:e, hk]))
            vs.append(f64(vcache[b, a:e, hk]))
        kk = np.concatenate(ks, axis=0)
        vv = np.concatenate(vs, axis=0)
        o[b, h], lse[b, h] = attend(f64(q[b, h]), kk, vv, scale)
    out = {"o": o, "lse": lse, "sel": sel}
    if return_scores:
        out["scores"] = scores
    return out


class PagedCache:
    """A paged KV cache presented as the logical [B, Lc, Hkv, D] cache that
    decode() slices.

    The pages describe no storage layout for the cache; this is the plain
    definition of the paged one: the cache is split into pages of `block`
    tokens, and token t of sequence b is row t mod block of page
    table[b, t div block].  pages: [P, block, Hkv, D] (anything that slices as
    pages[p, a:e, h], e.g. a lazily fetched device tensor); table: [B, >= Nb]
    integers.  Only the slices decode() asks for are supported:
    [b, a:e, h] with 0 <= a <= e <= Lc; a slice may cross page boundaries.
    """

    def __init__(self, pages, table, block: int, Lc: int):
        self.pages = pages
        self.table = _int(table)
        self.block = int(block)
        self.shape = (self.table.shape[0], int(Lc), pages.shape[2], pages.shape[3])

    def __getitem__(self, key):
        b, sl, h = key
        a, e = sl.start, sl.stop
        parts = []
        t = a
        while t < e:
            j = t // self.block
            stop = min(e, (j + 1) * self.block)
            page = int(self.table[b, j])
            parts.append(f64(self.pages[page, t - j * self.block:stop - j * self.block, h]))
            t = stop
        if not parts:
            return np.zeros((0, self.shape[3]))
        return np.concatenate(parts, axis=0)


# ---------------------------------------------------------------------------
# gradients through a fixed selection
# ---------------------------------------------------------------------------

def attend_grad(q_row, keys, values, do_row, scale: float):
    """Gradient of o = sum_u p_u v_u, p = softmax_u(scale * q . k_u), for one
    query, given g = dL/do.

    Differentiating: dL/dv_u = p_u g; with d_u = g . v_u and
    ds_u = p_u (d_u - sum_w p_w d_w) (the softmax Jacobian),
    dL/dq = scale * sum_u ds_u k_u and dL/dk_u = scale * ds_u q.
    Returns (dq [D], dK [n, D], dV [n, D]); an empty key set gives zeros.
    """
    q = f64(q_row)
    K = f64(keys)
    V = f64(values)
    g = f64(do_row)
    if K.shape[0] == 0:
        return np.zeros_like(q), np.zeros_like(K), np.zeros_like(V)
    z = (K @ q) * scale
    w = np.exp(z - z.max())
    pr = w / w.sum()
    dV = pr[:, None] * g[None, :]
    dpr = V @ g
    ds = pr * (dpr - pr @ dpr)
    return scale * (ds @ K), scale * ds[:, None] * q[None, :], dV


def prefill_backward(q, k, v, dout, sel, *, block: int, causal: bool, gate: str = "head",
                     scale: float | None = None, rows=None):
    """Gradients of the prefill output w.r.t. q, k and v with the selection
    held fixed.

    q: [B, Lq, Hq, D]; k, v: [B, Lk, Hkv, D]; dout = dL/do [B, Lq, Hq, D];
    sel [B, Hs, Lq, w]: the blocks each selection row attended (-1 padded),
    e.g. the prefill's own sel.  Each query (b, t, h) attends the union of its
    selection row's blocks, with keys after the query masked inside its own
    block when causal (absolute query position Lk - Lq + t), exactly as in
    prefill(); its gradient contributions are summed into dk, dv over the
    keys it attended.  q and k are the attended (already position-encoded)
    tensors.  rows: optional list of (b, t, h) query rows to evaluate (default
    all); dq is then filled for those rows only and dk, dv hold only their
    contributions.  Returns dict dq [B, Lq, Hq, D], dk, dv [B, Lk, Hkv, D].
    """
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    per_group = gate == "group"
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    sel = _int(sel)
    dq = np.zeros((B, Lq, Hq, D))
    dk = np.zeros((B, Lk, Hkv, D))
    dv = np.zeros((B, Lk, Hkv, D))
    if rows is None:
        rows = [(b, t, h) for b in range(B) for t in range(Lq) for h in range(Hq)]
    for b, t, h in rows:
        qabs = Lk - Lq + t
        cur = current_block(qabs, block) if causal else None
        hk = h // G
        hs = hk if per_group else h
        idx = []
        for j in sel[b, hs, t]:
            if j < 0:
                continue
            a, e = _block_tokens(int(j), block, Lk)
            if causal and j == cur:
                e = min(e, qabs + 1)
            idx.extend(range(a, e))
        idx = np.asarray(idx, dtype=np.int64)
        if idx.size == 0:
            continue
        gq, gk, gv = attend_grad(q[b, t, h], _rows(k, b, idx, hk), _rows(v, b, idx, hk),
                                 dout[b, t, h], scale)
        dq[b, t, h] = gq
        dk[b, idx, hk] += gk
        dv[b, idx, hk] += gv
    return {"dq": dq, "dk": dk, "dv": dv}
