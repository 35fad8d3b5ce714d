"""Benchmark of the block-sparse attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
  * prefill at 128K -- MiniMax-style index/main branch: batch 1, 131072
    tokens, 64 query heads / 8 KV heads, head dim 128, block 64, index q/k of
    dim 64, gate scores summed over each group's 8 heads, top-16 blocks per
    group plus the own block, causal, bf16 N(0,1);
  * decode -- 16 sequences x 1 new token over 1,048,576-token caches
    (stored head-major),
    32/8 heads, head dim 128, block 128, bf16 routing keys (8192 blocks)
    precomputed once by the library's block summary, top-32 per query head
    plus the own block, bf16 N(0,1).
Inputs are generated on the device and resident in HBM before timing.

Prints one JSON line.  `value` is whole-step token throughput (prefill
tokens + decode tokens per second); `breakdown` splits prefill and decode;
`roofline` covers the dominant kernel; `cpu_baseline` times the float64
oracle on a bounded sample of the prefill.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

PREFILL = dict(B=1, L=131072, Hq=64, Hkv=8, D=128, block=64, Di=64, topk=16, causal=True, gate="group", sigma=1.0)
DECODE = dict(B=16, Lc=1048576, Hq=32, Hkv=8, D=128, block=128, topk=32, gate="head", sigma=1.0)
SEED = 0


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def make_prefill_inputs():
    import synth

    c = PREFILL
    t = synth.TID
    q = synth.device_tensor((c["B"], c["L"], c["Hq"], c["D"]), c["sigma"], SEED, t["q"], "bf16")
    k = synth.device_tensor((c["B"], c["L"], c["Hkv"], c["D"]), c["sigma"], SEED, t["k"], "bf16")
    v = synth.device_tensor((c["B"], c["L"], c["Hkv"], c["D"]), c["sigma"], SEED, t["v"], "bf16")
    iq = synth.device_tensor((c["B"], c["L"], c["Hq"], c["Di"]), c["sigma"], SEED, t["index_q"], "bf16")
    ik = synth.device_tensor((c["B"], c["L"], c["Hkv"], c["Di"]), c["sigma"], SEED, t["index_k"], "bf16")
    return q, k, v, iq, ik


def make_decode_inputs(m):
    import synth

    c = DECODE
    t = synth.TID
    # distinct seed stream from the prefill inputs
    q = synth.device_tensor((c["B"], c["Hq"], c["D"]), c["sigma"], SEED + 1, t["q"], "bf16")
    # caches stored head-major ([B, Hkv, Lc, D], passed as [B, Lc, Hkv, D]
    # views): a block of one KV head is then 32 contiguous KB in HBM
    kc = synth.device_tensor((c["B"], c["Hkv"], c["Lc"], c["D"]), c["sigma"], SEED + 1, t["k"], "bf16").transpose(1, 2)
    vc = synth.device_tensor((c["B"], c["Hkv"], c["Lc"], c["D"]), c["sigma"], SEED + 1, t["v"], "bf16").transpose(1, 2)
    import torch

    pooled = m.block_summary(kc, c["block"], out_dtype=torch.bfloat16)  # routing keys, computed once
    return q, kc, vc, pooled


MOBA = dict(B=1, L=32768, Hq=32, Hkv=8, D=128, block=512, topk=3, sigma=128 ** -0.5)
MEMORY = dict(Lk=10_000_000, docs=2000, doc_mean=5000.0, doc_sigma=0.8, Lq=512, Hq=32, Hkv=8, D=128, block=64,
              topk=64)


def causal_pairs(L, bs, k):
    """(query, key) pairs a causal top-k + own-block prefill attends per head."""
    n = 0
    for t in range(L):
        cur = t // bs
        n += min(k, cur) * bs + (t - cur * bs + 1)
    return n


def time_call(fn, reps):
    import torch

    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def other_workloads(m, reps):
    """Times the MoBA-style 32K prefill and the 10M-token memory-bank prefill
    (reported beside the benchmark step, not part of it)."""
    import numpy as np
    import torch

    import synth

    t = synth.TID
    out = {}
    c = MOBA
    q = synth.device_tensor((c["B"], c["L"], c["Hq"], c["D"]), c["sigma"], SEED, t["q"], "bf16")
    k = synth.device_tensor((c["B"], c["L"], c["Hkv"], c["D"]), c["sigma"], SEED, t["k"], "bf16")
    v = synth.device_tensor((c["B"], c["L"], c["Hkv"], c["D"]), c["sigma"], SEED, t["v"], "bf16")
    o = torch.empty_like(q)
    ws = torch.empty(m.prefill_workspace_bytes(q, k, block=c["block"], topk=c["topk"], causal=True),
                     dtype=torch.uint8, device="cuda")
    ms = time_call(lambda: m.sparse_attn_prefill(q, k, v, c["block"], c["topk"], True, out=o, workspace=ws), reps)
    flops = 4.0 * c["D"] * c["Hq"] * causal_pairs(c["L"], c["block"], c["topk"])
    out["moba_32k_prefill"] = {"ms": round(ms, 4), "tokens_per_s": round(c["L"] / (ms * 1e-3), 1),
                               "attended_tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
    _log(f"MoBA-style 32K prefill: {ms:.3f} ms")
    # its backward through the selection (a training step's attention part)
    g = synth.device_tensor((c["B"], c["L"], c["Hq"], c["D"]), 1.0, SEED, t["dout"], "bf16")
    o, sel, lse = m.sparse_attn_prefill(q, k, v, c["block"], c["topk"], True, return_sel=True, return_lse=True)
    grads = (torch.empty(q.shape, dtype=torch.float32, device="cuda"),
             torch.empty(k.shape, dtype=torch.float32, device="cuda"),
             torch.empty(v.shape, dtype=torch.float32, device="cuda"))
    bws = torch.empty(m.backward_workspace_bytes(q, k, sel, block=c["block"], causal=True), dtype=torch.uint8,
                      device="cuda")
    bms = time_call(lambda: m.sparse_attn_backward(q, k, v, o, lse, sel, g, c["block"], True, out=grads,
                                                   workspace=bws), reps)
    m.timer_enable(1)
    m.timer_reset()
    for _ in range(2):
        m.sparse_attn_backward(q, k, v, o, lse, sel, g, c["block"], True, out=grads, workspace=bws)
    torch.cuda.synchronize()
    dkv_ms = m.timer_report("attn_bwd_dkv")[0] / 2
    dq_ms = m.timer_report("attn_bwd_dq")[0] / 2
    kms = dkv_ms + dq_ms
    m.timer_enable(0)
    bflops = 2.5 * flops  # per attended pair: q.k, g.v and the three products for dq, dk, dv = 10 D
    out["moba_32k_backward"] = {"ms": round(bms, 4), "attn_bwd_dkv_ms": round(dkv_ms, 4),
                                "attn_bwd_dq_ms": round(dq_ms, 4),
                                "attended_tflops": round(bflops / (bms * 1e-3) / 1e12, 2),
                                "kernel_tflops": round(bflops / (kms * 1e-3) / 1e12, 2),
                                "kernel_frac_bf16_peak": round(bflops / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                "note": "gradients through the forward's selection; bf16 MFMA, fp32 accumulation; "
                                        "the dk/dv and dq kernels form 7 products per attended pair (S and dP "
                                        "in both), the flops counted are the 5 the gradient needs"}
    _log(f"MoBA-style 32K backward: {bms:.3f} ms (dk/dv {dkv_ms:.3f} ms, dq {dq_ms:.3f} ms, "
         f"{bflops / (kms * 1e-3) / 1e12:.1f} TFLOP/s)")
    del q, k, v, o, ws, g, sel, lse, grads, bws
    c = MEMORY
    ids = synth.doc_ids_from_lengths(synth.doc_lengths(c["Lk"], c["docs"], c["doc_mean"], c["doc_sigma"], SEED))
    dk = torch.from_numpy(ids[None]).cuda()
    dq = torch.zeros((1, c["Lq"]), dtype=torch.int32, device="cuda")
    q = synth.device_tensor((1, c["Lq"], c["Hq"], c["D"]), 1.0, SEED, t["q"], "bf16")
    k = synth.device_tensor((1, c["Lk"], c["Hkv"], c["D"]), 1.0, SEED, t["k"], "bf16")
    v = synth.device_tensor((1, c["Lk"], c["Hkv"], c["D"]), 1.0, SEED, t["v"], "bf16")
    ms_sum = time_call(lambda: m.block_summary(k, c["block"], doc_ids=dk), reps)
    # the memory's offline encoding: routing keys (stored as the gate's bf16
    # hi / lo planes) and document-wise rotated content keys, stored once
    pooled, k_rot, planes = m.block_summary(k, c["block"], doc_ids=dk, return_k_rot=True, return_planes=True)
    del k
    o = torch.empty_like(q)
    kw = dict(doc_ids_q=dq, pooled=planes)  # keys arrive rotated; the query chunk is rotated per call
    ws = torch.empty(m.prefill_workspace_bytes(q, k_rot, block=c["block"], topk=c["topk"], causal=False, **kw),
                     dtype=torch.uint8, device="cuda")
    ms = time_call(lambda: m.sparse_attn_prefill(q, k_rot, v, c["block"], c["topk"], False, out=o, workspace=ws,
                                                 **kw), reps)
    out["memory_10m_summary"] = {"ms": round(ms_sum, 4),
                                 "read_gbs": round(2 * c["Lk"] * c["Hkv"] * c["D"] / (ms_sum * 1e-3) / 1e9, 1)}
    out["memory_10m_query_chunk"] = {"ms": round(ms, 4), "query_tokens_per_s": round(c["Lq"] / (ms * 1e-3), 1),
                                     "note": "keys stored rotated, routing keys stored as the gate's bf16 hi / lo planes (offline encoding)"}
    _log(f"memory bank: summaries {ms_sum:.3f} ms, 512-token query chunk {ms:.3f} ms")
    # host content tier: the memory's rotated keys and its values (41 GB) in
    # pinned host RAM, its routing keys in GPU memory; only the chosen blocks
    # cross the host link
    # (stored head-major there, so one block of one KV head is 16 contiguous KB)
    _log("host tier: moving the memory's keys and values to pinned host RAM")
    hm = (1, c["Hkv"], c["Lk"], c["D"])
    kh = torch.empty(hm, dtype=k_rot.dtype, pin_memory=True)
    kh.copy_(k_rot.transpose(1, 2))
    del k_rot
    vh = torch.empty(hm, dtype=v.dtype, pin_memory=True)
    vh.copy_(v.transpose(1, 2))
    del v
    kh, vh = kh.transpose(1, 2), vh.transpose(1, 2)
    torch.cuda.empty_cache()

    def hosted_chunk():
        return m.sparse_attn_prefill(q, kh, vh, c["block"], c["topk"], False, out=o, workspace=ws, **kw)

    ms_h = time_call(hosted_chunk, reps)
    sel = m.select_blocks(q, kh, c["block"], c["topk"], False, **kw)  # [1, Hq, Lq, topk]
    hk = torch.arange(c["Hq"], device="cuda").view(1, c["Hq"], 1, 1) // (c["Hq"] // c["Hkv"])
    nbm = pooled.shape[1]
    keys = (hk * nbm + sel.long()).masked_select(sel >= 0)
    distinct = int(torch.unique(keys).numel())
    m.timer_enable(1)
    m.timer_reset()
    for _ in range(2):
        hosted_chunk()
    torch.cuda.synchronize()
    att_ms = m.timer_report("attn")[0] / 2
    m.timer_enable(0)
    kv_bytes = distinct * c["block"] * c["D"] * 2 * 2
    out["memory_10m_query_chunk_host_tier"] = {
        "ms": round(ms_h, 4), "attn_ms": round(att_ms, 4), "host_bytes_gb": round(kv_bytes / 1e9, 3),
        "host_link_gbs": round(kv_bytes / (att_ms * 1e-3) / 1e9, 1), "distinct_blocks": distinct,
        "note": "memory keys/values in pinned host RAM (head-major), routing keys in HBM; host_link_gbs = chosen K/V bytes "
                "(each distinct (kv head, block) once) / attention-phase time"}
    _log(f"host-tier memory bank query chunk: {ms_h:.3f} ms, attention {att_ms:.3f} ms, "
         f"{kv_bytes / (att_ms * 1e-3) / 1e9:.1f} GB/s over the host link")
    del q, kh, vh, o, ws, pooled, planes, dk, dq, sel, keys
    torch.cuda.empty_cache()
    # the decode workload over a paged cache: the same 1,048,576-token caches
    # cut into 128-token pages (head-major inside a page) stored in a seeded
    # random order, one table row of 8192 pages per sequence
    c = DECODE
    nb = c["Lc"] // c["block"]
    npg = c["B"] * nb
    kp = synth.device_tensor((npg, c["Hkv"], c["block"], c["D"]), c["sigma"], SEED + 2, t["k"], "bf16").transpose(1, 2)
    vp = synth.device_tensor((npg, c["Hkv"], c["block"], c["D"]), c["sigma"], SEED + 2, t["v"], "bf16").transpose(1, 2)
    perm = np.random.default_rng(SEED + 2).permutation(npg).astype(np.int32)
    table = torch.from_numpy(perm.reshape(c["B"], nb)).cuda()
    qd = synth.device_tensor((c["B"], c["Hq"], c["D"]), c["sigma"], SEED + 2, t["q"], "bf16")
    # routing keys: each page summarised as a one-block sequence, then laid out by the table
    page_sum = m.block_summary(kp, c["block"], out_dtype=torch.bfloat16)  # [pages, 1, Hkv, D]
    pooled = page_sum[table.long(), 0]  # [B, nb, Hkv, D]
    od = torch.empty_like(qd)
    ws = torch.empty(m.decode_workspace_bytes(qd, kp, vp, pooled, block=c["block"], topk=c["topk"], block_table=table),
                     dtype=torch.uint8, device="cuda")

    def paged():
        return m.sparse_attn_decode(qd, kp, vp, pooled, c["topk"], c["block"], out=od, workspace=ws,
                                    block_table=table, return_sel=True)

    ms = time_call(paged, max(reps, 10))
    _, sel = paged()
    torch.cuda.synchronize()
    nbytes, distinct = decode_bytes(sel)
    out["paged_decode_1m"] = {"ms": round(ms, 4), "hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                              "algorithmic_gb": round(nbytes / 1e9, 4), "distinct_blocks": distinct,
                              "note": "128-token pages in a random order, block table per sequence"}
    _log(f"paged decode (1M caches, shuffled 128-token pages): {ms:.3f} ms, {nbytes / (ms * 1e-3) / 1e9:.1f} GB/s")
    # the same paged caches with one selection per GQA group (the group's query
    # heads' scores summed): one block list per (sequence, kv head)
    wsg = torch.empty(m.decode_workspace_bytes(qd, kp, vp, pooled, block=c["block"], topk=c["topk"], gate="group",
                                               block_table=table), dtype=torch.uint8, device="cuda")

    def grouped():
        return m.sparse_attn_decode(qd, kp, vp, pooled, c["topk"], c["block"], gate="group", out=od, workspace=wsg,
                                    block_table=table, return_sel=True)

    msg = time_call(grouped, max(reps, 10))
    _, gsel = grouped()
    torch.cuda.synchronize()
    gs = gsel.cpu().numpy()  # [B, Hkv, topk + 1]
    gdist = sum(len(set(int(x) for x in gs[b, hk] if x >= 0)) for b in range(c["B"]) for hk in range(c["Hkv"]))
    gbytes = (c["B"] * (nb - 1) * c["Hkv"] * c["D"] * 2 + gdist * c["block"] * c["D"] * 2 * 2
              + 2 * c["B"] * c["Hq"] * c["D"] * 2)
    out["paged_decode_1m_per_group"] = {"ms": round(msg, 4), "hbm_gbs": round(gbytes / (msg * 1e-3) / 1e9, 1),
                                        "algorithmic_gb": round(gbytes / 1e9, 4), "distinct_blocks": gdist,
                                        "note": "per-group gating (group scores summed) on the same paged caches"}
    _log(f"paged decode, per-group gating: {msg:.3f} ms, {gbytes / (msg * 1e-3) / 1e9:.1f} GB/s")
    del wsg, gsel
    del kp, vp, od, ws
    torch.cuda.empty_cache()
    # host content tier: the same decode with its 68.7 GB of caches in pinned
    # host RAM (read by the kernels over the host link, only the chosen blocks)
    # and the routing keys in GPU memory
    _log("host tier: filling 68.7 GB of pinned host caches")
    shape = (c["B"], c["Hkv"], c["Lc"], c["D"])
    host = []
    for tid in (t["k"], t["v"]):
        h = torch.empty(shape, dtype=torch.bfloat16, pin_memory=True)
        for b in range(c["B"]):  # one sequence at a time through a device staging tensor
            h[b].copy_(synth.device_tensor(shape[1:], c["sigma"], SEED + 4 + 16 * b, tid, "bf16"))
        host.append(h.transpose(1, 2))
    kh, vh = host
    qd = synth.device_tensor((c["B"], c["Hq"], c["D"]), c["sigma"], SEED + 4, t["q"], "bf16")
    pooled = m.block_summary(kh, c["block"], out_dtype=torch.bfloat16)
    od = torch.empty_like(qd)
    ws = torch.empty(m.decode_workspace_bytes(qd, kh, vh, pooled, block=c["block"], topk=c["topk"]),
                     dtype=torch.uint8, device="cuda")

    def hosted():
        return m.sparse_attn_decode(qd, kh, vh, pooled, c["topk"], c["block"], out=od, workspace=ws,
                                    return_sel=True)

    ms = time_call(hosted, max(reps, 10))
    _, sel = hosted()
    torch.cuda.synchronize()
    nbytes, distinct = decode_bytes(sel)
    kv_bytes = distinct * c["block"] * c["D"] * 2 * 2
    m.timer_enable(2)
    m.timer_reset()
    for _ in range(3):
        hosted()
    torch.cuda.synchronize()
    att_ms = m.timer_report("decode_attend")[0] / 3
    m.timer_enable(0)
    out["host_tier_decode_1m"] = {
        "ms": round(ms, 4), "decode_attend_ms": round(att_ms, 4),
        "host_link_gbs": round(kv_bytes / (att_ms * 1e-3) / 1e9, 1), "host_bytes_gb": round(kv_bytes / 1e9, 4),
        "distinct_blocks": distinct,
        "note": "caches in pinned host RAM, routing keys in HBM; host_link_gbs = chosen K/V bytes / decode_attend time"}
    _log(f"host-tier decode (1M caches in host RAM): {ms:.3f} ms, attend {att_ms:.3f} ms, "
         f"{kv_bytes / (att_ms * 1e-3) / 1e9:.1f} GB/s over the host link")
    return out


def prefill_pairs():
    """Exact attended (query, key) pair counts of the prefill workload:
    (pairs in gate-chosen blocks, pairs in own blocks)."""
    c = PREFILL
    L, bs, k = c["L"], c["block"], c["topk"]
    gate = 0
    diag = 0
    for t in range(L):
        cur = t // bs
        gate += min(k, cur) * bs  # earlier blocks are always full
        diag += t - cur * bs + 1
    return gate * c["Hq"] * c["B"], diag * c["Hq"] * c["B"]


def decode_bytes(sel):
    """Algorithmic HBM bytes of one decode step: routing keys streamed once,
    every distinct chosen block's keys and values once per KV head, q and o."""
    import numpy as np

    c = DECODE
    nb = -(-c["Lc"] // c["block"])
    G = c["Hq"] // c["Hkv"]
    s = sel.cpu().numpy()  # [B, Hq, topk+1]
    distinct = 0
    for b in range(c["B"]):
        for hk in range(c["Hkv"]):
            blk = s[b, hk * G:(hk + 1) * G].reshape(-1)
            distinct += len(set(int(x) for x in blk if x >= 0))
    pooled = c["B"] * (nb - 1) * c["Hkv"] * c["D"] * 2  # blocks before the own block are scored
    kv = distinct * c["block"] * c["D"] * 2 * 2
    qo = 2 * c["B"] * c["Hq"] * c["D"] * 2
    return pooled + kv + qo, distinct


def _host_info():
    """CPU model, logical CPU count and the BLAS NumPy uses (threadpoolctl)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info

        libs = [f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                for i in threadpool_info() if i.get("user_api") == "blas"]
        blas = "; ".join(libs) or blas
    except Exception:
        pass
    return model, os.cpu_count() or 1, blas


def _oracle_rate(q, kh, vh, iq, ikh, toks_all, budget_s, threads):
    """Oracle tokens/s over a seeded sample of prefill tokens; returns (rate, done, seconds, outputs)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle

    c = PREFILL
    outs = {}
    with threadpool_limits(limits=threads):
        torch.set_num_threads(threads)
        t0 = time.perf_counter()
        pooled = oracle.block_pool(ikh, c["block"])
        t_pool = time.perf_counter() - t0
        done = 0
        t1 = time.perf_counter()
        step = 16
        while done < len(toks_all) and time.perf_counter() - t1 < budget_s:
            toks = [int(t) for t in toks_all[done:done + step]]
            qh = q[:, toks].cpu()
            iqh = iq[:, toks].cpu()
            r = oracle.prefill(_RowView(qh, toks, c["L"]), kh, vh, block=c["block"], topk=c["topk"], causal=True,
                               gate="group", index_q=_RowView(iqh, toks, c["L"]), index_k=ikh, pooled=pooled,
                               tokens=toks)
            for i, t in enumerate(toks):
                outs[t] = (r["o"][:, i], r["sel"][:, :, i])
            done += len(toks)
        t_rows = time.perf_counter() - t1
    total = t_pool + t_rows / done * c["L"]
    return c["L"] / total, done, t_rows, t_pool, outs


def cpu_baseline(q, k, v, iq, ik, o_gpu, sel_gpu, budget_s=12.0):
    """The float64 oracle timed on a seeded sample of prefill tokens, once on one
    thread and once with BLAS threads on every host core; the sampled rows'
    outputs are compared with the GPU's (plain max-abs over rows whose
    selection matches the oracle's exactly)."""
    import numpy as np

    c = PREFILL
    rng = np.random.default_rng(1234)
    toks_all = np.sort(rng.choice(c["L"], size=4096, replace=False))
    kh, vh, ikh = k.cpu(), v.cpu(), ik.cpu()
    model, ncpu, blas = _host_info()
    r1, d1, s1, p1, _ = _oracle_rate(q, kh, vh, iq, ikh, toks_all, budget_s, 1)
    rn, dn, sn, pn, outs = _oracle_rate(q, kh, vh, iq, ikh, toks_all, budget_s, ncpu)
    toks = sorted(outs)
    og = o_gpu[:, toks].float().cpu().numpy().astype(np.float64)  # [B, T, Hq, D]
    sg = sel_gpu[:, :, toks].cpu().numpy()  # [B, Hs, T, W]
    max_abs, same_rows, G = 0.0, 0, c["Hq"] // c["Hkv"]
    for i, t in enumerate(toks):
        o_ref, s_ref = outs[t]
        for hs in range(c["Hkv"]):
            if np.array_equal(sg[0, hs, i], s_ref[0, hs]):
                same_rows += 1
                err = np.abs(og[0, i, hs * G:(hs + 1) * G] - o_ref[0, hs * G:(hs + 1) * G]).max()
                max_abs = max(max_abs, float(err))
    return {
        "value": round(rn, 3),
        "unit": "tokens/s",
        "cores": ncpu,
        "kind": "oracle",
        "sample": f"{dn} of {c['L']} prefill tokens (seeded, all 64 heads) in {sn:.1f} s plus one full index-key "
                  f"pooling pass in {pn:.1f} s, BLAS threads = {ncpu} (every logical CPU of the host); "
                  f"whole-sequence time extrapolated linearly; float64 NumPy",
        "one_thread": {"value": round(r1, 3), "tokens": d1, "seconds": round(s1, 1)},
        "host": {"cpu_model": model, "logical_cpus": ncpu, "blas": blas},
        "gpu_parity_on_sample": {"rows": len(toks) * c["Hkv"], "rows_same_selection": same_rows,
                                 "max_abs": max_abs},
    }


def copy_calibration(mib):
    """A kernel of known traffic: neg over `mib` MiB of bf16 reads and writes
    exactly that many bytes; its counter readings scale the gather's."""
    import torch

    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n * 2, "bytes_written": n * 2, "launches": 3}}), flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_gather_128k_traffic.md")
GATHER_SOURCES = ["api.hip", "attn.hip", "csr.hip", "bsa_device.h", "bsa_internal.h"]


def gather_sources_digest():
    import hashlib

    h = hashlib.sha256()
    for name in GATHER_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_long_mean_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes of one attn_gather launch of the 128K prefill, from the
    committed counter summary, or None when the sources have changed since
    the counters were taken."""
    import re

    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    got = {}
    for key in ("sources_digest", "hbm_bytes_per_launch"):
        mt = re.search(rf"^{key}:\s*(\S+)\s*$", text, re.M)
        if not mt:
            return None
        got[key] = mt.group(1)
    if got["sources_digest"] != gather_sources_digest():
        return None
    return float(got["hbm_bytes_per_launch"])


class _RowView:
    """Presents sampled query rows at their true positions to the oracle."""

    def __init__(self, rows, toks, L):
        self.rows = rows
        self.index = {t: i for i, t in enumerate(toks)}
        self.shape = (rows.shape[0], L) + tuple(rows.shape[2:])

    def __getitem__(self, key):
        b, t = key
        return self.rows[b, self.index[t]]


def make_workload(m, name):
    """Inputs of one workload on the device and a function that runs one call
    of it (the tensors stay alive through the function's closure)."""
    import numpy as np
    import torch

    import synth

    t = synth.TID
    if name == "prefill128k":
        c = PREFILL
        q, k, v, iq, ik = make_prefill_inputs()
        o = torch.empty_like(q)
        ws = torch.empty(m.prefill_workspace_bytes(q, k, block=c["block"], topk=c["topk"], causal=True,
                                                   gate="group", index_q=iq, index_k=ik), dtype=torch.uint8,
                         device="cuda")
        fn = lambda: m.sparse_attn_prefill(q, k, v, c["block"], c["topk"], True, gate="group", index_q=iq,
                                           index_k=ik, out=o, workspace=ws)
    elif name == "decode1m":
        d = DECODE
        dq, kc, vc, pooled = make_decode_inputs(m)
        do = torch.empty_like(dq)
        ws = torch.empty(m.decode_workspace_bytes(dq, kc, vc, pooled, block=d["block"], topk=d["topk"]),
                         dtype=torch.uint8, device="cuda")
        fn = lambda: m.sparse_attn_decode(dq, kc, vc, pooled, d["topk"], d["block"], out=do, workspace=ws)
    elif name in ("moba32k", "moba32k_backward"):
        c = MOBA
        q = synth.device_tensor((c["B"], c["L"], c["Hq"], c["D"]), c["sigma"], SEED, t["q"], "bf16")
        k = synth.device_tensor((c["B"], c["L"], c["Hkv"], c["D"]), c["sigma"], SEED, t["k"], "bf16")
        v = synth.device_tensor((c["B"], c["L"], c["Hkv"], c["D"]), c["sigma"], SEED, t["v"], "bf16")
        if name == "moba32k":
            o = torch.empty_like(q)
            ws = torch.empty(m.prefill_workspace_bytes(q, k, block=c["block"], topk=c["topk"], causal=True),
                             dtype=torch.uint8, device="cuda")
            fn = lambda: m.sparse_attn_prefill(q, k, v, c["block"], c["topk"], True, out=o, workspace=ws)
        else:
            g = synth.device_tensor((c["B"], c["L"], c["Hq"], c["D"]), 1.0, SEED, t["dout"], "bf16")
            o, sel, lse = m.sparse_attn_prefill(q, k, v, c["block"], c["topk"], True, return_sel=True,
                                                return_lse=True)
            grads = tuple(torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in (q, k, v))
            ws = torch.empty(m.backward_workspace_bytes(q, k, sel, block=c["block"], causal=True), dtype=torch.uint8,
                             device="cuda")
            fn = lambda: m.sparse_attn_backward(q, k, v, o, lse, sel, g, c["block"], True, out=grads, workspace=ws)
    elif name in ("memory_summary", "memory_chunk"):
        c = MEMORY
        ids = synth.doc_ids_from_lengths(synth.doc_lengths(c["Lk"], c["docs"], c["doc_mean"], c["doc_sigma"], SEED))
        dk = torch.from_numpy(ids[None]).cuda()
        k = synth.device_tensor((1, c["Lk"], c["Hkv"], c["D"]), 1.0, SEED, t["k"], "bf16")
        if name == "memory_summary":
            fn = lambda: m.block_summary(k, c["block"], doc_ids=dk)
        else:
            q = synth.device_tensor((1, c["Lq"], c["Hq"], c["D"]), 1.0, SEED, t["q"], "bf16")
            v = synth.device_tensor((1, c["Lk"], c["Hkv"], c["D"]), 1.0, SEED, t["v"], "bf16")
            # the memory's offline encoding: rotated keys and the routing keys as the gate's planes
            _, k_rot, planes = m.block_summary(k, c["block"], doc_ids=dk, return_k_rot=True, return_planes=True)
            del k
            dq = torch.zeros((1, c["Lq"]), dtype=torch.int32, device="cuda")
            o = torch.empty_like(q)
            kw = dict(doc_ids_q=dq, pooled=planes)
            ws = torch.empty(m.prefill_workspace_bytes(q, k_rot, block=c["block"], topk=c["topk"], causal=False,
                                                       **kw), dtype=torch.uint8, device="cuda")
            fn = lambda: m.sparse_attn_prefill(q, k_rot, v, c["block"], c["topk"], False, out=o, workspace=ws, **kw)
    else:
        raise SystemExit(f"unknown workload {name}")
    torch.cuda.synchronize()
    return fn


def profile_workload(m, name, reps):
    """Runs one workload `reps` times after one warm-up call (for rocprofv3:
    its kernel trace or counters then cover only this workload)."""
    import torch

    fn = make_workload(m, name)
    fn()
    torch.cuda.synchronize()
    _log(f"profile {name}: warm-up done")
    for i in range(reps):
        fn()
        torch.cuda.synchronize()
        _log(f"profile {name}: call {i + 1}/{reps} done")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work per CPU-baseline leg (one thread, then every core)")
    ap.add_argument("--also", action="store_true",
                    help="also time the MoBA-style 32K prefill, the 10M-token memory bank and the paged decode "
                         "(extra field)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run an elementwise negation over MIB MiB (read once, written once) -- the "
                         "known-size kernel that scales the HBM byte counters -- and exit")
    ap.add_argument("--profile", default=None, metavar="WORKLOAD",
                    help="only run WORKLOAD (prefill128k, decode1m, moba32k, moba32k_backward, memory_summary, "
                         "memory_chunk) --steps times after one warm-up call, for rocprofv3, and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the path shards by KV head or "
              f"sequence with no exchange, see the design notes", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import block_sparse_long_mean_amd as m

    m.lib()
    torch.cuda.set_device(0)
    if args.profile:
        profile_workload(m, args.profile, args.steps)
        return
    _log("generating prefill inputs")
    q, k, v, iq, ik = make_prefill_inputs()
    _log("generating decode inputs (68.7 GB of KV cache)")
    dq, kc, vc, pooled = make_decode_inputs(m)
    torch.cuda.synchronize()
    c, d = PREFILL, DECODE
    o = torch.empty_like(q)
    do = torch.empty_like(dq)
    pws = torch.empty(m.prefill_workspace_bytes(q, k, block=c["block"], topk=c["topk"], causal=True, gate="group",
                                                index_q=iq, index_k=ik), dtype=torch.uint8, device="cuda")
    dws = torch.empty(m.decode_workspace_bytes(dq, kc, vc, pooled, block=d["block"], topk=d["topk"]),
                      dtype=torch.uint8, device="cuda")
    _log(f"workspaces: prefill {pws.numel() / 1e9:.2f} GB, decode {dws.numel() / 1e6:.1f} MB")

    def prefill():
        m.sparse_attn_prefill(q, k, v, c["block"], c["topk"], True, gate="group", index_q=iq, index_k=ik, out=o,
                              workspace=pws)

    def decode():
        r = m.sparse_attn_decode(dq, kc, vc, pooled, d["topk"], d["block"], out=do, workspace=dws,
                                 return_sel=True)
        return r

    for i in range(args.warmup):
        prefill()
        decode()
        torch.cuda.synchronize()
        _log(f"warmup {i + 1}/{args.warmup} done")
    st = torch.cuda.current_stream()

    def run_steps(n):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        sel = None
        for i in range(n):
            ev[i][0].record(st)
            prefill()
            ev[i][1].record(st)
            _, sel = decode()
            ev[i][2].record(st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        pre = sum(a.elapsed_time(b) for a, b, _ in ev) / n
        dec = sum(b.elapsed_time(c2) for _, b, c2 in ev) / n
        stp = sum(a.elapsed_time(c2) for a, _, c2 in ev) / n
        return pre, dec, stp, wall, sel

    # the headline: K steps with nothing but the work on the stream
    pre_ms, dec_ms, step_ms, wall, last_sel = run_steps(args.steps)
    _log(f"timed {args.steps} steps: prefill {pre_ms:.3f} ms, decode {dec_ms:.3f} ms, step {step_ms:.3f} ms "
         f"(host wall {wall * 1e3 / args.steps:.3f} ms/step)")
    # the breakdown: the same K steps again with the library's launch timer
    # (HIP events on the launch stream around every launch; "attn" brackets
    # the attention passes, gathers and merges, as one phase)
    m.timer_reset()
    m.timer_enable(2)
    run_steps(args.steps)
    m.timer_enable(0)

    kernels = ["doc_chunk_last", "doc_positions", "rope_q", "block_summary", "pooled_to_planes", "gate_topk",
               "gate_merge", "decode_scores", "decode_select", "csr_fill", "csr_count", "csr_scan", "csr_scatter",
               "attn_gather", "attn_merge", "attn", "decode_attend", "decode_combine"]
    per_kernel = {}
    for name in kernels:
        ms, n = m.timer_report(name)
        if n:
            per_kernel[name] = {"ms_total": round(ms, 4), "launches": n, "ms_avg": round(ms / n, 4)}
    m.timer_reset()
    for name, r in sorted(per_kernel.items(), key=lambda x: -x[1]["ms_total"]):
        _log(f"  {name:18s} avg {r['ms_avg']:.4f} ms x{r['launches']}")

    gate_pairs, diag_pairs = prefill_pairs()
    flops_total = 4.0 * c["D"] * (gate_pairs + diag_pairs)
    dbytes, distinct = decode_bytes(last_sel)
    pre_tflops = flops_total / (pre_ms * 1e-3) / 1e12
    dec_gbs = dbytes / (dec_ms * 1e-3) / 1e9
    tokens = c["B"] * c["L"] + d["B"]
    value = tokens / (step_ms * 1e-3)

    # the dominant kernel: the gather, which runs every attended (query, key)
    # pair of the prefill on MFMA (4*D flops per pair, own blocks included;
    # one launch per call at this size)
    single = [n for n, r in per_kernel.items() if n != "attn"]
    dom = max(single, key=lambda n: per_kernel[n]["ms_total"])
    if dom == "attn_gather":
        g_ms = per_kernel[dom]["ms_total"] / args.steps  # per prefill call
        achieved = flops_total / (g_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                "kernel": "attn_gather_kernel (every attended pair of the 128K prefill)",
                "kernel_ms": round(g_ms, 4), "launches_per_call": per_kernel[dom]["launches"] // args.steps}
    else:
        roof = {"bound": "unknown", "achieved": None, "peak": None, "unit": None, "frac": None, "traffic": None,
                "kernel": dom, "kernel_ms": per_kernel[dom]["ms_avg"]}
    attn_ms = per_kernel.get("attn", {}).get("ms_avg")

    cpu = None
    if not args.no_cpu_baseline:
        _log("timing the float64 oracle on a sample of the prefill (CPU), one thread then every core")
        o_chk, sel_chk = m.sparse_attn_prefill(q, k, v, c["block"], c["topk"], True, gate="group", index_q=iq,
                                               index_k=ik, return_sel=True)
        torch.cuda.synchronize()
        cpu = cpu_baseline(q, k, v, iq, ik, o_chk, sel_chk, args.cpu_budget)
        del o_chk, sel_chk

    others = None
    if args.also:
        del q, k, v, iq, ik, o, pws, dq, kc, vc, pooled, dws
        torch.cuda.empty_cache()
        others = other_workloads(m, max(1, args.steps))

    out = {
        "metric": "block-sparse attn prefill tokens/s + MFMA TFLOP/s at 128K; decode HBM GB/s",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "128K MiniMax-style prefill (B1 L131072 H64/8 D128 block64 index-dim64 group-summed "
                        "top16+own causal) + decode (B16 x 1 token, 1,048,576-token head-major caches, H32/8 D128 "
                        "block128 top32+own)",
            "global_batch": c["B"],
            "seq_len": c["L"],
            "parallelism": "single GPU",
        },
        "breakdown": {
            "prefill_ms": round(pre_ms, 4),
            "prefill_tokens_per_s": round(c["B"] * c["L"] / (pre_ms * 1e-3), 1),
            "prefill_attended_tflops": round(pre_tflops, 2),
            "prefill_attended_tflop": round(flops_total / 1e12, 4),
            "attention_phase_ms": attn_ms,
            "attention_phase_tflops": round(flops_total / (attn_ms * 1e-3) / 1e12, 2) if attn_ms else None,
            "decode_ms": round(dec_ms, 4),
            "decode_tokens_per_s": round(d["B"] / (dec_ms * 1e-3), 1),
            "decode_hbm_gbs": round(dec_gbs, 1),
            "decode_hbm_frac": round(dec_gbs / PEAK_HBM_GBS, 4),
            "decode_algorithmic_gb": round(dbytes / 1e9, 4),
            "decode_distinct_blocks": distinct,
            "kernels_ms_avg": {k2: v2["ms_avg"] for k2, v2 in per_kernel.items()},
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if others is not None:
        out["other_workloads"] = others
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
