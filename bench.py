#!/usr/bin/env python3
"""Benchmark of the DSA sparse-attention layer on one MI355X.

Headline: DSA decode queries/s at a 1,048,576-token context (batch 4, top-512, planted low-rank
bias on 2% of regions), one step = compress the region the query token completes -> indexer
score + top-512 selection -> sparse GQA over the selected regions, inputs resident in HBM.
Also measured in the same run: prefill tokens/s of a 2048-token chunk appended to a 63,488-token
prefix (64K total).  Each figure carries the roofline of its dominant kernel (bytes or flops the
method needs / the kernel's average hipEvent-timed duration, against the MI355X peak) and the
CPU oracle's rate on a bounded sample of the same work.

Further objects in the same line: the two workloads over paged caches and with FP8 K/V caches, the
neighbour-merged prefill on a correlated chunk, the indexer front-end, the 3:1 sliding-window/DSA layer
mix and a sliding-window prefill chunk (each can be skipped with its --no-* flag).

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-prefill] [--no-paged] [--no-fp8] [--no-merged]
                [--no-frontend] [--no-swa] [--no-cpu] [--graph] [--profile-run]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
G, P, HI, HQ, D, REG, TOPK = 4, 256, 16, 64, 192, 8, 512

DECODE = dict(name="DSA decode, batch 4, 1,048,576-token context, top-512, planted bias on 2% of regions",
              batch=4, context=1048576, topk=TOPK, planted=True, seed_index=3)
PREFILL = dict(name="DSA chunked prefill, 2048 new tokens after a 63,488-token prefix (64K), top-512",
               prefix=63488, chunk=2048, topk=TOPK, seed_index=2)
MIX = dict(name="3:1 layer mix, decode: three sliding-window layers (512-token rings) then one DSA layer, "
                "batch 8, 262,144-token context, top-512",
           batch=8, context=262144, topk=TOPK, planted=False, seed_index=4, swa_layers=3)
SWA_PREFILL = dict(name="sliding-window layer, chunked prefill: 2048 new tokens after 63,488 (512-token ring)",
                   prefix=63488, chunk=2048, seed_index=4)
DECODE_8K = dict(name="DSA decode, batch 1, 8,192-token context, top-512 (32 independent input copies in "
                      "rotation so the 13.7 MB step is not served from the 256 MB Infinity Cache)",
                 batch=1, context=8192, topk=TOPK, planted=False, seed_index=0, copies=32)
DECODE_128K = dict(name="DSA decode, batch 16, 131,072-token context, top-512",
                   batch=16, context=131072, topk=TOPK, planted=False, seed_index=1)
QUERY_SETS = 8  # distinct query sets per decode workload, one per step in rotation
W = 512
# correlated variant of the prefill chunk: anchors every 64 queries, 10% of each query's own i.i.d.
# index_q mixed in (adjacent selections then share ~88% of their regions)
CORRELATED = dict(every=64, noise=0.1)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------------------------
# algorithmic work (bytes / flops the method needs; implementation scratch traffic is not counted)
# ------------------------------------------------------------------------------------------------
def decode_bytes(B, L, topk):
    """Per decode step.  compress: 8 index_k rows x 4 groups in, codes+scales out; score: every
    candidate region's 4 group summaries (256 B codes + 4 B scale each) + the query's index_q/z;
    select: the selection out; attention: K and V of the selected tokens + q in + out."""
    R = L // REG
    compress = B * (REG * G * P * 2 + G * (P + 4))
    score = B * ((R - 1) * G * (P + 4) + HI * P * 2 + HI * 4)
    select = B * G * (topk + 1) * 4
    tokens = min(topk, R) * REG  # L % 8 == 0: every selected region is complete
    attend = B * (G * tokens * D * 2 * 2 + HQ * D * 2 * 2)
    return dict(compress=compress, score=score, select=select, attend=attend,
                total=compress + score + select + attend)


def prefill_flops(prefix, chunk, topk):
    """Per chunk: indexer dot products (4 heads x 256 channels per candidate region and group) and
    sparse attention (QK^T and PV over the attended tokens, 16 heads per group)."""
    score = attend = gather = 0
    for p in range(prefix, prefix + chunk):
        c = p // REG
        score += c * G * 4 * P * 2
        tokens = min(topk - 1, c) * REG + (p % REG + 1)
        attend += G * tokens * 16 * D * 2 * 2
        gather += G * tokens * D * 2 * 2  # bf16 K and V rows of the attended tokens
    return dict(score=score, attend=attend, total=score + attend, gather=gather)


def swa_decode_bytes(B):
    """Per sliding-window layer and decode step: the window's K and V (511 ring rows + the new one) for
    4 groups, q in and out, the new row's K/V in and its ring write."""
    return B * (W * G * D * 2 * 2 + HQ * D * 2 * 2 + G * D * 2 * 2 * 2)


def swa_prefill_flops(prefix, chunk):
    """QK^T and PV over each query's band of min(512, p+1) keys, 64 heads."""
    return sum(min(W, p + 1) for p in range(prefix, prefix + chunk)) * HQ * D * 2 * 2


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "dsa_sparse_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_profile_json(kernel, workload_key, tag, src_hash):
    """A 'tag: {...}' line of profiles/<kernel>__<workload>.md (rocprofv3 counter figures), or None if absent or
    taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload_key}.md")
    if not os.path.exists(path):
        return None
    for line in open(path, encoding="utf-8"):
        if line.startswith(tag + ":"):
            d = json.loads(line.split(":", 1)[1])
            if d.get("source_hash") != src_hash:
                return None
            return {k: v for k, v in d.items() if k != "source_hash"}
    return None


def load_traffic(kernel, workload_key, src_hash):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/<kernel>__<workload>.md holds
    a line 'traffic_json: {...}'); None if absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload_key}.md")
    if not os.path.exists(path):
        return None
    for line in open(path, encoding="utf-8"):
        if line.startswith("traffic_json:"):
            d = json.loads(line.split(":", 1)[1])
            if d.get("source_hash") != src_hash:
                return None
            return d.get("bytes_per_launch")
    return None


# ------------------------------------------------------------------------------------------------
class Calls:
    """Pre-marshalled C-ABI calls (argument checks done once by the binding's conventions)."""

    def __init__(self, dsa):
        self.L = dsa.load()

    @staticmethod
    def p(t):
        return ctypes.c_void_p(t.data_ptr())


def setup_decode(cfg, steps_hint=1):
    """Decode inputs resident in HBM.  cfg["copies"] independent input sets (caches, summaries and
    queries of cfg["batch"] sequences each; a step uses copy i mod copies, so a workload smaller than
    the 256 MB Infinity Cache is not served from it), and cfg["query_sets"] distinct query sets per
    copy (q, index_q, z; a step uses set i mod query_sets, so neither the selection nor the gathered
    K/V repeats from one step to the next)."""
    import torch
    import dsa_inputs as gi
    import dsa_sparse_attention_amd as dsa

    B, Lc, topk = cfg["batch"], cfg["context"], cfg["topk"]
    copies, nqs = cfg.get("copies", 1), cfg.get("query_sets", QUERY_SETS)
    tcap, R = Lc, Lc // REG
    seed = gi.SEED_BASE + cfg["seed_index"]
    s = torch.cuda.current_stream().cuda_stream
    geom = dsa.geometry(topk=topk)
    t0 = time.time()
    NB = B * copies  # sequences of all copies: copy j holds sequences j*B .. j*B+B-1
    ik = torch.empty(NB * G * tcap * P, dtype=torch.bfloat16, device="cuda")
    K = torch.empty(NB * G * tcap * D, dtype=torch.bfloat16, device="cuda")
    V = torch.empty(NB * G * tcap * D, dtype=torch.bfloat16, device="cuda")
    gi.dev_tokens(ik.data_ptr(), s, seed, gi.TID_IK, NB, tcap, G, P, 0, tcap, tcap, tcap, gi.LAYOUT_GROUP_MAJOR,
                  gi.IK_SCALE, cfg["planted"])
    gi.dev_tokens(K.data_ptr(), s, seed, gi.TID_K, NB, tcap, G, D, 0, tcap, tcap, tcap, gi.LAYOUT_KTILED)
    gi.dev_tokens(V.data_ptr(), s, seed, gi.TID_V, NB, tcap, G, D, 0, tcap, tcap, tcap, gi.LAYOUT_REGION_T)
    # query set u of copy j: queries of sequences j*B.. in the generator's query index space u*NB + j*B + b
    NQ = NB * nqs
    q = torch.empty(NQ * HQ * D, dtype=torch.bfloat16, device="cuda")
    iq = torch.empty(NQ * HI * P, dtype=torch.bfloat16, device="cuda")
    z = torch.empty(NQ * HI, dtype=torch.float32, device="cuda")
    gi.dev_flat(q.data_ptr(), s, seed, gi.TID_Q, q.numel(), 0, 1.0)
    gi.dev_flat(iq.data_ptr(), s, seed, gi.TID_IQ, iq.numel(), 0, gi.IK_SCALE)
    gi.dev_flat(z.data_ptr(), s, seed, gi.TID_Z, z.numel(), 1)
    summ = torch.zeros(NB * G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(NB * G * R, dtype=torch.float32, device="cuda")
    i32 = lambda v: torch.tensor(v, dtype=torch.int32, device="cuda")
    # untimed: summaries of every region before the one the query token completes
    dsa.dsa_compress_regions(geom, ik, tcap, i32([0] * NB), i32([R - 1] * NB), R - 1, summ, scale)
    torch.cuda.synchronize()
    log(f"decode setup ({B} x {Lc}, {copies} copies, {nqs} query sets): {time.time() - t0:.1f}s")
    rb, re_ = i32([R - 1] * B), i32([R] * B)
    qseq, qpos, slen = i32(list(range(B))), i32([Lc - 1] * B), i32([Lc] * B)
    sel = torch.empty(NB * G * topk, dtype=torch.int32, device="cuda")
    nsel = torch.empty(NB * G, dtype=torch.int32, device="cuda")
    out = torch.empty(NB * HQ * D, dtype=torch.bfloat16, device="cuda")
    ws1 = dsa.workspace(dsa.dsa_score_topk_workspace_size(geom, B, R))
    ws2 = dsa.workspace(dsa.dsa_sparse_gqa_workspace_size(geom, B))
    ws3 = dsa.workspace(dsa.dsa_decode_step_workspace_size(geom, B, R))
    L = dsa.load()
    gp = ctypes.byref(geom)

    def at(t, elems):  # pointer to element offset `elems` of tensor t
        return ctypes.c_void_p(t.data_ptr() + elems * t.element_size())

    variants = []  # (separate-call argument tuples, fused-call arguments) per (copy, query set)
    for u in range(nqs):
        for j in range(copies):
            b0 = j * B  # first sequence of copy j
            qi = u * NB + b0  # first query of set u, copy j
            cq, ciq, cz = at(q, qi * HQ * D), at(iq, qi * HI * P), at(z, qi * HI)
            cik, cK, cV = at(ik, b0 * G * tcap * P), at(K, b0 * G * tcap * D), at(V, b0 * G * tcap * D)
            cs, csc = at(summ, b0 * G * R * P), at(scale, b0 * G * R)
            csel, cns, co = at(sel, b0 * G * topk), at(nsel, b0 * G), at(out, b0 * HQ * D)
            a_comp = (gp, B, cik, tcap, Calls.p(rb), Calls.p(re_), 1, cs, csc)
            a_score = (gp, B, ciq, cz, Calls.p(qseq), Calls.p(qpos), B, cs, csc, tcap, R, csel, cns, None,
                       Calls.p(ws1), ws1.numel())
            a_attn = (gp, B, cq, cK, cV, tcap, Calls.p(slen), csel, cns, co, Calls.p(ws2), ws2.numel())
            a_fused = (gp, B, cq, ciq, cz, cik, cK, cV, tcap, Calls.p(slen), cs, csc, R, csel, cns, co,
                       Calls.p(ws3), ws3.numel())
            variants.append((a_comp, a_score, a_attn, a_fused))
    # interleave copies first: consecutive steps use different copies, then different query sets
    order = [u * copies + j for u in range(nqs) for j in range(copies)]
    state = {"i": 0}

    def step(st):
        # the whole step through one entry point (compression folded into the scoring launch), or
        # the three separate calls
        a_comp, a_score, a_attn, a_fused = variants[order[state["i"] % len(order)]]
        state["i"] += 1
        if cfg.get("separate"):
            rc = (L.dsa_compress_regions(*a_comp, st) or L.dsa_score_topk(*a_score, st)
                  or L.dsa_sparse_gqa_decode(*a_attn, st))
        else:
            rc = L.dsa_decode_step(*a_fused, st)
        if rc:
            raise RuntimeError(f"decode step failed: {rc} {L.dsa_last_error().decode()}")

    step.variants = len(order)
    keep = (ik, K, V, q, iq, z, summ, scale, rb, re_, qseq, qpos, slen, sel, nsel, out, ws1, ws2, ws3, geom)
    return step, keep


def rotate_queries(make_args, q, iq, z, B, fn, what):
    """A step over QUERY_SETS argument tuples, one per query set u (queries u*B .. u*B+B-1 of q,
    index_q and z); make_args(q_ptr, iq_ptr, z_ptr) builds one tuple."""
    def at(t, elems):
        return ctypes.c_void_p(t.data_ptr() + elems * t.element_size())
    nqs = q.numel() // (B * HQ * D)
    variants = [make_args(at(q, u * B * HQ * D), at(iq, u * B * HI * P), at(z, u * B * HI)) for u in range(nqs)]
    state = {"i": 0}

    def step(st):
        args = variants[state["i"] % nqs]
        state["i"] += 1
        rc = fn(*args, st)
        if rc:
            raise RuntimeError(f"{what} failed: {rc} {dsa_error()}")

    step.variants = nqs
    return step


def dsa_error():
    import dsa_sparse_attention_amd as dsa
    return dsa.load().dsa_last_error().decode()


PAGE = 128  # positions per page of the paged caches
PAGE_ELEMS = {"k": 16 * 1536, "v": 16 * 1536, "ik": PAGE * P, "summ": 4096, "scale": 16}  # per (page, group)


def to_pools(tensors, n_seqs, tcap, seed, n_extra=64, order="interleaved"):
    """Copies contiguous caches into paged pools of n_seqs*pages + n_extra pages.  order "interleaved":
    page ids in the order a serving cache hands them out when the sequences of a batch grow together
    (page n of sequence s is id n*n_seqs + s); "shuffled": random distinct ids (a cache after heavy
    churn, the worst case for locality).  Returns (pools, Pages)."""
    import numpy as np
    import torch
    import dsa_sparse_attention_amd as dsa
    npg = tcap // PAGE
    n_pages = n_seqs * npg + n_extra
    if order == "shuffled":
        ids = np.random.default_rng(seed).permutation(n_pages)[:n_seqs * npg].reshape(n_seqs, npg)
    else:
        ids = (np.arange(npg)[None, :] * n_seqs + np.arange(n_seqs)[:, None]).astype(np.int64)
    bt = torch.tensor(ids, dtype=torch.int32, device="cuda")
    pools = dsa.paged_pools(n_pages, index_k="ik" in tensors)
    idx = bt.reshape(-1).long()
    for name, t in tensors.items():
        per = PAGE_ELEMS[name]
        src = t.view(n_seqs, G, npg, per).permute(0, 2, 1, 3).reshape(n_seqs * npg, G * per)
        pools[name].view(-1, G * per)[idx] = src
        del src
    torch.cuda.synchronize()
    return pools, dsa.Pages(bt, n_pages)


def paged_decode(cfg, order="interleaved"):
    """The decode workload with every cache of the layer in 128-position pages
    (dsa_decode_step_paged)."""
    import torch
    import dsa_inputs as gi
    import dsa_sparse_attention_amd as dsa
    _, keep = setup_decode(cfg)
    ik, K, V, q, iq, z, summ, scale = keep[:8]
    slen, sel, nsel, out = keep[12], keep[13], keep[14], keep[15]
    B, tcap = cfg["batch"], cfg["context"]
    R = tcap // REG
    pools, pages = to_pools(dict(ik=ik, k=K, v=V, summ=summ, scale=scale), B, tcap, gi.SEED_BASE + 99, order=order)
    del keep, ik, K, V, summ, scale
    torch.cuda.empty_cache()
    geom = dsa.geometry(topk=cfg["topk"])
    ws = dsa.workspace(dsa.dsa_decode_step_workspace_size(geom, B, R))
    L = dsa.load()
    p = Calls.p
    step = rotate_queries(
        lambda cq, ciq, cz: (ctypes.byref(geom), B, cq, ciq, cz, ctypes.byref(pages.struct), p(pools["ik"]),
                             p(pools["k"]), p(pools["v"]), p(slen), p(pools["summ"]), p(pools["scale"]), R, p(sel),
                             p(nsel), p(out), p(ws), ws.numel()),
        q, iq, z, B, L.dsa_decode_step_paged, "paged decode step")
    return step, (pools, pages, q, iq, z, slen, sel, nsel, out, ws, geom)


def paged_prefill(cfg, order="interleaved"):
    """The prefill workload over 128-position pages (compress, score_topk and sparse GQA through
    their _paged entry points)."""
    import torch
    import dsa_inputs as gi
    import dsa_sparse_attention_amd as dsa
    _, keep = setup_prefill(cfg)
    ik, K, V, q, iq, z, summ, scale, rb, re_, qseq, qpos, sel, nsel, out = keep[:15]
    P0, n, topk = cfg["prefix"], cfg["chunk"], cfg["topk"]
    tcap = P0 + n
    R = tcap // REG
    pools, pages = to_pools(dict(ik=ik, k=K, v=V, summ=summ, scale=scale), 1, tcap, gi.SEED_BASE + 98, order=order)
    del keep, ik, K, V, summ, scale
    torch.cuda.empty_cache()
    geom = dsa.geometry(topk=topk)
    ws1 = dsa.workspace(dsa.dsa_score_topk_workspace_size(geom, n, R))
    ws3 = dsa.workspace(dsa.dsa_sparse_gqa_prefill_workspace_size(geom, n))
    L = dsa.load()
    p = Calls.p
    gp, pt = ctypes.byref(geom), ctypes.byref(pages.struct)
    a_comp = (gp, 1, pt, p(pools["ik"]), p(rb), p(re_), tcap // REG - P0 // REG, p(pools["summ"]), p(pools["scale"]))
    a_score = (gp, n, p(iq), p(z), p(qseq), p(qpos), 1, pt, p(pools["summ"]), p(pools["scale"]), R, p(sel), p(nsel),
               None, p(ws1), ws1.numel())
    a_attn = (gp, n, p(q), p(qseq), p(qpos), 1, pt, p(pools["k"]), p(pools["v"]), p(sel), p(nsel), p(out), p(ws3),
              ws3.numel())

    def step(st):
        rc = (L.dsa_compress_regions_paged(*a_comp, st) or L.dsa_score_topk_paged(*a_score, st)
              or L.dsa_sparse_gqa_prefill_paged(*a_attn, st))
        if rc:
            raise RuntimeError(f"paged prefill step failed: {rc} {L.dsa_last_error().decode()}")

    return step, (pools, pages, q, iq, z, rb, re_, qseq, qpos, sel, nsel, out, ws1, ws3, geom)


def fp8_kv(seed, B, tcap):
    """FP8 K/V caches of B sequences filled through dsa_cache_write_fp8 with the generator's K/V rows
    (token-major rows generated on the GPU, written, then freed)."""
    import numpy as np
    import torch
    import dsa_inputs as gi
    import dsa_sparse_attention_amd as dsa
    s = torch.cuda.current_stream().cuda_stream
    geom = dsa.geometry()
    k8, v8, kvs = dsa.fp8_caches(B, tcap)
    tok_seq = torch.tensor(np.repeat(np.arange(B), tcap).astype(np.int32), device="cuda")
    tok_pos = torch.tensor(np.tile(np.arange(tcap), B).astype(np.int32), device="cuda")
    rows = {}
    for tid in (gi.TID_K, gi.TID_V):
        t = torch.empty(B * tcap * G * D, dtype=torch.bfloat16, device="cuda")
        gi.dev_tokens(t.data_ptr(), s, seed, tid, B, tcap, G, D, 0, tcap, tcap, tcap, gi.LAYOUT_TOKEN_MAJOR)
        rows[tid] = t
    dsa.dsa_cache_write_fp8(geom, tok_seq, tok_pos, rows[gi.TID_K], rows[gi.TID_V], k8, v8, kvs, B, tcap)
    torch.cuda.synchronize()
    del rows, tok_seq, tok_pos
    torch.cuda.empty_cache()
    return k8, v8, kvs


def fp8_decode(cfg):
    """The decode workload with FP8 K/V caches (dsa_decode_step_fp8)."""
    import torch
    import dsa_inputs as gi
    import dsa_sparse_attention_amd as dsa
    _, keep = setup_decode(cfg)
    ik, K, V, q, iq, z, summ, scale = keep[:8]
    slen, sel, nsel, out = keep[12], keep[13], keep[14], keep[15]
    B, tcap = cfg["batch"], cfg["context"]
    R = tcap // REG
    del keep, K, V
    torch.cuda.empty_cache()
    k8, v8, kvs = fp8_kv(gi.SEED_BASE + cfg["seed_index"], B, tcap)
    geom = dsa.geometry(topk=cfg["topk"])
    ws = dsa.workspace(dsa.dsa_decode_step_workspace_size(geom, B, R))
    L = dsa.load()
    p = Calls.p
    step = rotate_queries(
        lambda cq, ciq, cz: (ctypes.byref(geom), B, cq, ciq, cz, p(ik), p(k8), p(v8), p(kvs), tcap, p(slen),
                             p(summ), p(scale), R, p(sel), p(nsel), p(out), p(ws), ws.numel()),
        q, iq, z, B, L.dsa_decode_step_fp8, "fp8 decode step")
    return step, (ik, q, iq, z, summ, scale, slen, sel, nsel, out, k8, v8, kvs, ws, geom)


def fp8_prefill(cfg):
    """The prefill workload with FP8 K/V caches (dsa_sparse_gqa_prefill_fp8)."""
    import torch
    import dsa_inputs as gi
    import dsa_sparse_attention_amd as dsa
    _, keep = setup_prefill(cfg)
    ik, K, V, q, iq, z, summ, scale, rb, re_, qseq, qpos, sel, nsel, out = keep[:15]
    P0, n, topk = cfg["prefix"], cfg["chunk"], cfg["topk"]
    tcap = P0 + n
    R = tcap // REG
    del keep, K, V
    torch.cuda.empty_cache()
    k8, v8, kvs = fp8_kv(gi.SEED_BASE + cfg["seed_index"], 1, tcap)
    geom = dsa.geometry(topk=topk)
    ws1 = dsa.workspace(dsa.dsa_score_topk_workspace_size(geom, n, R))
    ws3 = dsa.workspace(dsa.dsa_sparse_gqa_prefill_workspace_size(geom, n))
    L = dsa.load()
    p = Calls.p
    gp = ctypes.byref(geom)
    a_comp = (gp, 1, p(ik), tcap, p(rb), p(re_), tcap // REG - P0 // REG, p(summ), p(scale))
    a_score = (gp, n, p(iq), p(z), p(qseq), p(qpos), 1, p(summ), p(scale), tcap, R, p(sel), p(nsel), None, p(ws1),
               ws1.numel())
    a_attn = (gp, n, p(q), p(qseq), p(qpos), 1, p(k8), p(v8), p(kvs), tcap, p(sel), p(nsel), p(out), p(ws3),
              ws3.numel())

    def step(st):
        rc = (L.dsa_compress_regions(*a_comp, st) or L.dsa_score_topk(*a_score, st)
              or L.dsa_sparse_gqa_prefill_fp8(*a_attn, st))
        if rc:
            raise RuntimeError(f"fp8 prefill step failed: {rc} {L.dsa_last_error().decode()}")

    return step, (ik, q, iq, z, summ, scale, rb, re_, qseq, qpos, sel, nsel, out, k8, v8, kvs, ws1, ws3, geom)


def measure_fp8(args, result):
    """Both headline workloads with FP8 K/V caches (the attention gathers half the bytes; results
    differ from the bf16 ones by the E4M3 rounding of K and V, ~4% rel-RMS)."""
    import torch
    res = {}
    for key, setup, cfg, unit_n, kern in (("decode", fp8_decode, DECODE, DECODE["batch"], "k_sgqa_decode"),
                                          ("prefill", fp8_prefill, PREFILL, PREFILL["chunk"], "k_sgqa_prefill")):
        if key == "prefill" and args.no_prefill:
            continue
        step, keep = setup(cfg)
        steps = args.steps if key == "decode" else max(3, args.steps // 3)
        secs, eager, st = timed(step, steps, max(1, args.warmup // 2), [kern], graph=args.graph)
        del keep
        torch.cuda.empty_cache()
        ms = secs * 1e3 / steps
        base = result.get("ms_per_step") if key == "decode" else result.get("prefill", {}).get("ms_per_step")
        res[key] = {"workload": cfg["name"] + ", K/V caches in FP8 (E4M3, one scale per token row)",
                    "value": round(unit_n * steps / secs, 1), "unit": "queries/s" if key == "decode" else "tokens/s",
                    "ms_per_step": round(ms, 4), "vs_bf16": round(base / ms, 4) if base else None,
                    "attention_us": round(st[kern][0] * 1e3, 2)}
        log(f"fp8 {key}: {unit_n * steps / secs:.0f}/s, {ms:.3f} ms/step")
    result["fp8_kv"] = res


def measure_paged(args, result):
    """Both headline workloads again with the caches in 128-position pages handed out in batch
    order, and the decode step once more with shuffled pages: the cost of the block-table
    indirection."""
    import torch
    res = {}
    for key, setup, cfg, unit_n, order in (("decode", paged_decode, DECODE, DECODE["batch"], "interleaved"),
                                           ("decode_shuffled", paged_decode, DECODE, DECODE["batch"], "shuffled"),
                                           ("prefill", paged_prefill, PREFILL, PREFILL["chunk"], "interleaved")):
        if key == "prefill" and args.no_prefill:
            continue
        step, keep = setup(cfg, order)
        steps = args.steps if key == "decode" else max(3, args.steps // 3)
        secs, eager, _ = timed(step, steps, max(1, args.warmup // 2), [], graph=args.graph)
        del keep
        torch.cuda.empty_cache()
        ms = secs * 1e3 / steps
        base = result.get("ms_per_step") if key != "prefill" else result.get("prefill", {}).get("ms_per_step")
        res[key] = {"workload": cfg["name"] + f", caches in 128-position pages ({order} page ids)",
                    "value": round(unit_n * steps / secs, 1), "unit": "tokens/s" if key == "prefill" else "queries/s",
                    "ms_per_step": round(ms, 4), "vs_contiguous": round(base / ms, 4) if base else None}
        log(f"paged {key}: {unit_n * steps / secs:.0f}/s, {ms:.3f} ms/step")
    result["paged"] = res


def setup_prefill(cfg, correlated=False, merged=False):
    import torch
    import dsa_inputs as gi
    import dsa_sparse_attention_amd as dsa

    P0, n, topk = cfg["prefix"], cfg["chunk"], cfg["topk"]
    Lc = P0 + n
    tcap, R = Lc, Lc // REG
    seed = gi.SEED_BASE + cfg["seed_index"]
    s = torch.cuda.current_stream().cuda_stream
    geom = dsa.geometry(topk=topk)
    ik = torch.empty(G * tcap * P, dtype=torch.bfloat16, device="cuda")
    K = torch.empty(G * tcap * D, dtype=torch.bfloat16, device="cuda")
    V = torch.empty(G * tcap * D, dtype=torch.bfloat16, device="cuda")
    gi.dev_tokens(ik.data_ptr(), s, seed, gi.TID_IK, 1, tcap, G, P, 0, tcap, tcap, tcap, gi.LAYOUT_GROUP_MAJOR,
                  gi.IK_SCALE)
    gi.dev_tokens(K.data_ptr(), s, seed, gi.TID_K, 1, tcap, G, D, 0, tcap, tcap, tcap, gi.LAYOUT_KTILED)
    gi.dev_tokens(V.data_ptr(), s, seed, gi.TID_V, 1, tcap, G, D, 0, tcap, tcap, tcap, gi.LAYOUT_REGION_T)
    q = torch.empty(n * HQ * D, dtype=torch.bfloat16, device="cuda")
    iq = torch.empty(n * HI * P, dtype=torch.bfloat16, device="cuda")
    z = torch.empty(n * HI, dtype=torch.float32, device="cuda")
    gi.dev_flat(q.data_ptr(), s, seed, gi.TID_Q, q.numel(), 0, 1.0)
    gi.dev_flat(iq.data_ptr(), s, seed, gi.TID_IQ, iq.numel(), 0, gi.IK_SCALE)
    gi.dev_flat(z.data_ptr(), s, seed, gi.TID_Z, z.numel(), 1)
    if correlated:  # neighbouring queries select overlapping regions
        iqh, zh = gi.host_correlated_index_queries(seed, n, HI, P, **CORRELATED)
        iq.copy_(torch.from_numpy(iqh.view("int16").ravel()).view(torch.bfloat16))
        z.copy_(torch.from_numpy(zh.ravel()))
    summ = torch.zeros(G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(G * R, dtype=torch.float32, device="cuda")
    i32 = lambda v: torch.tensor(v, dtype=torch.int32, device="cuda")
    dsa.dsa_compress_regions(geom, ik, tcap, i32([0]), i32([P0 // REG]), P0 // REG, summ, scale)  # prefix
    torch.cuda.synchronize()
    rb, re_ = i32([P0 // REG]), i32([Lc // REG])
    span = Lc // REG - P0 // REG
    qseq, qpos = i32([0] * n), i32(list(range(P0, Lc)))
    sel = torch.empty(n * G * topk, dtype=torch.int32, device="cuda")
    nsel = torch.empty(n * G, dtype=torch.int32, device="cuda")
    out = torch.empty(n * HQ * D, dtype=torch.bfloat16, device="cuda")
    ws1 = dsa.workspace(dsa.dsa_score_topk_workspace_size(geom, n, R))
    ws3 = dsa.workspace(dsa.dsa_sparse_gqa_prefill_workspace_size(geom, n))
    L = dsa.load()
    p = Calls.p
    gp = ctypes.byref(geom)
    a_comp = (gp, 1, p(ik), tcap, p(rb), p(re_), span, p(summ), p(scale))
    a_score = (gp, n, p(iq), p(z), p(qseq), p(qpos), 1, p(summ), p(scale), tcap, R, p(sel), p(nsel), None,
               p(ws1), ws1.numel())
    a_attn = (gp, n, p(q), p(qseq), p(qpos), 1, p(K), p(V), tcap, p(sel), p(nsel), p(out), p(ws3), ws3.numel())

    attend = L.dsa_sparse_gqa_prefill_merged if merged else L.dsa_sparse_gqa_prefill

    def step(st):
        rc = (L.dsa_compress_regions(*a_comp, st) or L.dsa_score_topk(*a_score, st) or attend(*a_attn, st))
        if rc:
            raise RuntimeError(f"prefill step failed: {rc} {L.dsa_last_error().decode()}")

    keep = (ik, K, V, q, iq, z, summ, scale, rb, re_, qseq, qpos, sel, nsel, out, ws1, ws3, geom)
    return step, keep


def setup_swa(seed, layer, n_seqs, p0, n_new, geom):
    """One sliding-window layer: rings holding positions p0-512..p0-1 of every sequence (written by the
    generator in the ring layouts), n_new new rows per sequence at p0.. (token-major K/V, q), output and
    workspace.  Returns the marshalled swa_attention and swa_ring_append arguments and the tensors."""
    import torch
    import dsa_inputs as gi
    import dsa_sparse_attention_amd as dsa

    s = torch.cuda.current_stream().cuda_stream
    tq, tk, tv = (gi.tid_swa(t, layer) for t in (gi.TID_Q, gi.TID_K, gi.TID_V))
    T = p0 + n_new
    kr = torch.empty(n_seqs * G * W * D, dtype=torch.bfloat16, device="cuda")
    vr = torch.empty(n_seqs * G * W * D, dtype=torch.bfloat16, device="cuda")
    t0 = max(0, p0 - W)
    if p0 > t0:
        gi.dev_tokens(kr.data_ptr(), s, seed, tk, n_seqs, T, G, D, t0, p0 - t0, W, W, gi.LAYOUT_KTILED)
        gi.dev_tokens(vr.data_ptr(), s, seed, tv, n_seqs, T, G, D, t0, p0 - t0, W, W, gi.LAYOUT_REGION_T)
    rows = n_seqs * n_new
    kn = torch.empty(rows * G * D, dtype=torch.bfloat16, device="cuda")
    vn = torch.empty(rows * G * D, dtype=torch.bfloat16, device="cuda")
    gi.dev_tokens(kn.data_ptr(), s, seed, tk, n_seqs, T, G, D, p0, n_new, n_new, n_new, gi.LAYOUT_TOKEN_MAJOR)
    gi.dev_tokens(vn.data_ptr(), s, seed, tv, n_seqs, T, G, D, p0, n_new, n_new, n_new, gi.LAYOUT_TOKEN_MAJOR)
    q = torch.empty(rows * HQ * D, dtype=torch.bfloat16, device="cuda")
    gi.dev_flat(q.data_ptr(), s, seed, tq, q.numel(), 0, 1.0)
    out = torch.empty(rows * HQ * D, dtype=torch.bfloat16, device="cuda")
    pos0 = torch.tensor([p0] * n_seqs, dtype=torch.int32, device="cuda")
    row0 = torch.tensor([n_new * i for i in range(n_seqs + 1)], dtype=torch.int32, device="cuda")
    ws = dsa.workspace(dsa.swa_attention_workspace_size(geom, W, n_seqs, n_new))
    p = Calls.p
    gp = ctypes.byref(geom)
    a_att = (gp, W, n_seqs, n_new, p(pos0), p(row0), p(q), p(kn), p(vn), p(kr), p(vr), p(out), p(ws), ws.numel())
    a_app = (gp, W, n_seqs, n_new, p(pos0), p(row0), p(kn), p(vn), p(kr), p(vr))
    a_dec = (gp, W, n_seqs, p(pos0), p(q), p(kn), p(vn), p(kr), p(vr), p(out)) if n_new == 1 else None
    return a_att, a_app, a_dec, (kr, vr, kn, vn, q, out, pos0, row0, ws)


def setup_mix(cfg):
    """The 3:1 stack: three sliding-window layers (decode: one new token per sequence at L-1, rings
    holding L-513..L-2), then the DSA decode step of the same batch.  Each layer's ring append rewrites
    the same slot every step, so repeated steps see identical inputs."""
    import torch
    import dsa_inputs as gi
    import dsa_sparse_attention_amd as dsa

    B, Lc = cfg["batch"], cfg["context"]
    seed = gi.SEED_BASE + cfg["seed_index"]
    dsa_step, keep = setup_decode(cfg)
    geom = keep[-1]
    L = dsa.load()
    layers = [setup_swa(seed, l, B, Lc - 1, 1, geom) for l in range(cfg["swa_layers"])]

    def step(st):
        # each sliding-window layer: attention over its window and the ring append, one launch
        for _, _, a_dec, _ in layers:
            rc = L.swa_decode_step(*a_dec, st)
            if rc:
                raise RuntimeError(f"sliding-window layer failed: {rc} {L.dsa_last_error().decode()}")
        dsa_step(st)

    return step, (keep, layers)


def setup_swa_prefill(cfg):
    import dsa_inputs as gi
    import dsa_sparse_attention_amd as dsa

    seed = gi.SEED_BASE + cfg["seed_index"]
    geom = dsa.geometry()
    a_att, a_app, _, tens = setup_swa(seed, 0, 1, cfg["prefix"], cfg["chunk"], geom)
    L = dsa.load()

    def step(st):
        rc = L.swa_attention(*a_att, st) or L.swa_ring_append(*a_app, st)
        if rc:
            raise RuntimeError(f"sliding-window prefill failed: {rc} {L.dsa_last_error().decode()}")

    return step, (tens, geom)


def cur_stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def timed(step, steps, warmup, kernels, graph=True):
    """Warmup, then three passes of exactly `steps` steps, each between two synchronisations:
    (1) eager launches; (2) replays of a HIP graph holding one step (the timed headline when
    graph=True); (3) eager launches with the library's per-kernel hipEvents on (roofline).
    Returns (seconds_headline, seconds_eager, {kernel: (avg_ms, launches)})."""
    import torch
    import dsa_sparse_attention_amd as dsa

    for _ in range(warmup):
        step(cur_stream())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(cur_stream())
    torch.cuda.synchronize()
    eager = time.perf_counter() - t0
    head = eager
    if graph:
        # one graph per input variant of the step (rotating inputs), replayed in turn
        nv = getattr(step, "variants", 1)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(nv):
                step(cur_stream())
        torch.cuda.current_stream().wait_stream(side)
        gs = []
        for _ in range(nv):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(cur_stream())
            gs.append(g)
        for g in gs:
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            gs[i % nv].replay()
        torch.cuda.synchronize()
        head = time.perf_counter() - t0
        del gs
    dsa.profile_enable(True)
    torch.cuda.synchronize()
    for _ in range(steps):
        step(cur_stream())
    torch.cuda.synchronize()
    stats = {}
    for k in kernels:
        ms, n = dsa.profile_kernel_stats(k)
        stats[k] = (ms / max(n, 1), n)
    dsa.profile_enable(False)
    return head, eager, stats


def host_cpu():
    """The host CPU the oracle runs on: model name (as lscpu reports it, from /proc/cpuinfo) and the
    number of processors this process may run on (nproc)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return {"cpu_model": model, "nproc": nproc}


def cpu_baseline_decode(cfg, budget_s=15.0):
    """The oracle on the host cores: one decode query of sequence 0 of the workload (compress the
    completed region, score every candidate region x 4 groups, top-512, sparse GQA), repeated until
    about budget_s of CPU time.  The prefix summaries are built untimed, as on the GPU."""
    import numpy as np
    import dsa_inputs as gi
    import oracle as O

    B, Lc, topk = cfg["batch"], cfg["context"], cfg["topk"]
    R = Lc // REG
    seed = gi.SEED_BASE + cfg["seed_index"]
    t0 = time.time()
    ik = gi.host_index_k(seed, Lc, G, P, 0, 0, Lc, cfg["planted"])
    K = gi.host_tokens_bf16(seed, gi.TID_K, Lc, G, D, 0, 0, Lc)
    V = gi.host_tokens_bf16(seed, gi.TID_V, Lc, G, D, 0, 0, Lc)
    q = gi.host_normal_bf16(seed, gi.TID_Q, HQ * D).reshape(HQ, D)
    iq = gi.host_normal_bf16(seed, gi.TID_IQ, HI * P, gi.IK_SCALE).reshape(HI, P)
    z = gi.host_uniform_f32(seed, gi.TID_Z, HI)
    codes, scales = O.compress_regions(ik, 0, R - 1, np.zeros((R, G, P), np.uint8), np.zeros((R, G), np.float32))
    log(f"cpu baseline setup: {time.time() - t0:.1f}s")
    n = 0
    t1 = time.perf_counter()
    while True:
        O.compress_regions(ik, R - 1, R, codes, scales)
        O.dsa_query(iq, z, codes, scales, q, K, V, Lc - 1, k=topk)
        n += 1
        el = time.perf_counter() - t1
        if el >= budget_s or n >= 200:
            break
    return dict(value=n / el, unit="queries/s", cores=O.num_threads(), kind="oracle",
                sample=f"{n} decode queries of one sequence at {Lc} tokens (compress 1 region, score {R - 1} "
                       f"regions x 4 groups, top-{topk}, sparse GQA), fp64 C with OpenMP; prefix summaries untimed",
                **host_cpu())


def cpu_baseline_prefill(cfg, n_queries=24):
    """The oracle on a bounded sample of the 64K prefill chunk: compress the chunk's complete regions,
    then n_queries evenly spaced chunk queries end to end."""
    import numpy as np
    import dsa_inputs as gi
    import oracle as O

    P0, n, topk = cfg["prefix"], cfg["chunk"], cfg["topk"]
    Lc = P0 + n
    R = Lc // REG
    seed = gi.SEED_BASE + cfg["seed_index"]
    ik = gi.host_index_k(seed, Lc, G, P, 0, 0, Lc)
    K = gi.host_tokens_bf16(seed, gi.TID_K, Lc, G, D, 0, 0, Lc)
    V = gi.host_tokens_bf16(seed, gi.TID_V, Lc, G, D, 0, 0, Lc)
    q = gi.host_normal_bf16(seed, gi.TID_Q, n * HQ * D).reshape(n, HQ, D)
    iq = gi.host_normal_bf16(seed, gi.TID_IQ, n * HI * P, gi.IK_SCALE).reshape(n, HI, P)
    z = gi.host_uniform_f32(seed, gi.TID_Z, n * HI).reshape(n, HI)
    codes, scales = O.compress_regions(ik, 0, P0 // REG, np.zeros((R, G, P), np.uint8), np.zeros((R, G), np.float32))
    qs = np.linspace(0, n - 1, n_queries).astype(int)
    t1 = time.perf_counter()
    O.compress_regions(ik, P0 // REG, R, codes, scales)
    for i in qs:
        O.dsa_query(iq[i], z[i], codes, scales, q[i], K, V, P0 + int(i), k=topk)
    el = time.perf_counter() - t1
    return dict(value=len(qs) / el, unit="tokens/s", cores=O.num_threads(), kind="oracle",
                sample=f"{len(qs)} of the {n} chunk queries (evenly spaced) end to end, after compressing the "
                       f"chunk's {R - P0 // REG} complete regions; fp64 C with OpenMP",
                **host_cpu())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-shapes", action="store_true", help="skip the 8K batch-1 and 128K batch-16 decode lines")
    ap.add_argument("--no-swa", action="store_true", help="skip the 3:1 layer mix and sliding-window prefill lines")
    ap.add_argument("--swa-only", action="store_true",
                    help="only the 3:1 layer mix and sliding-window prefill (for per-workload profiles)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-cache runs of the two headline workloads")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 K/V cache runs of the two headline workloads")
    ap.add_argument("--no-merged", action="store_true",
                    help="skip the neighbour-merged prefill runs (correlated and i.i.d. chunks)")
    ap.add_argument("--no-frontend", action="store_true", help="skip the indexer front-end runs")
    ap.add_argument("--graph", action="store_true", help="time replays of a HIP graph holding one step")
    ap.add_argument("--separate", action="store_true",
                    help="decode step as three calls (compress, score_topk, sparse_gqa_decode) instead of dsa_decode_step")
    ap.add_argument("--profile-run", action="store_true",
                    help="setup + a few steps of each workload + a 1 GiB copy kernel, for rocprofv3")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only: the DSA layer here runs on a single MI355X "
              f"(requested --gpus {args.gpus}); multi-GPU sharding is described, not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    import dsa_sparse_attention_amd as dsa

    torch.cuda.set_device(0)
    dsa.load()

    if args.swa_only:
        args.no_prefill, args.no_swa = True, False
    if args.profile_run:
        if not args.swa_only:
            # the 1M batch-4 decode, then (unless --no-shapes) the 8K batch-1 and 128K batch-16 ones:
            # three steps each, in this order
            for cfg in (DECODE,) + (() if args.no_shapes else (DECODE_8K, DECODE_128K)):
                step, keep = setup_decode(cfg)
                for _ in range(3):
                    step(cur_stream())
                torch.cuda.synchronize()
                del keep
                torch.cuda.empty_cache()
        if not args.no_prefill:
            step, keep = setup_prefill(PREFILL)
            for _ in range(2):
                step(cur_stream())
            torch.cuda.synchronize()
            del keep
            if not args.no_merged:
                step, keep = setup_prefill(PREFILL, correlated=True, merged=True)
                for _ in range(2):
                    step(cur_stream())
                torch.cuda.synchronize()
                del keep
        if not args.no_frontend and not args.swa_only:
            for T in (PREFILL["chunk"], DECODE["batch"]):
                step, keep = setup_frontend(T)
                for _ in range(2):
                    step(cur_stream())
                torch.cuda.synchronize()
                del keep
        if not args.no_swa:
            for setup, cfg in ((setup_mix, MIX), (setup_swa_prefill, SWA_PREFILL)):
                step, keep = setup(cfg)
                for _ in range(2):
                    step(cur_stream())
                torch.cuda.synchronize()
                del keep
        # calibration: a plain elementwise shader kernel that reads exactly 1 GiB and writes
        # exactly 1 GiB (torch.bitwise_not on uint8), for scaling the FETCH/WRITE counters
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            torch.bitwise_not(a, out=b)
        torch.cuda.synchronize()
        log("profile run done")
        return

    result = {} if args.swa_only else measure_decode(args)
    if not args.swa_only and not args.no_shapes:
        measure_decode_shapes(args, result)
    # ---- prefill at 64K
    if not args.no_prefill:
        measure_prefill(args, result)
    # ---- the same two workloads over paged caches, and with FP8 K/V caches
    if not args.no_paged and not args.swa_only:
        measure_paged(args, result)
    if not args.no_fp8 and not args.swa_only:
        measure_fp8(args, result)
    if not args.no_merged and not args.no_prefill:
        measure_merged(args, result)
    if not args.no_frontend and not args.swa_only:
        measure_frontend(args, result)
    # ---- the 3:1 sliding-window / DSA stack (decode) and a sliding-window prefill chunk
    if not args.no_swa:
        measure_swa(args, result)
    if not args.no_cpu and not args.swa_only:
        result["cpu_baseline"] = cpu_baseline_decode(DECODE)
        if "prefill" in result:
            result["prefill"]["cpu_baseline"] = cpu_baseline_prefill(PREFILL)
    print(json.dumps(result), flush=True)


def decode_workload(args, cfg, steps, warmup, traffic_key=None):
    """Times one decode workload (rotating inputs, see setup_decode).  The roofline is the kernel that
    moves the most algorithmic bytes: the score stream at long contexts, the K/V gather at short ones."""
    import torch
    step, keep = setup_decode(cfg)
    cfg["separate"] = args.separate
    kn = ["k_compress", "k_score_decode", "k_select", "k_sgqa_decode", "k_sgqa_merge"]
    secs, eager, st = timed(step, steps, warmup, kn, graph=args.graph)
    st = {k: v for k, v in st.items() if v[1]}
    del keep
    torch.cuda.empty_cache()
    B, Lc = cfg["batch"], cfg["context"]
    ms_step = secs * 1e3 / steps
    byt = decode_bytes(B, Lc, cfg["topk"])
    # (the fused step's compression runs inside the selection launch, not the scoring one)
    if byt["score"] >= byt["attend"]:
        kern, kbytes, src = "k_score_decode", byt["score"], source_hash("score_topk.hip")
    else:
        kern, kbytes, src = "k_sgqa_decode", byt["attend"], source_hash("attention.hip")
    kms = st[kern][0]
    achieved = kbytes / (kms * 1e-3) / 1e9
    out = {
        "value": round(B * steps / secs, 2), "unit": "queries/s", "steps": steps,
        "ms_per_step": round(ms_step, 4), "eager_ms_per_step": round(eager * 1e3 / steps, 4),
        "config": {"workload": cfg["name"], "batch": B, "context_tokens": Lc, "topk": cfg["topk"],
                   "regions_per_sequence": Lc // REG, "input_copies": cfg.get("copies", 1),
                   "query_sets": cfg.get("query_sets", QUERY_SETS),
                   "entry": "separate calls" if args.separate else "dsa_decode_step"},
        "roofline": {"bound": "hbm", "kernel": kern, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(kern, traffic_key, src) if traffic_key else None,
                     "algorithmic_bytes_per_launch": kbytes, "avg_launch_us": round(kms * 1e3, 2),
                     "counters": (load_profile_json(kern, traffic_key, "mem_json", src)
                                  or load_profile_json(kern, traffic_key, "mfma_json", src)) if traffic_key else None},
        "step_hbm": {"algorithmic_bytes": byt["total"],
                     "achieved_GBs": round(byt["total"] / (ms_step * 1e-3) / 1e9, 1),
                     "frac": round(byt["total"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "kernels_us": {k: round(v[0] * 1e3, 2) for k, v in st.items()},
    }
    log(f"decode {B} x {Lc}: {B * steps / secs:.1f} q/s, {ms_step:.4f} ms/step, {kern} {achieved:.0f} GB/s")
    return out


def measure_decode(args):
    d = decode_workload(args, DECODE, args.steps, args.warmup, traffic_key="decode_b4_1m")
    result = {
        "metric": "DSA layer decode queries/s @1M ctx + prefill tok/s @64K, % HBM/MFMA roofline",
        "value": d["value"], "unit": "queries/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": d["ms_per_step"], "timing": "graph replay" if args.graph else "eager",
        "eager_ms_per_step": d["eager_ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": d["config"], "roofline": d["roofline"], "step_hbm": d["step_hbm"], "kernels_us": d["kernels_us"],
    }
    return result


def measure_decode_shapes(args, result):
    """The 8K single-query and 128K batch-16 decode workloads, as objects of their own."""
    for key, cfg, tk in (("decode_8k", DECODE_8K, "decode_b1_8k"), ("decode_128k", DECODE_128K, "decode_b16_128k")):
        steps = max(args.steps, cfg.get("copies", 1) * 2) if key == "decode_8k" else args.steps
        d = decode_workload(args, cfg, steps, args.warmup, traffic_key=tk)
        d["workload"] = d["config"].pop("workload")
        if not args.no_cpu:
            d["cpu_baseline"] = cpu_baseline_decode(cfg, budget_s=4.0)
        result[key] = d


def measure_prefill(args, result):
    import torch
    step, keep = setup_prefill(PREFILL)
    kp = ["k_compress", "k_score_prefill", "k_select", "k_sgqa_prefill", "k_sgqa_merge"]
    psteps = max(3, args.steps // 3)
    psecs, peager, pst = timed(step, psteps, max(1, args.warmup // 2), kp, graph=args.graph)
    del keep
    torch.cuda.empty_cache()
    n = PREFILL["chunk"]
    fl = prefill_flops(PREFILL["prefix"], n, PREFILL["topk"])
    pms = psecs * 1e3 / psteps
    att_ms, sc_ms, mg_ms = pst["k_sgqa_prefill"][0], pst["k_score_prefill"][0], pst["k_sgqa_merge"][0]
    att_tf = fl["attend"] / (att_ms * 1e-3) / 1e12
    sc_tf = fl["score"] / (sc_ms * 1e-3) / 1e12
    step_tf = fl["total"] / (pms * 1e-3) / 1e12
    result["prefill"] = {
        "workload": PREFILL["name"], "value": round(n * psteps / psecs, 1), "unit": "tokens/s",
        "steps": psteps, "ms_per_step": round(pms, 3), "eager_ms_per_step": round(peager * 1e3 / psteps, 3),
        "roofline": {"bound": "mfma", "kernel": "k_sgqa_prefill", "achieved": round(att_tf, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(att_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": load_traffic("k_sgqa_prefill", "prefill_64k", source_hash("attention.hip")),
                     "algorithmic_flops_per_launch": fl["attend"], "avg_launch_us": round(att_ms * 1e3, 1),
                     "counters": load_profile_json("k_sgqa_prefill", "prefill_64k", "mfma_json",
                                                   source_hash("attention.hip"))},
        "attention_with_merge": {
            "kernels": ["k_sgqa_prefill", "k_sgqa_merge"],
            "achieved_TFLOPs": round(fl["attend"] / ((att_ms + mg_ms) * 1e-3) / 1e12, 2),
            "frac": round(fl["attend"] / ((att_ms + mg_ms) * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "gathered_kv_bytes": fl["gather"],
            "gather_GBs": round(fl["gather"] / (att_ms * 1e-3) / 1e9, 1)},
        "score_kernel": {"kernel": "k_score_prefill", "achieved_TFLOPs": round(sc_tf, 2),
                         "frac": round(sc_tf / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": fl["score"],
                         "avg_launch_us": round(sc_ms * 1e3, 1),
                         "counters": load_profile_json("k_score_prefill", "prefill_64k", "mfma_json",
                                                       source_hash("score_topk.hip"))},
        "step_mfma": {"algorithmic_flops": fl["total"], "achieved_TFLOPs": round(step_tf, 2),
                      "frac": round(step_tf / MFMA_BF16_PEAK_TFLOPS, 4)},
        "kernels_us": {k: round(v[0] * 1e3, 2) for k, v in pst.items()},
    }
    log(f"prefill: {n * psteps / psecs:.0f} tok/s, {pms:.3f} ms/step")


def union_of_neighbours(sel, nsel, n, topk, width=2):
    """Mean number of distinct regions per group in the selections of `width` consecutive queries."""
    import numpy as np
    s = sel.view(n, G, topk).cpu().numpy()
    c = nsel.view(n, G).cpu().numpy()
    us = [len(set().union(*[set(s[i, g, :c[i, g]].tolist()) for i in range(i0, i0 + width)]))
          for i0 in range(0, n - width + 1, width) for g in range(G)]
    return float(np.mean(us))


def measure_merged(args, result):
    """Neighbour-merged prefill (dsa_sparse_gqa_prefill_merged) against the per-query attention on the
    prefill chunk with correlated neighbouring queries, and on the unrelated (i.i.d.) chunk."""
    import torch
    n = PREFILL["chunk"]
    fl = prefill_flops(PREFILL["prefix"], n, PREFILL["topk"])
    res = {}
    for key, corr, merged in (("correlated_per_query", True, False), ("correlated_merged", True, True),
                              ("iid_merged", False, True)):
        step, keep = setup_prefill(PREFILL, correlated=corr, merged=merged)
        kern = "k_sgqa_prefill_merged" if merged else "k_sgqa_prefill"
        steps = max(3, args.steps // 3)
        secs, _, st = timed(step, steps, max(1, args.warmup // 2), [kern, "k_sgqa_merge"], graph=args.graph)
        sel, nsel = keep[12], keep[13]
        union = union_of_neighbours(sel, nsel, n, PREFILL["topk"]) if merged else None
        del keep
        torch.cuda.empty_cache()
        att_ms = st[kern][0]
        tf = fl["attend"] / (att_ms * 1e-3) / 1e12
        res[key] = {"workload": PREFILL["name"] + (", correlated neighbouring queries (anchors every "
                                                   f"{CORRELATED['every']}, noise {CORRELATED['noise']})"
                                                   if corr else ", i.i.d. queries"),
                    "value": round(n * steps / secs, 1), "unit": "tokens/s", "ms_per_step": round(secs * 1e3 / steps, 3),
                    "attention": {"kernel": kern, "avg_launch_us": round(att_ms * 1e3, 1),
                                  "achieved_TFLOPs": round(tf, 2), "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                  "merge_us": round(st["k_sgqa_merge"][0] * 1e3, 1)}}
        if key == "correlated_merged":  # rocprofv3 counters of this kernel on this chunk
            res[key]["attention"]["counters"] = load_profile_json(
                kern, "prefill_64k_correlated", "mfma_json", source_hash("attention.hip"))
        if union is not None:
            res[key]["mean_union_of_2_neighbours_per_group"] = round(union, 1)
        log(f"{key}: {n * steps / secs:.0f} tok/s, attention {att_ms * 1e3:.0f} us")
    result["merged_prefill"] = res


FRONTEND = dict(hidden=6144, seed_index=5)  # the pages give no hidden size: 6144 = 32 x 192 stands in


def setup_frontend(T):
    """Indexer front-end of T tokens (hidden states -> index_q, index_k, z) at positions 63,488.."""
    import numpy as np
    import torch
    import dsa_inputs as gi
    import dsa_sparse_attention_amd as dsa
    Hd = FRONTEND["hidden"]
    seed = gi.SEED_BASE + FRONTEND["seed_index"]
    x, w, gq, gk = gi.host_frontend_inputs(seed, T, Hd, dsa.IDX_PROJ_ROWS)
    up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16).ravel()).cuda().view(torch.bfloat16)
    xd, wd = up(x), up(w)
    gqd, gkd = torch.from_numpy(gq).cuda(), torch.from_numpy(gk).cuda()
    pos = torch.arange(63488, 63488 + T, dtype=torch.int32, device="cuda")
    iq = torch.empty(T * HI * P, dtype=torch.bfloat16, device="cuda")
    ik = torch.empty(T * G * P, dtype=torch.bfloat16, device="cuda")
    z = torch.empty(T * HI, dtype=torch.float32, device="cuda")
    ws = dsa.workspace(dsa.dsa_indexer_workspace_size(T, Hd))
    rope = dsa.rope_config()
    L = dsa.load()
    p = Calls.p
    args = (ctypes.byref(rope), T, Hd, p(xd), p(wd), p(gqd), p(gkd), p(pos), p(iq), p(ik), p(z), p(ws), ws.numel())

    def step(st):
        rc = L.dsa_indexer_project(*args, st)
        if rc:
            raise RuntimeError(f"front-end step failed: {rc} {L.dsa_last_error().decode()}")

    return step, (xd, wd, gqd, gkd, pos, iq, ik, z, ws, rope)


def measure_frontend(args, result):
    """The indexer front-end (projection GEMM, then RMSNorm + partial RoPE) for the 2048-token prefill chunk
    and for one decode step of batch 4: MFMA rate of the projection kernel, and for decode the weight
    bytes it streams."""
    import torch
    import dsa_sparse_attention_amd as dsa
    Hd = FRONTEND["hidden"]
    res = {}
    for key, T in (("prefill_chunk", PREFILL["chunk"]), ("decode_batch4", DECODE["batch"])):
        step, keep = setup_frontend(T)
        steps = max(3, args.steps // 3)
        secs, _, st = timed(step, steps, max(1, args.warmup // 2),
                            ["k_indexer_proj", "k_indexer_finish"], graph=args.graph)
        st = {k: v for k, v in st.items() if v[1]}
        del keep
        torch.cuda.empty_cache()
        proj_ms = st["k_indexer_proj"][0]
        flops = 2.0 * T * Hd * (HI + G) * P
        wbytes = (HI + G) * P * Hd * 2
        tf = flops / (proj_ms * 1e-3) / 1e12
        res[key] = {"workload": f"indexer front-end, {T} tokens, hidden {Hd} (stand-in), 16 index_q heads + 4 "
                                f"index_k groups of 256 + 16 z, RMSNorm + 64-dim llama3 RoPE",
                    "value": round(T * steps / secs, 1), "unit": "tokens/s", "ms_per_step": round(secs * 1e3 / steps, 4),
                    "projection": {"kernel": "k_indexer_proj", "avg_launch_us": round(proj_ms * 1e3, 1),
                                   "algorithmic_flops": flops, "achieved_TFLOPs": round(tf, 2),
                                   "frac_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                   "weight_bytes": wbytes,
                                   "weight_GBs": round(wbytes / (proj_ms * 1e-3) / 1e9, 1)},
                    "kernels_us": {k: round(v[0] * 1e3, 2) for k, v in st.items()}}
        if key == "prefill_chunk":  # the tiled GEMM's rocprofv3 counters (MFMA busy and executed flops)
            res[key]["projection"]["counters"] = load_profile_json(
                "k_indexer_gemm", f"frontend_{T}_h{Hd}", "mfma_json", source_hash("frontend.hip"))
        log(f"front-end {key}: projection {proj_ms * 1e3:.1f} us, {tf:.0f} TFLOP/s")
    result["indexer_frontend"] = res


def measure_swa(args, result):
    import torch
    step, keep = setup_mix(MIX)
    km = ["k_swa_decode", "k_score_decode", "k_select", "k_sgqa_decode",
          "k_sgqa_merge"]
    msteps = max(3, args.steps // 3)
    msecs, meager, mst = timed(step, msteps, max(1, args.warmup // 2), km, graph=args.graph)
    del keep
    torch.cuda.empty_cache()
    B, Lc = MIX["batch"], MIX["context"]
    mms = msecs * 1e3 / msteps
    sbytes = swa_decode_bytes(B)
    dbytes = decode_bytes(B, Lc, MIX["topk"])["total"]
    tot = MIX["swa_layers"] * sbytes + dbytes
    swa_us = mst["k_swa_decode"][0] * 1e3  # per layer: attention and ring append in one launch
    result["mix_decode"] = {
        "workload": MIX["name"], "value": round(B * msteps / msecs, 1), "unit": "queries/s (4-layer stack)",
        "steps": msteps, "ms_per_step": round(mms, 4), "eager_ms_per_step": round(meager * 1e3 / msteps, 4),
        "roofline": {"bound": "hbm", "kernel": "whole stack", "achieved": round(tot / (mms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(tot / (mms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_step": tot},
        "swa_layer": {"algorithmic_bytes": sbytes, "us_per_layer": round(swa_us, 2),
                      "achieved_GBs": round(sbytes / (swa_us * 1e-6) / 1e9, 1)},
        "kernels_us": {k: round(v[0] * 1e3, 2) for k, v in mst.items()},
    }
    log(f"mix decode: {B * msteps / msecs:.0f} q/s, {mms:.3f} ms/step")
    step, keep = setup_swa_prefill(SWA_PREFILL)
    ks = ["k_swa_stage", "k_swa_band", "k_ring_append"]
    ssteps = max(3, args.steps // 3)
    ssecs, seager, sst = timed(step, ssteps, max(1, args.warmup // 2), ks, graph=args.graph)
    del keep
    torch.cuda.empty_cache()
    n = SWA_PREFILL["chunk"]
    fl = swa_prefill_flops(SWA_PREFILL["prefix"], n)
    sms = ssecs * 1e3 / ssteps
    att_ms = sst["k_swa_band"][0]
    result["swa_prefill"] = {
        "workload": SWA_PREFILL["name"], "value": round(n * ssteps / ssecs, 1), "unit": "tokens/s",
        "steps": ssteps, "ms_per_step": round(sms, 4), "eager_ms_per_step": round(seager * 1e3 / ssteps, 4),
        "roofline": {"bound": "mfma", "kernel": "k_swa_band",
                     "achieved": round(fl / (att_ms * 1e-3) / 1e12, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fl / (att_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "algorithmic_flops_per_launch": fl, "avg_launch_us": round(att_ms * 1e3, 1),
                     "counters": load_profile_json("k_swa_band", "swa_prefill_2048", "mfma_json",
                                                   source_hash("attention.hip"))},
        "kernels_us": {k: round(v[0] * 1e3, 2) for k, v in sst.items()},
    }
    log(f"swa prefill: {n * ssteps / ssecs:.0f} tok/s, {sms:.3f} ms/step")


if __name__ == "__main__":
    main()
