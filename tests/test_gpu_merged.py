"""Neighbour-merged prefill (2 consecutive queries walk the union of their selections) through the
C ABI: each query's output meets the oracle's attention over its own selection, on correlated chunks
(neighbouring selections overlap, the case the merge is for) and on unrelated ones; queries of
several sequences may be neighbours; lists are sets (order, repeats and out-of-range ids do not
matter); the paged form is bit-identical to the contiguous one."""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
import dsa_sparse_attention_amd as dsa
import oracle as O

import _harness as H
import test_gpu_paged as TP

pytestmark = pytest.mark.gpu

G, P, HQ, D, HI = H.G, H.P, H.HQ, H.D, H.HI


def _upload_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).ravel()).cuda().view(H.BF16)


def _chunk(seed, seqs, order="chunk", correlated=True, topk=512):
    """Caches holding every position of each sequence (p0 + n tokens), queries at p0..p0+n-1 of every
    sequence (sequence after sequence, or interleaved), correlated or i.i.d. indexer inputs, and the
    selection of dsa_score_topk."""
    B = len(seqs)
    end = np.array([p0 + n for p0, n in seqs], dtype=np.int32)
    tcap = H.round128(int(end.max()))
    R = tcap // 8
    geom = dsa.geometry(topk=topk)
    ik = H.dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE)
    K = H.dev_cache(seed, gi.TID_K, B, tcap, D, tcap, gi.LAYOUT_KTILED)
    V = H.dev_cache(seed, gi.TID_V, B, tcap, D, tcap, gi.LAYOUT_REGION_T)
    summ = torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(B * G * R, dtype=torch.float32, device="cuda")
    dsa.dsa_compress_regions(geom, ik, tcap, H.i32(np.zeros(B)), H.i32(end // 8), R, summ, scale)
    qs, qp = [], []
    if order == "chunk":
        for b, (p0, n) in enumerate(seqs):
            qs += [b] * n
            qp += list(range(p0, p0 + n))
    else:
        for i in range(max(n for _, n in seqs)):
            for b, (p0, n) in enumerate(seqs):
                if i < n:
                    qs.append(b)
                    qp.append(p0 + i)
    nq = len(qs)
    q = H.dev_flat_bf16(seed, gi.TID_Q, nq * HQ * D)
    if correlated:
        iqh, zh = gi.host_correlated_index_queries(seed, nq)
        iq, z = _upload_bf16(iqh), torch.from_numpy(zh.ravel()).cuda()
    else:
        _, iq, z = H.dev_queries(seed, nq)
    sel = torch.empty(nq * G * topk, dtype=torch.int32, device="cuda")
    nsel = torch.empty(nq * G, dtype=torch.int32, device="cuda")
    dsa.dsa_score_topk(geom, iq, z, H.i32(qs), H.i32(qp), B, summ, scale, tcap, R, sel, nsel)
    return dict(B=B, tcap=tcap, R=R, geom=geom, K=K, V=V, q=q, qs=qs, qp=qp, nq=nq, sel=sel, nsel=nsel,
                end=end, topk=topk)


def _run(c, merged, sel=None, nsel=None):
    out = torch.empty(c["nq"] * HQ * D, dtype=H.BF16, device="cuda")
    f = dsa.dsa_sparse_gqa_prefill_merged if merged else dsa.dsa_sparse_gqa_prefill
    f(c["geom"], c["q"], H.i32(c["qs"]), H.i32(c["qp"]), c["B"], c["K"], c["V"], c["tcap"],
      c["sel"] if sel is None else sel, c["nsel"] if nsel is None else nsel, out)
    torch.cuda.synchronize()
    return H.bf16_np(out).reshape(c["nq"], HQ, D)


def _oracle_check(seed, c, out, step, lists_of=None, what="merged"):
    """Sampled queries against the oracle's attention over the GPU's own selection lists."""
    hq = gi.host_normal_bf16(seed, gi.TID_Q, c["nq"] * HQ * D).reshape(c["nq"], HQ, D)
    gsel = c["sel"].cpu().numpy().reshape(c["nq"], G, c["topk"])
    gn = c["nsel"].cpu().numpy().reshape(c["nq"], G)
    host = {}
    worst = [0.0, 0.0]
    for i in range(0, c["nq"], step):
        b, p = c["qs"][i], c["qp"][i]
        if b not in host:
            L = int(c["end"][b])
            host[b] = (gi.host_tokens_bf16(seed, gi.TID_K, c["tcap"], G, D, b, 0, L),
                       gi.host_tokens_bf16(seed, gi.TID_V, c["tcap"], G, D, b, 0, L))
        lists = lists_of(i) if lists_of else [gsel[i, g, :gn[i, g]] for g in range(G)]
        ref = O.attend(hq[i], host[b][0], host[b][1], p, lists, k=c["topk"])
        mx, rr = H.assert_attn(out[i], ref, f"{what} query {i}")
        worst = [max(worst[0], mx), max(worst[1], rr)]
    print(f"{what}: worst max abs {worst[0]:.2e}, rel rms {worst[1]:.2e}")


def _union_stats(c, width=2):
    gsel = c["sel"].cpu().numpy().reshape(c["nq"], G, c["topk"])
    gn = c["nsel"].cpu().numpy().reshape(c["nq"], G)
    us = []
    for i0 in range(0, c["nq"] - width + 1, width):
        for g in range(G):
            us.append(len(set().union(*[set(gsel[i, g, :gn[i, g]].tolist()) for i in range(i0, i0 + width)])))
    return float(np.mean(us))


@pytest.mark.parametrize("seqs,correlated", [
    ([(4003, 300)], True),             # one sequence, partial regions at both ends
    ([(4003, 300)], False),            # unrelated neighbouring selections
    ([(63488, 2048)], True),           # the 64K prefill chunk, correlated queries
])
def test_merged_prefill_matches_oracle(seqs, correlated):
    seed = 0xA10 + len(seqs) + int(correlated) + seqs[0][1]
    c = _chunk(seed, seqs, correlated=correlated)
    out = _run(c, True)
    ref = _run(c, False)
    # same maths as the per-query kernel, another summation order
    H.assert_attn(out.reshape(-1, D), ref.reshape(-1, D).astype(np.float64), "merged vs per-query")
    print(f"mean union of 2 neighbours: {_union_stats(c):.0f} regions per group")
    _oracle_check(seed, c, out, 97 if c["nq"] > 1000 else 7)


def test_merged_prefill_mixed_sequences_and_ragged():
    """Interleaved queries of 3 sequences (each pair of neighbours spans two sequences), a count that is
    not a multiple of 8, and topk 37."""
    seed = 0xA20
    c = _chunk(seed, [(1000, 33), (130, 5), (4096, 21)], order="interleaved", correlated=False, topk=37)
    out = _run(c, True)
    _oracle_check(seed, c, out, 1, what="merged mixed")


@pytest.mark.parametrize("merged", [True, False])
def test_prefill_lists_are_sets(merged):
    """Unsorted lists with repeats, ids past the query's region and negative ids: both prefill calls
    (neighbour-merged and per-query) attend each valid region once."""
    seed = 0xA30
    c = _chunk(seed, [(2000, 40)], correlated=True, topk=64)
    nq, k = c["nq"], 64
    rng = np.random.default_rng(seed)
    sel = np.full((nq, G, k), -1, dtype=np.int32)
    nsel = np.zeros((nq, G), dtype=np.int32)
    valid = {}
    for i in range(nq):
        cur = c["qp"][i] // 8
        for g in range(G):
            base = rng.choice(cur + 1, size=40, replace=False)
            lst = list(base) + list(base[:10]) + [cur + 1, cur + 500, -3, -1]  # repeats, out of range
            lst = [int(x) for x in rng.permutation(lst)][:k]
            sel[i, g, :len(lst)] = lst
            nsel[i, g] = len(lst)
            valid[(i, g)] = sorted(set(x for x in lst if 0 <= x <= cur))
    c["sel"], c["nsel"] = H.i32(sel.ravel()), H.i32(nsel.ravel())
    out = _run(c, merged)
    _oracle_check(seed, c, out, 1, lists_of=lambda i: [valid[(i, g)] for g in range(G)],
                  what="merged sets" if merged else "per-query sets")


def test_merged_prefill_paged_matches_contiguous():
    seed = 0xA40
    seqs = [(4003, 300), (1000, 77)]
    c = _chunk(seed, seqs, correlated=True)
    pools, pages, _ = TP._to_pools(dict(k=c["K"], v=c["V"], ik=None, summ=None, scale=None),
                                   [int(e) for e in c["end"]], c["tcap"], seed)
    o1 = _run(c, True)
    out = torch.empty(c["nq"] * HQ * D, dtype=H.BF16, device="cuda")
    dsa.dsa_sparse_gqa_prefill_merged_paged(c["geom"], c["q"], H.i32(c["qs"]), H.i32(c["qp"]), c["B"], pages,
                                            pools["k"], pools["v"], c["sel"], c["nsel"], out)
    torch.cuda.synchronize()
    assert np.array_equal(o1.view(np.uint32), H.bf16_np(out).reshape(o1.shape).view(np.uint32))


def test_merged_prefill_edge_cases():
    """A chunk at the very start of a sequence (positions 0..11: partial regions 0 and 1), top-1 (only
    the forced current region), then the same chunk with empty lists for one group of every query and
    for every group of odd queries (their output is 0, as the oracle defines it)."""
    seed = 0xA50
    c = _chunk(seed, [(0, 12)], correlated=False, topk=1)
    out = _run(c, True)
    _oracle_check(seed, c, out, 1, what="merged start of sequence")
    nq = c["nq"]
    sel = c["sel"].cpu().numpy().reshape(nq, G, 1).copy()
    nsel = c["nsel"].cpu().numpy().reshape(nq, G).copy()
    nsel[:, 1] = 0
    nsel[1::2, :] = 0
    c["sel"], c["nsel"] = H.i32(sel.ravel()), H.i32(nsel.ravel())
    out = _run(c, True)
    assert np.all(out[1::2] == 0.0)
    assert np.all(out[:, 16:32] == 0.0)
    _oracle_check(seed, c, out, 1, what="merged empty lists")
