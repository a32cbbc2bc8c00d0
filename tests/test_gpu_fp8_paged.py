"""FP8 K/V caches in pages: every paged FP8 entry point gives bit for bit what its contiguous FP8
counterpart gives on the same logical data (the contiguous FP8 calls meet the oracle in
test_gpu_fp8.py).  Pages sit at random ids of pools whose unused pages hold random bytes; block-table
entries past a sequence's last page are -1."""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
import dsa_sparse_attention_amd as dsa

import _harness as H
import test_gpu_fp8 as F
import test_gpu_paged as TP

pytestmark = pytest.mark.gpu

G, P, HQ, D = H.G, H.P, H.HQ, H.D
PG = dsa.PAGE_POSITIONS
# per (page, group) elements of each pool
PER = {"k8": 16 * 1536, "v8": 16 * 1536, "kvs": 16 * 16, "ik": PG * P, "summ": 4096, "scale": 16}


def _junk(t, gen):
    t.view(torch.uint8).copy_(torch.randint(0, 256, (t.numel() * t.element_size(),), dtype=torch.uint8,
                                            device="cuda", generator=gen))
    return t


def _fp8_pools(contig, lens, tcap, seed, n_extra=5):
    """Paged pools holding the used pages of the contiguous caches in `contig` (names of PER)."""
    bt, n_pages = TP._page_tables(lens, tcap, n_extra, seed)
    gen = torch.Generator(device="cuda").manual_seed(seed)
    k8, v8, kvs = dsa.fp8_pools(n_pages)
    pools = {"k8": k8, "v8": v8, "kvs": kvs,
             "ik": torch.empty(n_pages * G * PER["ik"], dtype=H.BF16, device="cuda"),
             "summ": torch.empty(n_pages * G * PER["summ"], dtype=torch.uint8, device="cuda"),
             "scale": torch.empty(n_pages * G * PER["scale"], dtype=torch.float32, device="cuda")}
    pools = {n: _junk(t, gen) for n, t in pools.items() if n in contig}
    B = len(lens)
    for name, t in contig.items():
        TP._scatter(pools[name], t, bt, B, tcap, PER[name])
    return pools, dsa.Pages(torch.tensor(bt, device="cuda"), n_pages), bt


def test_fp8_paged_cache_write_matches_contiguous():
    seed, lens = 0xFC0, [1000, 259, 8, 130]
    B, tcap = len(lens), 1024
    geom = dsa.geometry()
    rows = sum(lens)
    tok_seq = np.concatenate([np.full(L, b) for b, L in enumerate(lens)]).astype(np.int32)
    tok_pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int32)
    k_new = H.dev_flat_bf16(seed, gi.TID_K, rows * G * D)
    v_new = H.dev_flat_bf16(seed, gi.TID_V, rows * G * D)
    k8, v8, kvs = dsa.fp8_caches(B, tcap)
    dsa.dsa_cache_write_fp8(geom, H.i32(tok_seq), H.i32(tok_pos), k_new, v_new, k8, v8, kvs, B, tcap)
    bt, n_pages = TP._page_tables(lens, tcap, 3, seed)
    gen = torch.Generator(device="cuda").manual_seed(seed)
    pk8, pv8, pkvs = (_junk(t, gen) for t in dsa.fp8_pools(n_pages))
    pages = dsa.Pages(torch.tensor(bt, device="cuda"), n_pages)
    dsa.dsa_cache_write_fp8_paged(geom, H.i32(tok_seq), H.i32(tok_pos), k_new, v_new, pages, B, pk8, pv8, pkvs)
    torch.cuda.synchronize()
    bk8 = TP._gather(pk8, bt, B, tcap, PER["k8"], torch.uint8)
    bv8 = TP._gather(pv8, bt, B, tcap, PER["v8"], torch.uint8)
    bkvs = TP._gather(pkvs, bt, B, tcap, PER["kvs"], torch.float32)
    for b, L in enumerate(lens):  # the written positions only (the rest of a last page is junk)
        got = F._logical(bk8, bv8, bkvs, B, tcap, b, L)
        ref = F._logical(k8, v8, kvs, B, tcap, b, L)
        for x, y in zip(got, ref):
            x, y = np.ascontiguousarray(x), np.ascontiguousarray(y)
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), b


@pytest.mark.parametrize("lens,topk", [([5003, 1000, 17, 1], 512), ([131072, 70001, 9000], 512),
                                       ([3000, 2047, 4096], 37)])
def test_fp8_paged_decode_matches_contiguous(lens, topk):
    seed = 0xFD0 + len(lens) + topk
    r = H.run_dsa_decode(seed, lens, topk=topk, check_seqs=[])
    B, tcap = r["B"], r["tcap"]
    k8, v8, kvs = F._write_fp8(seed, B, tcap)
    pools, pages, _ = _fp8_pools(dict(k8=k8, v8=v8, kvs=kvs), lens, tcap, seed)
    geom, q = r["dev"]["geom"], r["dev"]["q"]
    sel, nsel, slen = H.i32(r["sel"].ravel()), H.i32(r["nsel"].ravel()), H.i32(lens)
    o1 = torch.empty(B * HQ * D, dtype=H.BF16, device="cuda")
    o2 = torch.empty_like(o1)
    dsa.dsa_sparse_gqa_decode_fp8(geom, q, k8, v8, kvs, tcap, slen, sel, nsel, o1)
    dsa.dsa_sparse_gqa_decode_fp8_paged(geom, q, pages, pools["k8"], pools["v8"], pools["kvs"], slen, sel, nsel, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("lens", [[1 << 20] * 4, [131072, 70001, 9000, 8192, 17, 1]])
def test_fp8_paged_decode_step_matches_contiguous(lens):
    """Selections, outputs and the summaries the step writes, paged FP8 vs contiguous FP8."""
    seed = 0xFE0 + len(lens)
    B, tcap = len(lens), H.round128(max(lens))
    R = tcap // 8
    geom = dsa.geometry()
    ik = H.dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE, True)
    q, iq, z = H.dev_queries(seed, B)
    lens_np = np.asarray(lens, dtype=np.int32)
    slen = H.i32(lens_np)
    summ = torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(B * G * R, dtype=torch.float32, device="cuda")
    dsa.dsa_compress_regions(geom, ik, tcap, H.i32(np.zeros(B)), H.i32((lens_np - 1) // 8), R, summ, scale)
    k8, v8, kvs = F._write_fp8(seed, B, tcap)
    pools, pages, bt = _fp8_pools(dict(k8=k8, v8=v8, kvs=kvs, ik=ik, summ=summ, scale=scale), lens, tcap, seed)
    sel1 = torch.empty(B * G * 512, dtype=torch.int32, device="cuda")
    n1 = torch.empty(B * G, dtype=torch.int32, device="cuda")
    o1 = torch.empty(B * HQ * D, dtype=H.BF16, device="cuda")
    dsa.dsa_decode_step_fp8(geom, q, iq, z, ik, k8, v8, kvs, tcap, slen, summ, scale, R, sel1, n1, o1)
    sel2, n2, o2 = torch.empty_like(sel1), torch.empty_like(n1), torch.empty_like(o1)
    dsa.dsa_decode_step_fp8_paged(geom, q, iq, z, pages, pools["ik"], pools["k8"], pools["v8"], pools["kvs"], slen,
                                  pools["summ"], pools["scale"], R, sel2, n2, o2)
    torch.cuda.synchronize()
    assert torch.equal(n1, n2) and torch.equal(sel1, sel2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    back_s = TP._gather(pools["summ"], bt, B, tcap, 4096, torch.uint8).view(B, G, R // 16, 4, 4, 16, 16)
    back_c = TP._gather(pools["scale"], bt, B, tcap, 16, torch.float32).view(B, G, R)
    sv, cv = summ.view(B, G, R // 16, 4, 4, 16, 16), scale.view(B, G, R)
    for b, L in enumerate(lens):
        nr = (L - 1) // 8 + (1 if L % 8 == 0 else 0)  # regions with a summary after the step
        assert torch.equal(back_c[b, :, :nr].view(torch.int32), cv[b, :, :nr].view(torch.int32)), b
        ft = nr // 16
        assert torch.equal(back_s[b, :, :ft], sv[b, :, :ft]), b
        if nr % 16:
            assert torch.equal(back_s[b, :, ft, :, :, :nr % 16], sv[b, :, ft, :, :, :nr % 16]), b


def test_fp8_paged_prefill_matches_contiguous():
    seed, seqs = 0xFF0, [(4003, 300), (1000, 77), (130, 5)]
    B = len(seqs)
    tcap = H.round128(max(p0 + n for p0, n in seqs))
    R = tcap // 8
    geom = dsa.geometry()
    ik = H.dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE)
    summ = torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(B * G * R, dtype=torch.float32, device="cuda")
    end = np.array([p0 + n for p0, n in seqs], dtype=np.int32)
    dsa.dsa_compress_regions(geom, ik, tcap, H.i32(np.zeros(B)), H.i32(end // 8), R, summ, scale)
    qs, qp = [], []
    for i in range(max(n for _, n in seqs)):
        for b, (s0, n) in enumerate(seqs):
            if i < n:
                qs.append(b)
                qp.append(s0 + i)
    nq = len(qs)
    q, iq, z = H.dev_queries(seed, nq)
    sel = torch.empty(nq * G * 512, dtype=torch.int32, device="cuda")
    nsel = torch.empty(nq * G, dtype=torch.int32, device="cuda")
    dsa.dsa_score_topk(geom, iq, z, H.i32(qs), H.i32(qp), B, summ, scale, tcap, R, sel, nsel)
    k8, v8, kvs = F._write_fp8(seed, B, tcap)
    pools, pages, _ = _fp8_pools(dict(k8=k8, v8=v8, kvs=kvs), [int(e) for e in end], tcap, seed)
    o1 = torch.empty(nq * HQ * D, dtype=H.BF16, device="cuda")
    o2 = torch.empty_like(o1)
    dsa.dsa_sparse_gqa_prefill_fp8(geom, q, H.i32(qs), H.i32(qp), B, k8, v8, kvs, tcap, sel, nsel, o1)
    dsa.dsa_sparse_gqa_prefill_fp8_paged(geom, q, H.i32(qs), H.i32(qp), B, pages, pools["k8"], pools["v8"],
                                         pools["kvs"], sel, nsel, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
