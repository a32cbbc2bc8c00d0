"""Paged caches (128-position pages under a block table) through the C ABI: every paged entry point
gives bit for bit what its contiguous counterpart gives on the same logical data, and the paged
results meet the oracle directly.  Pages are assigned in a random order inside pools that also hold
unused pages of random bytes, and block-table entries past a sequence's last page are -1."""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
import dsa_sparse_attention_amd as dsa
import oracle as O

import _harness as H

pytestmark = pytest.mark.gpu

G, P, HQ, D = H.G, H.P, H.HQ, H.D
PG = dsa.PAGE_POSITIONS


def _page_tables(lens, tcap, n_extra, seed):
    """Block table [B][tcap/128] with each sequence's used pages at random distinct ids of a pool of
    sum(used) + n_extra pages; entries past a sequence's last used page are -1."""
    B, npg = len(lens), tcap // PG
    used = [(L + PG - 1) // PG for L in lens]
    n_pages = sum(used) + n_extra
    rng = np.random.default_rng(seed)
    ids = rng.permutation(n_pages)
    bt = np.full((B, npg), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        bt[b, :used[b]] = ids[k:k + used[b]]
        k += used[b]
    return bt, n_pages


def _junk_pools(n_pages, seed, index_k=True):
    """Pools of n_pages pages filled with random bytes (finite bf16 / fp32 values are not needed:
    unused pages are never read)."""
    pools = dsa.paged_pools(n_pages, index_k=index_k)
    g = torch.Generator(device="cuda").manual_seed(seed)
    for t in pools.values():
        if t is not None:
            t.view(torch.uint8).copy_(torch.randint(0, 256, (t.numel() * t.element_size(),), dtype=torch.uint8,
                                                    device="cuda", generator=g))
    return pools


# contiguous tensor -> [B][pages][per-page elements] in the paged order (group inside page)
def _by_page(t, B, tcap, per_group_page):
    return t.view(B, G, tcap // PG, per_group_page).permute(0, 2, 1, 3)


def _scatter(pool, contig, bt, B, tcap, per_group_page):
    """Copies the used pages of a contiguous cache into the pool at the block table's ids."""
    src = _by_page(contig, B, tcap, per_group_page).reshape(B * (tcap // PG), G * per_group_page)
    ids = torch.tensor(bt.reshape(-1), dtype=torch.int64, device="cuda")
    used = ids >= 0
    pool.view(-1, G * per_group_page)[ids[used]] = src[used]


def _gather(pool, bt, B, tcap, per_group_page, dtype):
    """The logical contiguous cache (pages without an id left zero) read back from a pool."""
    ids = torch.tensor(bt.reshape(-1), dtype=torch.int64, device="cuda")
    used = ids >= 0
    out = torch.zeros(B * (tcap // PG), G * per_group_page, dtype=dtype, device="cuda")
    out[used] = pool.view(-1, G * per_group_page)[ids[used]]
    return out.view(B, tcap // PG, G, per_group_page).permute(0, 2, 1, 3).reshape(-1)


SIZES = {"k": 16 * 1536, "v": 16 * 1536, "ik": PG * P, "summ": 4096, "scale": 16}


def _to_pools(contig, lens, tcap, seed, n_extra=5):
    bt, n_pages = _page_tables(lens, tcap, n_extra, seed)
    pools = _junk_pools(n_pages, seed, index_k=contig.get("ik") is not None)
    B = len(lens)
    for name, t in contig.items():
        if t is not None:
            _scatter(pools[name], t, bt, B, tcap, SIZES[name])
    pages = dsa.Pages(torch.tensor(bt, device="cuda"), n_pages)
    return pools, pages, bt


@pytest.mark.parametrize("lens,topk", [
    ([5003, 1000, 17, 1], 512),     # ragged, partial current regions, p = 0
    ([131072, 70001, 9000], 512),   # tile-maxima selection (16,384-region capacity)
    ([3000, 2047, 4096], 37),
])
def test_paged_decode_matches_contiguous_and_oracle(lens, topk):
    seed = 0x9A0 + len(lens) + topk
    r = H.run_dsa_decode(seed, lens, topk=topk)
    dev, B, tcap, R = r["dev"], r["B"], r["tcap"], r["R"]
    geom = dev["geom"]
    pools, pages, bt = _to_pools(dict(k=dev["K"], v=dev["V"], summ=dev["summ"], scale=dev["scale"], ik=None),
                                 lens, tcap, seed)
    lens_np = np.asarray(lens, dtype=np.int32)
    sel = torch.empty(B * G * topk, dtype=torch.int32, device="cuda")
    nsel = torch.empty(B * G, dtype=torch.int32, device="cuda")
    scores = torch.full((B * G * R,), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_score_topk_paged(geom, dev["iq"], dev["z"], H.i32(np.arange(B)), H.i32(lens_np - 1), B, pages,
                             pools["summ"], pools["scale"], R, sel, nsel, scores_out=scores)
    out = torch.empty(B * HQ * D, dtype=H.BF16, device="cuda")
    dsa.dsa_sparse_gqa_decode_paged(geom, dev["q"], pages, pools["k"], pools["v"], H.i32(lens_np), sel, nsel, out)
    torch.cuda.synchronize()
    got = dict(sel=sel.cpu().numpy().reshape(B, G, topk), nsel=nsel.cpu().numpy().reshape(B, G),
               scores=scores.cpu().numpy().reshape(B, G, R), out=H.bf16_np(out).reshape(B, HQ, D))
    assert np.array_equal(got["nsel"], r["nsel"])
    for b in range(B):
        for g in range(G):
            n = r["nsel"][b, g]
            assert np.array_equal(got["sel"][b, g, :n], r["sel"][b, g, :n])
            c = (lens[b] - 1) // 8
            assert np.array_equal(got["scores"][b, g, :c].view(np.uint32), r["scores"][b, g, :c].view(np.uint32))
    assert np.array_equal(got["out"].view(np.uint16), r["out"].view(np.uint16))
    # and directly against the oracle
    rp = dict(r)
    rp.update(got)
    H.assert_decode_parity(rp)


def test_paged_cache_write_and_compress():
    """Token rows written into paged pools land where the contiguous layouts put them, and the
    summaries compressed from the pools are the contiguous ones (and the oracle's)."""
    seed = 0x9B0
    lens = [1000, 259, 8]
    B, tcap = len(lens), H.round128(max(lens))
    R = tcap // 8
    geom = dsa.geometry()
    rows = sum(lens)
    tok_seq = np.concatenate([np.full(L, b) for b, L in enumerate(lens)]).astype(np.int32)
    tok_pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int32)
    k_new = H.dev_flat_bf16(seed, gi.TID_K, rows * G * D)
    v_new = H.dev_flat_bf16(seed, gi.TID_V, rows * G * D)
    ik_new = H.dev_flat_bf16(seed, gi.TID_IK, rows * G * P, gi.IK_SCALE)
    kc = torch.zeros(B * G * tcap * D, dtype=H.BF16, device="cuda")
    vc, ikc = torch.zeros_like(kc), torch.zeros(B * G * tcap * P, dtype=H.BF16, device="cuda")
    dsa.dsa_cache_write(geom, H.i32(tok_seq), H.i32(tok_pos), k_new, v_new, ik_new, kc, vc, ikc, B, tcap)
    bt, n_pages = _page_tables(lens, tcap, 3, seed)
    pools = _junk_pools(n_pages, seed)
    pages = dsa.Pages(torch.tensor(bt, device="cuda"), n_pages)
    dsa.dsa_cache_write_paged(geom, H.i32(tok_seq), H.i32(tok_pos), k_new, v_new, ik_new, pages, B, pools["k"],
                              pools["v"], pools["ik"])
    # compression of every complete region, both ways
    summ = torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(B * G * R, dtype=torch.float32, device="cuda")
    ends = H.i32(np.asarray(lens) // 8)
    dsa.dsa_compress_regions(geom, ikc, tcap, H.i32(np.zeros(B)), ends, R, summ, scale)
    dsa.dsa_compress_regions_paged(geom, pages, pools["ik"], H.i32(np.zeros(B)), ends, R, pools["summ"],
                                   pools["scale"])
    torch.cuda.synchronize()

    def used(t, per):  # the contiguous tensor restricted to each sequence's used pages
        v = t.view(B, G, tcap // PG, per).clone()
        for b in range(B):
            v[b, :, (lens[b] + PG - 1) // PG:] = 0
        return v.reshape(-1)

    for name, contig, dt in (("k", kc, H.BF16), ("v", vc, H.BF16), ("ik", ikc, H.BF16),
                             ("summ", summ, torch.uint8), ("scale", scale, torch.float32)):
        back = _gather(pools[name], bt, B, tcap, SIZES[name], dt)
        ref = used(contig, SIZES[name])
        # the tail of a sequence's last page was never written in the pool (random bytes there) and
        # is zero in the contiguous cache: compare the written positions only
        bv, rv = back.view(B, G, tcap // PG, SIZES[name]), ref.view(B, G, tcap // PG, SIZES[name])
        for b, L in enumerate(lens):
            if name in ("k", "v", "ik"):
                per_tok = SIZES[name] // PG
                full = L // PG
                assert torch.equal(bv[b, :, :full].view(torch.uint8), rv[b, :, :full].view(torch.uint8)), name
                if L % PG:
                    a = bv[b, :, full].reshape(G, -1)
                    c = rv[b, :, full].reshape(G, -1)
                    if name == "ik":
                        assert torch.equal(a[:, :(L % PG) * per_tok].view(torch.uint8),
                                           c[:, :(L % PG) * per_tok].view(torch.uint8)), name
                    else:  # region-tiled: compare the complete regions and the written slots of the partial one
                        nreg = (L % PG) // 8
                        assert torch.equal(a[:, :nreg * 1536].view(torch.uint8), c[:, :nreg * 1536].view(torch.uint8))
            else:
                nreg = L // 8
                per_reg = SIZES[name] // 16
                s_b = bv[b].reshape(G, -1)
                s_r = rv[b].reshape(G, -1)
                if name == "scale":
                    assert torch.equal(s_b[:, :nreg].view(torch.int32), s_r[:, :nreg].view(torch.int32))
                else:
                    full = nreg // 16
                    assert torch.equal(s_b[:, :full * 4096], s_r[:, :full * 4096])
    # the summaries also meet the oracle
    sl = H.summ_logical(_gather(pools["summ"], bt, B, tcap, 4096, torch.uint8).cpu().numpy(), B, R)
    ikh_all = ik_new.view(torch.int16).cpu().numpy().view(np.uint16).reshape(rows, G, P)  # bf16 bits
    off = 0
    for b, L in enumerate(lens):
        codes, scales = O.compress_regions(ikh_all[off:off + L], 0, L // 8)
        off += L
        assert np.array_equal(sl[b, :, :L // 8], codes.transpose(1, 0, 2))


@pytest.mark.parametrize("lens", [[1 << 20] * 4, [131072, 70001, 9000, 8192, 17, 1],
                                  [8192, 1000, 4096, 17, 8, 1]])
def test_paged_decode_step_matches_contiguous(lens):
    """dsa_decode_step_paged (folded compression writing into the pools) gives bit for bit what
    dsa_decode_step gives on contiguous caches: selections, outputs and the new summaries."""
    seed = 0x9C0 + len(lens)
    B, tcap = len(lens), H.round128(max(lens))
    R = tcap // 8
    geom = dsa.geometry()
    ik = H.dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE, True)
    K = H.dev_cache(seed, gi.TID_K, B, tcap, D, tcap, gi.LAYOUT_KTILED)
    V = H.dev_cache(seed, gi.TID_V, B, tcap, D, tcap, gi.LAYOUT_REGION_T)
    q, iq, z = H.dev_queries(seed, B)
    lens_np = np.asarray(lens, dtype=np.int32)
    slen = H.i32(lens_np)
    summ = torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(B * G * R, dtype=torch.float32, device="cuda")
    dsa.dsa_compress_regions(geom, ik, tcap, H.i32(np.zeros(B)), H.i32((lens_np - 1) // 8), R, summ, scale)
    pools, pages, bt = _to_pools(dict(k=K, v=V, ik=ik, summ=summ, scale=scale), lens, tcap, seed)
    sel1 = torch.empty(B * G * 512, dtype=torch.int32, device="cuda")
    n1 = torch.empty(B * G, dtype=torch.int32, device="cuda")
    o1 = torch.empty(B * HQ * D, dtype=H.BF16, device="cuda")
    dsa.dsa_decode_step(geom, q, iq, z, ik, K, V, tcap, slen, summ, scale, R, sel1, n1, o1)
    sel2, n2, o2 = torch.empty_like(sel1), torch.empty_like(n1), torch.empty_like(o1)
    dsa.dsa_decode_step_paged(geom, q, iq, z, pages, pools["ik"], pools["k"], pools["v"], slen, pools["summ"],
                              pools["scale"], R, sel2, n2, o2)
    torch.cuda.synchronize()
    assert torch.equal(n1, n2) and torch.equal(sel1, sel2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    # the summaries: the prefix ones and the one the step wrote (region (L-1)/8 when L is a multiple
    # of 8); a tile's bytes are [64-channel quarter][16-channel piece][region][16], so region rr of a
    # tile is [:, :, rr, :] of its (4, 4, 16, 16) view
    back_s = _gather(pools["summ"], bt, B, tcap, 4096, torch.uint8).view(B, G, R // 16, 4, 4, 16, 16)
    back_c = _gather(pools["scale"], bt, B, tcap, 16, torch.float32).view(B, G, R)
    sv, cv = summ.view(B, G, R // 16, 4, 4, 16, 16), scale.view(B, G, R)
    for b, L in enumerate(lens):
        nr = (L - 1) // 8 + (1 if L % 8 == 0 else 0)  # regions with a summary after the step
        assert torch.equal(back_c[b, :, :nr].view(torch.int32), cv[b, :, :nr].view(torch.int32)), b
        ft = nr // 16
        assert torch.equal(back_s[b, :, :ft], sv[b, :, :ft]), b
        if nr % 16:
            assert torch.equal(back_s[b, :, ft, :, :, :nr % 16], sv[b, :, ft, :, :, :nr % 16]), b


def test_paged_prefill_matches_contiguous():
    """Prefill scoring, selection and attention over paged pools, mixed sequences in one call."""
    seed = 0x9D0
    seqs = [(4003, 300), (1000, 77), (130, 5)]
    B = len(seqs)
    tcap = H.round128(max(p0 + n for p0, n in seqs))
    R = tcap // 8
    geom = dsa.geometry()
    ik = H.dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE)
    K = H.dev_cache(seed, gi.TID_K, B, tcap, D, tcap, gi.LAYOUT_KTILED)
    V = H.dev_cache(seed, gi.TID_V, B, tcap, D, tcap, gi.LAYOUT_REGION_T)
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
    pools, pages, bt = _to_pools(dict(k=K, v=V, ik=None, summ=summ, scale=scale), [int(e) for e in end], tcap, seed)

    def run(paged):
        sel = torch.empty(nq * G * 512, dtype=torch.int32, device="cuda")
        nsel = torch.empty(nq * G, dtype=torch.int32, device="cuda")
        out = torch.empty(nq * HQ * D, dtype=H.BF16, device="cuda")
        if paged:
            dsa.dsa_score_topk_paged(geom, iq, z, H.i32(qs), H.i32(qp), B, pages, pools["summ"], pools["scale"], R,
                                     sel, nsel)
            dsa.dsa_sparse_gqa_prefill_paged(geom, q, H.i32(qs), H.i32(qp), B, pages, pools["k"], pools["v"], sel,
                                             nsel, out)
        else:
            dsa.dsa_score_topk(geom, iq, z, H.i32(qs), H.i32(qp), B, summ, scale, tcap, R, sel, nsel)
            dsa.dsa_sparse_gqa_prefill(geom, q, H.i32(qs), H.i32(qp), B, K, V, tcap, sel, nsel, out)
        torch.cuda.synchronize()
        return sel.cpu().numpy().reshape(nq, G, 512), nsel.cpu().numpy().reshape(nq, G), H.bf16_np(out)

    s1, n1, o1 = run(False)
    s2, n2, o2 = run(True)
    assert np.array_equal(n1, n2)
    live = np.arange(512)[None, None, :] < n1[:, :, None]
    assert np.array_equal(np.where(live, s1, -1), np.where(live, s2, -1))
    assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16))
    # a sample of queries against the oracle
    hq, hiq, hz = H.host_queries(seed, nq)
    go = o2.reshape(nq, HQ, D)
    for i in range(0, nq, 23):
        b, p = qs[i], qp[i]
        L = int(end[b])
        ikh = gi.host_index_k(seed, tcap, G, P, b, 0, L)
        codes, scales = O.compress_regions(ikh, 0, L // 8)
        Kh = gi.host_tokens_bf16(seed, gi.TID_K, tcap, G, D, b, 0, L)
        Vh = gi.host_tokens_bf16(seed, gi.TID_V, tcap, G, D, b, 0, L)
        osel, on, oout, osc = O.dsa_query(hiq[i], hz[i], codes, scales, hq[i], Kh, Vh, p, k=512, want_scores=True)
        for g in range(G):
            assert n2[i, g] == on[g]
            if H.check_selection(s2[i, g, :n2[i, g]], osel[g, :on[g]], osc[g], p // 8):
                H.assert_attn(go[i, 16 * g:16 * g + 16], oout[16 * g:16 * g + 16], f"query {i} group {g}")
