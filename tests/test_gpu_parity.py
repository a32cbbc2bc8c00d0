"""GPU vs oracle parity through the C ABI, at sizes the oracle finishes in seconds (several tiles,
ragged tails, partial regions, short contexts, small top-k), plus determinism."""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
import dsa_sparse_attention_amd as dsa
import oracle as O

import _harness as H

pytestmark = pytest.mark.gpu

G, P, HQ, D = H.G, H.P, H.HQ, H.D


def test_compress_bit_exact_in_two_calls():
    seed = 0xC0
    lens = [8192, 1003, 64, 7]
    B, tcap = len(lens), 8192
    R = tcap // 8
    geom = dsa.geometry()
    ik = H.dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE)
    summ = torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(B * G * R, dtype=torch.float32, device="cuda")
    ends = np.array([L // 8 for L in lens], dtype=np.int32)
    mids = ends // 2
    dsa.dsa_compress_regions(geom, ik, tcap, H.i32(np.zeros(B)), H.i32(mids), R, summ, scale)
    dsa.dsa_compress_regions(geom, ik, tcap, H.i32(mids), H.i32(ends), R, summ, scale)
    torch.cuda.synchronize()
    s = H.summ_logical(summ.cpu().numpy(), B, R)
    sc = scale.cpu().numpy().reshape(B, G, R)
    for b, L in enumerate(lens):
        nr = L // 8
        ikh = gi.host_index_k(seed, tcap, G, P, b, 0, L)
        codes, scales = O.compress_regions(ikh, 0, nr)
        assert np.array_equal(s[b, :, :nr], codes[:nr].transpose(1, 0, 2))
        assert np.array_equal(sc[b, :, :nr].view(np.uint32), scales[:nr].T.copy().view(np.uint32))
        assert not s[b, :, nr:].any() and not sc[b, :, nr:].any()  # partial tail held back


def test_compress_planted_bit_exact():
    r = H.run_dsa_decode(0xC1, [4096, 4096], topk=64, planted=True)
    H.assert_decode_parity(r)


@pytest.mark.parametrize("lens,topk", [
    ([8192], 512),                     # the 8K single-query decode workload
    ([5003, 1000, 17, 1], 512),        # ragged: partial current regions, short contexts, p = 0
    ([3000, 2047, 4096], 37),          # odd top-k (splits partially filled)
    ([600, 4104], 1),                  # top-1: only the current region
])
def test_decode_end_to_end(lens, topk):
    r = H.run_dsa_decode(0xD0 + len(lens) + topk, lens, topk=topk)
    H.assert_decode_parity(r)


@pytest.mark.parametrize("lens", [
    [40000, 9000],   # <= 8192 regions: every key ranked in registers
    [70000, 9000],   # > 8192 regions: every tile maximum ties, the lowest 511 tiles are kept
])
def test_decode_all_equal_scores_take_the_lowest_regions(lens):
    """Every score is 0 (z = 0): ties go to the lowest regions."""
    r = H.run_dsa_decode(0xDE, lens, topk=512, zero_z=True)
    H.assert_decode_parity(r)
    for b, L in enumerate(lens):
        c = (L - 1) // 8
        for g in range(G):
            assert r["sel"][b, g, :512].tolist() == list(range(511)) + [c]


def test_decode_long_contexts_select_through_tile_maxima():
    """16,384-region capacity: the best 511 tiles by their maxima, then exact ranking inside them
    (and every tile kept for the 9,000-token sequence)."""
    r = H.run_dsa_decode(0xD7, [131072, 70001, 9000], topk=512, planted=True)
    H.assert_decode_parity(r)


def test_decode_1m_context_batch_of_4():
    """The 1,048,576-token batch-4 decode shape with the planted bias, in the launch configuration
    the benchmark times (8,192 tiles per problem: the tile selection at full capacity); sequences 0
    and 3 are checked against the oracle."""
    r = H.run_dsa_decode(0xD8, [1 << 20] * 4, topk=512, planted=True, check_seqs=[0, 3])
    H.assert_decode_parity(r)


def test_decode_128k_context_batch_of_16():
    """The 131,072-token batch-16 decode shape (16,384 regions per sequence, 1,024 tiles per problem)
    in the launch configuration the benchmark times; sequences 0, 7 and 15 are checked against the
    oracle."""
    r = H.run_dsa_decode(0xDC, [131072] * 16, topk=512, check_seqs=[0, 7, 15])
    H.assert_decode_parity(r)


def test_decode_crowded_boundary_digit():
    """A selection whose boundary bin of the 12-bit score key is crowded: more than 1,024 regions score
    at or above the bin of the 511th best (1,057 for sequence 1, group 2 of this input: the 1M
    batch-4 workload, planted bias, with queries 20..23).  The selection still takes its fast path
    (up to 2,048 candidates) and matches the oracle."""
    seed = gi.SEED_BASE + 3
    r = H.run_dsa_decode(seed, [1 << 20] * 4, topk=512, planted=True, check_seqs=[1], q_start=20)
    H.assert_decode_parity(r)


def test_decode_layer_mix_shape_batch_8_at_256k():
    """The DSA layer of the 3:1 layer-mix workload as the benchmark times it: batch 8 at 262,144
    tokens (2,048 tiles per problem); sequences 0 and 7 are checked against the oracle."""
    r = H.run_dsa_decode(0xDA, [262144] * 8, topk=512, check_seqs=[0, 7])
    H.assert_decode_parity(r)


def test_decode_beyond_tile_capacity_uses_radix_fallback():
    """More than 8,192 tiles of 16 regions (a context just over 1M tokens): exact selection by radix
    narrowing over the scores in global memory."""
    r = H.run_dsa_decode(0xD9, [(1 << 20) + 72], topk=512, planted=True)
    H.assert_decode_parity(r)


def test_decode_selection_does_not_depend_on_workspace_contents():
    """The decode selection reads only what the score kernel of the same call wrote into the
    workspace (scores and tile maxima): a workspace full of random bytes gives the same selection as
    a zeroed one, on the first call and on the next call over the same bytes."""
    seed, lens = 0xDA, [131072, 100003, 70001]
    B, tcap = len(lens), H.round128(max(lens))
    R = tcap // 8
    geom = dsa.geometry()
    ik = H.dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE, True)
    _, iq, z = H.dev_queries(seed, B)
    summ = torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(B * G * R, dtype=torch.float32, device="cuda")
    lens_np = np.asarray(lens, dtype=np.int32)
    dsa.dsa_compress_regions(geom, ik, tcap, H.i32(np.zeros(B)), H.i32(lens_np // 8), R, summ, scale)
    qseq, qpos = H.i32(np.arange(B)), H.i32(lens_np - 1)
    nbytes = dsa.dsa_score_topk_workspace_size(geom, B, R)

    def run(ws):
        sel = torch.empty(B * G * 512, dtype=torch.int32, device="cuda")
        nsel = torch.empty(B * G, dtype=torch.int32, device="cuda")
        dsa.dsa_score_topk(geom, iq, z, qseq, qpos, B, summ, scale, tcap, R, sel, nsel, workspace=ws)
        torch.cuda.synchronize()
        return sel.cpu().numpy(), nsel.cpu().numpy()

    ref_sel, ref_n = run(dsa.workspace(nbytes))
    junk = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        sel, n = run(junk)
        assert np.array_equal(n, ref_n)
        assert np.array_equal(sel, ref_sel)


@pytest.mark.parametrize("lens", [[1 << 20] * 4, [131072, 70001, 9000, 8192, 17, 1],
                                  [8192, 1000, 4096, 17, 8, 1]])
def test_decode_step_matches_the_separate_calls(lens):
    """dsa_decode_step, whose compression of the completed region runs inside the selection launch,
    gives bit for bit what dsa_compress_regions + dsa_score_topk + dsa_sparse_gqa_decode give,
    summaries included (only the region a query token completes is written).  The last case (1,024
    regions of capacity: the short-context scoring and the register selection, which holds the folded
    compression blocks) has tokens completing regions 8191 // 8, 999 // 8, 4095 // 8 and 7 // 8."""
    seed = 0xDB + len(lens)
    B, tcap = len(lens), H.round128(max(lens))
    R = tcap // 8
    geom = dsa.geometry()
    ik = H.dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE, True)
    K = H.dev_cache(seed, gi.TID_K, B, tcap, D, tcap, gi.LAYOUT_KTILED)
    V = H.dev_cache(seed, gi.TID_V, B, tcap, D, tcap, gi.LAYOUT_REGION_T)
    q, iq, z = H.dev_queries(seed, B)
    lens_np = np.asarray(lens, dtype=np.int32)
    slen = H.i32(lens_np)

    def prefix_summaries():
        summ = torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda")
        scale = torch.zeros(B * G * R, dtype=torch.float32, device="cuda")
        dsa.dsa_compress_regions(geom, ik, tcap, H.i32(np.zeros(B)), H.i32((lens_np - 1) // 8), R, summ, scale)
        return summ, scale

    def outputs():
        return (torch.empty(B * G * 512, dtype=torch.int32, device="cuda"),
                torch.empty(B * G, dtype=torch.int32, device="cuda"),
                torch.empty(B * HQ * D, dtype=torch.bfloat16, device="cuda"))

    s1, c1 = prefix_summaries()
    sel1, n1, o1 = outputs()
    dsa.dsa_compress_regions(geom, ik, tcap, H.i32((lens_np - 1) // 8), H.i32(lens_np // 8), 1, s1, c1)
    dsa.dsa_score_topk(geom, iq, z, H.i32(np.arange(B)), H.i32(lens_np - 1), B, s1, c1, tcap, R, sel1, n1)
    dsa.dsa_sparse_gqa_decode(geom, q, K, V, tcap, slen, sel1, n1, o1)
    s2, c2 = prefix_summaries()
    sel2, n2, o2 = outputs()
    dsa.dsa_decode_step(geom, q, iq, z, ik, K, V, tcap, slen, s2, c2, R, sel2, n2, o2)
    torch.cuda.synchronize()
    assert torch.equal(n1, n2) and torch.equal(sel1, sel2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(s1, s2) and torch.equal(c1.view(torch.int32), c2.view(torch.int32))


def test_decode_step_in_a_partial_region_with_tight_max_regions():
    """Queries in a partial region (seq_len not a multiple of 8) with max_regions = max(seq_len // 8),
    the documented bound: the current region seq_len // 8 is still selected and attended, and the
    result equals a call with a generous max_regions bit for bit and the oracle within tolerance."""
    seed = 0xDF
    lens = [8195, 1003, 4099, 13]
    B, tcap = len(lens), H.round128(max(lens))
    R = tcap // 8
    tight = max(L // 8 for L in lens)
    assert tight < R
    geom = dsa.geometry()
    ik = H.dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE)
    K = H.dev_cache(seed, gi.TID_K, B, tcap, D, tcap, gi.LAYOUT_KTILED)
    V = H.dev_cache(seed, gi.TID_V, B, tcap, D, tcap, gi.LAYOUT_REGION_T)
    q, iq, z = H.dev_queries(seed, B)
    lens_np = np.asarray(lens, dtype=np.int32)
    res = []
    for mr in (tight, R):
        summ = torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda")
        scale = torch.zeros(B * G * R, dtype=torch.float32, device="cuda")
        dsa.dsa_compress_regions(geom, ik, tcap, H.i32(np.zeros(B)), H.i32(lens_np // 8), R, summ, scale)
        sel = torch.empty(B * G * 512, dtype=torch.int32, device="cuda")
        nsel = torch.empty(B * G, dtype=torch.int32, device="cuda")
        out = torch.empty(B * HQ * D, dtype=H.BF16, device="cuda")
        dsa.dsa_decode_step(geom, q, iq, z, ik, K, V, tcap, H.i32(lens_np), summ, scale, mr, sel, nsel, out)
        res.append((sel, nsel, out))
    torch.cuda.synchronize()
    (s1, n1, o1), (s2, n2, o2) = res
    assert torch.equal(n1, n2) and torch.equal(s1, s2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    gsel = s1.cpu().numpy().reshape(B, G, 512)
    gn = n1.cpu().numpy().reshape(B, G)
    go = H.bf16_np(o1).reshape(B, HQ, D)
    hq, hiq, hz = H.host_queries(seed, B)
    for b in (0, 1):
        L = lens[b]
        c = (L - 1) // 8
        for g in range(G):
            assert c in gsel[b, g, :gn[b, g]].tolist(), "current region not selected"
        ikh = gi.host_index_k(seed, tcap, G, P, b, 0, L)
        Kh = gi.host_tokens_bf16(seed, gi.TID_K, tcap, G, D, b, 0, L)
        Vh = gi.host_tokens_bf16(seed, gi.TID_V, tcap, G, D, b, 0, L)
        codes, scales = O.compress_regions(ikh, 0, L // 8)
        ref = O.attend(hq[b], Kh, Vh, L - 1, [gsel[b, g, :gn[b, g]] for g in range(G)])
        H.assert_attn(go[b], ref, f"seq {b}")
        osel, on, _, _ = O.dsa_query(hiq[b], hz[b], codes, scales, hq[b], Kh, Vh, L - 1)
        assert np.array_equal(on, gn[b])


def test_decode_attention_on_oracle_selection():
    """Sparse GQA alone: the oracle's selection is fed to the GPU kernel, every head compared."""
    seed = 0xD7
    lens = [4096, 1001, 9]
    r = H.run_dsa_decode(seed, lens, topk=512)
    B, tcap, topk = len(lens), r["tcap"], 512
    sel = np.full((B, G, topk), -1, dtype=np.int32)
    nsel = np.zeros((B, G), dtype=np.int32)
    for b in range(B):
        sel[b] = r["oracle"][b]["sel"]
        nsel[b] = r["oracle"][b]["nsel"]
    out = torch.empty(B * HQ * D, dtype=H.BF16, device="cuda")
    dsa.dsa_sparse_gqa_decode(r["dev"]["geom"], r["dev"]["q"], r["dev"]["K"], r["dev"]["V"], tcap,
                              H.i32(lens), H.i32(sel.ravel()), H.i32(nsel.ravel()), out)
    go = H.bf16_np(out).reshape(B, HQ, D)
    for b in range(B):
        H.assert_attn(go[b], r["oracle"][b]["out"], f"seq {b}")


def _prefill(seed, seqs, topk=512, check_every=1, zero_z=False):
    """seqs: list of (P0, n) -- each sequence has a prefix of P0 tokens and a chunk of n new queries.
    Queries of all sequences are interleaved to exercise mixed-sequence query blocks when len(seqs)>1."""
    B = len(seqs)
    tcap = H.round128(max(p0 + n for p0, n in seqs))
    R = tcap // 8
    geom = dsa.geometry(topk=topk)
    ik = H.dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE)
    K = H.dev_cache(seed, gi.TID_K, B, tcap, D, tcap, gi.LAYOUT_KTILED)
    V = H.dev_cache(seed, gi.TID_V, B, tcap, D, tcap, gi.LAYOUT_REGION_T)
    summ = torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(B * G * R, dtype=torch.float32, device="cuda")
    p0 = np.array([s[0] for s in seqs], dtype=np.int32)
    end = np.array([s[0] + s[1] for s in seqs], dtype=np.int32)
    dsa.dsa_compress_regions(geom, ik, tcap, H.i32(np.zeros(B)), H.i32(p0 // 8), R, summ, scale)  # prefix
    dsa.dsa_compress_regions(geom, ik, tcap, H.i32(p0 // 8), H.i32(end // 8), R, summ, scale)  # in-chunk
    qs, qp = [], []
    for i in range(max(n for _, n in seqs)):
        for b, (s0, n) in enumerate(seqs):
            if i < n:
                qs.append(b)
                qp.append(s0 + i)
    nq = len(qs)
    q, iq, z = H.dev_queries(seed, nq)
    if zero_z:  # every score 0: selection falls to the lowest regions (tie rule)
        z.zero_()
    sel = torch.empty(nq * G * topk, dtype=torch.int32, device="cuda")
    nsel = torch.empty(nq * G, dtype=torch.int32, device="cuda")
    scores = torch.full((nq * G * R,), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_score_topk(geom, iq, z, H.i32(qs), H.i32(qp), B, summ, scale, tcap, R, sel, nsel, scores_out=scores)
    # the same call without the caller's score array takes the other scoring variant
    sel_b = torch.empty_like(sel)
    nsel_b = torch.empty_like(nsel)
    dsa.dsa_score_topk(geom, iq, z, H.i32(qs), H.i32(qp), B, summ, scale, tcap, R, sel_b, nsel_b)
    na, nb = nsel.cpu().numpy(), nsel_b.cpu().numpy()
    assert np.array_equal(na, nb)
    sa, sb = sel.cpu().numpy().reshape(-1, topk), sel_b.cpu().numpy().reshape(-1, topk)
    live = np.arange(topk)[None, :] < na[:, None]
    assert np.array_equal(np.where(live, sa, -1), np.where(live, sb, -1))
    out = torch.empty(nq * HQ * D, dtype=H.BF16, device="cuda")
    dsa.dsa_sparse_gqa_prefill(geom, q, H.i32(qs), H.i32(qp), B, K, V, tcap, sel, nsel, out)
    torch.cuda.synchronize()
    gsel = sel.cpu().numpy().reshape(nq, G, topk)
    gnsel = nsel.cpu().numpy().reshape(nq, G)
    gsc = scores.cpu().numpy().reshape(nq, G, R)
    gout = H.bf16_np(out).reshape(nq, HQ, D)
    hq, hiq, hz = H.host_queries(seed, nq)
    if zero_z:
        hz = np.zeros_like(hz)
    host = {}
    for b, (s0, n) in enumerate(seqs):
        L = s0 + n
        ikh = gi.host_index_k(seed, tcap, G, P, b, 0, L)
        host[b] = (O.compress_regions(ikh, 0, L // 8), gi.host_tokens_bf16(seed, gi.TID_K, tcap, G, D, b, 0, L),
                   gi.host_tokens_bf16(seed, gi.TID_V, tcap, G, D, b, 0, L))
    n_same = n_tot = 0
    worst = []
    osels = np.full((nq, G, topk), -1, dtype=np.int32)
    onsel = np.zeros((nq, G), dtype=np.int32)
    for i in range(0, nq, check_every):
        b, p = qs[i], qp[i]
        (codes, scales), Kh, Vh = host[b]
        osel, on, oout, osc = O.dsa_query(hiq[i], hz[i], codes, scales, hq[i], Kh, Vh, p, k=topk, want_scores=True)
        osels[i], onsel[i] = osel, on
        c = p // 8
        differ = []
        for g in range(G):
            if c:
                tol = 2e-5 * max(np.abs(osc[g]).max(), 1e-30)
                assert np.all(np.abs(gsc[i, g, :c] - osc[g]) <= tol), f"query {i} group {g}: scores"
            assert gnsel[i, g] == on[g]
            same = H.check_selection(gsel[i, g, :gnsel[i, g]], osel[g, :on[g]], osc[g], c)
            n_tot += 1
            if same:
                n_same += 1
                worst.append(H.assert_attn(gout[i, 16 * g:16 * g + 16], oout[16 * g:16 * g + 16],
                                           f"query {i} group {g}"))
            else:
                differ.append(g)
        if differ:  # selections differing inside the band: the oracle's attention on the GPU's selection
            ref = O.attend(hq[i], Kh, Vh, p, [gsel[i, g, :gnsel[i, g]] for g in range(G)], k=topk)
            for g in differ:
                worst.append(H.assert_attn(gout[i, 16 * g:16 * g + 16], ref[16 * g:16 * g + 16],
                                           f"query {i} group {g} (on the GPU's selection)"))
    assert n_same >= 0.9 * n_tot, (n_same, n_tot)
    print(f"prefill parity: {n_tot} (query, group) outputs checked, {n_tot - n_same} of them on the GPU's own "
          f"selection (differs from the oracle's inside the band)")
    # attention alone on the oracle's selection, every head
    out2 = torch.empty(nq * HQ * D, dtype=H.BF16, device="cuda")
    checked = list(range(0, nq, check_every))
    dsa.dsa_sparse_gqa_prefill(geom, q, H.i32(qs), H.i32(qp), B, K, V, tcap, H.i32(osels.ravel()),
                               H.i32(onsel.ravel()), out2)
    g2 = H.bf16_np(out2).reshape(nq, HQ, D)
    for i in checked:
        b, p = qs[i], qp[i]
        (codes, scales), Kh, Vh = host[b]
        ref = O.attend(hq[i], Kh, Vh, p, [osels[i, g, :onsel[i, g]] for g in range(G)], k=topk)
        worst.append(H.assert_attn(g2[i], ref, f"query {i} on oracle selection"))
    if worst:
        print(f"attention error: worst max abs {max(w[0] for w in worst):.3e}, "
              f"worst rel rms {max(w[1] for w in worst):.3e} over {len(worst)} checks")
    return gsel, gnsel, qp


def test_prefill_chunk_one_sequence():
    # prefix of 4003 tokens (partial region), 300 new queries: several 16-query blocks + a ragged one
    _prefill(0xE0, [(4003, 300)], check_every=7)


def test_prefill_64k_chunk_sampled():
    # the 64K prefill workload as timed: 2048 queries after a 63,488-token prefix; every 64th query
    # is checked against the oracle
    _prefill(0xE5, [(63488, 2048)], topk=512, check_every=64)


def test_prefill_64k_chunk_with_held_back_tail_sampled():
    """The 64K prefill at its hold-back shape: a 63,485-token prefix (its last region partial, so not
    yet summarised) and 2,051 new tokens; the chunk completes that region and 256 more, which are
    summarised in the chunk, and queries in the partial region attend it under the causal mask.
    Every 64th query is checked against the oracle."""
    _prefill(0xE7, [(63485, 2051)], topk=512, check_every=64)


@pytest.mark.parametrize("seqs", [
    [(8000, 80)],    # ~1000 candidates, all in one digit: finished in LDS
    [(40000, 80)],   # ~5000 candidates, all in one digit: bisection on the keys in registers
])
def test_prefill_all_equal_scores_take_the_lowest_regions(seqs):
    gsel, gnsel, qp = _prefill(0xE6, seqs, topk=512, check_every=5, zero_z=True)
    for i, p in enumerate(qp):
        c = p // 8
        for g in range(G):
            want = list(range(c + 1)) if c < 512 else list(range(511)) + [c]
            assert gsel[i, g, :gnsel[i, g]].tolist() == want


def test_prefill_mixed_sequences_and_small_topk():
    _prefill(0xE1, [(2000, 40), (511, 37), (8, 20)], topk=100, check_every=3)


def test_prefill_beyond_8192_regions():
    # ~8,750 candidate regions per query: selection through the tile maxima
    _prefill(0xE3, [(69997, 70)], topk=512, check_every=7)


def test_prefill_beyond_32768_regions():
    # ~33,800 candidate regions per query: 2,110 tiles ranked by their maxima
    _prefill(0xE4, [(270001, 64)], topk=512, check_every=16)


def test_prefill_short_chunk_uses_decode_tiling():
    _prefill(0xE2, [(1200, 20)], topk=512)


@pytest.mark.parametrize("chunks", [[530, 40, 1], [1, 1, 1, 600], [700, 513, 3]])
def test_swa_chunks_and_decode(chunks):
    H.check_swa_sequence(0xF0 + sum(chunks), chunks, check_from=0, sample=48)


def test_swa_prefill_chunk_at_64k_sampled():
    """The sliding-window prefill workload as the benchmark times it: a 2048-token chunk after
    63,488 tokens (the prefix itself is run as one chunk first to fill the ring); 24 sampled
    queries of the timed chunk are checked."""
    worst = H.check_swa_sequence(0xF8, [63488, 2048], check_from=1, sample=24)
    print(f"swa 64K chunk: worst max abs {worst[0]:.3e}, rel rms {worst[1]:.3e}")


def _swa_decode_inputs(seed, pos, layer):
    """Rings of len(pos) sequences holding positions p-512..p-1 (generator-written, NaN elsewhere),
    and one new token per sequence at p: q (row s), k_new, v_new."""
    S = len(pos)
    T = max(pos) + 1
    tq, tk, tv = H.swa_tids(layer)
    per = G * H.W * D
    k_ring = torch.full((S * per,), float("nan"), dtype=H.BF16, device="cuda")
    v_ring = torch.full((S * per,), float("nan"), dtype=H.BF16, device="cuda")
    for s, p in enumerate(pos):
        t0 = max(0, p - H.W)
        if p > t0:
            for layout, ring, tid in ((gi.LAYOUT_KTILED, k_ring, tk), (gi.LAYOUT_REGION_T, v_ring, tv)):
                tmp = torch.empty((s + 1) * per, dtype=H.BF16, device="cuda")
                gi.dev_tokens(tmp.data_ptr(), H.stream_ptr(), seed, tid, s + 1, T, G, D, t0, p - t0, H.W, H.W,
                              layout, 1.0)
                ring[s * per:(s + 1) * per] = tmp[s * per:(s + 1) * per]
    q = torch.empty(S * HQ * D, dtype=H.BF16, device="cuda")
    kn = torch.empty(S * G * D, dtype=H.BF16, device="cuda")
    vn = torch.empty(S * G * D, dtype=H.BF16, device="cuda")
    for s, p in enumerate(pos):
        gi.dev_flat(q[s * HQ * D:].data_ptr(), H.stream_ptr(), seed, tq, HQ * D, 0, 1.0, start=(s * T + p) * HQ * D)
        tmpk = H.dev_cache(seed, tk, s + 1, T, D, 0, gi.LAYOUT_TOKEN_MAJOR, t0=p, nt=1)
        tmpv = H.dev_cache(seed, tv, s + 1, T, D, 0, gi.LAYOUT_TOKEN_MAJOR, t0=p, nt=1)
        kn[s * G * D:(s + 1) * G * D] = tmpk[s * G * D:(s + 1) * G * D]
        vn[s * G * D:(s + 1) * G * D] = tmpv[s * G * D:(s + 1) * G * D]
    return k_ring, v_ring, q, kn, vn, T, (tq, tk, tv)


def _swa_decode_oracle(seed, tids, T, s, p, q_row_start):
    tq, tk, tv = tids
    Kh = gi.host_tokens_bf16(seed, tk, T, G, D, s, 0, p + 1)
    Vh = gi.host_tokens_bf16(seed, tv, T, G, D, s, 0, p + 1)
    hq = gi.host_normal_bf16(seed, tq, HQ * D, 1.0, start=q_row_start).reshape(HQ, D)
    return O.swa(hq, Kh, Vh, p, H.W)


def test_swa_decode_skips_sequences_without_a_new_row():
    """swa_attention with one new row per sequence at most (the single-launch decode kernel): a
    sequence whose row range is empty writes nothing (its output row keeps a sentinel), the others
    match the oracle; one sequence sits at p mod 8 = 7 with a full ring, one at the ring's first
    region."""
    seed = 0xFA
    pos = [1023, 4096, 6, 2047]
    S = len(pos)
    k_ring, v_ring, q, kn, vn, T, tids = _swa_decode_inputs(seed, pos, 1)
    geom = dsa.geometry()
    # rows: sequence 1 has none, the others take rows 0, 1, 2 (their inputs moved down by one row
    # after sequence 1)
    keep = [0, 2, 3]
    q2 = torch.zeros_like(q)
    kn2, vn2 = torch.zeros_like(kn), torch.zeros_like(vn)
    for r, s in enumerate(keep):
        q2[r * HQ * D:(r + 1) * HQ * D] = q[s * HQ * D:(s + 1) * HQ * D]
        kn2[r * G * D:(r + 1) * G * D] = kn[s * G * D:(s + 1) * G * D]
        vn2[r * G * D:(r + 1) * G * D] = vn[s * G * D:(s + 1) * G * D]
    row0 = H.i32([0, 1, 1, 2, 3])
    out = torch.full((S * HQ * D,), 7.0, dtype=H.BF16, device="cuda")
    dsa.swa_attention(geom, H.W, 1, H.i32(pos), row0, q2, kn2, vn2, k_ring, v_ring, out)
    torch.cuda.synchronize()
    go = H.bf16_np(out).reshape(S, HQ, D)
    for r, s in enumerate(keep):
        p = pos[s]
        H.assert_attn(go[r], _swa_decode_oracle(seed, tids, T, s, p, (s * T + p) * HQ * D), f"seq {s} at {p}")
    assert np.all(go[3] == 7.0), "the row past the last sequence's was written"


def test_swa_batched_decode_with_prefilled_rings():
    """Several sequences, one new token each, rings written directly by the generator."""
    seed = 0xF5
    pos = [0, 7, 300, 511, 512, 519, 5000]
    S = len(pos)
    T = max(pos) + 1
    tq, tk, tv = H.swa_tids(0)
    geom = dsa.geometry()
    k_ring = torch.full((S * G * H.W * D,), float("nan"), dtype=H.BF16, device="cuda")
    v_ring = torch.full((S * G * H.W * D,), float("nan"), dtype=H.BF16, device="cuda")
    per = G * H.W * D
    for s, p in enumerate(pos):
        t0 = max(0, p - H.W)
        if p > t0:
            # write positions t0..p-1 of sequence s (logical batch index s) into its ring
            for layout, ring, tid in ((gi.LAYOUT_KTILED, k_ring, tk), (gi.LAYOUT_REGION_T, v_ring, tv)):
                tmp = torch.empty((s + 1) * per, dtype=H.BF16, device="cuda")
                gi.dev_tokens(tmp.data_ptr(), H.stream_ptr(), seed, tid, s + 1, T, G, D, t0, p - t0, H.W, H.W,
                              layout, 1.0)
                ring[s * per:(s + 1) * per] = tmp[s * per:(s + 1) * per]
    rows = []
    q = torch.empty(S * HQ * D, dtype=H.BF16, device="cuda")
    kn = torch.empty(S * G * D, dtype=H.BF16, device="cuda")
    vn = torch.empty(S * G * D, dtype=H.BF16, device="cuda")
    for s, p in enumerate(pos):
        gi.dev_flat(q[s * HQ * D:].data_ptr(), H.stream_ptr(), seed, tq, HQ * D, 0, 1.0, start=(s * T + p) * HQ * D)
        tmpk = H.dev_cache(seed, tk, s + 1, T, D, 0, gi.LAYOUT_TOKEN_MAJOR, t0=p, nt=1)
        tmpv = H.dev_cache(seed, tv, s + 1, T, D, 0, gi.LAYOUT_TOKEN_MAJOR, t0=p, nt=1)
        kn[s * G * D:(s + 1) * G * D] = tmpk[s * G * D:(s + 1) * G * D]
        vn[s * G * D:(s + 1) * G * D] = tmpv[s * G * D:(s + 1) * G * D]
    out = torch.empty(S * HQ * D, dtype=H.BF16, device="cuda")
    dsa.swa_attention(geom, H.W, 1, H.i32(pos), H.i32(np.arange(S + 1)), q, kn, vn, k_ring, v_ring, out)
    torch.cuda.synchronize()
    go = H.bf16_np(out).reshape(S, HQ, D)
    for s, p in enumerate(pos):
        Kh = gi.host_tokens_bf16(seed, tk, T, G, D, s, 0, p + 1)
        Vh = gi.host_tokens_bf16(seed, tv, T, G, D, s, 0, p + 1)
        hq = gi.host_normal_bf16(seed, tq, HQ * D, 1.0, start=(s * T + p) * HQ * D).reshape(HQ, D)
        H.assert_attn(go[s], O.swa(hq, Kh, Vh, p, H.W), f"seq {s} at {p}")
    # the append then leaves each ring holding positions p-511..p
    dsa.swa_ring_append(geom, H.W, 1, H.i32(pos), H.i32(np.arange(S + 1)), kn, vn, k_ring, v_ring)
    torch.cuda.synchronize()
    kr = H.ktiled_logical(k_ring.view(torch.int16).cpu().numpy().view(np.uint16), S, H.W)
    for s, p in enumerate(pos):
        Kh = gi.host_tokens_bf16(seed, tk, T, G, D, s, 0, p + 1)
        for t in range(max(0, p - H.W + 1), p + 1):
            assert np.array_equal(kr[s, :, t % H.W, :], Kh[t])


def test_swa_decode_step_equals_attention_then_append():
    """swa_decode_step (attention and ring append in one launch) against swa_attention followed by
    swa_ring_append on copies of the same rings: the same output bit for bit, the same rings, and the
    oracle's window attention; positions at the ring's start, just before and after it fills, region
    edges, and a full ring whose current slot still holds the window's first region."""
    seed = 0xF9
    pos = [0, 5, 8, 510, 511, 512, 513, 1023, 4100, 4103]
    S = len(pos)
    T = max(pos) + 1
    tq, tk, tv = H.swa_tids(2)
    geom = dsa.geometry()
    per = G * H.W * D
    k_ring = torch.full((S * per,), float("nan"), dtype=H.BF16, device="cuda")
    v_ring = torch.full((S * per,), float("nan"), dtype=H.BF16, device="cuda")
    for s, p in enumerate(pos):
        t0 = max(0, p - H.W)
        if p > t0:
            for layout, ring, tid in ((gi.LAYOUT_KTILED, k_ring, tk), (gi.LAYOUT_REGION_T, v_ring, tv)):
                tmp = torch.empty((s + 1) * per, dtype=H.BF16, device="cuda")
                gi.dev_tokens(tmp.data_ptr(), H.stream_ptr(), seed, tid, s + 1, T, G, D, t0, p - t0, H.W, H.W,
                              layout, 1.0)
                ring[s * per:(s + 1) * per] = tmp[s * per:(s + 1) * per]
    q = torch.empty(S * HQ * D, dtype=H.BF16, device="cuda")
    kn = torch.empty(S * G * D, dtype=H.BF16, device="cuda")
    vn = torch.empty(S * G * D, dtype=H.BF16, device="cuda")
    for s, p in enumerate(pos):
        gi.dev_flat(q[s * HQ * D:].data_ptr(), H.stream_ptr(), seed, tq, HQ * D, 0, 1.0, start=(s * T + p) * HQ * D)
        tmpk = H.dev_cache(seed, tk, s + 1, T, D, 0, gi.LAYOUT_TOKEN_MAJOR, t0=p, nt=1)
        tmpv = H.dev_cache(seed, tv, s + 1, T, D, 0, gi.LAYOUT_TOKEN_MAJOR, t0=p, nt=1)
        kn[s * G * D:(s + 1) * G * D] = tmpk[s * G * D:(s + 1) * G * D]
        vn[s * G * D:(s + 1) * G * D] = tmpv[s * G * D:(s + 1) * G * D]
    kr1, vr1 = k_ring.clone(), v_ring.clone()
    out1 = torch.empty(S * HQ * D, dtype=H.BF16, device="cuda")
    dsa.swa_attention(geom, H.W, 1, H.i32(pos), H.i32(np.arange(S + 1)), q, kn, vn, kr1, vr1, out1)
    dsa.swa_ring_append(geom, H.W, 1, H.i32(pos), H.i32(np.arange(S + 1)), kn, vn, kr1, vr1)
    kr2, vr2 = k_ring.clone(), v_ring.clone()
    out2 = torch.empty(S * HQ * D, dtype=H.BF16, device="cuda")
    dsa.swa_decode_step(geom, H.W, H.i32(pos), q, kn, vn, kr2, vr2, out2)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(kr1.view(torch.int16), kr2.view(torch.int16))
    assert torch.equal(vr1.view(torch.int16), vr2.view(torch.int16))
    go = H.bf16_np(out2).reshape(S, HQ, D)
    for s, p in enumerate(pos):
        Kh = gi.host_tokens_bf16(seed, tk, T, G, D, s, 0, p + 1)
        Vh = gi.host_tokens_bf16(seed, tv, T, G, D, s, 0, p + 1)
        hq = gi.host_normal_bf16(seed, tq, HQ * D, 1.0, start=(s * T + p) * HQ * D).reshape(HQ, D)
        H.assert_attn(go[s], O.swa(hq, Kh, Vh, p, H.W), f"seq {s} at {p}")


def test_swa_prefill_chunks_of_several_sequences_in_one_call():
    """Chunks of different lengths for sequences at different positions in one call (the banded
    prefill kernel: tiles of 8 tokens, partial last tiles, short and full rings)."""
    seed = 0xF7
    p0s, ns = [0, 300, 1000, 4093], [50, 37, 64, 17]
    S, M = len(p0s), max(ns)
    T = max(p + n for p, n in zip(p0s, ns))
    tq, tk, tv = H.swa_tids(1)
    geom = dsa.geometry()
    per = G * H.W * D
    k_ring = torch.full((S * per,), float("nan"), dtype=H.BF16, device="cuda")
    v_ring = torch.full((S * per,), float("nan"), dtype=H.BF16, device="cuda")
    for s, p in enumerate(p0s):
        t0 = max(0, p - H.W)
        if p > t0:
            for layout, ring, tid in ((gi.LAYOUT_KTILED, k_ring, tk), (gi.LAYOUT_REGION_T, v_ring, tv)):
                tmp = torch.empty((s + 1) * per, dtype=H.BF16, device="cuda")
                gi.dev_tokens(tmp.data_ptr(), H.stream_ptr(), seed, tid, s + 1, T, G, D, t0, p - t0, H.W, H.W,
                              layout, 1.0)
                ring[s * per:(s + 1) * per] = tmp[s * per:(s + 1) * per]
    row0 = np.concatenate([[0], np.cumsum(ns)]).astype(np.int32)
    rows = int(row0[-1])
    q = torch.empty(S * M * HQ * D, dtype=H.BF16, device="cuda")
    kn = torch.empty(S * M * G * D, dtype=H.BF16, device="cuda")
    vn = torch.empty(S * M * G * D, dtype=H.BF16, device="cuda")
    for s, (p, n) in enumerate(zip(p0s, ns)):
        r = int(row0[s])
        gi.dev_flat(q[r * HQ * D:].data_ptr(), H.stream_ptr(), seed, tq, n * HQ * D, 0, 1.0,
                    start=(s * T + p) * HQ * D)
        tmpk = H.dev_cache(seed, tk, s + 1, T, D, 0, gi.LAYOUT_TOKEN_MAJOR, t0=p, nt=n)
        tmpv = H.dev_cache(seed, tv, s + 1, T, D, 0, gi.LAYOUT_TOKEN_MAJOR, t0=p, nt=n)
        kn[r * G * D:(r + n) * G * D] = tmpk[s * n * G * D:(s + 1) * n * G * D]
        vn[r * G * D:(r + n) * G * D] = tmpv[s * n * G * D:(s + 1) * n * G * D]
    out = torch.empty(S * M * HQ * D, dtype=H.BF16, device="cuda")
    dsa.swa_attention(geom, H.W, M, H.i32(p0s), H.i32(row0), q, kn, vn, k_ring, v_ring, out)
    torch.cuda.synchronize()
    go = H.bf16_np(out)[:rows * HQ * D].reshape(rows, HQ, D)
    for s, (p, n) in enumerate(zip(p0s, ns)):
        Kh = gi.host_tokens_bf16(seed, tk, T, G, D, s, 0, p + n)
        Vh = gi.host_tokens_bf16(seed, tv, T, G, D, s, 0, p + n)
        hq = gi.host_normal_bf16(seed, tq, n * HQ * D, 1.0, start=(s * T + p) * HQ * D).reshape(n, HQ, D)
        for i in sorted(set([0, 1, 15, 16, n // 2, n - 1])):
            if i < n:
                H.assert_attn(go[int(row0[s]) + i], O.swa(hq[i], Kh, Vh, p + i, H.W), f"seq {s} token {p + i}")


def test_decode_is_deterministic():
    a = H.run_dsa_decode(0xAA, [6000, 3001], topk=512, check_seqs=[])
    b = H.run_dsa_decode(0xAA, [6000, 3001], topk=512, check_seqs=[])
    for k in ("summ", "scale", "sel", "nsel", "out"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


def _prefill_inputs(seed, p0, n, topk=512):
    """One sequence: prefix p0 summarised, chunk of n queries scored and selected on the GPU."""
    tcap = H.round128(p0 + n)
    R = tcap // 8
    geom = dsa.geometry(topk=topk)
    ik = H.dev_cache(seed, gi.TID_IK, 1, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE)
    K = H.dev_cache(seed, gi.TID_K, 1, tcap, D, tcap, gi.LAYOUT_KTILED)
    V = H.dev_cache(seed, gi.TID_V, 1, tcap, D, tcap, gi.LAYOUT_REGION_T)
    summ = torch.zeros(G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(G * R, dtype=torch.float32, device="cuda")
    dsa.dsa_compress_regions(geom, ik, tcap, H.i32([0]), H.i32([(p0 + n) // 8]), R, summ, scale)
    q, iq, z = H.dev_queries(seed, n)
    qs, qp = H.i32(np.zeros(n)), H.i32(np.arange(p0, p0 + n))
    return dict(geom=geom, tcap=tcap, R=R, K=K, V=V, summ=summ, scale=scale, q=q, iq=iq, z=z, qs=qs, qp=qp, n=n,
                topk=topk)


def _prefill_select(a):
    sel = torch.empty(a["n"] * G * a["topk"], dtype=torch.int32, device="cuda")
    nsel = torch.empty(a["n"] * G, dtype=torch.int32, device="cuda")
    dsa.dsa_score_topk(a["geom"], a["iq"], a["z"], a["qs"], a["qp"], 1, a["summ"],
                       a["scale"], a["tcap"], a["R"], sel, nsel)
    return sel, nsel


def _prefill_attend(a, sel, nsel, ws=None, merged=False):
    out = torch.empty(a["n"] * HQ * D, dtype=H.BF16, device="cuda")
    f = dsa.dsa_sparse_gqa_prefill_merged if merged else dsa.dsa_sparse_gqa_prefill
    f(a["geom"], a["q"], a["qs"], a["qp"], 1, a["K"], a["V"], a["tcap"], sel, nsel, out, workspace=ws)
    return out


def test_prefill_is_deterministic():
    """Selection and attention of a prefill chunk are bitwise identical from run to run (the 64K
    prefill shape, every query of the chunk)."""
    a = _prefill_inputs(0xAC, 63488, 2048)
    s1, n1 = _prefill_select(a)
    o1 = _prefill_attend(a, s1, n1)
    s2, n2 = _prefill_select(a)
    o2 = _prefill_attend(a, s2, n2)
    torch.cuda.synchronize()
    assert torch.equal(n1, n2) and torch.equal(s1, s2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_attention_does_not_depend_on_workspace_contents():
    """The split partials of sparse GQA decode and the region-range partials of prefill (both in the
    caller's workspace) are fully written before they are read: a workspace filled with NaN bytes
    gives the same output, bit for bit, as a zeroed one."""
    # decode: partial last splits (top-37), short and partial-region contexts
    r = H.run_dsa_decode(0xAD, [3000, 2047, 17, 1], topk=37, check_seqs=[])
    d = r["dev"]
    B = r["B"]
    lens = H.i32(r["lens"])
    sel, nsel = H.i32(r["sel"].ravel()), H.i32(r["nsel"].ravel())
    nb = dsa.dsa_sparse_gqa_workspace_size(d["geom"], B)
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((nb,), fill, dtype=torch.uint8, device="cuda")
        out = torch.empty(B * HQ * D, dtype=H.BF16, device="cuda")
        dsa.dsa_sparse_gqa_decode(d["geom"], d["q"], d["K"], d["V"], r["tcap"], lens, sel, nsel, out, workspace=ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert not torch.isnan(outs[0].float()).any()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    # prefill (per-query and neighbour-merged): a chunk with a partial trailing region
    a = _prefill_inputs(0xAE, 4003, 300)
    s, n = _prefill_select(a)
    nb = dsa.dsa_sparse_gqa_prefill_workspace_size(a["geom"], a["n"])
    for merged in (False, True):
        outs = [_prefill_attend(a, s, n, torch.full((nb,), fill, dtype=torch.uint8, device="cuda"), merged)
                for fill in (0x00, 0xFF)]
        torch.cuda.synchronize()
        assert not torch.isnan(outs[0].float()).any()
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), f"merged={merged}"


def test_decode_step_replays_from_a_hip_graph():
    """The whole decode step captured once and replayed several times, with eager work and
    synchronisations in between, gives the eager result bit for bit on every replay."""
    seed = 0xAB
    lens = [3000, 1505]
    B, topk = len(lens), 512
    tcap = H.round128(max(lens))
    R = tcap // 8
    geom = dsa.geometry(topk=topk)
    ik = H.dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE)
    K = H.dev_cache(seed, gi.TID_K, B, tcap, D, tcap, gi.LAYOUT_KTILED)
    V = H.dev_cache(seed, gi.TID_V, B, tcap, D, tcap, gi.LAYOUT_REGION_T)
    q, iq, z = H.dev_queries(seed, B)
    lens_np = np.asarray(lens, dtype=np.int32)
    zero, rend = H.i32(np.zeros(B)), H.i32(lens_np // 8)
    qs, qp, sl = H.i32(np.arange(B)), H.i32(lens_np - 1), H.i32(lens_np)
    ws1 = dsa.workspace(dsa.dsa_score_topk_workspace_size(geom, B, R))
    ws2 = dsa.workspace(dsa.dsa_sparse_gqa_workspace_size(geom, B))

    def make_bufs():
        return dict(summ=torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda"),
                    scale=torch.zeros(B * G * R, dtype=torch.float32, device="cuda"),
                    sel=torch.empty(B * G * topk, dtype=torch.int32, device="cuda"),
                    nsel=torch.empty(B * G, dtype=torch.int32, device="cuda"),
                    out=torch.empty(B * HQ * D, dtype=H.BF16, device="cuda"))

    def step(b):
        dsa.dsa_compress_regions(geom, ik, tcap, zero, rend, R, b["summ"], b["scale"])
        dsa.dsa_score_topk(geom, iq, z, qs, qp, B, b["summ"], b["scale"], tcap, R, b["sel"], b["nsel"],
                           workspace=ws1)
        dsa.dsa_sparse_gqa_decode(geom, q, K, V, tcap, sl, b["sel"], b["nsel"], b["out"], workspace=ws2)

    ref = make_bufs()
    step(ref)
    torch.cuda.synchronize()
    gb = make_bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(gb)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(gb)
    for rep in range(3):
        for t in gb.values():
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(gb[k].view(torch.uint8), ref[k].view(torch.uint8)), (rep, k)
        other = make_bufs()  # eager work between replays, sharing the workspaces
        step(other)
        torch.cuda.synchronize()
        assert torch.equal(other["out"].view(torch.uint8), ref["out"].view(torch.uint8))


def test_swa_decode_step_replays_from_a_hip_graph():
    """The sliding-window decode step (attention and ring append in one launch) captured once and
    replayed several times, with eager steps on other rings in between: every replay gives the eager
    output and rings bit for bit (a replay appends the same token to the same slot, which the step
    itself never reads)."""
    seed = 0xAC
    pos = [700, 1023, 40, 512]
    S = len(pos)
    k_ring, v_ring, q, kn, vn, T, tids = _swa_decode_inputs(seed, pos, 3)
    geom = dsa.geometry()
    p32 = H.i32(pos)

    def make_bufs():
        return dict(kr=k_ring.clone(), vr=v_ring.clone(), out=torch.empty(S * HQ * D, dtype=H.BF16, device="cuda"))

    def step(b):
        dsa.swa_decode_step(geom, H.W, p32, q, kn, vn, b["kr"], b["vr"], b["out"])

    ref = make_bufs()
    step(ref)
    torch.cuda.synchronize()
    gb = make_bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(gb)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(gb)
    for rep in range(3):
        gb["out"].zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(gb[k].view(torch.int16), ref[k].view(torch.int16)), (rep, k)
        other = make_bufs()
        step(other)
        torch.cuda.synchronize()
        assert torch.equal(other["out"].view(torch.int16), ref["out"].view(torch.int16))
    go = H.bf16_np(ref["out"]).reshape(S, HQ, D)
    for s_, p in enumerate(pos):
        H.assert_attn(go[s_], _swa_decode_oracle(seed, tids, T, s_, p, (s_ * T + p) * HQ * D), f"seq {s_} at {p}")


def test_cache_write_produces_the_documented_layouts():
    """dsa_cache_write of token-major rows gives the same bytes as the generator's direct fill of the
    group-major index_k, region-tiled K and region-transposed V caches."""
    seed = 0xCA
    B, T, tcap = 2, 300, 384
    geom = dsa.geometry()
    ref_k = H.dev_cache(seed, gi.TID_K, B, T, D, tcap, gi.LAYOUT_KTILED)
    ref_v = H.dev_cache(seed, gi.TID_V, B, T, D, tcap, gi.LAYOUT_REGION_T)
    ref_ik = H.dev_cache(seed, gi.TID_IK, B, T, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE)
    kn = H.dev_cache(seed, gi.TID_K, B, T, D, 0, gi.LAYOUT_TOKEN_MAJOR)
    vn = H.dev_cache(seed, gi.TID_V, B, T, D, 0, gi.LAYOUT_TOKEN_MAJOR)
    ikn = H.dev_cache(seed, gi.TID_IK, B, T, P, 0, gi.LAYOUT_TOKEN_MAJOR, gi.IK_SCALE)
    k = torch.zeros_like(ref_k)
    v = torch.zeros_like(ref_v)
    ik = torch.zeros_like(ref_ik)
    seqs = np.repeat(np.arange(B), T).astype(np.int32)
    pos = np.tile(np.arange(T), B).astype(np.int32)
    perm = np.random.default_rng(0).permutation(B * T)  # rows in any order
    dsa.dsa_cache_write(geom, H.i32(seqs[perm]), H.i32(pos[perm]), kn.view(B * T, -1)[perm].contiguous().view(-1),
                        vn.view(B * T, -1)[perm].contiguous().view(-1), ikn.view(B * T, -1)[perm].contiguous().view(-1),
                        k, v, ik, B, tcap)
    torch.cuda.synchronize()
    # compare the written token range only (positions >= T stay zero in the written caches)
    kt = H.ktiled_logical(k.view(torch.int16).cpu().numpy().view(np.uint16), B, tcap)
    rt = H.ktiled_logical(ref_k.view(torch.int16).cpu().numpy().view(np.uint16), B, tcap)
    assert np.array_equal(kt[:, :, :T], rt[:, :, :T]) and not kt[:, :, T:].any()
    vv = v.view(torch.int16).cpu().numpy().reshape(B, G, tcap // 8, D, 8)
    rv = ref_v.view(torch.int16).cpu().numpy().reshape(B, G, tcap // 8, D, 8)
    vl = vv.transpose(0, 1, 2, 4, 3).reshape(B, G, tcap, D)
    rl = rv.transpose(0, 1, 2, 4, 3).reshape(B, G, tcap, D)
    assert np.array_equal(vl[:, :, :T], rl[:, :, :T])
    ikw = ik.view(torch.int16).cpu().numpy().reshape(B, G, tcap, P)
    ikr = ref_ik.view(torch.int16).cpu().numpy().reshape(B, G, tcap, P)
    assert np.array_equal(ikw[:, :, :T], ikr[:, :, :T])
