"""Shared test harness: builds the same seeded inputs for the GPU library and the CPU oracle, runs
both, and applies the acceptance rules.

Acceptance (the task's stated bar):
  * summaries: E4M3 codes and fp32 scales bit-exact;
  * selection: GPU and oracle sets equal except for regions whose oracle score lies within 1e-4
    (relative) of s_k, the smallest oracle score among the oracle's selected non-forced regions;
  * attention: max |err| <= 2e-2 and ||err||_2 / ||ref||_2 <= 5e-3 against the fp64 oracle.
Input layouts differ between the two sides (the library's group-major / region-transposed caches,
the oracle's token-major arrays); both are filled from the same generator definition.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import dsa_inputs as gi
import dsa_sparse_attention_amd as dsa
import oracle as O

G, P, HI, HQ, D, W = 4, 256, 16, 64, 192, 512
MAX_ABS, REL_RMS, BAND = 2e-2, 5e-3, 1e-4
BF16 = torch.bfloat16


def stream_ptr():
    return torch.cuda.current_stream().cuda_stream


def round8(x):
    return (x + 7) // 8 * 8


def round128(x):
    """Cache capacities are multiples of 128 tokens (16 regions = one summary tile)."""
    return (x + 127) // 128 * 128


def ktiled_logical(k_np, B, T):
    """Region-tiled keys [B][G][T/8][1536] -> [B][G][T][D] (layout of include/dsa.h)."""
    t = k_np.reshape(B, G, T // 8, 2, 6, 4, 4, 8)  # region, pos/4, (d%48)/8, d/48, pos%4, d%8
    return t.transpose(0, 1, 2, 3, 6, 5, 4, 7).reshape(B, G, T, D)


def summ_logical(summ_np, B, R):
    """The library's tiled summary bytes [B][G][R/16][4096] -> [B][G][R][P] (layout of include/dsa.h)."""
    t = summ_np.reshape(B, G, R // 16, 4, 4, 16, 16)  # tile, j/64, (j%64)/16, r%16, j%16
    return t.transpose(0, 1, 2, 5, 3, 4, 6).reshape(B, G, R, P)


# ------------------------------------------------------------------------------------------------
# device inputs (dsa_inputs HIP generator) and host inputs (dsa_inputs C generator)
# ------------------------------------------------------------------------------------------------
def dev_cache(seed, tid, B, T, C, tcap, layout, scale=1.0, planted=False, t0=0, nt=None, tmod=None):
    nt = T - t0 if nt is None else nt
    if layout == gi.LAYOUT_TOKEN_MAJOR:
        out = torch.empty(B * nt * G * C, dtype=BF16, device="cuda")
    else:
        out = torch.empty(B * G * tcap * C, dtype=BF16, device="cuda")
    gi.dev_tokens(out.data_ptr(), stream_ptr(), seed, tid, B, T, G, C, t0, nt, tcap, tmod or tcap, layout, scale,
                  planted)
    return out


def dev_flat_bf16(seed, tid, n, scale=1.0):
    out = torch.empty(n, dtype=BF16, device="cuda")
    gi.dev_flat(out.data_ptr(), stream_ptr(), seed, tid, n, 0, scale)
    return out


def dev_flat_uniform(seed, tid, n):
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    gi.dev_flat(out.data_ptr(), stream_ptr(), seed, tid, n, 1)
    return out


def host_queries(seed, nq, q_start=0):
    """q [nq][64][192], index_q [nq][16][256], z [nq][16] for query indices q_start.."""
    q = gi.host_normal_bf16(seed, gi.TID_Q, nq * HQ * D, 1.0, start=q_start * HQ * D).reshape(nq, HQ, D)
    iq = gi.host_normal_bf16(seed, gi.TID_IQ, nq * HI * P, gi.IK_SCALE, start=q_start * HI * P).reshape(nq, HI, P)
    z = gi.host_uniform_f32(seed, gi.TID_Z, nq * HI, start=q_start * HI).reshape(nq, HI)
    return q, iq, z


def dev_queries(seed, nq, q_start=0):
    """q, index_q, z of query indices q_start .. q_start+nq-1 (device generator)."""
    q = torch.empty(nq * HQ * D, dtype=BF16, device="cuda")
    gi.dev_flat(q.data_ptr(), stream_ptr(), seed, gi.TID_Q, nq * HQ * D, 0, 1.0, start=q_start * HQ * D)
    iq = torch.empty(nq * HI * P, dtype=BF16, device="cuda")
    gi.dev_flat(iq.data_ptr(), stream_ptr(), seed, gi.TID_IQ, nq * HI * P, 0, gi.IK_SCALE, start=q_start * HI * P)
    z = torch.empty(nq * HI, dtype=torch.float32, device="cuda")
    gi.dev_flat(z.data_ptr(), stream_ptr(), seed, gi.TID_Z, nq * HI, 1, start=q_start * HI)
    return q, iq, z


def i32(x):
    return torch.tensor(np.asarray(x, dtype=np.int32), dtype=torch.int32, device="cuda")


# ------------------------------------------------------------------------------------------------
# comparisons
# ------------------------------------------------------------------------------------------------
def attn_errors(gpu: np.ndarray, ref: np.ndarray):
    err = gpu.astype(np.float64) - ref
    return float(np.abs(err).max()), float(math.sqrt((err ** 2).sum() / max((ref ** 2).sum(), 1e-300)))


def assert_attn(gpu, ref, what=""):
    mx, rr = attn_errors(gpu, ref)
    assert mx <= MAX_ABS and rr <= REL_RMS, f"{what}: max abs {mx:.3e}, rel rms {rr:.3e}"
    return mx, rr


def bf16_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def check_selection(gsel, or_sel, or_scores_g, c):
    """Band rule. gsel/or_sel: ascending region lists; or_scores_g: oracle scores of regions 0..c-1.
    Returns True when the sets are identical."""
    gsel = [int(x) for x in gsel]
    assert gsel == sorted(set(gsel)), "GPU selection not ascending/unique"
    assert c in gsel, "current region missing from GPU selection"
    assert len(gsel) == len(or_sel), (len(gsel), len(or_sel))
    sym = set(gsel) ^ set(int(x) for x in or_sel)
    if not sym:
        return True
    nonforced = [int(r) for r in or_sel if r != c]
    s_k = min(or_scores_g[r] for r in nonforced)
    for r in sym:
        assert r != c and r < c, f"region {r} outside the candidates"
        assert abs(or_scores_g[r] - s_k) <= BAND * abs(s_k), \
            f"region {r}: score {or_scores_g[r]!r} outside the band around s_k={s_k!r}"
    return False


# ------------------------------------------------------------------------------------------------
# DSA decode end to end
# ------------------------------------------------------------------------------------------------
def run_dsa_decode(seed, lens, topk=512, tcap=None, planted=False, check_seqs=None, zero_z=False, q_start=0):
    """Runs compress -> score_topk -> sparse GQA decode on the GPU for len(lens) sequences (query b at
    position lens[b]-1, generated as query index q_start + b), and the oracle for the sequences in
    check_seqs (default all)."""
    B = len(lens)
    tcap = tcap or round128(max(lens))
    R = tcap // 8
    geom = dsa.geometry(topk=topk)
    ik = dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE, planted)
    K = dev_cache(seed, gi.TID_K, B, tcap, D, tcap, gi.LAYOUT_KTILED)
    V = dev_cache(seed, gi.TID_V, B, tcap, D, tcap, gi.LAYOUT_REGION_T)
    q, iq, z = dev_queries(seed, B, q_start)
    if zero_z:  # every score 0: selection falls to the lowest regions (tie rule)
        z.zero_()
    summ = torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(B * G * R, dtype=torch.float32, device="cuda")
    lens_np = np.asarray(lens, dtype=np.int32)
    dsa.dsa_compress_regions(geom, ik, tcap, i32(np.zeros(B)), i32(lens_np // 8), R, summ, scale)
    sel = torch.empty(B * G * topk, dtype=torch.int32, device="cuda")
    nsel = torch.empty(B * G, dtype=torch.int32, device="cuda")
    scores = torch.full((B * G * R,), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_score_topk(geom, iq, z, i32(np.arange(B)), i32(lens_np - 1), B, summ, scale, tcap, R, sel, nsel,
                       scores_out=scores)
    out = torch.empty(B * HQ * D, dtype=BF16, device="cuda")
    dsa.dsa_sparse_gqa_decode(geom, q, K, V, tcap, i32(lens_np), sel, nsel, out)
    torch.cuda.synchronize()
    res = dict(lens=list(lens), topk=topk, tcap=tcap, R=R, B=B,
               summ=summ_logical(summ.cpu().numpy(), B, R), scale=scale.cpu().numpy().reshape(B, G, R),
               sel=sel.cpu().numpy().reshape(B, G, topk), nsel=nsel.cpu().numpy().reshape(B, G),
               scores=scores.cpu().numpy().reshape(B, G, R), out=bf16_np(out).reshape(B, HQ, D),
               oracle={}, dev=dict(K=K, V=V, q=q, geom=geom, ik=ik, iq=iq, z=z, summ=summ, scale=scale))
    hq, hiq, hz = host_queries(seed, B, q_start)
    if zero_z:
        hz = np.zeros_like(hz)
    for b in (range(B) if check_seqs is None else check_seqs):
        L = lens[b]
        ikh = gi.host_index_k(seed, tcap, G, P, b, 0, L, planted)
        Kh = gi.host_tokens_bf16(seed, gi.TID_K, tcap, G, D, b, 0, L)
        Vh = gi.host_tokens_bf16(seed, gi.TID_V, tcap, G, D, b, 0, L)
        codes, scales = O.compress_regions(ikh, 0, L // 8)
        osel, onsel, oout, osc = O.dsa_query(hiq[b], hz[b], codes, scales, hq[b], Kh, Vh, L - 1, k=topk,
                                             want_scores=True)
        res["oracle"][b] = dict(codes=codes, scales=scales, sel=osel, nsel=onsel, out=oout, scores=osc, K=Kh,
                                V=Vh, q=hq[b])
    return res


def assert_decode_parity(r, min_identical_frac=0.9, report=True):
    """Every (sequence, group) is checked end to end.  Where the GPU's selection equals the oracle's,
    its output is compared with the oracle's output; where the two differ inside the band (both
    correct), with the oracle's attention recomputed on the GPU's own selection.  Selections that
    differ stay rare (at least min_identical_frac identical); their count is returned and printed."""
    n_same = n_groups = 0
    for b, o in r["oracle"].items():
        L = r["lens"][b]
        nr = L // 8
        # summaries bit-exact
        assert np.array_equal(r["summ"][b][:, :nr, :], o["codes"][:nr].transpose(1, 0, 2)), f"seq {b}: codes differ"
        assert np.array_equal(r["scale"][b][:, :nr].view(np.uint32),
                              o["scales"][:nr].T.copy().view(np.uint32)), f"seq {b}: scales differ"
        c = (L - 1) // 8
        differ = []
        gpu_lists = []
        for g in range(G):
            osc = o["scores"][g]
            gsc = r["scores"][b, g, :c].astype(np.float64)
            if c:
                tol = 2e-5 * max(np.abs(osc).max(), 1e-30)
                assert np.all(np.abs(gsc - osc) <= tol), f"seq {b} group {g}: scores differ"
            gs = r["sel"][b, g, :r["nsel"][b, g]]
            gpu_lists.append(gs.copy())
            assert np.all(r["sel"][b, g, r["nsel"][b, g]:] == -1)
            assert r["nsel"][b, g] == o["nsel"][g] == min(r["topk"], c + 1)
            same = check_selection(gs, o["sel"][g, :o["nsel"][g]], osc, c)
            n_groups += 1
            if same:
                n_same += 1
                assert_attn(r["out"][b, 16 * g:16 * g + 16], o["out"][16 * g:16 * g + 16], f"seq {b} group {g}")
            else:
                differ.append(g)
        if differ:  # the oracle's attention on the GPU's selection
            ref = O.attend(o["q"], o["K"], o["V"], L - 1, gpu_lists, k=r["topk"])
            for g in differ:
                assert_attn(r["out"][b, 16 * g:16 * g + 16], ref[16 * g:16 * g + 16],
                            f"seq {b} group {g} (on the GPU's selection)")
    assert n_same >= min_identical_frac * n_groups, f"only {n_same}/{n_groups} selections identical"
    if report:
        print(f"decode parity: {n_groups} (sequence, group) outputs checked, {n_groups - n_same} of them on the "
              f"GPU's own selection (differs from the oracle's inside the band)")
    return n_same, n_groups


# ------------------------------------------------------------------------------------------------
# sliding window
# ------------------------------------------------------------------------------------------------
def swa_tids(layer=0):
    return gi.tid_swa(gi.TID_Q, layer), gi.tid_swa(gi.TID_K, layer), gi.tid_swa(gi.TID_V, layer)


def check_swa_sequence(seed, chunks, check_from=0, layer=0, sample=None, rng_seed=0):
    """One sequence processed as consecutive chunks (prefill chunks and decode steps): swa_attention on
    each chunk then swa_ring_append.  The ring starts filled with NaN so a stale slot would show.
    Outputs of chunks >= check_from are compared with the oracle over the full K/V history."""
    T = sum(chunks)
    tq, tk, tv = swa_tids(layer)
    geom = dsa.geometry()
    k_ring = torch.full((G * W * D,), float("nan"), dtype=BF16, device="cuda")
    v_ring = torch.full((G * W * D,), float("nan"), dtype=BF16, device="cuda")
    Kh = gi.host_tokens_bf16(seed, tk, T, G, D, 0, 0, T)
    Vh = gi.host_tokens_bf16(seed, tv, T, G, D, 0, 0, T)
    rng = np.random.default_rng(rng_seed)
    pos = 0
    worst = (0.0, 0.0)
    for ci, n in enumerate(chunks):
        q = torch.empty(n * HQ * D, dtype=BF16, device="cuda")
        gi.dev_flat(q.data_ptr(), stream_ptr(), seed, tq, n * HQ * D, 0, 1.0, start=pos * HQ * D)
        kn = dev_cache(seed, tk, 1, T, D, 0, gi.LAYOUT_TOKEN_MAJOR, t0=pos, nt=n)
        vn = dev_cache(seed, tv, 1, T, D, 0, gi.LAYOUT_TOKEN_MAJOR, t0=pos, nt=n)
        out = torch.empty(n * HQ * D, dtype=BF16, device="cuda")
        dsa.swa_attention(geom, W, n, i32([pos]), i32([0, n]), q, kn, vn, k_ring, v_ring, out)
        dsa.swa_ring_append(geom, W, n, i32([pos]), i32([0, n]), kn, vn, k_ring, v_ring)
        if ci >= check_from:
            go = bf16_np(out).reshape(n, HQ, D)
            hq = gi.host_normal_bf16(seed, tq, n * HQ * D, 1.0, start=pos * HQ * D).reshape(n, HQ, D)
            idx = range(n) if sample is None or n <= sample else sorted(rng.choice(n, sample, replace=False))
            for i in idx:
                p = pos + i
                ref = O.swa(hq[i], Kh[:p + 1], Vh[:p + 1], p, W)
                mx, rr = assert_attn(go[i], ref, f"swa chunk {ci} position {p}")
                worst = (max(worst[0], mx), max(worst[1], rr))
        pos += n
    return worst
