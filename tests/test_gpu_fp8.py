"""FP8 K/V caches through the C ABI: the cache write is bit-exact with the oracle's row quantiser, and
sparse attention over the FP8 caches (decode, the decode step, prefill) meets the oracle's attention
over the same dequantised values within the attention tolerance.  The quantisation error itself
(FP8 result vs the bf16 oracle) is reported, with a loose bound of its own."""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
import dsa_sparse_attention_amd as dsa
import oracle as O

import _harness as H

pytestmark = pytest.mark.gpu

G, P, HQ, D = H.G, H.P, H.HQ, H.D
FP8_VS_BF16_REL_RMS = 0.06  # E4M3 keeps 3 mantissa bits: the own tolerance of the FP8 cache vs bf16


def _k8_offset(pos, d):
    return ((((pos >> 2) * 3 + (d % 48) // 16) * 4 + d // 48) * 4 + (pos & 3)) * 16 + (d & 15)


K8_PERM = np.array([[_k8_offset(pos, d) for d in range(D)] for pos in range(8)])  # [pos][d] -> byte


def _write_fp8(seed, B, tcap):
    """FP8 caches of B sequences holding the generator's K/V rows at every position < tcap."""
    geom = dsa.geometry()
    Kt = H.dev_cache(seed, gi.TID_K, B, tcap, D, tcap, gi.LAYOUT_TOKEN_MAJOR)
    Vt = H.dev_cache(seed, gi.TID_V, B, tcap, D, tcap, gi.LAYOUT_TOKEN_MAJOR)
    k8, v8, kvs = dsa.fp8_caches(B, tcap)
    tok_seq = np.repeat(np.arange(B), tcap).astype(np.int32)
    tok_pos = np.tile(np.arange(tcap), B).astype(np.int32)
    dsa.dsa_cache_write_fp8(geom, H.i32(tok_seq), H.i32(tok_pos), Kt, Vt, k8, v8, kvs, B, tcap)
    torch.cuda.synchronize()
    del Kt, Vt
    return k8, v8, kvs


def _logical(k8, v8, kvs, B, tcap, b, L):
    """Codes [L][G][D] and scales [L][G] of sequence b read back from the FP8 caches."""
    R = tcap // 8
    nr = (L + 7) // 8
    k = k8.view(B, G, R, 1536)[b, :, :nr].cpu().numpy()          # [G][nr][1536]
    v = v8.view(B, G, R, D, 8)[b, :, :nr].cpu().numpy()          # [G][nr][D][8]
    s = kvs.view(B, G, R, 16)[b, :, :nr].cpu().numpy()           # [G][nr][16]
    kc = k[:, :, K8_PERM]                                        # [G][nr][8][D]
    vc = v.transpose(0, 1, 3, 2)                                 # [G][nr][8][D]
    Kc = kc.reshape(G, nr * 8, D).transpose(1, 0, 2)[:L]
    Vc = vc.reshape(G, nr * 8, D).transpose(1, 0, 2)[:L]
    Ks = s[:, :, :8].reshape(G, nr * 8).T[:L]
    Vs = s[:, :, 8:].reshape(G, nr * 8).T[:L]
    return Kc, Ks, Vc, Vs


def test_fp8_cache_write_is_bit_exact():
    seed, lens = 0xF80, [1000, 259, 8]
    B, tcap = len(lens), 1024
    k8, v8, kvs = _write_fp8(seed, B, tcap)
    for b, L in enumerate(lens):
        Kh = gi.host_tokens_bf16(seed, gi.TID_K, tcap, G, D, b, 0, L)
        Vh = gi.host_tokens_bf16(seed, gi.TID_V, tcap, G, D, b, 0, L)
        okc, oks = O.quantize_rows(Kh)
        ovc, ovs = O.quantize_rows(Vh)
        Kc, Ks, Vc, Vs = _logical(k8, v8, kvs, B, tcap, b, L)
        assert np.array_equal(Kc, okc) and np.array_equal(Vc, ovc), b
        assert np.array_equal(Ks.view(np.uint32), oks.view(np.uint32)), b
        assert np.array_equal(Vs.view(np.uint32), ovs.view(np.uint32)), b


def _check_fp8_outputs(seed, out, lens, tcap, sel, nsel, topk, hq, seqs, what):
    worst = [0.0, 0.0, 0.0]
    for b in seqs:
        L = lens[b]
        Kh = gi.host_tokens_bf16(seed, gi.TID_K, tcap, G, D, b, 0, L)
        Vh = gi.host_tokens_bf16(seed, gi.TID_V, tcap, G, D, b, 0, L)
        Kc, Ks = O.quantize_rows(Kh)
        Vc, Vs = O.quantize_rows(Vh)
        lists = [sel[b, g, :nsel[b, g]] for g in range(G)]
        ref = O.attend_fp8(hq[b], Kc, Ks, Vc, Vs, L - 1, lists, k=topk)
        mx, rr = H.assert_attn(out[b], ref, f"{what} seq {b}")
        exact = O.attend(hq[b], Kh, Vh, L - 1, lists, k=topk)
        q_err = H.attn_errors(ref, exact)[1]
        assert q_err <= FP8_VS_BF16_REL_RMS, f"{what} seq {b}: quantisation error {q_err:.3e}"
        worst = [max(worst[0], mx), max(worst[1], rr), max(worst[2], q_err)]
    print(f"{what}: worst max abs {worst[0]:.2e}, rel rms {worst[1]:.2e} vs the FP8 oracle; "
          f"FP8 vs bf16 rel rms {worst[2]:.2e}")


@pytest.mark.parametrize("lens,topk", [([5003, 1000, 17, 1], 512), ([3000, 2047, 4096], 37), ([600, 4104], 1)])
def test_fp8_decode_matches_oracle(lens, topk):
    seed = 0xF90 + len(lens) + topk
    r = H.run_dsa_decode(seed, lens, topk=topk, check_seqs=[])  # the (bf16) selection feeds both paths
    B, tcap = r["B"], r["tcap"]
    k8, v8, kvs = _write_fp8(seed, B, tcap)
    out = torch.empty(B * HQ * D, dtype=H.BF16, device="cuda")
    dsa.dsa_sparse_gqa_decode_fp8(r["dev"]["geom"], r["dev"]["q"], k8, v8, kvs, tcap, H.i32(lens),
                                  H.i32(r["sel"].ravel()), H.i32(r["nsel"].ravel()), out)
    torch.cuda.synchronize()
    hq, _, _ = H.host_queries(seed, B)
    _check_fp8_outputs(seed, H.bf16_np(out).reshape(B, HQ, D), lens, tcap, r["sel"], r["nsel"], topk, hq,
                       range(B), "fp8 decode")


def test_fp8_decode_step_1m_batch_of_4():
    """dsa_decode_step_fp8 at the benchmark's decode shape: the selection is bit for bit the bf16
    step's (the indexer path does not touch K/V), and sequences 0 and 3 meet the FP8 oracle."""
    seed, lens = 0xFA0, [1 << 20] * 4
    B, tcap = len(lens), 1 << 20
    R = tcap // 8
    geom = dsa.geometry()
    ik = H.dev_cache(seed, gi.TID_IK, B, tcap, P, tcap, gi.LAYOUT_GROUP_MAJOR, gi.IK_SCALE, True)
    q, iq, z = H.dev_queries(seed, B)
    lens_np = np.asarray(lens, dtype=np.int32)
    summ = torch.zeros(B * G * R * P, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(B * G * R, dtype=torch.float32, device="cuda")
    dsa.dsa_compress_regions(geom, ik, tcap, H.i32(np.zeros(B)), H.i32((lens_np - 1) // 8), R, summ, scale)
    summ2, scale2 = summ.clone(), scale.clone()
    k8, v8, kvs = _write_fp8(seed, B, tcap)
    sel1 = torch.empty(B * G * 512, dtype=torch.int32, device="cuda")
    n1 = torch.empty(B * G, dtype=torch.int32, device="cuda")
    o1 = torch.empty(B * HQ * D, dtype=H.BF16, device="cuda")
    dsa.dsa_decode_step_fp8(geom, q, iq, z, ik, k8, v8, kvs, tcap, H.i32(lens_np), summ, scale, R, sel1, n1, o1)
    del k8, v8, kvs
    torch.cuda.empty_cache()
    K = H.dev_cache(seed, gi.TID_K, B, tcap, D, tcap, gi.LAYOUT_KTILED)
    V = H.dev_cache(seed, gi.TID_V, B, tcap, D, tcap, gi.LAYOUT_REGION_T)
    sel2, n2, o2 = torch.empty_like(sel1), torch.empty_like(n1), torch.empty_like(o1)
    dsa.dsa_decode_step(geom, q, iq, z, ik, K, V, tcap, H.i32(lens_np), summ2, scale2, R, sel2, n2, o2)
    torch.cuda.synchronize()
    assert torch.equal(n1, n2) and torch.equal(sel1, sel2)
    assert torch.equal(summ, summ2) and torch.equal(scale.view(torch.int32), scale2.view(torch.int32))
    hq, _, _ = H.host_queries(seed, B)
    sel = sel1.cpu().numpy().reshape(B, G, 512)
    nsel = n1.cpu().numpy().reshape(B, G)
    _check_fp8_outputs(seed, H.bf16_np(o1).reshape(B, HQ, D), lens, tcap, sel, nsel, 512, hq, [0, 3],
                       "fp8 decode step 1M")


def test_fp8_prefill_matches_oracle():
    """Prefill chunks of two sequences (partial regions, mixed query blocks) over FP8 caches."""
    seed, seqs = 0xFB0, [(4003, 300), (1000, 77)]
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
    k8, v8, kvs = _write_fp8(seed, B, tcap)
    out = torch.empty(nq * HQ * D, dtype=H.BF16, device="cuda")
    dsa.dsa_sparse_gqa_prefill_fp8(geom, q, H.i32(qs), H.i32(qp), B, k8, v8, kvs, tcap, sel, nsel, out)
    torch.cuda.synchronize()
    gsel = sel.cpu().numpy().reshape(nq, G, 512)
    gn = nsel.cpu().numpy().reshape(nq, G)
    go = H.bf16_np(out).reshape(nq, HQ, D)
    hq, _, _ = H.host_queries(seed, nq)
    host = {}
    for b, (s0, n) in enumerate(seqs):
        L = s0 + n
        Kh = gi.host_tokens_bf16(seed, gi.TID_K, tcap, G, D, b, 0, L)
        Vh = gi.host_tokens_bf16(seed, gi.TID_V, tcap, G, D, b, 0, L)
        host[b] = (Kh, Vh) + O.quantize_rows(Kh) + O.quantize_rows(Vh)
    worst = 0.0
    for i in range(0, nq, 9):
        b, p = qs[i], qp[i]
        Kh, Vh, Kc, Ks, Vc, Vs = host[b]
        lists = [gsel[i, g, :gn[i, g]] for g in range(G)]
        ref = O.attend_fp8(hq[i], Kc, Ks, Vc, Vs, p, lists)
        H.assert_attn(go[i], ref, f"fp8 prefill query {i}")
        worst = max(worst, H.attn_errors(ref, O.attend(hq[i], Kh, Vh, p, lists))[1])
    assert worst <= FP8_VS_BF16_REL_RMS
    print(f"fp8 prefill: FP8 vs bf16 rel rms {worst:.2e}")
