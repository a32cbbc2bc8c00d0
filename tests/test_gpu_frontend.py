"""Indexer front-end (projection, RMSNorm, partial RoPE) and the attention's partial RoPE through
the C ABI, against the fp64 oracle of oracle/frontend.py on seeded inputs: ragged token counts around
the 128-token tile, positions from 0 to 2^20 - 1, and the 2048-token chunk at hidden 6144 (sampled
tokens).  Tolerances: the index vectors and rotated Q/K are bf16 (one rounding of values near 1: at
most 2^-8 relative, plus 2e-3 absolute for the fp32 GEMM and rotation); z is fp32, within 1e-5 of the
sum of |x_i w_i|."""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
import dsa_sparse_attention_amd as dsa
from oracle import frontend as F

import _harness as H

pytestmark = pytest.mark.gpu


def _up_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).ravel()).cuda().view(torch.bfloat16)


def _check_bf16(gpu, ref, what):
    err = np.abs(gpu - ref)
    bad = err > 2.0 ** -8 * np.abs(ref) + 2e-3
    assert not bad.any(), f"{what}: {bad.sum()} elements off, worst {err.max():.3e}"
    rr = np.sqrt((err ** 2).sum() / (ref ** 2).sum())
    assert rr <= 3e-3, f"{what}: rel rms {rr:.3e}"
    return err.max(), rr


def _positions(seed, T):
    rng = np.random.default_rng(seed)
    p = rng.integers(0, 1 << 20, T).astype(np.int32)
    p[0] = 0
    if T > 1:
        p[-1] = (1 << 20) - 1
    return p


@pytest.mark.parametrize("T,Hd,sample", [
    (1, 128, None), (4, 6144, None), (37, 256, None), (64, 512, None),   # split-K path (<= 64 tokens)
    (65, 256, None), (300, 1024, None), (2048, 6144, 61),                # tiled path (ragged 128-token tiles)
])
def test_indexer_project_matches_oracle(T, Hd, sample):
    seed = 0xE00 + T
    rows = dsa.IDX_PROJ_ROWS
    x, w, gq, gk = gi.host_frontend_inputs(seed, T, Hd, rows)
    pos = _positions(seed, T)
    rope = dsa.rope_config()
    iq = torch.empty(T * 16 * 256, dtype=torch.bfloat16, device="cuda")
    ik = torch.empty(T * 4 * 256, dtype=torch.bfloat16, device="cuda")
    z = torch.empty(T * 16, dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_project(rope, _up_bf16(x), _up_bf16(w), torch.from_numpy(gq).cuda(),
                            torch.from_numpy(gk).cuda(), H.i32(pos), iq, ik, z, Hd)
    torch.cuda.synchronize()
    toks = np.arange(T) if sample is None else np.unique(np.r_[0, np.arange(1, T, sample), T - 1])
    giq = H.bf16_np(iq).reshape(T, 16, 256)[toks]
    gik = H.bf16_np(ik).reshape(T, 4, 256)[toks]
    gz = z.cpu().numpy().reshape(T, 16)[toks]
    oiq, oik, oz = F.indexer_frontend(x[toks], w, gq, gk, pos[toks])
    m1 = _check_bf16(giq, oiq, "index_q")
    m2 = _check_bf16(gik, oik, "index_k")
    xf, wf = F.bf16_to_f64(x[toks]), F.bf16_to_f64(w[-16:])
    bound = 1e-5 * (np.abs(xf) @ np.abs(wf).T)
    assert np.all(np.abs(gz - oz) <= bound), f"z off by {np.abs(gz - oz).max():.3e}"
    print(f"T={T} H={Hd}: index_q max {m1[0]:.2e} rel-rms {m1[1]:.2e}; index_k max {m2[0]:.2e}")


def test_rope_qk_matches_oracle():
    seed, T = 0xE80, 67
    q = gi.host_normal_bf16(seed, gi.TID_Q, T * 64 * 192).reshape(T, 64, 192)
    k = gi.host_normal_bf16(seed, gi.TID_K, T * 4 * 192).reshape(T, 4, 192)
    pos = _positions(seed, T)
    qd, kd = _up_bf16(q), _up_bf16(k)
    dsa.dsa_rope_qk(dsa.rope_config(), H.i32(pos), qd, kd)
    torch.cuda.synchronize()
    gq = qd.view(torch.int16).cpu().numpy().view(np.uint16).reshape(T, 64, 192)
    gk = kd.view(torch.int16).cpu().numpy().view(np.uint16).reshape(T, 4, 192)
    oq, ok = F.rope_qk(q, k, pos)
    _check_bf16(F.bf16_to_f64(gq), oq, "q")
    _check_bf16(F.bf16_to_f64(gk), ok, "k")
    # dimensions 64.. are untouched, bit for bit; position 0 is the identity
    assert np.array_equal(gq[:, :, 64:], q[:, :, 64:]) and np.array_equal(gk[:, :, 64:], k[:, :, 64:])
    assert np.array_equal(gq[0], q[0]) and np.array_equal(gk[0], k[0])


def test_frontend_feeds_the_selection():
    """index_q / index_k / z from the front-end go straight into cache write, compression and
    score_topk (layouts agree): the selection meets the oracle's selection over the same vectors."""
    import oracle as O
    seed, L, Hd = 0xE90, 1024, 256
    rows = dsa.IDX_PROJ_ROWS
    x, w, gq, gk = gi.host_frontend_inputs(seed, L, Hd, rows)
    pos = np.arange(L, dtype=np.int32)
    iq = torch.empty(L * 16 * 256, dtype=torch.bfloat16, device="cuda")
    ik = torch.empty(L * 4 * 256, dtype=torch.bfloat16, device="cuda")
    z = torch.empty(L * 16, dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_project(dsa.rope_config(), _up_bf16(x), _up_bf16(w), torch.from_numpy(gq).cuda(),
                            torch.from_numpy(gk).cuda(), H.i32(pos), iq, ik, z, Hd)
    geom = dsa.geometry(topk=64)
    tcap, R = L, L // 8
    K = torch.zeros(4 * tcap * 192, dtype=torch.bfloat16, device="cuda")
    V = torch.zeros_like(K)
    ikc = torch.zeros(4 * tcap * 256, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(L * 4 * 192, dtype=torch.bfloat16, device="cuda")
    dsa.dsa_cache_write(geom, H.i32(np.zeros(L)), H.i32(pos), kv, kv, ik, K, V, ikc, 1, tcap)
    summ = torch.zeros(4 * R * 256, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(4 * R, dtype=torch.float32, device="cuda")
    dsa.dsa_compress_regions(geom, ikc, tcap, H.i32([0]), H.i32([R]), R, summ, scale)
    qi = L - 1
    sel = torch.empty(4 * 64, dtype=torch.int32, device="cuda")
    nsel = torch.empty(4, dtype=torch.int32, device="cuda")
    scores = torch.zeros(4 * R, dtype=torch.float32, device="cuda")
    dsa.dsa_score_topk(geom, iq[qi * 4096:(qi + 1) * 4096], z[qi * 16:(qi + 1) * 16], H.i32([0]), H.i32([qi]), 1,
                       summ, scale, tcap, R, sel, nsel, scores_out=scores)
    torch.cuda.synchronize()
    ikh = ik.view(torch.int16).cpu().numpy().view(np.uint16).reshape(L, 4, 256)
    codes, scs = O.compress_regions(ikh, 0, R)
    iqh = iq.view(torch.int16).cpu().numpy().view(np.uint16).reshape(L, 16, 256)[qi]
    osc = O.scores(iqh, z.cpu().numpy().reshape(L, 16)[qi], codes, scs, qi // 8)
    gsel = sel.cpu().numpy().reshape(4, 64)
    gn = nsel.cpu().numpy()
    for g in range(4):
        osel = O.select(osc[g], qi // 8, k=64)
        assert gn[g] == len(osel)
        assert H.check_selection(sorted(gsel[g, :gn[g]].tolist()), sorted(osel), osc[g], qi // 8), g
