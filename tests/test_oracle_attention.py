"""Pins the oracle's sparse GQA and sliding-window attention to textbook dense attention.

* topk >= number of regions  =>  sparse GQA equals dense causal GQA (torch SDPA, fp64, CPU);
* sliding window            =>  dense attention with a band mask (SDPA with an explicit mask);
* p = 0 => o = V[0]; identical keys => o = mean of V over the attended tokens; outputs are convex
  combinations of the attended V rows; at most 4096 tokens per query with k = 512.
"""
import math

import numpy as np
import pytest
import torch

from dsa_inputs import bf16_rne, bf16_to_f32

G, D, HQ, P, HI = 4, 192, 64, 256, 16
TAU = 1.0 / math.sqrt(D)


def _qkv(gen, seed, T, nq=1):
    q = gen.host_tokens_bf16(seed, 1, nq, HQ, D, 0, 0, 1)[0] if nq == 1 else None
    K = gen.host_tokens_bf16(seed, 2, T, G, D, 0, 0, T)
    V = gen.host_tokens_bf16(seed, 3, T, G, D, 0, 0, T)
    return q, K, V


def _sdpa(q, K, V, p, lo=0):
    """Dense GQA attention of one query at p over positions lo..p, fp64 CPU."""
    qt = torch.from_numpy(bf16_to_f32(q).astype(np.float64)).reshape(1, HQ, 1, D)
    Kt = torch.from_numpy(bf16_to_f32(K[lo:p + 1]).astype(np.float64)).permute(1, 0, 2)  # [G][n][D]
    Vt = torch.from_numpy(bf16_to_f32(V[lo:p + 1]).astype(np.float64)).permute(1, 0, 2)
    Kt = Kt.repeat_interleave(HQ // G, dim=0).unsqueeze(0)
    Vt = Vt.repeat_interleave(HQ // G, dim=0).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=TAU)
    return o.reshape(HQ, D).numpy()


@pytest.mark.parametrize("p", [0, 5, 7, 8, 63, 100, 257])
def test_all_regions_selected_equals_dense_causal(oracle_lib, gen_host, p):
    o = oracle_lib
    T = p + 1
    q, K, V = _qkv(gen_host, 31 + p, T)
    c = p // 8
    sel = [list(range(c + 1))] * G
    out = o.attend(q, K, V, p, sel)
    ref = _sdpa(q, K, V, p)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_end_to_end_query_dense_when_topk_covers(oracle_lib, gen_host):
    o = oracle_lib
    p = 150
    T = p + 1
    q, K, V = _qkv(gen_host, 41, T)
    ik = gen_host.host_index_k(41, T, G, P, 0, 0, T)
    codes, scales = o.compress_regions(ik, 0, T // 8)
    iq = gen_host.host_tokens_bf16(41, 5, 1, HI, P, 0, 0, 1, 1 / 16)[0]
    z = gen_host.host_uniform_f32(41, 6, HI)
    sel, nsel, out, _ = o.dsa_query(iq, z, codes, scales, q, K, V, p, k=512)
    assert np.all(nsel == p // 8 + 1)
    assert np.max(np.abs(out - _sdpa(q, K, V, p))) < 1e-12


def test_first_token_returns_its_value(oracle_lib, gen_host):
    q, K, V = _qkv(gen_host, 51, 1)
    out = oracle_lib.attend(q, K, V, 0, [[0]] * G)
    want = np.repeat(bf16_to_f32(V[0]).astype(np.float64), HQ // G, axis=0)
    assert np.array_equal(out, want)


def test_identical_keys_average_values(oracle_lib, gen_host):
    o = oracle_lib
    T = 40
    q, K, V = _qkv(gen_host, 52, T)
    K[:] = K[0]
    sel = [[0, 2, 4]] * G  # regions 0, 2, 4 -> tokens 0..7, 16..23, 32..39 (p = 39)
    out = o.attend(q, K, V, 39, sel)
    toks = list(range(0, 8)) + list(range(16, 24)) + list(range(32, 40))
    mean = bf16_to_f32(V[toks]).astype(np.float64).mean(axis=0)  # [G][D]
    want = np.repeat(mean, HQ // G, axis=0)
    assert np.max(np.abs(out - want)) < 1e-12


def test_sparse_is_dense_over_selected_tokens_and_convex(oracle_lib, gen_host):
    o = oracle_lib
    T = 200
    p = 197  # current region 24 is partial (192..197)
    q, K, V = _qkv(gen_host, 53, T)
    rng = np.random.default_rng(0)
    sel = [sorted(rng.choice(24, size=5, replace=False).tolist() + [24]) for _ in range(G)]
    out = o.attend(q, K, V, p, sel, k=6)
    Vf = bf16_to_f32(V).astype(np.float64)
    for h in range(HQ):
        g = h // (HQ // G)
        toks = [t for r in sel[g] for t in range(8 * r, 8 * r + 8) if t <= p]
        assert len(toks) <= 4096
        lo = Vf[toks, g].min(axis=0)
        hi = Vf[toks, g].max(axis=0)
        assert np.all(out[h] >= lo - 1e-12) and np.all(out[h] <= hi + 1e-12)
    # group 0's output = dense attention restricted to its tokens (gather then SDPA)
    toks = [t for r in sel[0] for t in range(8 * r, 8 * r + 8) if t <= p]
    qt = torch.from_numpy(bf16_to_f32(q[:16]).astype(np.float64)).unsqueeze(1)
    Kt = torch.from_numpy(bf16_to_f32(K[toks, 0]).astype(np.float64)).unsqueeze(0).expand(16, -1, -1)
    Vt = torch.from_numpy(bf16_to_f32(V[toks, 0]).astype(np.float64)).unsqueeze(0).expand(16, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=TAU).squeeze(1).numpy()
    assert np.max(np.abs(out[:16] - ref)) < 1e-12


@pytest.mark.parametrize("p,W", [(0, 512), (300, 512), (511, 512), (512, 512), (1500, 512), (90, 64)])
def test_swa_equals_band_masked_dense(oracle_lib, gen_host, p, W):
    o = oracle_lib
    T = p + 1
    q, K, V = _qkv(gen_host, 61 + p, T)
    out = o.swa(q, K, V, p, W)
    # dense attention over all 0..p with an explicit band mask
    qt = torch.from_numpy(bf16_to_f32(q).astype(np.float64)).reshape(1, HQ, 1, D)
    Kt = torch.from_numpy(bf16_to_f32(K).astype(np.float64)).permute(1, 0, 2).repeat_interleave(16, 0)[None]
    Vt = torch.from_numpy(bf16_to_f32(V).astype(np.float64)).permute(1, 0, 2).repeat_interleave(16, 0)[None]
    pos = torch.arange(T)
    mask = (pos <= p) & (pos > p - W)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask.view(1, 1, 1, T), scale=TAU)
    assert np.max(np.abs(out - ref.reshape(HQ, D).numpy())) < 1e-12


def test_swa_wide_window_is_full_causal(oracle_lib, gen_host):
    q, K, V = _qkv(gen_host, 70, 300)
    out = oracle_lib.swa(q, K, V, 299, 10_000)
    assert np.max(np.abs(out - _sdpa(q, K, V, 299))) < 1e-12
