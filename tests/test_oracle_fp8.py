"""Pins the oracle's FP8 K/V cache path (the pages: an FP8 KV cache halves it; the per-row rule is the
stand-in of the summaries applied to each cached (token, group) row):

* the row quantiser against closed forms and against a brute-force nearest-code search over the
  E4M3 value table (pinned to the OCP spec by test_oracle_e4m3);
* sparse attention over the FP8 cache equals the bf16 oracle when every row is exactly representable
  (row maxima 448 * 2^e, values = E4M3 values * 2^e), so the dequantisation has no error to hide;
* p = 0 gives the dequantised V row; outputs are convex combinations of the dequantised V rows.
"""
import math

import numpy as np
import pytest

from dsa_inputs import bf16_rne, bf16_to_f32

G, D, HQ = 4, 192, 64
TAU = 1.0 / math.sqrt(D)


def _table(o):
    codes = np.array([c for c in range(128) if not math.isnan(o.e4m3_value(c))])
    return codes, np.array([o.e4m3_value(c) for c in codes])


def _nearest(x, codes, values):
    """Nearest non-negative code to |x| (ties to the even code), sign from x, saturating at 448."""
    a = abs(float(x))
    d = np.abs(values - a)
    best = d.min()
    tied = codes[d == best]
    if len(tied) > 1:
        tied = tied[tied % 2 == 0]
    c = int(tied[0])
    return c | (0x80 if (x < 0 or (x == 0 and math.copysign(1.0, x) < 0)) else 0)


def test_quantize_rows_closed_forms(oracle_lib):
    o = oracle_lib
    rows = np.zeros((4, D), dtype=np.float32)
    rows[0, :] = 0.75                 # equal values: every code is the largest, scale = 0.75/448
    rows[1, :] = -2.5
    rows[2, 17] = 3.0                 # one non-zero element
    # rows[3] all zero: scale 0, codes 0
    codes, scales = o.quantize_rows(bf16_rne(rows))
    assert np.all(codes[0] == 0x7E) and scales[0] == np.float32(0.75) / np.float32(448.0)
    assert np.all(codes[1] == 0xFE) and scales[1] == np.float32(2.5) / np.float32(448.0)
    assert codes[2, 17] == 0x7E and not np.delete(codes[2], 17).any()
    assert scales[3] == 0.0 and not codes[3].any()


def test_quantize_rows_matches_brute_force(oracle_lib, gen_host):
    o = oracle_lib
    X = gen_host.host_tokens_bf16(0xF8, 2, 64, G, D, 0, 0, 12)  # 12 tokens x 4 groups of N(0,1) rows
    codes, scales = o.quantize_rows(X)
    tab_c, tab_v = _table(o)
    xf = bf16_to_f32(X).reshape(-1, D)
    for i in range(xf.shape[0]):
        amax = np.float32(np.abs(xf[i]).max())
        sc = np.float32(amax / np.float32(448.0))
        assert scales.reshape(-1)[i] == sc
        for d in range(0, D, 7):
            q = np.float32(xf[i, d] / sc)
            assert codes.reshape(-1, D)[i, d] == _nearest(q, tab_c, tab_v), (i, d)
        # the row maximum always lands on the largest code
        assert (codes.reshape(-1, D)[i] & 0x7F).max() == 0x7E


def _exact_rows(rng, T):
    """[T][G][D] bf16 rows whose values are E4M3 values times 2^e with one element of magnitude 448*2^e."""
    o_codes = rng.integers(0, 0x7F, size=(T, G, D))
    o_codes = np.where(o_codes == 0x7F, 0x7E, o_codes) | (rng.integers(0, 2, size=(T, G, D)) << 7)
    e = rng.integers(-12, -6, size=(T, G, 1))
    o_codes[:, :, 5] = 0x7E | (rng.integers(0, 2, size=(T, G)) << 7)
    return o_codes.astype(np.uint8), e


def test_attend_fp8_equals_bf16_attention_on_exact_rows(oracle_lib, gen_host):
    o = oracle_lib
    rng = np.random.default_rng(3)
    T, p = 40, 37
    kc, ke = _exact_rows(rng, T)
    vc, ve = _exact_rows(rng, T)
    val = np.vectorize(o.e4m3_value)
    K = bf16_rne((val(kc) * np.exp2(ke)).astype(np.float32))
    V = bf16_rne((val(vc) * np.exp2(ve)).astype(np.float32))
    q = gen_host.host_tokens_bf16(0xF9, 1, 1, HQ, D, 0, 0, 1)[0]
    Kc, Ks = o.quantize_rows(K)
    Vc, Vs = o.quantize_rows(V)
    # the quantiser recovers the codes and the power-of-two scales exactly
    assert np.array_equal(Kc, kc) and np.array_equal(Vc, vc)
    assert np.array_equal(Ks, np.exp2(ke[..., 0]).astype(np.float32))
    sel = [np.array([0, 2, 4], dtype=np.int32)] * G  # region 4 holds the partial current region (p = 37)
    a = o.attend_fp8(q, Kc, Ks, Vc, Vs, p, sel, k=8)
    b = o.attend(q, K, V, p, sel, k=8)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)


def test_attend_fp8_first_token_and_convexity(oracle_lib, gen_host):
    o = oracle_lib
    T = 24
    K = gen_host.host_tokens_bf16(0xFA, 2, T, G, D, 0, 0, T)
    V = gen_host.host_tokens_bf16(0xFA, 3, T, G, D, 0, 0, T)
    q = gen_host.host_tokens_bf16(0xFA, 1, 1, HQ, D, 0, 0, 1)[0]
    Kc, Ks = o.quantize_rows(K)
    Vc, Vs = o.quantize_rows(V)
    val = np.vectorize(o.e4m3_value)
    Vd = val(Vc) * Vs[..., None].astype(np.float64)  # dequantised V [T][G][D]
    out0 = o.attend_fp8(q, Kc, Ks, Vc, Vs, 0, [np.array([0])] * G, k=4)
    for h in range(HQ):
        assert np.allclose(out0[h], Vd[0, h // 16], rtol=0, atol=1e-15)
    p = 20
    out = o.attend_fp8(q, Kc, Ks, Vc, Vs, p, [np.array([0, 1, 2])] * G, k=4)
    for h in range(HQ):
        vv = Vd[:p + 1, h // 16]
        assert np.all(out[h] <= vv.max(axis=0) + 1e-12) and np.all(out[h] >= vv.min(axis=0) - 1e-12)
