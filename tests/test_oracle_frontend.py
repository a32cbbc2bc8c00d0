"""Pins of the oracle's indexer front-end (oracle/frontend.py) against facts other than its own formulas:
hand-derived values of the llama3 frequency scaling, the continuity of its three branches, special cases
that reduce to plain RoPE, the rotation's invariants (identity at position 0, pair norms, dependence on
the position difference only, the rotate-half pairing and sign on unit vectors), a worked RMSNorm
example and its invariances, and a brute-force projection."""
import math

import numpy as np

from oracle import frontend as F

L3 = dict(F.LLAMA3)


def _freq_with_wavelen(w):
    return 2.0 * math.pi / w


def test_llama3_worked_value():
    # wavelength 65536 with original 1,048,576 positions, factors 1 and 32, factor 8: the position in the
    # ramp is (1,048,576/65,536 - 1)/(32 - 1) = 15/31, so the frequency becomes
    # (16/31)/8 + 15/31 = 17/31 of the base one (worked by hand)
    f = _freq_with_wavelen(65536.0)
    assert math.isclose(F.llama3_scale_freq(f, **L3), f * 17.0 / 31.0, rel_tol=1e-12)
    # wavelength 32768 sits on the upper edge (ramp position 1): unchanged; 1,048,576 on the lower edge
    # (ramp position 0): divided by the factor
    for w, want in ((32768.0, 1.0), (1048576.0, 1.0 / 8.0)):
        f = _freq_with_wavelen(w)
        assert math.isclose(F.llama3_scale_freq(f, **L3), f * want, rel_tol=1e-12)


def test_llama3_branches_are_continuous_and_monotone():
    for edge in (32768.0, 1048576.0):
        lo = F.llama3_scale_freq(_freq_with_wavelen(edge * (1 - 1e-9)), **L3)
        hi = F.llama3_scale_freq(_freq_with_wavelen(edge * (1 + 1e-9)), **L3)
        assert math.isclose(lo, hi, rel_tol=1e-6)
    ws = np.geomspace(2 * math.pi, 1e8, 400)
    fs = [F.llama3_scale_freq(_freq_with_wavelen(w), **L3) for w in ws]
    assert all(a > b for a, b in zip(fs, fs[1:]))  # longer wavelength, lower frequency
    assert fs[0] == _freq_with_wavelen(ws[0])      # short wavelengths untouched


def test_factor_one_is_plain_rope():
    fr = F.inv_freq(64, 10000.0, factor=1.0)
    plain = 10000.0 ** (-np.arange(32) / 32.0)
    assert np.allclose(fr, plain, rtol=1e-14, atol=0)
    # the default: the 32 base frequencies' wavelengths run from 2*pi to about 47,000 positions, so only
    # those above 32,768 (the last two) are scaled, and none reaches the lower edge
    fr = F.inv_freq()
    base = 10000.0 ** (-np.arange(32) / 32.0)
    changed = ~np.isclose(fr, base, rtol=1e-15, atol=0)
    assert changed.tolist() == [False] * 30 + [True, True]
    assert np.all(fr[30:] > base[30:] / 8) and np.all(fr[30:] < base[30:])


def test_rope_invariants():
    rng = np.random.default_rng(1)
    fr = F.inv_freq()
    x = rng.standard_normal((5, 3, 256))
    pos = np.array([0, 1, 17, 65535, 1048575])
    y = F.rope(x, pos, fr)
    assert np.array_equal(y[0], x[0])                        # position 0: identity
    assert np.array_equal(y[:, :, 64:], x[:, :, 64:])        # only the first 64 dims rotate
    nx = x[:, :, :32] ** 2 + x[:, :, 32:64] ** 2             # each pair keeps its length
    ny = y[:, :, :32] ** 2 + y[:, :, 32:64] ** 2
    assert np.allclose(nx, ny, rtol=1e-12, atol=1e-12)
    # scores depend on the position difference only
    q, k = rng.standard_normal(256), rng.standard_normal(256)
    for m, n, d in ((5, 2, 100), (70000, 3, 900000), (1, 1, 12345)):
        a = F.rope(q[None, None], [m], fr)[0, 0] @ F.rope(k[None, None], [n], fr)[0, 0]
        b = F.rope(q[None, None], [m + d], fr)[0, 0] @ F.rope(k[None, None], [n + d], fr)[0, 0]
        assert math.isclose(a, b, rel_tol=1e-9, abs_tol=1e-9)


def test_rope_pairing_and_sign_on_unit_vectors():
    fr = F.inv_freq()
    p = 1234
    for i in (0, 7, 31):
        e = np.zeros((1, 1, 256))
        e[0, 0, i] = 1.0
        y = F.rope(e, [p], fr)[0, 0]
        a = p * fr[i]
        want = np.zeros(256)
        want[i], want[i + 32] = math.cos(a), math.sin(a)   # e_i turns towards e_{i+32}
        assert np.allclose(y, want, atol=1e-15)
        e2 = np.zeros((1, 1, 256))
        e2[0, 0, i + 32] = 1.0
        y2 = F.rope(e2, [p], fr)[0, 0]
        want2 = np.zeros(256)
        want2[i], want2[i + 32] = -math.sin(a), math.cos(a)
        assert np.allclose(y2, want2, atol=1e-15)


def test_rms_norm_worked_example_and_invariances():
    # [3, 4]: mean square 12.5, root 3.5355339...; with eps 0: [0.8485281, 1.1313708]
    y = F.rms_norm(np.array([3.0, 4.0]), np.ones(2), eps=0.0)
    assert np.allclose(y, [0.848528137423857, 1.131370849898476], rtol=1e-14)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 256))
    g = rng.uniform(0.5, 1.5, 256)
    assert np.allclose(F.rms_norm(7.5 * x, g, eps=0.0), F.rms_norm(x, g, eps=0.0), rtol=1e-13)
    assert np.allclose(np.sqrt((F.rms_norm(x, np.ones(256), eps=0.0) ** 2).mean(-1)), 1.0, rtol=1e-13)


def _bits(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_frontend_projection_brute_force_and_norms():
    rng = np.random.default_rng(3)
    T, H = 3, 16
    N = 16 * 256 + 4 * 256 + 16
    xb = _bits(rng.standard_normal((T, H)))
    wb = _bits(rng.standard_normal((N, H)) / 4)
    pos = [0, 5, 1000]
    iq, ik, z = F.indexer_frontend(xb, wb, np.ones(256), np.ones(256), pos)
    x, w = F.bf16_to_f64(xb), F.bf16_to_f64(wb)
    # z: brute-force dot products
    for t in range(T):
        for h in range(16):
            acc = 0.0
            for c in range(H):
                acc += x[t, c] * w[16 * 256 + 4 * 256 + h, c]
            assert math.isclose(z[t, h], acc, rel_tol=1e-12, abs_tol=1e-12)
    # unit gains: every index vector has length 16 (= sqrt(256)) up to eps, rotation included
    assert np.allclose(np.linalg.norm(iq, axis=-1), 16.0, rtol=1e-5)
    assert np.allclose(np.linalg.norm(ik, axis=-1), 16.0, rtol=1e-5)
    # position 0 is not rotated: token 0's vectors are the normalised projections themselves
    for h in range(16):
        y = np.array([sum(x[0, c] * w[h * 256 + j, c] for c in range(H)) for j in range(256)])
        assert np.allclose(iq[0, h], y / math.sqrt((y * y).mean() + F.EPS), rtol=1e-10)
    # the un-rotated tail of a later token matches its normalised projection
    y = np.array([sum(x[2, c] * w[16 * 256 + 2 * 256 + j, c] for c in range(H)) for j in range(256)])
    assert np.allclose(ik[2, 2, 64:], (y / math.sqrt((y * y).mean() + F.EPS))[64:], rtol=1e-10)
