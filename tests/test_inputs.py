"""The C host generator reproduces the numpy definition bit for bit; recipe statistics are sane."""
import numpy as np

import dsa_inputs as gi


def test_host_normal_matches_reference(gen_host):
    idx = np.arange(1000, 5000, dtype=np.uint64)
    ref = gi.bf16_rne(gi.ref_normal_f32(77, 4, idx) * np.float32(1 / 16))
    got = gi.host_normal_bf16(77, 4, 4000, 1 / 16, start=1000)
    assert np.array_equal(ref, got)


def test_host_tokens_and_uniform_match_reference(gen_host):
    assert np.array_equal(gi.ref_tokens_bf16(9, 2, 100, 4, 192, 1, 37, 6), gi.host_tokens_bf16(9, 2, 100, 4, 192, 1, 37, 6))
    idx = np.arange(300, dtype=np.uint64)
    assert np.array_equal(gi.ref_uniform_f32(9, 6, idx), gi.host_uniform_f32(9, 6, 300))


def test_host_index_k_planted_matches_reference(gen_host):
    T = 8 * 400
    # find a planted region of sequence 1 and compare a slice around it
    mask = gi.host_bernoulli(5, gi.TID_MASK, 400, start=400)
    r = int(np.flatnonzero(mask)[0])
    ref = gi.ref_index_k(5, T, 4, 256, 1, 8 * r - 8, 24, planted=True)
    got = gi.host_index_k(5, T, 4, 256, 1, 8 * r - 8, 24, planted=True)
    assert np.array_equal(ref, got)
    plain = gi.host_index_k(5, T, 4, 256, 1, 8 * r - 8, 24, planted=False)
    assert np.array_equal(plain[:8], got[:8]) and not np.array_equal(plain[8:16], got[8:16])


def test_recipe_statistics(gen_host):
    x = gi.bf16_to_f32(gi.host_normal_bf16(1, 2, 200_000))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01 and np.abs(x).max() <= 6
    u = gi.host_uniform_f32(1, 6, 100_000)
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.01
    b = gi.host_bernoulli(1, 7, 200_000)
    assert abs(b.mean() - 0.02) < 0.002


def test_hadamard_rows_orthonormal():
    d = np.arange(256, dtype=np.uint32)
    H = np.stack([gi.ref_hadamard16(r, d) for r in range(1, 17)]).astype(np.float64)
    assert np.allclose(H @ H.T, np.eye(16))
