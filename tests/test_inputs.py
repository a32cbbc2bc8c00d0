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


def test_correlated_chunk_recipe(gen_host):
    """The correlated prefill chunk: noise 1 gives the i.i.d. index_q back bit for bit; with no noise,
    query 64a is anchor a itself (t = 0) and z runs linearly between anchors; neighbouring queries are
    far closer than unrelated ones."""
    import dsa_inputs as gi
    seed, n = 0xC0, 200
    iq1, _ = gi.host_correlated_index_queries(seed, n, noise=1.0)
    own = gi.host_normal_bf16(seed, gi.TID_IQ, n * 16 * 256, gi.IK_SCALE).reshape(n, 16, 256)
    assert np.array_equal(iq1, own)
    iq0, z0 = gi.host_correlated_index_queries(seed, n, noise=0.0)
    anchors = gi.host_normal_bf16(seed, gi.TID_IQ_ANCHOR, (n // 64 + 2) * 16 * 256, gi.IK_SCALE).reshape(-1, 16, 256)
    za = gi.host_uniform_f32(seed, gi.TID_Z_ANCHOR, (n // 64 + 2) * 16).reshape(-1, 16)
    for a in range(n // 64 + 1):
        if 64 * a < n:
            assert np.array_equal(iq0[64 * a], anchors[a])
            assert np.array_equal(z0[64 * a], za[a])
    assert np.allclose(z0[32], 0.5 * (za[0] + za[1]), rtol=1e-6)
    iq, _ = gi.host_correlated_index_queries(seed, n)
    f = gi.bf16_to_f32(iq).reshape(n, -1)
    near = np.mean([np.corrcoef(f[i], f[i + 1])[0, 1] for i in range(0, n - 1, 7)])
    far = np.mean([np.corrcoef(f[i], f[(i + 97) % n])[0, 1] for i in range(0, n, 7)])
    assert near > 0.95 and far < 0.6, (near, far)
