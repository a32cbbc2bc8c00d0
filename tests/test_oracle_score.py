"""Pins the oracle's indexer score to closed forms (one-hot queries) and to its algebraic properties.

Stand-in rule: s_g(r) = sum_{h in 4g..4g+3} z_h * ReLU(q_h . S_g[r]), S = dequantised summary.
"""
import numpy as np

from dsa_inputs import bf16_rne

G, P, HI = 4, 256, 16


def _summaries(o, gen, seed, R):
    ik = gen.host_index_k(seed, 8 * R, G, P, 0, 0, 8 * R)
    return o.compress_regions(ik, 0, R)


def test_one_hot_queries(oracle_lib, gen_host):
    o = oracle_lib
    R = 6
    codes, scales = _summaries(o, gen_host, 21, R)
    rng = np.random.default_rng(3)
    for trial in range(20):
        h = int(rng.integers(0, HI))
        d = int(rng.integers(0, P))
        iq = np.zeros((HI, P), dtype=np.float32)
        iq[h, d] = 1.0
        z = rng.uniform(0, 1, HI).astype(np.float32)
        s = o.scores(bf16_rne(iq), z, codes, scales, R)
        g_h = h // 4
        for g in range(G):
            for r in range(R):
                want = 0.0
                if g == g_h:
                    want = float(z[h]) * max(0.0, o.e4m3_value(codes[r, g, d]) * float(scales[r, g]))
                assert s[g, r] == want


def test_heads_add_with_their_weights(oracle_lib, gen_host):
    o = oracle_lib
    R = 5
    codes, scales = _summaries(o, gen_host, 22, R)
    iq = np.zeros((HI, P), dtype=np.float32)
    # heads 4..7 (group 1) one-hot at different channels, negative on head 6
    chans = {4: 3, 5: 100, 6: 200, 7: 255}
    for h, d in chans.items():
        iq[h, d] = -2.0 if h == 6 else 0.5
    z = np.array([0.1 * (i + 1) for i in range(HI)], dtype=np.float32)
    s = o.scores(bf16_rne(iq), z, codes, scales, R)
    for r in range(R):
        want = 0.0
        for h, d in chans.items():
            v = float(iq[h, d]) * (o.e4m3_value(codes[r, 1, d]) * float(scales[r, 1]))
            want += float(z[h]) * max(0.0, v)
        assert abs(s[1, r] - want) <= 1e-15 * max(1.0, abs(want))
        assert s[0, r] == 0 and s[2, r] == 0 and s[3, r] == 0


def test_scaling_and_relu_properties(oracle_lib, gen_host):
    o = oracle_lib
    R = 32
    codes, scales = _summaries(o, gen_host, 23, R)
    iq = gen_host.host_tokens_bf16(24, 5, 1, HI, P, 0, 0, 1, 1 / 16)[0]
    z = gen_host.host_uniform_f32(24, 6, HI)
    s1 = o.scores(iq, z, codes, scales, R)
    s2 = o.scores(iq, (2 * z).astype(np.float32), codes, scales, R)
    assert np.allclose(s2, 2 * s1, rtol=1e-15, atol=0)
    assert np.all(s1 >= 0)
    # negating every query head flips each dot's sign: s(q) + s(-q) = sum z |q.S|
    neg = (iq ^ np.uint16(0x8000)).astype(np.uint16)
    s3 = o.scores(neg, z, codes, scales, R)
    assert np.all(s1 + s3 > 0)
    # doubling the scale of region 0 doubles its score only (dequantised summary is code * scale)
    sc2 = scales.copy()
    sc2[0] *= 2
    s4 = o.scores(iq, z, codes, sc2, R)
    assert np.allclose(s4[:, 0], 2 * s1[:, 0], rtol=1e-15) and np.array_equal(s4[:, 1:], s1[:, 1:])
