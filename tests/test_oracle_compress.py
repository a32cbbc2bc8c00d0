"""Pins the oracle's region compression to closed forms and invariants.

Stand-in rule (the pages give no maths for the summary): mean of the region's 8 index_k rows of the
group, E4M3 codes with one fp32 scale amax/448 per (region, group).
"""
import numpy as np
import pytest

from dsa_inputs import bf16_rne, bf16_to_f32

G, P = 4, 256


def _rows(vals):
    """vals [8][G][P] float32 -> bf16 bits (values chosen bf16-exact)."""
    return bf16_rne(np.asarray(vals, dtype=np.float32))


def test_equal_rows_give_the_row(oracle_lib):
    o = oracle_lib
    rng = np.random.default_rng(1)
    x = bf16_to_f32(bf16_rne(rng.normal(0, 0.1, (G, P)).astype(np.float32)))
    ik = _rows(np.broadcast_to(x, (8, G, P)))
    codes, scales = o.compress_regions(ik, 0, 1)
    for g in range(G):
        amax = np.abs(x[g]).max()
        assert scales[0, g] == np.float32(amax) / np.float32(448.0)
        deq = np.array([o.e4m3_value(c) for c in codes[0, g]]) * float(scales[0, g])
        # E4M3 keeps 4 significant bits: relative error <= 2^-4 for normals, absolute 2^-10*scale below
        err = np.abs(deq - x[g])
        bound = np.maximum(np.abs(x[g]) * 2.0 ** -4, 2.0 ** -10 * float(scales[0, g]))
        assert np.all(err <= bound * (1 + 1e-12))
        # the largest element maps exactly to +-448
        j = int(np.argmax(np.abs(x[g])))
        assert codes[0, g, j] in (0x7E, 0xFE)
        assert (codes[0, g, j] == 0xFE) == (x[g, j] < 0)


def test_single_nonzero_element(oracle_lib):
    o = oracle_lib
    vals = np.zeros((8, G, P), dtype=np.float32)
    vals[3, 2, 17] = -0.75  # only token 3, group 2, channel 17
    codes, scales = o.compress_regions(_rows(vals), 0, 1)
    assert scales[0, 2] == np.float32(0.75 / 8) / np.float32(448)
    assert codes[0, 2, 17] == 0xFE
    assert np.count_nonzero(codes[0, 2]) == 1
    for g in (0, 1, 3):  # other groups untouched: amax 0 -> scale 0, codes 0
        assert scales[0, g] == 0 and not codes[0, g].any()


def test_mean_uses_all_eight_rows_in_order(oracle_lib):
    o = oracle_lib
    # row t holds 2^t at channel 0 of group 0: mean = 255/8
    vals = np.zeros((8, G, P), dtype=np.float32)
    for t in range(8):
        vals[t, 0, 0] = 2.0 ** t
    vals[:, 0, 1] = 1.0  # channel 1: mean 1
    codes, scales = o.compress_regions(_rows(vals), 0, 1)
    assert scales[0, 0] == np.float32(255.0 / 8) / np.float32(448)
    assert codes[0, 0, 0] == 0x7E
    deq1 = o.e4m3_value(codes[0, 0, 1]) * float(scales[0, 0])
    assert abs(deq1 - 1.0) <= 2.0 ** -4


def test_invariants_on_random_regions(oracle_lib, gen_host):
    o = oracle_lib
    T = 64
    ik = gen_host.host_index_k(11, T, G, P, 0, 0, T)
    codes, scales = o.compress_regions(ik, 0, T // 8)
    x = bf16_to_f32(ik).astype(np.float64)
    for r in range(T // 8):
        mean = x[8 * r:8 * r + 8].mean(axis=0)  # exact fp64 mean
        for g in range(G):
            a = np.abs(mean[g]).max()
            # fp32 summation in order differs from the exact mean by a few ulp at most
            assert abs(float(scales[r, g]) * 448 - a) <= 1e-6 * a
            assert np.any((codes[r, g] & 0x7F) == 0x7E)  # someone hits the top code
            assert not np.any((codes[r, g] & 0x7F) == 0x7F)  # never NaN
            deq = np.array([o.e4m3_value(c) for c in codes[r, g]]) * float(scales[r, g])
            bound = np.maximum(np.abs(mean[g]) * 2.0 ** -4, 2.0 ** -10 * float(scales[r, g])) + 1e-6 * a
            assert np.all(np.abs(deq - mean[g]) <= bound)
            # sign of every non-zero code follows the mean
            nz = (codes[r, g] & 0x7F) != 0
            assert np.all(((codes[r, g] & 0x80) != 0)[nz] == (mean[g] < 0)[nz])


def test_appending_tokens_never_changes_existing_summaries(oracle_lib, gen_host):
    o = oracle_lib
    ik = gen_host.host_index_k(12, 96, G, P, 0, 0, 96)
    c1, s1 = o.compress_regions(ik[:40], 0, 5)  # 40 tokens -> 5 complete regions
    c2, s2 = o.compress_regions(ik, 0, 12)
    assert np.array_equal(c1, c2[:5]) and np.array_equal(s1, s2[:5])


def test_partial_regions_are_refused(oracle_lib, gen_host):
    ik = gen_host.host_index_k(13, 20, G, P, 0, 0, 20)
    with pytest.raises(AssertionError):
        oracle_lib.compress_regions(ik, 0, 3)  # region 2 holds only tokens 16..19
