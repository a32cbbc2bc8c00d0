"""Pins the oracle's E4M3 (OCP e4m3fn) encoder/decoder to brute force and to the format's definition.

The format is OCP "8-bit Floating Point Specification (OFP8)", rev 1.0, E4M3: bias 7, no infinities,
S.1111.111 = NaN, max normal 448, min normal 2^-6, min subnormal 2^-9 (tests/golden/e4m3_spec.txt).
The pages fix only that region summaries are 8-bit floating point.
"""
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_spec.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split("=")
            vals[k.strip()] = v.strip()
    return vals


def _all_finite_codes(oracle):
    codes = [c for c in range(256) if not math.isnan(oracle.e4m3_value(c))]
    return np.array(codes), np.array([oracle.e4m3_value(c) for c in codes])


def _brute(x, codes, values):
    """Nearest finite code, ties to the code with an even mantissa LSB; |x| beyond range -> 448."""
    if x == 0.0:
        return 0x80 if math.copysign(1.0, x) < 0 else 0x00
    sign = 0x80 if x < 0 else 0x00
    a = abs(x)
    pos = [(c, v) for c, v in zip(codes, values) if c < 0x80]
    d = [abs(v - a) for _, v in pos]
    best = min(d)
    tied = [c for (c, _), dd in zip(pos, d) if dd == best]
    if len(tied) > 1:
        tied = [c for c in tied if c % 2 == 0]
    return sign | tied[0]


def test_decode_matches_spec_constants(oracle_lib):
    g = _golden()
    o = oracle_lib
    assert o.e4m3_value(0x7E) == float(g["max_normal"])
    assert o.e4m3_value(0x08) == 2.0 ** int(g["min_normal_log2"])
    assert o.e4m3_value(0x01) == 2.0 ** int(g["min_subnormal_log2"])
    assert o.e4m3_value(0x38) == 1.0
    assert math.isnan(o.e4m3_value(0x7F)) and math.isnan(o.e4m3_value(0xFF))
    assert o.e4m3_value(0x80) == 0.0 and math.copysign(1, o.e4m3_value(0x80)) < 0
    # 253 finite non-NaN codes + the two zeros are distinct values except +-0
    codes, values = _all_finite_codes(o)
    assert len(codes) == 254
    assert len(set(values.tolist())) == 253
    # monotone in the positive half
    pos = values[codes < 0x80]
    assert np.all(np.diff(pos) > 0)


def test_encode_special_cases(oracle_lib):
    o = oracle_lib
    enc = lambda v: int(o.e4m3_encode([v])[0])
    assert enc(448.0) == 0x7E
    assert enc(464.0) == 0x7E  # tie between 448 and (unrepresentable) 480 -> saturate, never NaN
    assert enc(1e30) == 0x7E and enc(-1e30) == 0xFE
    assert enc(2.0 ** -9) == 0x01
    assert enc(2.0 ** -10) == 0x00  # tie between 0 and 2^-9 -> even code
    assert enc(3 * 2.0 ** -10) == 0x02  # tie between 2^-9 and 2^-8 -> even code
    assert enc(-0.0) == 0x80
    assert enc(-1e-30) == 0x80  # negative values rounding to zero keep their sign
    assert enc(1.0) == 0x38
    assert enc(1.0625) == 0x38  # tie 1.0 / 1.125 -> even
    assert enc(1.1875) == 0x3A  # tie 1.125 / 1.25 -> even


def test_encode_matches_brute_force(oracle_lib):
    o = oracle_lib
    codes, values = _all_finite_codes(o)
    pos = np.sort(values[codes < 0x80])
    xs = list(pos) + list((pos[1:] + pos[:-1]) / 2)  # every value and every midpoint
    mids = (pos[1:] + pos[:-1]) / 2
    xs += list(np.nextafter(mids.astype(np.float32), np.float32(0)))
    xs += list(np.nextafter(mids.astype(np.float32), np.float32(1000)))
    rng = np.random.default_rng(7)
    xs += list(rng.normal(0, 1, 3000) * 2.0 ** rng.integers(-12, 10, 3000))
    xs += [470.0, 500.0, 1e6, 1e-12, 2.0 ** -11]
    xs = np.array(xs, dtype=np.float32)
    xs = np.concatenate([xs, -xs])
    got = o.e4m3_encode(xs)
    for x, c in zip(xs.tolist(), got.tolist()):
        assert c == _brute(float(x), codes, values), (x, hex(c))
