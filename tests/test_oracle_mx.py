"""Pins for the oracle's MX-fp8 arithmetic (E4M3 FN elements, E8M0 scales).

The pins come from the OCP Microscaling Formats (MX) v1.0 specification:
the E4M3 element table, and worked examples derived by hand from its
quantisation rule (tests/golden/mxq_examples.txt).
"""
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxq_examples.txt")


def _golden_blocks():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, vals, scale, codes = [p.strip() for p in line.split("|")]
            v = np.zeros(32, np.float32)
            if vals.startswith("all:"):
                v[:] = np.float32(vals[4:])
            elif vals:
                for item in vals.split(","):
                    i, x = item.split(":")
                    v[int(i)] = np.float32(x)
            c = np.zeros(32, np.uint8)
            if codes.startswith("all:"):
                c[:] = int(codes[4:], 16)
            elif codes:
                for item in codes.split(","):
                    i, x = item.split(":")
                    c[int(i)] = int(x, 16)
            out.append((name, v, int(scale), c))
    return out


@pytest.mark.parametrize("name,v,scale,codes", _golden_blocks(), ids=lambda p: p if isinstance(p, str) else "")
def test_mxq_worked_examples(orc, name, v, scale, codes):
    q, s = orc.mxq(v)
    assert int(s[0]) == scale, name
    np.testing.assert_array_equal(q, codes, err_msg=name)


def test_tiny_clamped_input_is_exact():
    # the golden file's tiny value must be exactly 2^-130 after parsing
    assert np.float32("7.346839692639297e-40") == np.float32(2.0 ** -130)


def test_e4m3_table_values(orc):
    # OCP MX v1.0, E4M3 element table
    assert orc.e4m3_decode(0x7E) == 448.0            # max normal S.1111.110
    assert orc.e4m3_decode(0xFE) == -448.0
    assert orc.e4m3_decode(0x08) == 2.0 ** -6        # min normal S.0001.000
    assert orc.e4m3_decode(0x07) == 0.875 * 2.0 ** -6  # max subnormal S.0000.111
    assert orc.e4m3_decode(0x01) == 2.0 ** -9        # min subnormal S.0000.001
    assert orc.e4m3_decode(0x38) == 1.0              # exponent field 7 = bias
    assert orc.e4m3_decode(0x00) == 0.0
    assert math.copysign(1.0, orc.e4m3_decode(0x80)) == -1.0
    assert math.isnan(orc.e4m3_decode(0x7F)) and math.isnan(orc.e4m3_decode(0xFF))


def test_e4m3_encode_inverts_decode(orc):
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert orc.e4m3_encode(orc.e4m3_decode(c)) == c, hex(c)


def test_e4m3_decode_is_monotone(orc):
    pos = [orc.e4m3_decode(c) for c in range(0x00, 0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))


def test_e4m3_midpoints_round_to_even(orc):
    # the exact midpoint between adjacent codes goes to the code with an even
    # mantissa field; just above / below the midpoint goes to the nearer code
    for c in range(0x00, 0x7E):
        lo, hi = orc.e4m3_decode(c), orc.e4m3_decode(c + 1)
        mid = (lo + hi) / 2
        want = c if (c & 1) == 0 else c + 1
        assert orc.e4m3_encode(mid) == want, hex(c)
        assert orc.e4m3_encode(math.nextafter(mid, 0.0)) == c
        assert orc.e4m3_encode(math.nextafter(mid, 1e9)) == c + 1


def test_e4m3_saturates(orc):
    for v in (448.0, 449.0, 463.9, 464.0, 479.0, 500.0, 1e30):
        assert orc.e4m3_encode(v) == 0x7E
        assert orc.e4m3_encode(-v) == 0xFE


def test_mx_roundtrip_error_bounds(orc):
    rng = np.random.default_rng(123)
    v = (rng.standard_normal((64, 32)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    q, s = orc.mxq(v)
    d = orc.mx_dequant(q, s)
    X = s.astype(np.int64) - 127
    for b in range(v.shape[0]):
        # the block's largest magnitude scales into [256, 512)
        a = np.abs(v[b]).max()
        assert 256.0 <= a / 2.0 ** X[b] < 512.0
        for i in range(32):
            vp = abs(float(v[b, i])) / 2.0 ** X[b]
            err = abs(float(v[b, i]) - float(d[b, i]))
            if vp >= 464.0:            # saturated to 448
                assert err < 64.0 * 2.0 ** X[b]
            elif vp >= 2.0 ** -6:        # normal: half an ulp of a 3-bit mantissa
                assert err <= 2.0 ** -4 * abs(float(v[b, i])) + 0.0
            else:                        # subnormal spacing 2^-9, half of it
                assert err <= 2.0 ** (X[b] - 10)


def test_mx_scale_is_block_local(orc):
    rng = np.random.default_rng(7)
    v = rng.standard_normal((3, 64)).astype(np.float32)
    q, s = orc.mxq(v)
    assert s.shape == (3, 2)
    for r in range(3):
        for b in range(2):
            q1, s1 = orc.mxq(v[r, 32 * b: 32 * b + 32])
            assert s1[0] == s[r, b]
            np.testing.assert_array_equal(q1, q[r, 32 * b: 32 * b + 32])
