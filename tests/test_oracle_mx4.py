"""Pins for the oracle's MXFP4 arithmetic (E2M1 elements, E8M0 scales) and
its W4A8 expert FFN (MXFP4 weights, MX-fp8 activations).

The pins come from the OCP Microscaling Formats (MX) v1.0 specification:
the E2M1 element table, worked examples derived by hand from its
quantisation rule (tests/golden/mxq4_examples.txt), a brute-force nearest
search, and round-trip error bounds.  The W4A8 recipe itself (routed experts
MXFP4 with 8-bit activations, shared expert W8A8) is the Hy3 guide's
section 8.2.
"""
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxq4_examples.txt")
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


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


@pytest.mark.parametrize("name,v,scale,codes", _golden_blocks(),
                         ids=lambda p: p if isinstance(p, str) else "")
def test_mxq4_worked_examples(orc, name, v, scale, codes):
    q, s = orc.mxq4(v)
    assert int(s[0]) == scale, name
    np.testing.assert_array_equal(q, codes, err_msg=name)


def test_golden_clamp_inputs_are_exact():
    assert np.float32("2.350988701644575e-38") == np.float32(2.0 ** -125)
    assert np.float32("2.938735877055719e-39") == np.float32(2.0 ** -128)


def test_e2m1_table(orc):
    # OCP MX v1.0, E2M1: max normal 6 = S.11.1, min normal 1 = S.01.0,
    # subnormal 0.5 = S.00.1
    for c, m in enumerate(E2M1_MAGNITUDES):
        assert orc.e2m1_decode(c) == m
        assert orc.e2m1_decode(c | 8) == -m
    assert math.copysign(1.0, orc.e2m1_decode(8)) == -1.0


def test_e2m1_encode_inverts_decode(orc):
    for c in range(16):
        assert orc.e2m1_encode(orc.e2m1_decode(c)) == c


def test_e2m1_midpoints_round_to_even(orc):
    for c in range(7):
        lo, hi = E2M1_MAGNITUDES[c], E2M1_MAGNITUDES[c + 1]
        mid = (lo + hi) / 2
        want = c if (c & 1) == 0 else c + 1
        assert orc.e2m1_encode(mid) == want, c
        assert orc.e2m1_encode(-mid) == 8 | want, c
        assert orc.e2m1_encode(math.nextafter(mid, 0.0)) == c
        assert orc.e2m1_encode(math.nextafter(mid, 1e9)) == c + 1


def test_e2m1_saturates(orc):
    for v in (6.0, 6.5, 7.0, 8.0, 1e30):
        assert orc.e2m1_encode(v) == 7
        assert orc.e2m1_encode(-v) == 15


def test_mxq4_matches_brute_force(orc):
    """Scale from frexp, element from an exhaustive nearest search (ties to
    the even code), over random blocks spanning many binades."""
    rng = np.random.default_rng(11)
    v = (rng.standard_normal((200, 32)) * np.exp(rng.uniform(-20, 20, (200, 1)))).astype(np.float32)
    v[3, :] = 0.0
    v[4, 5] = 0.0
    q, s = orc.mxq4(v)
    mags = np.array(E2M1_MAGNITUDES)
    for b in range(v.shape[0]):
        amax = float(np.abs(v[b]).max())
        X = -127 if amax == 0.0 else max(-127, min(127, int(np.frexp(amax)[1]) - 1 - 2))
        assert int(s[b, 0]) == X + 127
        for i in range(32):
            x = float(v[b, i])
            a = abs(x) / 2.0 ** X
            d = np.abs(mags - a)
            cands = np.flatnonzero(d == d.min())
            c = int(cands[0]) if len(cands) == 1 else int(cands[cands % 2 == 0][0])
            assert int(q[b, i]) == (8 if math.copysign(1.0, x) < 0 else 0) | c, (b, i, x)


def test_mx4_roundtrip_error_bounds(orc):
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((64, 32)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    q, s = orc.mxq4(v)
    d = orc.mx4_dequant(q, s)
    X = s.astype(np.int64) - 127
    for b in range(v.shape[0]):
        # the block's largest magnitude scales into [4, 8)
        assert 4.0 <= np.abs(v[b]).max() / 2.0 ** X[b] < 8.0
        for i in range(32):
            vp = abs(float(v[b, i])) / 2.0 ** X[b]
            err = abs(float(v[b, i]) - float(d[b, i]))
            if vp > 6.0:                 # saturated to 6
                assert err < 2.0 * 2.0 ** X[b]
            elif vp >= 1.0:              # normal: half an ulp of a 1-bit mantissa
                assert err <= 0.25 * abs(float(v[b, i]))
            else:                        # subnormal spacing 0.5, half of it
                assert err <= 0.25 * 2.0 ** X[b]


def _dense_ffn(x, Wg, Wu, Wd, orc, w4):
    """fp64 library matmuls on the dequantised operands: weights through
    MXFP4 (w4) or MX-fp8, activations x and h through MX-fp8."""
    wq = (lambda a: orc.mx4_dequant(*orc.mxq4(a))) if w4 else (lambda a: orc.mx_dequant(*orc.mxq(a)))
    aq = lambda a: orc.mx_dequant(*orc.mxq(a))
    xq = aq(x).astype(np.float64)
    g = xq @ wq(Wg).astype(np.float64).T
    u = xq @ wq(Wu).astype(np.float64).T
    h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
    return h, aq(h).astype(np.float64) @ wq(Wd).astype(np.float64).T


def test_w4a8_ffn_equals_dense_library_ffn(orc):
    rng = np.random.default_rng(3)
    H, I, M = 256, 128, 9
    x = rng.standard_normal((M, H)).astype(np.float32)
    Wg, Wu = (rng.standard_normal((2, I, H)) * 0.05).astype(np.float32)
    Wd = (rng.standard_normal((H, I)) * 0.05).astype(np.float32)
    h, y = orc.swiglu_rows(x, Wg, Wu, Wd, mx=orc.MX_W4A8)
    h_ref, y_ref = _dense_ffn(x, Wg, Wu, Wd, orc, w4=True)
    np.testing.assert_allclose(h, h_ref, rtol=1e-6, atol=1e-7)
    # h is re-quantised to MX-fp8 before the down projection: a one-ulp
    # difference in fp32 h could move a code, so compare with a tolerance of
    # one E4M3 step of the largest term instead of bit for bit
    err = np.abs(y - y_ref).max() / np.abs(y_ref).max()
    assert err < 1e-5
    # and W4A8 differs from W8A8 (the weights really go through 4 bits)
    _, y8 = orc.swiglu_rows(x, Wg, Wu, Wd, mx=orc.MX_FP8)
    assert np.abs(y8 - y).max() / np.abs(y8).max() > 1e-2


def test_w4a8_exact_weights_match_w8a8(orc):
    """Weights already on the MXFP4 grid (each 32-block holds 6 * 2^X and
    E2M1 multiples of 2^X) go through MXFP4 and MX-fp8 unchanged, so W4A8
    and W8A8 give identical results."""
    rng = np.random.default_rng(9)
    H, I, M = 256, 64, 4
    mags = np.array(E2M1_MAGNITUDES, np.float32)

    def grid(shape):
        k = rng.integers(0, 8, shape)
        sgn = np.where(rng.random(shape) < 0.5, -1.0, 1.0).astype(np.float32)
        a = (mags[k] * sgn).reshape(-1, 32)
        a[:, 0] = 6.0                     # block maximum 6 * 2^X
        X = rng.integers(-9, -5, (a.shape[0], 1))
        return (a * np.exp2(X)).astype(np.float32).reshape(shape)

    x = rng.standard_normal((M, H)).astype(np.float32)
    Wg, Wu, Wd = grid((I, H)), grid((I, H)), grid((H, I))
    q, s = orc.mxq4(Wg)
    np.testing.assert_array_equal(orc.mx4_dequant(q, s), Wg)
    _, y4 = orc.swiglu_rows(x, Wg, Wu, Wd, mx=orc.MX_W4A8)
    _, y8 = orc.swiglu_rows(x, Wg, Wu, Wd, mx=orc.MX_FP8)
    np.testing.assert_array_equal(y4, y8)


def test_w4a8_layer_identical_experts(orc):
    """All routed experts equal W: every token's output is rho * FFN_W(x)
    through W4A8 plus the shared expert through W8A8, whatever the routing."""
    rng = np.random.default_rng(21)
    T, H, E, k, I, Is, rho = 12, 256, 8, 2, 128, 128, 2.826
    x = rng.standard_normal((T, H)).astype(np.float32)
    Wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    W = [(rng.standard_normal(s) * 0.05).astype(np.float32) for s in ((I, H), (I, H), (H, I))]
    S = [(rng.standard_normal(s) * 0.05).astype(np.float32) for s in ((Is, H), (Is, H), (H, Is))]
    Wg, Wu, Wd = (np.broadcast_to(a, (E,) + a.shape).copy() for a in W)
    r = orc.layer_forward(x, Wr, None, Wg, Wu, Wd, *S, k=k, rho=rho, mx=orc.MX_W4A8)
    _, yw = _dense_ffn(x, *W, orc, w4=True)
    _, ys = _dense_ffn(x, *S, orc, w4=False)
    ref = rho * yw + ys
    assert np.abs(r["out"] - ref).max() / np.abs(ref).max() < 1e-5
    # the per-token definition agrees with the permuted layer bit for bit
    out_t, idx_t, _, _ = orc.layer_forward_tokens(
        np.arange(T), x, Wr, None, lambda e: (Wg[e], Wu[e], Wd[e]), S, k=k, rho=rho,
        mx=orc.MX_W4A8)
    np.testing.assert_array_equal(idx_t, r["topk_idx"])
    np.testing.assert_array_equal(out_t, r["out"])
