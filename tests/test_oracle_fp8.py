"""Pins for the oracle's static per-tensor FP8 (W8A8) arithmetic.

A weight tensor's scale is max|w| / 448 (E4M3's largest normal) in fp32; an
activation tensor uses a fixed scale.  Codes are E4M3 (OCP, FN variant) of
fp32(v / s).  The E4M3 encoder itself is pinned in test_oracle_mx.py; these
pins tie the per-tensor layer to it, to exact hand-derived scales, and to
dense library FFNs on the dequantised operands.
"""
import numpy as np
import pytest


def _e4m3_table(orc):
    return np.array([orc.e4m3_decode(c) if c not in (0x7F, 0xFF) else np.nan for c in range(256)])


def test_tensor_scale_examples(orc):
    assert orc.fp8_tensor_scale(np.array([448.0, -3.0], np.float32)) == 1.0
    assert orc.fp8_tensor_scale(np.array([1.0, -3.5, 0.25], np.float32)) == 2.0 ** -7
    assert orc.fp8_tensor_scale(np.zeros(7, np.float32)) == 1.0
    # not a power of two: the fp32 quotient
    assert orc.fp8_tensor_scale(np.array([-5.0, 2.0], np.float32)) == float(np.float32(5.0) / np.float32(448.0))


def test_quantize_with_unit_and_power_of_two_scales(orc):
    rng = np.random.default_rng(4)
    v = (rng.standard_normal(500) * np.exp(rng.uniform(-6, 6, 500))).astype(np.float32)
    q1 = orc.fp8_quantize(v, 1.0)
    assert all(int(q1[i]) == orc.e4m3_encode(float(v[i])) for i in range(v.size))
    q8 = orc.fp8_quantize(v, 2.0 ** -3)
    assert all(int(q8[i]) == orc.e4m3_encode(float(v[i]) * 8.0) for i in range(v.size))


def test_tensor_max_maps_to_largest_normal(orc):
    rng = np.random.default_rng(8)
    tab = _e4m3_table(orc)
    for t in range(20):
        w = (rng.standard_normal(300) * 10.0 ** rng.uniform(-4, 3)).astype(np.float32)
        s = orc.fp8_tensor_scale(w)
        q = orc.fp8_quantize(w, s)
        i = int(np.argmax(np.abs(w)))
        assert int(q[i]) & 0x7F == 0x7E
        assert np.nanmax(np.abs(tab[q])) == 448.0


def test_activation_saturates_beyond_scale(orc):
    s = 2.0 ** -5
    q = orc.fp8_quantize(np.array([14.0, 20.0, -1e6, 0.0], np.float32), s)
    assert list(q) == [0x7E, 0x7E, 0xFE, 0x00]      # 14 / 2^-5 = 448 exactly


def _dense_fp8_ffn(orc, x, Wg, Wu, Wd, s_x, s_h):
    tab = _e4m3_table(orc)
    dq = lambda a, s: tab[orc.fp8_quantize(a, s)] * np.float64(s)
    wq = lambda a: dq(a, orc.fp8_tensor_scale(a))
    g = dq(x, s_x) @ wq(Wg).T
    u = dq(x, s_x) @ wq(Wu).T
    h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
    return h, dq(h, s_h) @ wq(Wd).T


def test_fp8_ffn_equals_dense_library_ffn(orc):
    rng = np.random.default_rng(2)
    H, I, M, s_x, s_h = 256, 128, 7, 2.0 ** -5, 2.0 ** -6
    x = rng.standard_normal((M, H)).astype(np.float32)
    Wg, Wu = (rng.standard_normal((2, I, H)) * 0.05).astype(np.float32)
    Wd = (rng.standard_normal((H, I)) * 0.05).astype(np.float32)
    h, y = orc.swiglu_rows_fp8(x, Wg, Wu, Wd, s_x, s_h)
    h_ref, y_ref = _dense_fp8_ffn(orc, x, Wg, Wu, Wd, s_x, s_h)
    np.testing.assert_allclose(h, h_ref, rtol=1e-6, atol=1e-7)
    assert np.abs(y - y_ref).max() / np.abs(y_ref).max() < 1e-5
    # the activation scale matters: a scale that is not a power of two puts h
    # on another grid (a power of two would only shift exponents)
    _, y2 = orc.swiglu_rows_fp8(x, Wg, Wu, Wd, s_x, 0.0123)
    assert np.abs(y2 - y).max() / np.abs(y).max() > 1e-3


def test_fp8_layer_identical_experts(orc):
    """All routed experts equal W: out = rho * FFN8_W(x) + FFN8_sh(x), with the
    routed and the shared h scales each applied to their own expert."""
    rng = np.random.default_rng(31)
    T, H, E, k, I, rho = 10, 256, 8, 2, 128, 2.826
    s_x, s_h, s_hs = 2.0 ** -5, 2.0 ** -6, 2.0 ** -3
    x = rng.standard_normal((T, H)).astype(np.float32)
    Wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    W = [(rng.standard_normal(s) * 0.05).astype(np.float32) for s in ((I, H), (I, H), (H, I))]
    S = [(rng.standard_normal(s) * 0.05).astype(np.float32) for s in ((I, H), (I, H), (H, I))]
    out, idx, w, _ = orc.layer_forward_tokens(np.arange(T), x, Wr, None, lambda e: W, S, k=k,
                                              rho=rho, fp8=(s_x, s_h, s_hs))
    _, yw = _dense_fp8_ffn(orc, x, *W, s_x, s_h)
    _, ys = _dense_fp8_ffn(orc, x, *S, s_x, s_hs)
    ref = rho * yw + ys
    assert np.abs(out - ref).max() / np.abs(ref).max() < 1e-5
