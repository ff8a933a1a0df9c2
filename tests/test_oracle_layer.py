"""Pins for the oracle's expert FFN, combine and whole-layer composition.

Pinned against: library matmuls (numpy/BLAS, float64) for a single dense
SwiGLU FFN; the identical-experts special case, where routing drops out and
the layer is rho * FFN_W(x) + FFN_shared(x); linearity in the routed and
shared parts; the per-token definition of the output evaluated directly with
library matmuls (no permutation); token-order equivariance and expert
relabelling invariance.
"""
import numpy as np
import pytest

from mixture_experts_layer_19_amd import inputs as I

RHO = np.float32(2.826)


def dense_swiglu(x, Wg, Wu, Wd):
    x = x.astype(np.float64)
    g = x @ Wg.astype(np.float64).T
    u = x @ Wu.astype(np.float64).T
    h = (g / (1.0 + np.exp(-g))) * u
    return h.astype(np.float32).astype(np.float64) @ Wd.astype(np.float64).T


def _ffn(rng, H, Iw, scale=0.05):
    return ((rng.standard_normal((Iw, H)) * scale).astype(np.float32),
            (rng.standard_normal((Iw, H)) * scale).astype(np.float32),
            (rng.standard_normal((H, Iw)) * scale).astype(np.float32))


def rel_err(a, b):
    return float(np.abs(np.asarray(a, np.float64) - b).max() / np.abs(b).max())


def test_swiglu_rows_matches_library_dense_ffn(orc):
    rng = np.random.default_rng(10)
    H, Iw = 96, 64                     # H != I so a transposed operand cannot pass
    x = rng.standard_normal((13, H)).astype(np.float32)
    Wg, Wu, Wd = _ffn(rng, H, Iw)
    h, y = orc.swiglu_rows(x, Wg, Wu, Wd)
    g = x.astype(np.float64) @ Wg.T.astype(np.float64)
    u = x.astype(np.float64) @ Wu.T.astype(np.float64)
    np.testing.assert_allclose(h, ((g / (1 + np.exp(-g))) * u).astype(np.float32), rtol=1e-6,
                               atol=1e-9)
    assert rel_err(y, dense_swiglu(x, Wg, Wu, Wd)) < 1e-6


def test_swiglu_closed_forms(orc):
    rng = np.random.default_rng(11)
    H, Iw = 64, 32
    x = rng.standard_normal((4, H)).astype(np.float32)
    Wg, Wu, Wd = _ffn(rng, H, Iw)
    # silu(0) = 0: a zero gate projection gives h = 0 and y = 0
    h, y = orc.swiglu_rows(x, np.zeros_like(Wg), Wu, Wd)
    assert np.all(h == 0) and np.all(y == 0)
    # silu(g) -> g for large g: gate rows = 50 * e_0 on inputs with x_0 = 1
    x1 = np.zeros((1, H), np.float32)
    x1[0, 0] = 1.0
    Wg2 = np.zeros_like(Wg)
    Wg2[:, 0] = 50.0
    h, _ = orc.swiglu_rows(x1, Wg2, Wu, Wd)
    np.testing.assert_allclose(h[0], 50.0 * Wu[:, 0], rtol=1e-6)


def test_bf16_weights_are_widened_exactly(orc):
    rng = np.random.default_rng(12)
    H, Iw = 64, 32
    x = rng.standard_normal((5, H)).astype(np.float32)
    m = _ffn(rng, H, Iw)
    b = [I.bf16_round(a) for a in m]
    f = [I.bf16_widen(a) for a in b]
    h1, y1 = orc.swiglu_rows(x, *b)
    h2, y2 = orc.swiglu_rows(x, *f)
    np.testing.assert_array_equal(h1, h2)
    np.testing.assert_array_equal(y1, y2)


def test_mx_rows_equal_dense_ffn_on_dequantised_operands(orc):
    rng = np.random.default_rng(13)
    H, Iw = 128, 64
    x = rng.standard_normal((6, H)).astype(np.float32)
    Wg, Wu, Wd = _ffn(rng, H, Iw, 0.02)
    h, y = orc.swiglu_rows(x, Wg, Wu, Wd, mx=True)
    dq = lambda a: orc.mx_dequant(*orc.mxq(a))
    xq, gq, uq, dq_ = dq(x), dq(Wg), dq(Wu), dq(Wd)
    g = xq.astype(np.float64) @ gq.T.astype(np.float64)
    u = xq.astype(np.float64) @ uq.T.astype(np.float64)
    href = ((g / (1 + np.exp(-g))) * u).astype(np.float32)
    np.testing.assert_allclose(h, href, rtol=1e-5, atol=1e-7)
    yref = dq(href).astype(np.float64) @ dq_.T.astype(np.float64)
    assert rel_err(y, yref) < 1e-3
    # and MX really rounds: the unquantised FFN differs by more than fp32 noise
    assert rel_err(y, dense_swiglu(x, Wg, Wu, Wd)) > 1e-4


def _tiny_inputs(seed=0, E=16, k=4, T=64, H=256, Iw=128, bias=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    Wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    b = (rng.standard_normal(E) * 0.3).astype(np.float32) if bias else None
    Wg = (rng.standard_normal((E, Iw, H)) * 0.02).astype(np.float32)
    Wu = (rng.standard_normal((E, Iw, H)) * 0.02).astype(np.float32)
    Wd = (rng.standard_normal((E, H, Iw)) * 0.02).astype(np.float32)
    S = _ffn(rng, H, Iw, 0.02)
    return x, Wr, b, Wg, Wu, Wd, S


def test_identical_experts_reduce_to_dense_ffn(orc):
    x, Wr, b, Wg, Wu, Wd, S = _tiny_inputs(bias=True)
    for arr in (Wg, Wu, Wd):
        arr[:] = arr[3]
    r = orc.layer_forward(x, Wr, b, Wg, Wu, Wd, *S, k=4, rho=RHO)
    ref = float(RHO) * dense_swiglu(x, Wg[0], Wu[0], Wd[0]) + dense_swiglu(x, *S)
    assert rel_err(r["out"], ref) < 1e-6
    # with the shared expert equal to the routed one: (rho + 1) * FFN_W(x)
    r = orc.layer_forward(x, Wr, b, Wg, Wu, Wd, Wg[0], Wu[0], Wd[0], k=4, rho=RHO)
    ref = (float(RHO) + 1.0) * dense_swiglu(x, Wg[0], Wu[0], Wd[0])
    assert rel_err(r["out"], ref) < 1e-6


def test_layer_equals_per_token_definition(orc):
    # out[t] = sum_j w[t,j] FFN_{idx[t,j]}(x[t]) + FFN_sh(x[t]), evaluated per
    # token with library matmuls and no permutation
    x, Wr, b, Wg, Wu, Wd, S = _tiny_inputs(seed=1, bias=True)
    r = orc.layer_forward(x, Wr, b, Wg, Wu, Wd, *S, k=4, rho=RHO)
    idx, w, _, _ = orc.route(x, Wr, b, 4, RHO)
    np.testing.assert_array_equal(r["topk_idx"], idx)
    np.testing.assert_array_equal(r["topk_w"], w)
    sh = dense_swiglu(x, *S)
    ref = np.zeros(x.shape, np.float64)
    for t in range(x.shape[0]):
        for j in range(4):
            e = idx[t, j]
            ref[t] += float(w[t, j]) * dense_swiglu(x[t:t + 1], Wg[e], Wu[e], Wd[e])[0]
        ref[t] += sh[t]
    assert rel_err(r["out"], ref) < 1e-6
    # the pairs routed to all experts number T*k
    assert r["counts"].sum() == 64 * 4


def test_layer_linearity(orc):
    x, Wr, b, Wg, Wu, Wd, S = _tiny_inputs(seed=2)
    z = [np.zeros_like(a) for a in (Wg, Wu, Wd)]
    r = orc.layer_forward(x, Wr, b, *z, *S, k=4, rho=RHO)
    assert rel_err(r["out"], dense_swiglu(x, *S)) < 1e-6
    r0 = orc.layer_forward(x, Wr, b, Wg, Wu, Wd, *[np.zeros_like(a) for a in S], k=4, rho=RHO)
    r1 = orc.layer_forward(x, Wr, b, Wg, Wu, Wd, k=4, rho=RHO)
    np.testing.assert_array_equal(r0["out"], r1["out"])
    r2 = orc.layer_forward(x, Wr, b, Wg, Wu, Wd, *S, k=4, rho=RHO)
    assert rel_err(r2["out"], r1["out"].astype(np.float64) + dense_swiglu(x, *S)) < 1e-6


def test_token_permutation_equivariance(orc):
    x, Wr, b, Wg, Wu, Wd, S = _tiny_inputs(seed=3)
    perm = np.random.default_rng(99).permutation(x.shape[0])
    r = orc.layer_forward(x, Wr, b, Wg, Wu, Wd, *S, k=4, rho=RHO)
    rp = orc.layer_forward(x[perm], Wr, b, Wg, Wu, Wd, *S, k=4, rho=RHO)
    np.testing.assert_array_equal(rp["out"], r["out"][perm])


def test_expert_relabelling_invariance(orc):
    x, Wr, b, Wg, Wu, Wd, S = _tiny_inputs(seed=4, bias=True)
    r = orc.layer_forward(x, Wr, b, Wg, Wu, Wd, *S, k=4, rho=RHO)
    _, _, _, gap = orc.route(x, Wr, b, 4, RHO)
    assert np.all(gap > 0)          # no ties, so relabelling cannot change choices
    pi = np.random.default_rng(5).permutation(16)
    rp = orc.layer_forward(x, Wr[pi], b[pi], Wg[pi], Wu[pi], Wd[pi], *S, k=4, rho=RHO)
    np.testing.assert_array_equal(rp["out"], r["out"])
    np.testing.assert_array_equal(pi[rp["topk_idx"]], r["topk_idx"])


def test_sampled_tokens_match_whole_layer(orc):
    x, Wr, b, Wg, Wu, Wd, S = _tiny_inputs(seed=6, bias=True)
    r = orc.layer_forward(x, Wr, b, Wg, Wu, Wd, *S, k=4, rho=RHO)
    toks = [0, 5, 17, 63]
    out, idx, w, gap = orc.layer_forward_tokens(
        toks, x, Wr, b, lambda e: (Wg[e], Wu[e], Wd[e]), S, k=4, rho=RHO)
    np.testing.assert_array_equal(out, r["out"][toks])
    np.testing.assert_array_equal(idx, r["topk_idx"][toks])


def test_tiny_workload_layer_runs(orc):
    w = I.workload("tiny")
    xg, x = I.x_input(w)
    Wg, Wu, Wd = I.all_experts_stored(w)
    r = orc.layer_forward(x, I.router_weight(w), None, Wg, Wu, Wd, *I.shared_stored(w), k=w.k,
                          rho=w.rho)
    assert np.isfinite(r["out"]).all()
    assert r["counts"].sum() == w.T * w.k
    assert np.all(np.abs(r["topk_w"].astype(np.float64).sum(1) - 2.826) <= 1e-6)


def test_mx_layer_identical_experts(orc):
    # MX special case: identical experts still reduce to rho * FFN + shared,
    # with every operand rounded through MX-fp8 in both
    rng = np.random.default_rng(20)
    T, H, Iw, E, k = 8, 64, 32, 6, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    Wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    g, u, d = _ffn(rng, H, Iw, 0.02)
    Wg, Wu, Wd = (np.repeat(a[None], E, 0) for a in (g, u, d))
    r = orc.layer_forward(x, Wr, None, Wg, Wu, Wd, g, u, d, k=k, rho=RHO, mx=True)
    _, y = orc.swiglu_rows(x, g, u, d, mx=True)
    ref = (float(RHO) + 1.0) * y.astype(np.float64)
    assert rel_err(r["out"], ref) < 1e-6
