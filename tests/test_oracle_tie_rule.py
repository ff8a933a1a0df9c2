"""Pins for gating step 4 on a given selection (oracle.route_weights) and for
the tie-flip rule (oracle.parity) that decides when a GPU selection differing
from the oracle's is a near-tie rather than a mistake.

Pinned against: hand-computed closed forms (rho * s / sum s on a three-expert
example); the oracle's own gating on its own selection; the invariant
sum(w) = router_scaling_factor; hand-built selections that are, and are not,
a top-k within the 1e-6 margin.
"""
import numpy as np
import pytest

from oracle import parity

RHO = 2.826


def test_route_weights_closed_form(orc):
    s = np.array([[0.5, 0.25, 0.25]], np.float32)
    w = orc.route_weights(s, np.array([[1, 0]], np.int32), RHO)
    np.testing.assert_array_equal(w, np.array([[RHO * 0.25 / 0.75, RHO * 0.5 / 0.75]], np.float32))
    # route_norm off: rho * s
    w = orc.route_weights(s, np.array([[0, 2]], np.int32), RHO, route_norm=False)
    np.testing.assert_array_equal(w, np.array([[RHO * 0.5, RHO * 0.25]], np.float32))


def test_route_weights_equal_gating_on_its_own_selection(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, 128)).astype(np.float32)
    Wr = (rng.standard_normal((24, 128)) * 0.02).astype(np.float32)
    idx, w, s, _ = orc.route(x, Wr, None, 6, RHO)
    np.testing.assert_array_equal(orc.route_weights(s, idx, RHO), w)


def test_route_weights_of_another_selection(orc):
    # a selection other than the top-k still gets rho * s / sum s and sums to rho
    rng = np.random.default_rng(4)
    s = rng.random((7, 10)).astype(np.float32)
    idx = np.stack([rng.permutation(10)[:4] for _ in range(7)]).astype(np.int32)
    w = orc.route_weights(s, idx, RHO)
    sel = np.take_along_axis(s, idx, axis=1).astype(np.float64)
    np.testing.assert_allclose(w, RHO * sel / sel.sum(1, keepdims=True), rtol=1e-7)
    np.testing.assert_allclose(w.astype(np.float64).sum(1), RHO, rtol=1e-6)


@pytest.mark.parametrize("bad", [[[0, 0]], [[0, 3]], [[-1, 1]]])
def test_route_weights_rejects_invalid_selection(orc, bad):
    s = np.array([[0.5, 0.25, 0.25]], np.float32)
    with pytest.raises(ValueError):
        orc.route_weights(s, np.array(bad, np.int32), RHO)


def _scores():
    # expert 3 and 1 nearly tie at the top-3 boundary (gap 5e-7); experts 0
    # and 2 nearly tie inside the selection; expert 4 is far below
    return np.array([0.8, 0.6, 0.8000004, 0.6000005, 0.1], np.float64)


def test_exact_selection_is_no_mismatch():
    s = _scores()[None]
    o = np.array([[2, 0, 3]])
    mism, flips = parity.classify_routing(o, o, s)
    assert not mism.any() and not flips.any()


@pytest.mark.parametrize("gpu,flip", [
    ([2, 0, 1], True),     # boundary swap 3 <-> 1 within the margin
    ([0, 2, 3], True),     # slot order swap of two near-equal selected scores
    ([2, 3, 0], False),    # slot order violated by 0.2: not a tie
    ([2, 0, 4], False),    # 4 is far below 1 and 3: not a top-k
    ([2, 2, 3], False),    # duplicate expert
    ([2, 0, 5], False),    # out of range
])
def test_tie_flip_rule(gpu, flip):
    s = _scores()[None]
    o = np.array([[2, 0, 3]])
    mism, flips = parity.classify_routing(np.array([gpu]), o, s)
    assert mism[0]
    assert bool(flips[0]) == flip


def test_margin_is_inclusive_and_tight():
    s = np.array([[0.5, 0.5 - 1e-6, 0.1]])
    assert parity.is_near_top_k([1], s[0])               # gap exactly the margin
    s = np.array([[0.5, 0.5 - 2e-6, 0.1]])
    assert not parity.is_near_top_k([1], s[0])           # twice the margin
