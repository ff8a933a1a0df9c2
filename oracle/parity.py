"""Comparison rules between the GPU path and the oracle -- TEST INFRASTRUCTURE.

Used by the tests and by the benchmark's parity leg only.

Routing is an integer result decided by floating point: the selection of a
token is the k largest sigmoid scores (Hy3 guide, section 1: top-8 of the
sigmoid router scores).  The GPU sums the router logits in another order than
the oracle, so two experts whose scores differ by less than the rounding of
those sums can swap places.  One rule decides when a differing selection is
such a tie flip rather than a mistake: the GPU's selection must itself be a
top-k of the oracle's scores up to a margin of 1e-6 -- k distinct experts in
range, slots in non-increasing score order within the margin, and every
selected score at least every unselected score minus the margin.  A flipped
token is then evaluated by the oracle with the GPU's selection (weights from
the oracle's scores) and its output compared like any other token's.
"""
from __future__ import annotations

import numpy as np

TIE_MARGIN = 1e-6


def is_near_top_k(sel, scores, margin: float = TIE_MARGIN) -> bool:
    """True when the k experts ``sel`` of one token are a top-k of its scores
    [E] up to ``margin`` (distinct, in range, slot order and boundary)."""
    sel = np.asarray(sel, dtype=np.int64)
    s = np.asarray(scores, dtype=np.float64)
    k, E = len(sel), len(s)
    if k == 0 or len(set(sel.tolist())) != k or sel.min() < 0 or sel.max() >= E:
        return False
    ss = s[sel]
    if np.any(ss[1:] > ss[:-1] + margin):
        return False
    if k < E:
        rest = np.ones(E, dtype=bool)
        rest[sel] = False
        if ss.min() < s[rest].max() - margin:
            return False
    return True


def classify_routing(gpu_idx, oracle_idx, scores, margin: float = TIE_MARGIN):
    """Rows where the GPU's selection differs from the oracle's, and which of
    them are tie flips.  Returns (mismatch mask [T], tie-flip mask [T])."""
    g = np.asarray(gpu_idx)
    o = np.asarray(oracle_idx)
    mism = (g != o).any(axis=1)
    flips = np.zeros_like(mism)
    for t in np.nonzero(mism)[0]:
        flips[t] = is_near_top_k(g[t], scores[t], margin)
    return mism, flips
