"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws random numbers and rounds them to the storage type
(fp32 masters to bf16 with round-to-nearest-even).  It holds none of the
layer's arithmetic; both the GPU library's callers and the CPU oracle's
callers take their inputs from here.

Workloads (one Hunyuan-style MoE layer; sizes from the Hy3 guide, section 1,
and the Hy4-preview tutorial, section 1):

  tiny         T=64,   H=256,  E=16,  k=4, I=Is=128,  fp32
  hy3_decode   T=64,   H=4096, E=192, k=8, I=Is=1536, bf16
  hy3_prefill  T=8192, H=4096, E=192, k=8, I=Is=1536, bf16
  hy4_skew     T=2048, H=4096, E=256, k=8, I=Is=1536, bf16, Zipf logit bias
  mx           T=4096, H=4096, E=192, k=8, I=Is=1536, MX-fp8 experts
  w4a8_decode  T=64,   H=4096, E=192, k=8, I=Is=1536, MXFP4 routed experts (W4A8)
  w4a8         T=4096, H=4096, E=192, k=8, I=Is=1536, MXFP4 routed experts (W4A8)
  fp8_decode   T=64,   H=4096, E=192, k=8, I=Is=1536, static per-tensor FP8 (W8A8)
  fp8          T=4096, H=4096, E=192, k=8, I=Is=1536, static per-tensor FP8 (W8A8)

The static FP8 workloads fix their activation scales (the pages give no
calibration): x 2^-5 (N(0,1) activations stay below 448 * 2^-5 = 14) and h
2^-3 for the routed and the shared experts (h stays below 56; about 25
at most in these workloads).

Distributions: activations N(0,1); router and expert weights N(0, 0.02);
router weights stay fp32.  Every tensor has its own PCG64 stream derived from
(seed, tensor tag, expert) with numpy's SeedSequence, so any single expert's
weights can be regenerated on their own and large weight sets can be drawn on
several threads.

The skewed workload adds a per-expert logit bias b_e = beta * (-1.1 ln r_e -
mean), where r_e is a seeded permutation of the ranks 1..E; beta is fixed so
that the busiest expert receives about ten times the mean token count.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROUTER_SCALING_FACTOR = 2.826

# Stream tags (spawn keys) for SeedSequence.
_TAG_X, _TAG_ROUTER, _TAG_BIAS, _TAG_EXPERT, _TAG_SHARED, _TAG_AUX = 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    Is: int
    dtype: str                 # "f32", "bf16", "mxfp8" (expert weights + activations),
                               # "w4a8" (MXFP4 routed experts, MX-fp8 shared and activations)
                               # or "fp8" (static per-tensor E4M3 W8A8)
    rho: float = ROUTER_SCALING_FACTOR
    route_norm: bool = True
    zipf_beta: float = 0.0     # 0: no router bias
    seed: int = 0
    x_std: float = 1.0
    w_std: float = 0.02
    fp8_x_scale: float = 2.0 ** -5      # static activation scales ("fp8" only)
    fp8_h_scale: float = 2.0 ** -3
    fp8_sh_h_scale: float = 2.0 ** -3

    @property
    def P(self) -> int:
        return self.T * self.k


WORKLOADS = {
    "tiny": Workload("tiny", T=64, H=256, E=16, k=4, I=128, Is=128, dtype="f32"),
    "hy3_decode": Workload("hy3_decode", T=64, H=4096, E=192, k=8, I=1536, Is=1536, dtype="bf16"),
    "hy3_prefill": Workload("hy3_prefill", T=8192, H=4096, E=192, k=8, I=1536, Is=1536,
                            dtype="bf16"),
    "hy4_skew": Workload("hy4_skew", T=2048, H=4096, E=256, k=8, I=1536, Is=1536, dtype="bf16",
                         zipf_beta=0.38),
    "mx": Workload("mx", T=4096, H=4096, E=192, k=8, I=1536, Is=1536, dtype="mxfp8"),
    "w4a8_decode": Workload("w4a8_decode", T=64, H=4096, E=192, k=8, I=1536, Is=1536,
                            dtype="w4a8"),
    "w4a8": Workload("w4a8", T=4096, H=4096, E=192, k=8, I=1536, Is=1536, dtype="w4a8"),
    "fp8_decode": Workload("fp8_decode", T=64, H=4096, E=192, k=8, I=1536, Is=1536,
                           dtype="fp8"),
    "fp8": Workload("fp8", T=4096, H=4096, E=192, k=8, I=1536, Is=1536, dtype="fp8"),
}


def workload(name: str, **overrides) -> Workload:
    return dataclasses.replace(WORKLOADS[name], **overrides)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_widen(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


# ----------------------------------------------------------------------------- draws


def x_master(w: Workload, T: int | None = None) -> np.ndarray:
    """Activations [T,H] fp32 masters (the first T rows of the workload's stream)."""
    T = w.T if T is None else T
    return _normal(_rng(w.seed, _TAG_X), (T, w.H), w.x_std)


def x_input(w: Workload, T: int | None = None):
    """Activations as the layer receives them.  Returns (array for the GPU,
    exact fp32 widening for the oracle).  bf16/MX workloads hand over bf16."""
    xm = x_master(w, T)
    if w.dtype == "f32":
        return xm, xm
    b = bf16_round(xm)
    return b, bf16_widen(b)


def router_weight(w: Workload) -> np.ndarray:
    return _normal(_rng(w.seed, _TAG_ROUTER), (w.E, w.H), w.w_std)


def router_bias(w: Workload):
    """Per-expert logit bias, or None.  Zipf-shaped: rank r gets -1.1 ln r."""
    if w.zipf_beta == 0.0:
        return None
    rng = _rng(w.seed, _TAG_BIAS)
    ranks = rng.permutation(w.E).astype(np.float64) + 1.0
    v = -1.1 * np.log(ranks)
    v -= v.mean()
    return (w.zipf_beta * v).astype(np.float32)


def expert_master(w: Workload, e: int):
    """fp32 masters of expert e: (Wg [I,H], Wu [I,H], Wd [H,I])."""
    rng = _rng(w.seed, _TAG_EXPERT, e)
    return (_normal(rng, (w.I, w.H), w.w_std), _normal(rng, (w.I, w.H), w.w_std),
            _normal(rng, (w.H, w.I), w.w_std))


def shared_master(w: Workload):
    """fp32 masters of the shared expert: (Sg [Is,H], Su [Is,H], Sd [H,Is])."""
    rng = _rng(w.seed, _TAG_SHARED)
    return (_normal(rng, (w.Is, w.H), w.w_std), _normal(rng, (w.Is, w.H), w.w_std),
            _normal(rng, (w.H, w.Is), w.w_std))


def expert_stored(w: Workload, e: int):
    """Expert e as stored: fp32 for f32/MX workloads (MX is quantised by the
    consumer), bf16 bit patterns for bf16 workloads."""
    m = expert_master(w, e)
    if w.dtype == "bf16":
        return tuple(bf16_round(a) for a in m)
    return m


def shared_stored(w: Workload):
    m = shared_master(w)
    if w.dtype == "bf16":
        return tuple(bf16_round(a) for a in m)
    return m


def all_experts_stored(w: Workload, threads: int | None = None):
    """Stacked expert weights (Wg [E,I,H], Wu [E,I,H], Wd [E,H,I]) as stored,
    drawn on a thread pool (numpy releases the GIL while drawing)."""
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    Wg = np.empty((w.E, w.I, w.H), dt)
    Wu = np.empty((w.E, w.I, w.H), dt)
    Wd = np.empty((w.E, w.H, w.I), dt)

    def one(e):
        g, u, d = expert_stored(w, e)
        Wg[e], Wu[e], Wd[e] = g, u, d

    n = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(one, range(w.E)))
    return Wg, Wu, Wd


def aux_stream(w: Workload, tag: int = 0) -> np.random.Generator:
    """A spare seeded stream for synthetic stage inputs in tests
    (routing indices, weights, intermediate activations)."""
    return _rng(w.seed, _TAG_AUX, tag)


def random_topk(w: Workload, T: int, tag: int = 0) -> np.ndarray:
    """Seeded routing indices [T,k]: k distinct experts per token, uniform."""
    rng = aux_stream(w, 1000 + tag)
    keys = rng.random((T, w.E))
    return np.argsort(keys, axis=1)[:, : w.k].astype(np.int32)
