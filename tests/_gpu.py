"""Shared helpers for the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from mixture_experts_layer_19_amd import inputs as I
from oracle.parity import classify_routing

TOL = {"f32": 1e-5, "bf16": 1e-2, "mxfp8": 3e-2, "w4a8": 3e-2, "fp8": 3e-2}

_layers = {}


def oracle_mx(dtype: str, shared: bool = False) -> int:
    """Oracle MX mode for a workload dtype: 0 none, 1 MX-fp8, 2 W4A8 (whose
    shared expert is MX-fp8)."""
    m = {"mxfp8": 1, "w4a8": 2}.get(dtype, 0)
    return 1 if (shared and m == 2) else m


def device_layer(w: I.Workload):
    """One DeviceLayer per distinct weight set (decode and prefill share)."""
    from mixture_experts_layer_19_amd.layer import DeviceLayer
    key = (w.H, w.E, w.k, w.I, w.Is, w.dtype, w.seed, w.zipf_beta)
    if key not in _layers:
        print("[gpu] building layer %s" % (key,), flush=True)
        _layers[key] = DeviceLayer(w)
    lay = _layers[key]
    lay.w = w
    return lay


def to_numpy(t):
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def rel_max_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(gpu - ref).max() / np.abs(ref).max())


# per-workload parity margins of this session, printed by conftest's summary
MARGINS = []


def compare_layer(orc, w: I.Workload, x, out, g_idx, toks, label=None):
    """Compare the GPU layer output ``out`` [T,H] for tokens ``toks`` with the
    oracle.  The GPU's routing ``g_idx`` [T,k] must equal the oracle's except
    on tie flips (oracle.parity's rule); a flipped token is evaluated by the
    oracle with the GPU's selection, so every token in ``toks`` is compared.
    Returns the relative error max|gpu - oracle| / max|oracle| and records
    it with the token and flip counts in MARGINS."""
    Wr, b = I.router_weight(w), I.router_bias(w)
    o_idx, _, scores, _ = orc.route(x, Wr, b, w.k, w.rho, w.route_norm)
    mism, flips = classify_routing(g_idx, o_idx, scores)
    bad = np.nonzero(mism & ~flips)[0]
    assert len(bad) == 0, "routing differs beyond near-ties at tokens %s" % bad[:10].tolist()
    toks = np.asarray(toks)
    flipped = toks[flips[toks]]
    plain = toks[~flips[toks]]
    experts = np.concatenate([o_idx[plain].ravel(), g_idx[flipped].ravel()])
    ew = expert_weights_parallel(w, experts)
    kw = dict(k=w.k, rho=w.rho, route_norm=w.route_norm, mx=oracle_mx(w.dtype), fp8=oracle_fp8(w))
    shared = I.shared_stored(w) if w.Is else None
    ref = np.empty((len(toks), w.H), np.float32)
    where = {int(t): i for i, t in enumerate(toks)}
    if len(plain):
        r, idx, _, _ = orc.layer_forward_tokens(plain, x, Wr, b, lambda e: ew[e], shared, **kw)
        np.testing.assert_array_equal(idx, o_idx[plain])
        ref[[where[int(t)] for t in plain]] = r
    if len(flipped):
        r, _, _, _ = orc.layer_forward_tokens(flipped, x, Wr, b, lambda e: ew[e], shared,
                                              topk_idx=g_idx[flipped], **kw)
        ref[[where[int(t)] for t in flipped]] = r
    err = rel_max_err(out[toks], ref)
    MARGINS.append(dict(workload=label or w.name, T=w.T, compared=len(toks),
                        tie_flips=int(flips.sum()), flips_compared=len(flipped),
                        rel_err=err, tol=TOL[w.dtype]))
    print("[layer] %s T=%d: %d of %d tokens compared (%d tie flips, all re-evaluated), rel err %.3g"
          % (label or w.name, w.T, len(toks), w.T, int(flips.sum()), err), flush=True)
    return err


def expert_weights_parallel(w: I.Workload, experts, threads=None):
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    experts = sorted(set(int(e) for e in experts))
    with ThreadPoolExecutor(max_workers=threads) as ex:
        vals = list(ex.map(lambda e: I.expert_stored(w, e), experts))
    return dict(zip(experts, vals))


def unpack_blocks(packed: np.ndarray, E: int, N: int, row_bytes: int) -> np.ndarray:
    """Inverse of the packed fragment layout: bytes [E, N/16, K/256, piece 4,
    lane 64, 16] -> dense bytes [E, N, row_bytes], with lane l = row l % 16,
    lane group g = l / 16, and piece p at chunk byte 128 (p/2) + 64 (p%2) + 16 g."""
    nb, kc = N // 16, row_bytes // 256
    a = packed.reshape(E, nb, kc, 2, 2, 4, 16, 16)       # e nb kc ph pl g r byte
    a = a.transpose(0, 1, 6, 2, 3, 4, 5, 7)               # e nb r kc ph pl g byte
    return a.reshape(E, N, row_bytes)


def unpack_scales(packed: np.ndarray, E: int, N: int, K: int) -> np.ndarray:
    """Packed uint16 scale pairs [E, N/16, K/256, lane] -> E8M0 bytes [E, N, K/32].
    Byte h of lane l is the scale of 32-block 8 kc + 4 h + l / 16 of row l % 16."""
    nb, kc = N // 16, K // 256
    b = packed.view(np.uint8).reshape(E, nb, kc, 4, 16, 2)   # e nb kc g r h
    b = b.transpose(0, 1, 4, 2, 5, 3)                         # e nb r kc h g
    return b.reshape(E, N, K // 32)


def oracle_fp8(w: I.Workload):
    """Static FP8 activation scales (x, routed h, shared h) of an "fp8"
    workload, else None."""
    return (w.fp8_x_scale, w.fp8_h_scale, w.fp8_sh_h_scale) if w.dtype == "fp8" else None


def oracle_ffn(orc, w: I.Workload, x, weights, shared=False):
    """The oracle's SwiGLU FFN of one expert in the workload's format."""
    if w.dtype == "fp8":
        return orc.swiglu_rows_fp8(x, *weights, w.fp8_x_scale,
                                   w.fp8_sh_h_scale if shared else w.fp8_h_scale)
    return orc.swiglu_rows(x, *weights, mx=oracle_mx(w.dtype, shared))


def unpack_blocks_e2m1(packed: np.ndarray, E: int, N: int, K: int) -> np.ndarray:
    """Inverse of the MXFP4 packed layout: bytes [E, N/16, K/256, half 2,
    lane group 4, row 16, 16 bytes] -> E2M1 codes [E, N, K] (one per byte),
    where lane group g of half h holds K [128 h + 32 g, +32) of its row, two
    codes per byte, low nibble first."""
    nb, kc = N // 16, K // 256
    a = packed.reshape(E, nb, kc, 2, 4, 16, 16)               # e nb kc h g r byte
    codes = np.stack([a & 15, a >> 4], axis=-1).reshape(E, nb, kc, 2, 4, 16, 32)
    codes = codes.transpose(0, 1, 5, 2, 3, 4, 6)              # e nb r kc h g i
    return codes.reshape(E, N, K)


def virtual_to_gate_up(dense: np.ndarray, I_: int):
    """Split interleaved gate/up virtual rows (16-row blocks alternate)."""
    E = dense.shape[0]
    a = dense.reshape(E, I_ // 16, 2, 16, -1)
    return a[:, :, 0].reshape(E, I_, -1), a[:, :, 1].reshape(E, I_, -1)
