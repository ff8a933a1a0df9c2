"""Benchmark of one Hunyuan-style MoE layer forward pass on one MI355X.

A step is one moe_layer_forward call (gating, permutation, routed grouped
SwiGLU GEMM, shared expert on the side stream, combine) over one batch of
synthetic tokens, with weights and inputs already resident in HBM.  The
default workload is the Hy3-shape decode batch (T = 64, H = 4096, 192
experts, top-8, I = I_s = 1536, bf16); the same weights then run the T = 8192
prefill batch, reported under "prefill".  Prints one JSON line.

  roofline     dominant kernel (the routed gate/up + SwiGLU GEMM): algorithmic
               bytes (decode, HBM-bound) or flops (prefill, MFMA-bound) per
               launch over its mean duration from HIP events recorded around
               it on its own stream during profiled steps
  cpu_baseline the CPU oracle on a bounded sample of the same batch
  parity       that sample's oracle output against the timed batch's: routing
               index mismatches (and tie flips among them) and the largest
               relative output error
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + %HBM (T=64) / %MFMA peak (T=8192), Hy3 shape, 1 GPU"
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6        # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
FP8_PEAK_TFLOPS = 5033.2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="hy3_decode",
                    choices=["hy3_decode", "hy3_prefill", "hy4_skew", "mx", "tiny", "w4a8_decode",
                             "w4a8", "fp8_decode", "fp8"])
    ap.add_argument("--profile-steps", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the batch replayed from a captured HIP graph")
    ap.add_argument("--single-stream", action="store_true",
                    help="run the shared expert on the main stream (per-stage times then "
                         "measure each kernel alone)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def measured_traffic(workload: str):
    """HBM bytes per launch of the decode gate/up kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when the kernel's
    source has changed since those counters were taken."""
    import hashlib
    if workload != "hy3_decode":
        return None
    path = os.path.join(ROOT, "profiles", "hy3_decode_gate_up_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        kv[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in ("mixture_experts_layer_19_amd/csrc/gemm.hip",
              "mixture_experts_layer_19_amd/csrc/moe_common.hpp"):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if kv.get("source_sha256") != h.hexdigest():
        return None
    return int(kv["traffic_bytes"])


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU: the library runs the whole MoE layer on a single "
              "MI355X and has no multi-GPU path (--gpus %d requested)" % a.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixture_experts_layer_19_amd import binding as B
    from mixture_experts_layer_19_amd import inputs as I
    from mixture_experts_layer_19_amd.layer import DeviceLayer, to_device

    w = I.workload(a.workload)
    dev = torch.device("cuda", 0)
    t0 = time.time()
    log("drawing %s weights (E=%d, H=%d, I=%d, %s)" % (w.name, w.E, w.H, w.I, w.dtype))
    Wg, Wu, Wd = I.all_experts_stored(w)
    shared = I.shared_stored(w)
    Wr, bias = I.router_weight(w), I.router_bias(w)
    log("uploading and packing (%.1fs)" % (time.time() - t0))
    lay = DeviceLayer(w, expert_fn=lambda e: (Wg[e], Wu[e], Wd[e]), shared_fn=lambda: shared,
                      router=(Wr, bias), side_stream=not a.single_stream)
    main_stream = torch.cuda.current_stream(dev)

    def run(x_dev, T, steps, warmup):
        out = torch.empty((T, w.H), dtype=lay.out_dtype(), device=dev)
        for _ in range(warmup):
            lay.forward(x_dev, out)
        torch.cuda.synchronize(dev)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        h0 = time.perf_counter()
        e0.record(main_stream)
        for _ in range(steps):
            lay.forward(x_dev, out)
        e1.record(main_stream)
        torch.cuda.synchronize(dev)
        wall = (time.perf_counter() - h0) * 1e3
        return e0.elapsed_time(e1) / steps, wall / steps, out

    def run_graph(x_dev, T, steps, warmup):
        # the same forward captured once as a HIP graph and replayed on the
        # caller's stream: what a serving loop that records its decode step
        # would run
        out = torch.empty((T, w.H), dtype=lay.out_dtype(), device=dev)
        xs = x_dev.clone()
        graph = lay.capture(xs, out)
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize(dev)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(main_stream)
        for _ in range(steps):
            graph.replay()
        e1.record(main_stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / steps

    def stage_profile(x_dev, T, steps):
        B.moe_ctx_set_profiling(lay.ctx, True)
        out = torch.empty((T, w.H), dtype=lay.out_dtype(), device=dev)
        acc = {}
        for _ in range(steps):
            lay.forward(x_dev, out)
            ms = B.moe_ctx_stage_ms(lay.ctx)
            for k, v in ms.items():
                acc[k] = acc.get(k, 0.0) + v
        B.moe_ctx_set_profiling(lay.ctx, False)
        return {k: v / steps for k, v in acc.items()}

    def routed_experts(T):
        ws = lay.workspace(T)
        io, _ = B.moe_layer_ws_topk(lay.desc, T)
        idx = ws[io:io + 4 * T * w.k].view(torch.int32).cpu().numpy()
        return int(np.unique(idx).size)

    # bytes per weight of the routed and the shared experts (MX: + one scale
    # byte per 32); W4A8 keeps its shared expert in MX-fp8
    mxw = w.dtype in ("mxfp8", "w4a8")
    eight = mxw or w.dtype == "fp8"            # 8-bit (or 4-bit) products
    eb = {"bf16": 2, "f32": 4, "mxfp8": 1, "w4a8": 0.5, "fp8": 1}[w.dtype]
    ebs = 1 if w.dtype == "w4a8" else eb
    sb = (1.0 / 32.0) if mxw else 0.0
    ab = 1 if eight else eb                    # bytes per element of h
    ob = 4 if w.dtype == "f32" else 2
    xb = 4 if w.dtype == "f32" else 2

    # ------------------------------------------------------------------ decode-size batch
    xg, x32 = I.x_input(w)
    xd = to_device(xg, dev)
    T = w.T
    log("timing %s: T=%d, %d warm-up + %d steps" % (w.name, T, a.warmup, a.steps))
    ms, wall_ms, out_decode = run(xd, T, a.steps, a.warmup)
    out_host = out_decode.float().cpu().numpy()
    ws = lay.workspace(T)
    io, _ = B.moe_layer_ws_topk(lay.desc, T)
    idx_host = ws[io:io + 4 * T * w.k].view(torch.int32).reshape(T, w.k).cpu().numpy()
    touched = routed_experts(T)
    stages = stage_profile(xd, T, a.profile_steps)
    P = T * w.k
    # algorithmic bytes: weights of the touched experts, shared expert, router,
    # activations in, layer output
    expert_bytes = (3 * w.I * w.H) * (eb + sb)
    shared_bytes = (3 * w.Is * w.H) * (ebs + sb)
    layer_bytes = (touched * expert_bytes + shared_bytes + w.E * w.H * 4 + T * w.H * xb
                   + T * w.H * ob)
    gu_bytes = touched * (2 * w.I * w.H) * (eb + sb) + T * w.H * xb + P * w.I * (ab + sb)
    gu_ms = stages["gate_up"]
    flops = 2.0 * P * 3 * w.I * w.H + 2.0 * T * 3 * w.Is * w.H
    gu_flops = 2.0 * P * 2 * w.I * w.H
    tok_s = T / (ms * 1e-3)
    # MX products run at the fp8 rate (an E2M1 x E4M3 product is priced as fp8)
    mfma_peak = FP8_PEAK_TFLOPS if eight else BF16_PEAK_TFLOPS
    if w.name == "hy3_prefill":
        roof = {"bound": "mfma", "kernel": "routed gate/up + SwiGLU grouped GEMM",
                "achieved": round(gu_flops / (gu_ms * 1e-3) / 1e12, 1), "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": round(gu_flops / (gu_ms * 1e-3) / 1e12 / mfma_peak, 4),
                "traffic": None, "kernel_ms": round(gu_ms, 4), "algorithmic_flops": gu_flops}
    else:
        roof = {"bound": "hbm", "kernel": "routed gate/up + SwiGLU grouped GEMM",
                "achieved": round(gu_bytes / (gu_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(gu_bytes / (gu_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(w.name), "kernel_ms": round(gu_ms, 4),
                "algorithmic_bytes": int(gu_bytes)}
    result = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "mxfp8": "mxfp8-e4m3",
                  "w4a8": "mxfp4-e2m1 x mxfp8-e4m3", "fp8": "fp8-e4m3 per-tensor"}[w.dtype],
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": w.name, "tokens": T, "hidden": w.H, "experts": w.E,
                   "top_k": w.k, "inter": w.I, "shared_inter": w.Is,
                   "touched_experts": touched, "parallelism": "single GPU"},
        "roofline": roof,
        "layer": {"algorithmic_bytes": int(layer_bytes),
                  "hbm_GBps": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
                  "hbm_frac": round(layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                  "mfma_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
                  "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / mfma_peak, 4),
                  "host_wall_ms_per_step": round(wall_ms, 4)},
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
    }
    if not a.no_graph:
        gms = run_graph(xd, T, a.steps, a.warmup)
        result["graph_replay"] = {"ms_per_step": round(gms, 4),
                                  "tokens_per_s": round(T / (gms * 1e-3), 1),
                                  "hbm_frac": round(layer_bytes / (gms * 1e-3) / 1e9
                                                    / HBM_PEAK_GBPS, 4)}

    # ------------------------------------------------------------------ prefill batch
    if not a.no_prefill and w.name == "hy3_decode":
        wp = I.workload("hy3_prefill")
        lay.w = wp
        xpg, _ = I.x_input(wp)
        xpd = to_device(xpg, dev)
        Tp = wp.T
        log("timing hy3_prefill: T=%d" % Tp)
        msp, _, _ = run(xpd, Tp, max(5, a.steps // 5), max(2, a.warmup // 2))
        stp = stage_profile(xpd, Tp, max(3, a.profile_steps // 4))
        Pp = Tp * wp.k
        fl = 2.0 * Pp * 3 * wp.I * wp.H + 2.0 * Tp * 3 * wp.Is * wp.H
        gu_fl = 2.0 * Pp * 2 * wp.I * wp.H
        result["prefill"] = {
            "workload": wp.name, "tokens": Tp, "ms_per_step": round(msp, 4),
            "tokens_per_s": round(Tp / (msp * 1e-3), 1),
            "mfma_TFLOPs": round(fl / (msp * 1e-3) / 1e12, 1),
            "mfma_frac": round(fl / (msp * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "roofline": {"bound": "mfma", "kernel": "routed gate/up + SwiGLU grouped GEMM",
                         "achieved": round(gu_fl / (stp["gate_up"] * 1e-3) / 1e12, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(gu_fl / (stp["gate_up"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "traffic": None, "kernel_ms": round(stp["gate_up"], 4)},
            "stages_ms": {k: round(v, 4) for k, v in stp.items()},
        }
        lay.w = w
        del xpd

    if a.copy_calib:
        # plain device copy of a known size, for HBM counter calibration
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        del src, dst

    # ------------------------------------------------------------------ CPU oracle
    if not a.no_cpu:
        import oracle
        oracle.build(force=False)

        def oracle_tokens(toks):
            return oracle.layer_forward_tokens(toks, x32, Wr, bias, lambda e: (Wg[e], Wu[e], Wd[e]),
                                        shared, k=w.k, rho=w.rho, route_norm=w.route_norm,
                                        mx={"mxfp8": 1, "w4a8": 2}.get(w.dtype, 0),
                                        fp8=((w.fp8_x_scale, w.fp8_h_scale, w.fp8_sh_h_scale)
                                             if w.dtype == "fp8" else None))

        # a bounded sample: the first n tokens of the batch (all of them when
        # the batch is small), evaluated `reps` times back to back
        t1 = time.perf_counter()
        oracle_tokens(np.arange(1))
        one = time.perf_counter() - t1
        n = int(max(1, min(T, a.cpu_seconds / max(one, 1e-3))))
        t1 = time.perf_counter()
        oracle_tokens(np.arange(n))
        first = time.perf_counter() - t1
        reps = int(max(1, min(100, a.cpu_seconds / max(first, 1e-3))))
        t1 = time.perf_counter()
        for _ in range(reps):
            oracle_tokens(np.arange(n))
        dt = time.perf_counter() - t1
        # parity of the timed batch on the same sample: routing indices
        # (mismatches, and those inside the oracle's 1e-6 score gap at the
        # top-k boundary, i.e. tie flips) and the output relative to the
        # largest oracle magnitude, over the tokens whose routing agrees
        ref, o_idx, _, gap = oracle_tokens(np.arange(n))
        mism = (idx_host[:n] != o_idx).any(axis=1)
        keep = ~mism
        err = (float(np.abs(out_host[:n][keep].astype(np.float64) - ref[keep]).max()
                     / np.abs(ref[keep]).max()) if keep.any() else None)
        result["parity"] = {
            "tokens": n, "index_mismatches": int(mism.sum()),
            "tie_flips": int((mism & (gap <= 1e-6)).sum()),
            "max_rel_err": None if err is None else float("%.3g" % err),
            "tolerance": {"f32": 1e-5, "bf16": 1e-2}.get(w.dtype, 3e-2)}
        result["cpu_baseline"] = {
            "value": round(n * reps / dt, 3), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "first %d of the %d tokens of the %s batch, %d passes: fp64-accumulating "
                      "C oracle (gating, each token's %d expert FFNs, shared FFN, combine); "
                      "%.1f s" % (n, T, w.name, reps, w.k, dt)}

    lay.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
