"""Benchmark of one Hunyuan-style MoE layer forward pass on one MI355X.

A step is one moe_layer_forward call (gating, permutation, routed grouped
SwiGLU GEMM, shared expert -- on the side stream where that pays, else on
the caller's stream, folded into the routed GEMMs where it can be -- and
combine) over one batch of
synthetic tokens, with weights and inputs already resident in HBM.  The
default run times the five workloads (tiny fp32, Hy3 decode T = 64, Hy3
prefill T = 8192, Hy4-shape skewed T = 2048, MX-fp8 T = 4096) and prints one
JSON line whose headline is the Hy3 decode batch; every workload has its own
object under "workloads".

Timing: each timed step is bracketed by HIP events on the caller's stream;
before every step (outside the bracket) a 1 GiB read evicts L2 and the
256 MB MALL.  Reported: the median step, with p10 and p90.

  roofline     the dominant kernel (the routed gate/up + SwiGLU GEMM, with the
               shared expert's gate/up when that is folded into it): its
               algorithmic bytes (HBM-bound workloads) or flops (prefill) per
               launch over its duration, timed with HIP events recorded
               around it on its own stream (median of profiled steps)
  layer        the whole step against HBM and matrix-core peaks
  parity       the oracle on a sample of the timed batch's tokens against the
               GPU output: routing mismatches, tie flips (evaluated with the
               GPU's selection), largest relative error
  cpu_baseline the CPU oracle on a bounded sample of the headline batch

``--trace-summary DIR`` instead summarises a rocprofv3 kernel trace (no GPU).
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
FP8_PEAK_TFLOPS = 5033.2         # dense fp8 / MX-fp8
FP32_PEAK_TFLOPS = 157.3         # fp32 matrix / vector
DEFAULT_WORKLOADS = ["hy3_decode", "tiny", "hy3_prefill", "hy4_skew", "mx"]
# workloads whose binding roofline is the matrix cores (the others: HBM)
MFMA_BOUND = {"hy3_prefill"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "hy3_decode", "hy3_prefill", "hy4_skew", "mx", "tiny",
                             "w4a8_decode", "w4a8", "fp8_decode", "fp8"])
    ap.add_argument("--profile-steps", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the batch replayed from a captured HIP graph")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not evict the caches before each timed step")
    ap.add_argument("--single-stream", action="store_true",
                    help="run the shared expert on the main stream (per-stage times then "
                         "measure each kernel alone)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="summarise the rocprofv3 kernel trace under DIR and exit")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR", "JSON"),
                    help="write the gate/up traffic file of WORKLOAD from rocprofv3 FETCH_SIZE and "
                         "WRITE_SIZE runs and the FETCH_SIZE run's bench line, and exit")
    ap.add_argument("--counter-summary", metavar="DIR", nargs="+",
                    help="summarise rocprofv3 --pmc outputs under DIR(s) and exit")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def pct(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v, dtype=np.float64), q))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_traffic(workload: str):
    """HBM bytes per launch of the workload's gate/up kernel from its committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (profiles/<workload>_gate_up_traffic.txt,
    written by --traffic-summary), or None when there is none or the GEMM
    source has changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "%s_gate_up_traffic.txt" % workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != gemm_source_sha256():
        return None
    return int(kv["traffic_bytes"])


def traffic_summary(workload: str, fetch_dir: str, write_dir: str, bench_json: str) -> None:
    """The traffic file of the workload's gate/up kernel: the largest-grid
    grouped GEMM dispatch with the SwiGLU epilogue (template arguments
    <format, 0, ...>) in two rocprofv3 --pmc runs of bench.py (FETCH_SIZE,
    then WRITE_SIZE, both with --copy-calib), calibrated by the 1 GiB device
    copy of the same runs, against the algorithmic bytes the counter run's
    bench line reports."""
    import csv
    import glob
    import re

    def load(d, counter):
        vals = {}
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] != counter:
                        continue
                    name = re.sub(r"\(.*$", "", r["Kernel_Name"]).replace("void ", "").replace("moe::", "")
                    vals.setdefault((name, int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
        return vals

    fv, wv = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    gemm = [k for k in fv if re.match(r"gemm_(skinny|tile)_kernel<\d+, 0,", k[0])]
    if not gemm:
        sys.exit("no gate/up GEMM dispatch in %s" % fetch_dir)
    key = max(gemm, key=lambda k: k[1])
    def copy_kib(vals):
        # mean over the dispatches of the largest copy (the 1 GiB calibration)
        grids = [g for (n, g) in vals if n == "__amd_rocclr_copyBuffer"]
        if not grids:
            return 0.0
        v = vals[("__amd_rocclr_copyBuffer", max(grids))]
        return sum(v) / len(v)

    copy_f, copy_w = copy_kib(fv), copy_kib(wv)
    if copy_f <= 0 or copy_w <= 0 or key not in wv:
        sys.exit("the runs need --copy-calib and the kernel in both counter passes")
    ff, fw = (1 << 30) / (copy_f * 1024.0), (1 << 30) / (copy_w * 1024.0)
    fk, wk = sum(fv[key]) / len(fv[key]), sum(wv[key]) / len(wv[key])
    traffic = int(round(fk * 1024 * ff + wk * 1024 * fw))
    with open(bench_json) as fh:
        line = json.loads(fh.read().strip().splitlines()[-1])
    alg = int(line["roofline"]["algorithmic_bytes"])
    cmd = ("bench.py --workload %s --steps 3 --warmup 1 --profile-steps 1 --no-cpu --no-parity "
           "--no-graph --no-flush --copy-calib" % workload)
    print("# HBM traffic of the gate/up kernel of the %s workload" % workload)
    print("# Commands (from /tmp, TMPDIR=/tmp), one counter per run, then this summary:")
    print("#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <f> -o p -- python3 %s > <f>.json" % cmd)
    print("#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <w> -o p -- python3 %s" % cmd)
    print("#   python3 bench.py --traffic-summary %s <f> <w> <f>.json" % workload)
    print("# Calibration: the runs copy 1 GiB device-to-device; the counters read FETCH_SIZE %.1f KiB"
          % copy_f)
    print("# and WRITE_SIZE %.1f KiB for it, so bytes = FETCH_SIZE * 1024 * %.4f and WRITE_SIZE * 1024 * %.4f."
          % (copy_w, ff, fw))
    print("# Values are KiB per dispatch, averaged over %d dispatches.  Algorithmic bytes of the" % len(fv[key]))
    print("# kernel (from the counter run's bench line): %d; the measured traffic is %.4f x that." %
          (alg, traffic / alg))
    print("kernel: %s grid %d" % (key[0], key[1]))
    print("source_sha256: %s" % gemm_source_sha256())
    print("fetch_kib: %.1f" % fk)
    print("write_kib: %.1f" % wk)
    print("fetch_factor: %.4f" % ff)
    print("write_factor: %.4f" % fw)
    print("algorithmic_bytes: %d" % alg)
    print("traffic_bytes: %d" % traffic)


# ----------------------------------------------------------------------------- trace summary


def trace_summary(d: str) -> None:
    """Per-kernel statistics of a rocprofv3 kernel trace, with the routed and
    the shared-expert launches (the latter on the side stream) in separate
    rows, and the overlap of the shared expert with the main stream."""
    import csv
    import glob
    import re
    files = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        sys.exit("no *kernel_trace.csv under %s" % d)
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))

    def short(name):
        name = re.sub(r"\(.*$", "", name)
        name = re.sub(r"^void ", "", name)
        return name.replace("moe::", "").replace("(anonymous namespace)::", "")

    streams = sorted({int(r["Stream_Id"]) for r in rows})
    groups = {}
    for r in rows:
        key = (short(r["Kernel_Name"]), int(r["Stream_Id"]), int(r["Grid_Size_X"]))
        groups.setdefault(key, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    total = sum(e - s for v in groups.values() for s, e in v)
    print("| Kernel | Stream | Grid (threads) | Calls | Median (us) | Mean (us) | Min (us) | Max (us) | Share |")
    print("|---|---|---|---|---|---|---|---|---|")
    for key, v in sorted(groups.items(), key=lambda kv: -sum(e - s for s, e in kv[1])):
        durs = sorted((e - s) / 1e3 for s, e in v)
        print("| `%s` | %d | %d | %d | %.1f | %.1f | %.1f | %.1f | %.2f%% |"
              % (key[0], key[1], key[2], len(v), durs[len(durs) // 2], sum(durs) / len(durs),
                 durs[0], durs[-1], 100.0 * sum(durs) * 1e3 / total))
    if len(streams) > 1:
        # time the side-stream kernels spend running while a main-stream kernel runs
        main = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
                      if int(r["Stream_Id"]) == streams[0])
        side = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
                if int(r["Stream_Id"]) != streams[0]]
        busy = ov = 0
        for s, e in side:
            busy += e - s
            for ms, me in main:
                if me <= s:
                    continue
                if ms >= e:
                    break
                ov += min(e, me) - max(s, ms)
        print("\nSide-stream kernels: %.1f us in total, %.1f%% of it beside a main-stream kernel"
              % (busy / 1e3, 100.0 * ov / max(busy, 1)))


def _code_text(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def gemm_source_sha256() -> str:
    """SHA-256 of the grouped GEMM sources with comments and whitespace
    removed (to tie counter readings to the code they were taken with; a
    change of comments leaves it as it is)."""
    import hashlib
    h = hashlib.sha256()
    for f in ("mixture_experts_layer_19_amd/csrc/gemm.hip",
              "mixture_experts_layer_19_amd/csrc/gemm_common.hpp",
              "mixture_experts_layer_19_amd/csrc/moe_common.hpp"):
        h.update(_code_text(open(os.path.join(ROOT, f)).read()).encode())
    return h.hexdigest()


def counter_summary(dirs) -> None:
    """Mean per dispatch of every counter in rocprofv3 --pmc outputs, by kernel
    and grid size.  FETCH_SIZE / WRITE_SIZE (KiB) are also converted to bytes
    with the factor that makes a 1 GiB device copy in the same run (the
    largest __amd_rocclr_copyBuffer dispatch) read or write 1 GiB."""
    import csv
    import glob
    import re
    rows = []
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            with open(f) as fh:
                rows += list(csv.DictReader(fh))
    if not rows:
        sys.exit("no *counter_collection.csv under %s" % " ".join(dirs))

    def short(name):
        name = re.sub(r"\(.*$", "", name)
        return re.sub(r"^void ", "", name).replace("moe::", "")

    vals = {}
    for r in rows:
        key = (short(r["Kernel_Name"]), int(r["Grid_Size"]))
        vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    factor = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        copies = [max(v[c]) for (n, _), v in vals.items() if n == "__amd_rocclr_copyBuffer" and c in v]
        if copies and max(copies) > 0:
            factor[c] = (1 << 30) / (max(copies) * 1024.0)
    counters = sorted({c for v in vals.values() for c in v})
    print("GEMM source sha256: %s" % gemm_source_sha256())
    for c, f in factor.items():
        print("%s calibration: bytes = KiB x 1024 x %.4f (1 GiB copy)" % (c, f))
    print()
    print("| Kernel | Grid | Dispatches | " + " | ".join(counters) + " |")
    print("|---|---|---|" + "---|" * len(counters))
    for key in sorted(vals, key=lambda k: (k[0], k[1])):
        v = vals[key]
        n = max(len(x) for x in v.values())
        cells = []
        for c in counters:
            if c not in v:
                cells.append("")
                continue
            m = sum(v[c]) / len(v[c])
            cell = "%.1f" % m
            if c in factor:
                cell += " (%.3f GB)" % (m * 1024.0 * factor[c] / 1e9)
            cells.append(cell)
        print("| `%s` | %d | %d | %s |" % (key[0], key[1], n, " | ".join(cells)))


# ----------------------------------------------------------------------------- measurement


def main():
    a = parse()
    if a.trace_summary:
        trace_summary(a.trace_summary)
        return
    if a.counter_summary:
        counter_summary(a.counter_summary)
        return
    if a.traffic_summary:
        traffic_summary(*a.traffic_summary)
        return
    if a.gpus != 1:
        print("bench.py measures one GPU: the library runs the whole MoE layer on a single "
              "MI355X and has no multi-GPU path (--gpus %d requested)" % a.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixture_experts_layer_19_amd import binding as B
    from mixture_experts_layer_19_amd import inputs as I
    from mixture_experts_layer_19_amd.layer import DeviceLayer, to_device

    dev = torch.device("cuda", 0)
    main_stream = torch.cuda.current_stream(dev)
    flush_buf = None if a.no_flush else torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def flush():
        # a read of 1 GiB on the caller's stream, outside the bracket: it
        # evicts L2 and the MALL and leaves them holding clean lines (a fill
        # would leave dirty lines whose write-back lands inside the next step)
        if flush_buf is not None:
            torch.amax(flush_buf)

    def timed(step_fn, steps, warmup):
        for _ in range(warmup):
            step_fn()
        torch.cuda.synchronize(dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for e0, e1 in ev:
            flush()
            e0.record(main_stream)
            step_fn()
            e1.record(main_stream)
        torch.cuda.synchronize(dev)
        return [e0.elapsed_time(e1) for e0, e1 in ev]

    def stage_profile(lay, x_dev, out, steps):
        B.moe_ctx_set_profiling(lay.ctx, True)
        acc = {}
        for _ in range(steps):
            flush()
            lay.forward(x_dev, out)
            for k, v in B.moe_ctx_stage_ms(lay.ctx).items():
                acc.setdefault(k, []).append(v)
        B.moe_ctx_set_profiling(lay.ctx, False)
        return {k: float(np.median(v)) for k, v in acc.items()}

    def gpu_topk(lay, w, T):
        ws = lay.workspace(T)
        io, _ = B.moe_layer_ws_topk(lay.desc, T)
        return ws[io:io + 4 * T * w.k].view(torch.int32).reshape(T, w.k).cpu().numpy()

    orc = None
    if not (a.no_cpu and a.no_parity):
        import oracle
        from oracle import parity as par
        oracle.build(force=False)
        orc = oracle

    def oracle_kw(w):
        return dict(k=w.k, rho=w.rho, route_norm=w.route_norm,
                    mx={"mxfp8": 1, "w4a8": 2}.get(w.dtype, 0),
                    fp8=((w.fp8_x_scale, w.fp8_h_scale, w.fp8_sh_h_scale)
                         if w.dtype == "fp8" else None))

    def expert_cache(w):
        cache = {}

        def get(e):
            if e not in cache:
                cache[e] = I.expert_stored(w, e)
            return cache[e]
        return get

    def parity_sample(w, x32, out_host, g_idx, toks):
        """The oracle on tokens `toks` of the timed batch, with the tie rule
        and flipped tokens evaluated with the GPU's selection."""
        Wr, b = I.router_weight(w), I.router_bias(w)
        xs = x32[toks]
        o_idx, _, scores, _ = orc.route(xs, Wr, b, w.k, w.rho, w.route_norm)
        mism, flips = par.classify_routing(g_idx[toks], o_idx, scores)
        get = expert_cache(w)
        sh = I.shared_stored(w) if w.Is else None
        sel = np.where(flips[:, None], g_idx[toks], o_idx)
        ok = ~mism | flips
        ref, _, _, _ = orc.layer_forward_tokens(toks[ok], x32, Wr, b, get, sh, topk_idx=sel[ok],
                                                **oracle_kw(w))
        got = out_host[toks[ok]].astype(np.float64)
        err = float(np.abs(got - ref).max() / np.abs(ref).max()) if ok.any() else None
        return {"tokens": int(len(toks)), "index_mismatches": int(mism.sum()),
                "tie_flips": int(flips.sum()), "non_tie_mismatches": int((mism & ~flips).sum()),
                "max_rel_err": None if err is None else float("%.3g" % err),
                "tolerance": {"f32": 1e-5, "bf16": 1e-2}.get(w.dtype, 3e-2)}

    def bytes_per_weight(w):
        # routed and shared expert weights (MX: + one scale byte per 32; the
        # shared expert of a W4A8 layer is MX-fp8)
        mxw = w.dtype in ("mxfp8", "w4a8")
        eb = {"bf16": 2, "f32": 4, "mxfp8": 1, "w4a8": 0.5, "fp8": 1}[w.dtype]
        ebs = 1 if w.dtype == "w4a8" else eb
        sb = (1.0 / 32.0) if mxw else 0.0
        return eb + sb, ebs + sb

    def run_workload(w, lay, headline=False):
        T = w.T
        lay.w = w
        xg, x32 = I.x_input(w)
        x_dev = to_device(xg, dev)
        out = torch.empty((T, w.H), dtype=lay.out_dtype(), device=dev)
        log("timing %s: T=%d, %d warm-up + %d steps" % (w.name, T, a.warmup, a.steps))
        wall0 = time.perf_counter()
        ts = timed(lambda: lay.forward(x_dev, out), a.steps, a.warmup)
        wall = (time.perf_counter() - wall0) * 1e3 / (a.steps + a.warmup)
        torch.cuda.synchronize(dev)
        out_host = out.float().cpu().numpy()
        g_idx = gpu_topk(lay, w, T)
        touched = int(np.unique(g_idx).size)
        stages = stage_profile(lay, x_dev, out, a.profile_steps)
        ms = float(np.median(ts))
        P = T * w.k
        ew, ews = bytes_per_weight(w)
        eight = w.dtype in ("mxfp8", "w4a8", "fp8")
        ab = 1 if eight else {"f32": 4}.get(w.dtype, 2)       # bytes per element of x, h
        xb = 4 if w.dtype == "f32" else 2
        ob = xb
        layer_bytes = (touched * 3 * w.I * w.H * ew + 3 * w.Is * w.H * ews + w.E * w.H * 4
                       + T * w.H * xb + T * w.H * ob)
        flops = 2.0 * P * 3 * w.I * w.H + 2.0 * T * 3 * w.Is * w.H
        gu_bytes = touched * 2 * w.I * w.H * ew + T * w.H * xb + P * w.I * ab
        gu_flops = 2.0 * P * 2 * w.I * w.H
        gu_ms = stages["gate_up"]
        # a layer whose shared expert shows no time of its own ran it inside
        # the routed GEMMs (one more segment, on the caller's stream): the
        # gate/up kernel then also does the shared expert's gate/up work
        folded = w.Is > 0 and stages["shared_gate_up"] == 0.0
        gu_kernel = "routed gate/up + SwiGLU grouped GEMM"
        if folded:
            gu_bytes += 2 * w.Is * w.H * ews + T * w.Is * ab
            gu_flops += 2.0 * T * 2 * w.Is * w.H
            gu_kernel += " (with the shared expert's gate/up as one more segment)"
        mfma_peak = (FP8_PEAK_TFLOPS if eight else FP32_PEAK_TFLOPS if w.dtype == "f32"
                     else BF16_PEAK_TFLOPS)
        if w.name in MFMA_BOUND:
            ach = gu_flops / (gu_ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "kernel": gu_kernel,
                    "achieved": round(ach, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                    "frac": round(ach / mfma_peak, 4), "traffic": measured_traffic(w.name),
                    "kernel_ms": round(gu_ms, 4), "algorithmic_flops": gu_flops,
                    "algorithmic_bytes": int(gu_bytes)}
        else:
            ach = gu_bytes / (gu_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "kernel": gu_kernel,
                    "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(w.name),
                    "kernel_ms": round(gu_ms, 4), "algorithmic_bytes": int(gu_bytes)}
        res = {
            "workload": w.name, "tokens": T, "hidden": w.H, "experts": w.E, "top_k": w.k,
            "inter": w.I, "shared_inter": w.Is, "dtype": w.dtype, "touched_experts": touched,
            "ms_per_step": round(ms, 4), "p10_ms": round(pct(ts, 10), 4),
            "p90_ms": round(pct(ts, 90), 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "roofline": roof,
            "layer": {"algorithmic_bytes": int(layer_bytes),
                      "hbm_GBps": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
                      "hbm_frac": round(layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                      "algorithmic_flops": flops,
                      "mfma_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
                      "mfma_peak": mfma_peak,
                      "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / mfma_peak, 4),
                      "host_wall_ms_per_step": round(wall, 4)},
            "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        }
        if w.name == "hy4_skew":
            counts = np.bincount(g_idx.ravel(), minlength=w.E)
            res["load"] = {"max_rows": int(counts.max()), "mean_rows": float(counts.mean()),
                           "max_over_mean": round(float(counts.max() / counts.mean()), 2)}
        if not a.no_graph:
            xs = x_dev.clone()
            graph = lay.capture(xs, out)
            gt = timed(graph.replay, a.steps, a.warmup)
            gms = float(np.median(gt))
            res["graph_replay"] = {"ms_per_step": round(gms, 4), "p10_ms": round(pct(gt, 10), 4),
                                   "p90_ms": round(pct(gt, 90), 4),
                                   "tokens_per_s": round(T / (gms * 1e-3), 1)}
            del graph
        if orc is not None and not a.no_parity:
            if T <= 64:
                toks = np.arange(T)
            else:
                rng = np.random.default_rng(12345)
                toks = np.unique(np.concatenate([np.arange(8), np.arange(T - 8, T),
                                                 rng.choice(T, 16, replace=False)]))
            t0 = time.perf_counter()
            res["parity"] = parity_sample(w, x32, out_host, g_idx, toks)
            log("%s parity on %d tokens: %s (%.1fs)" % (w.name, len(toks), res["parity"],
                                                      time.perf_counter() - t0))
        if headline and orc is not None and not a.no_cpu:
            res["cpu_baseline"] = cpu_baseline(w, x32)
        del x_dev, out
        return res

    def cpu_baseline(w, x32):
        # the oracle as it stands on a bounded sample: the first n tokens of
        # the batch (all of them when the batch is small), `reps` passes
        Wr, b = I.router_weight(w), I.router_bias(w)
        get = expert_cache(w)
        sh = I.shared_stored(w) if w.Is else None
        kw = oracle_kw(w)

        def run(n):
            return orc.layer_forward_tokens(np.arange(n), x32, Wr, b, get, sh, **kw)

        t1 = time.perf_counter()
        run(1)
        one = time.perf_counter() - t1
        n = int(max(1, min(w.T, a.cpu_seconds / max(one, 1e-3))))
        run(n)                                          # draws the experts the sample needs
        t1 = time.perf_counter()
        run(n)
        first = time.perf_counter() - t1
        reps = int(max(1, min(1000, a.cpu_seconds / max(first, 1e-3))))
        t1 = time.perf_counter()
        for _ in range(reps):
            run(n)
        dt = time.perf_counter() - t1
        flops_tok = 2.0 * w.E * w.H + 2.0 * w.k * 3 * w.I * w.H + 2.0 * 3 * w.Is * w.H
        return {"value": round(n * reps / dt, 3), "unit": "tokens/s",
                "cores": orc.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
                "gflops": round(flops_tok * n * reps / dt / 1e9, 2),
                "sample": "first %d of the %d tokens of the %s batch, %d passes: fp64-accumulating "
                          "C oracle (gating, each token's %d expert FFNs, shared FFN, combine); "
                          "%.1f s" % (n, w.T, w.name, reps, w.k, dt)}

    names = DEFAULT_WORKLOADS if a.workload == "all" else [a.workload]
    headline = names[0]
    results = {}
    layers = {}
    for name in names:
        w = I.workload(name)
        key = (w.H, w.E, w.k, w.I, w.Is, w.dtype, w.seed, w.zipf_beta)
        if key not in layers:
            for k in list(layers):                    # one weight set on the device at a time
                layers.pop(k).close()
            torch.cuda.empty_cache()
            t0 = time.time()
            log("drawing and packing %s weights (E=%d, H=%d, I=%d, %s)" % (w.name, w.E, w.H, w.I,
                                                                           w.dtype))
            layers[key] = DeviceLayer(w, side_stream=not a.single_stream)
            log("packed in %.1fs" % (time.time() - t0))
        results[name] = run_workload(w, layers[key], headline=(name == headline))
    for lay in layers.values():
        lay.close()

    if a.copy_calib:
        # plain device copy of a known size, for HBM counter calibration
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        del src, dst

    h = results[headline]
    hw = I.workload(headline)
    line = {
        "metric": METRIC, "value": h["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": h["ms_per_step"],
        "p10_ms": h["p10_ms"], "p90_ms": h["p90_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "mxfp8": "mxfp8-e4m3",
                  "w4a8": "mxfp4-e2m1 x mxfp8-e4m3", "fp8": "fp8-e4m3 per-tensor"}[hw.dtype],
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": hw.name, "tokens": hw.T, "hidden": hw.H, "experts": hw.E,
                   "top_k": hw.k, "inter": hw.I, "shared_inter": hw.Is,
                   "touched_experts": h["touched_experts"], "parallelism": "single GPU",
                   "timing": "median of %d steps, caches evicted before each" % a.steps
                             if not a.no_flush else "median of %d steps" % a.steps},
        "roofline": h["roofline"],
        "layer": h["layer"],
        "stages_ms": h["stages_ms"],
    }
    for k in ("graph_replay", "parity", "cpu_baseline"):
        if k in h:
            line[k] = h[k]
    line["workloads"] = {n: r for n, r in results.items() if n != headline}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
