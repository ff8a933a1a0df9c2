"""The measurement tooling of bench.py on synthetic rocprofv3 outputs (CPU):
the kernel-trace summary (routed and side-stream launches in separate rows,
the side stream's overlap with the main stream), the gate/up traffic summary
(kernel choice, copy calibration, bytes) and the source hash that ties
counter readings to the GEMM code."""
import contextlib
import csv
import io
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
import bench  # noqa: E402

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
              "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"]
PMC_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Grid_Size", "Kernel_Name", "Counter_Name",
            "Counter_Value"]


def _write(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _run(fn, *args):
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        fn(*args)
    return out.getvalue()


def test_code_text_ignores_comments_and_layout():
    a = "int f(int x) {\n  // twice\n  return 2 * x; /* doubled */\n}\n"
    b = "/* header */ int f(int x) { return 2 * x; }"
    c = "int f(int x) { return 3 * x; }"
    assert bench._code_text(a) == bench._code_text(b)
    assert bench._code_text(a) != bench._code_text(c)


def test_trace_summary_rows_and_side_stream_overlap(tmp_path):
    k = "void moe::gemm_tile_kernel<1, 0, 1, 4, 1, 8, 1, 2>(moe::GemmArgs)"
    rows = [
        # main stream: two launches of the routed kernel (1000 ns, 3000 ns)
        dict(Stream_Id=0, Kernel_Name=k, Start_Timestamp=0, End_Timestamp=1000, Grid_Size_X=4096),
        dict(Stream_Id=0, Kernel_Name=k, Start_Timestamp=2000, End_Timestamp=5000, Grid_Size_X=4096),
        # side stream: the same kernel with another grid, 400 of its 1000 ns
        # beside a main-stream kernel
        dict(Stream_Id=1, Kernel_Name=k, Start_Timestamp=4600, End_Timestamp=5600, Grid_Size_X=512),
    ]
    for r in rows:
        r.update(Kind="KERNEL_DISPATCH", Agent_Id="Agent 1", Queue_Id=1, Thread_Id=1, Dispatch_Id=1,
                 Kernel_Id=1, Correlation_Id=1)
    _write(str(tmp_path / "t" / "run_kernel_trace.csv"), TRACE_COLS, rows)
    text = _run(bench.trace_summary, str(tmp_path))
    lines = [ln for ln in text.splitlines() if ln.startswith("| `gemm_tile_kernel")]
    assert len(lines) == 2                       # one row per (kernel, stream, grid)
    main = [ln for ln in lines if "| 0 | 4096 |" in ln][0]
    cells = [c.strip() for c in main.split("|")]
    assert cells[4] == "2"                       # calls
    assert cells[6] == "2.0"                     # mean of 1.0 and 3.0 us
    assert "1.0 us in total, 40.0% of it beside a main-stream kernel" in text


def _pmc_rows(counter, copy_kib, kernels):
    rows = [dict(Grid_Size=131072, Kernel_Name="__amd_rocclr_copyBuffer", Counter_Name=counter,
                 Counter_Value=v) for v in copy_kib]
    for name, grid, vals in kernels:
        rows += [dict(Grid_Size=grid, Kernel_Name=name, Counter_Name=counter, Counter_Value=v)
                 for v in vals]
    for i, r in enumerate(rows):
        r.update(Correlation_Id=i, Dispatch_Id=i, Agent_Id="Agent 1")
    return rows


def test_traffic_summary_kernel_choice_and_calibration(tmp_path):
    gu = "void moe::gemm_tile_kernel<1, 0, 1, 4, 1, 8, 1, 2>(moe::GemmArgs)"
    gu_small = "void moe::gemm_skinny_kernel<1, 0, 1, 4, 4, 4>(moe::GemmArgs)"
    down = "void moe::gemm_tile_kernel<1, 1, 1, 4, 1, 8, 1, 2>(moe::GemmArgs)"
    # the 1 GiB copy reads as 0.5 GiB of FETCH_SIZE (mean of two dispatches)
    # and 1 GiB of WRITE_SIZE: factors 2 and 1
    fetch = _pmc_rows("FETCH_SIZE", [524000.0, 524576.0],
                      [(gu, 8000, [1000.0, 3000.0]), (gu_small, 100, [9e9]), (down, 9000, [9e9])])
    write = _pmc_rows("WRITE_SIZE", [1048576.0],
                      [(gu, 8000, [10.0, 30.0]), (gu_small, 100, [9e9]), (down, 9000, [9e9])])
    _write(str(tmp_path / "f" / "p_counter_collection.csv"), PMC_COLS, fetch)
    _write(str(tmp_path / "w" / "p_counter_collection.csv"), PMC_COLS, write)
    jpath = tmp_path / "f.json"
    jpath.write_text(json.dumps({"roofline": {"algorithmic_bytes": 4000000}}) + "\n")
    text = _run(bench.traffic_summary, "wl", str(tmp_path / "f"), str(tmp_path / "w"), str(jpath))
    kv = dict(ln.split(": ", 1) for ln in text.splitlines() if not ln.startswith("#"))
    assert kv["kernel"] == "gemm_tile_kernel<1, 0, 1, 4, 1, 8, 1, 2> grid 8000"
    assert kv["fetch_factor"] == "2.0000" and kv["write_factor"] == "1.0000"
    # (mean 2000 KiB x 2) + (mean 20 KiB x 1), in bytes
    assert int(kv["traffic_bytes"]) == 2000 * 1024 * 2 + 20 * 1024
    assert kv["algorithmic_bytes"] == "4000000"
    assert kv["source_sha256"] == bench.gemm_source_sha256()


def test_traffic_summary_needs_the_copy_calibration(tmp_path):
    gu = "void moe::gemm_tile_kernel<1, 0, 1, 4, 1, 8, 1, 2>(moe::GemmArgs)"
    for d, c in (("f", "FETCH_SIZE"), ("w", "WRITE_SIZE")):
        rows = [dict(Correlation_Id=0, Dispatch_Id=0, Agent_Id="Agent 1", Grid_Size=8000,
                     Kernel_Name=gu, Counter_Name=c, Counter_Value=1.0)]
        _write(str(tmp_path / d / "p_counter_collection.csv"), PMC_COLS, rows)
    jpath = tmp_path / "f.json"
    jpath.write_text(json.dumps({"roofline": {"algorithmic_bytes": 1}}) + "\n")
    with pytest.raises(SystemExit):
        _run(bench.traffic_summary, "wl", str(tmp_path / "f"), str(tmp_path / "w"), str(jpath))
