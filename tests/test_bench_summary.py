"""Host logic of bench.py's profile summary: the calibration bracket, the
copy scaling and the per-call figures, on hand-made rocprofv3-style CSVs.
No GPU is used."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

# config 2 (4096 x 4096, K = 2) runs the matrix-core decode kernel by default
GEMV = "void mbok::(anonymous namespace)::gemv_f4_kernel<unsigned short, 2, 1>(...)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def _dispatches():
    # setup copy (large, must be ignored), timed calls, then the bracket:
    # copy in two chunks, 8 calls, copy in two chunks
    seq = [(COPY, 900000.0)] + [(GEMV, 1.0)] * 20
    seq += [(COPY, 65536.0), (COPY, 65536.0)]  # 131072 KiB counted for 262144 KiB copied
    seq += [(GEMV, 2500.0)] * bench.CAL_CALLS
    seq += [(COPY, 65536.0), (COPY, 65536.0)]
    return seq


def _make(tmp_path, counter):
    rows = []
    for i, (nm, v) in enumerate(_dispatches(), start=1):
        rows.append({"Dispatch_Id": i, "Kernel_Name": nm, "Counter_Name": counter,
                     "Counter_Value": v})
    d = tmp_path / counter
    _write(str(d / "run_counter_collection.csv"),
           ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    return str(d)


def test_bracket_finds_the_last_copy_calls_copy():
    seq = [(i, nm, v) for i, (nm, v) in enumerate(_dispatches())]
    copy, calls = bench.bracketed(seq, "gemv_f4_kernel")
    assert copy == [65536.0, 65536.0]
    assert calls == [2500.0] * bench.CAL_CALLS


def test_bracket_absent_pattern():
    assert bench.bracketed([(0, GEMV, 1.0), (1, GEMV, 1.0)], "gemv_") is None
    assert bench.bracketed([(0, COPY, 1.0), (1, GEMV, 1.0)], "gemv_") is None


def test_summary_scales_counters_by_the_copy(tmp_path):
    f = _make(tmp_path, "FETCH_SIZE")
    w = _make(tmp_path, "WRITE_SIZE")
    stats = tmp_path / "stats"
    _write(str(stats / "run_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"],
           [{"Name": GEMV, "Calls": 28, "TotalDurationNs": 140000, "AverageNs": 5000,
             "MinNs": 4000, "MaxNs": 6000}])
    trace_rows = []
    for i, (nm, _) in enumerate(_dispatches(), start=1):
        trace_rows.append({"Dispatch_Id": i, "Kernel_Name": nm, "Start_Timestamp": 1000 * i,
                           "End_Timestamp": 1000 * i + (5000 if nm == GEMV else 100)})
    _write(str(stats / "run_kernel_trace.csv"),
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace_rows)
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "2",
                          "--summarize", str(stats), f, w, "--command", "test"],
                         capture_output=True, text=True, check=True).stdout
    rec = dict(l.split(":", 1) for l in out.splitlines() if ":" in l and not l.startswith("#"))
    # the copy counted 131072 KiB for 256 MiB: scale 2; 8 calls of 2500 KiB
    assert float(rec["FETCH_SIZE_scale"]) == pytest.approx(2.0)
    assert float(rec["fetch_bytes_per_launch"]) == pytest.approx(2500 * 1024 * 2.0)
    assert float(rec["traffic_bytes_per_launch"]) == pytest.approx(2 * 2500 * 1024 * 2.0)
    assert float(rec["dominant_call_kernel_us"].split()[0]) == pytest.approx(5.0)
    assert rec["source_sha256"].strip() == bench.source_digest(1, 4096, 4096, 2)


def test_timed_regions_between_markers():
    M = "(anonymous namespace)::region_marker_kernel()"
    seq = [(1, "setup_kernel", 5.0), (2, "(anonymous namespace)::empty_kernel()", 1.0),
           (3, M, 1.0), (4, GEMV, 4.0), (5, GEMV, 6.0), (6, M, 1.0), (7, GEMV, 50.0),
           (8, "(anonymous namespace)::empty_kernel()", 1.0), (9, M, 1.0),
           (10, "gemm_mfma8_kernel", 100.0), (11, M, 1.0)]
    regs = bench.timed_regions(seq)
    # the launch-floor measurement's empty kernels are not markers
    assert regs == [{GEMV: [4.0, 6.0]}, {"gemm_mfma8_kernel": [100.0]}]
    assert bench.timed_regions([(1, GEMV, 1.0)]) == []


def test_code_digest_ignores_comments_only():
    """The kernel-source digest that ties a profile record to its kernel
    ignores comments and layout, and sees every code change."""
    import bench
    src = 'int f(int a) {  // scale\n  /* two\n     lines */ return a * 2; }\nconst char* s = "//x";\n'
    same = 'int f(int a)\n{\n  return a * 2;  /* other words */\n}\nconst char* s = "//x";\n'
    other = 'int f(int a) { return a * 3; }\nconst char* s = "//x";\n'
    assert bench.code_text(src) == bench.code_text(same)
    assert bench.code_text(src) != bench.code_text(other)
    assert '"//x"' in bench.code_text(src)  # string contents are code
