"""bench.py's command-line contract: one GPU only, and one JSON line with
the fields the measurement needs (value, roofline of the dominant kernel,
the oracle's CPU baseline)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=600):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          cwd=ROOT, capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.gpu
def test_bench_line_fields():
    r = _bench("--steps", "20", "--warmup", "5")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 5
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True
    assert d["vs_baseline"] is None
    assert "workload" in d["config"]
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    assert roof["traffic"] is None or roof["traffic"] > 0
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert cpu["unit"] == d["unit"] and cpu["sample"]
    for key in ("value_1_thread", "o1_quantize_s", "o2_dequantize_s", "o3_matmul_s",
                "cpu_model", "blas"):
        assert key in cpu, key
    # the timed copies were not touched by the upload or the warm-up and at
    # least 512 MB of other data was read before the region
    pool = d["config"]["pool"]
    assert pool["timed_copies"] == 20 and pool["read_before_timing_MB"] >= 512
    assert d["tokens_per_s"] == pytest.approx(1e3 / d["ms_per_step"])
    assert d["ceilings"]["launch_floor_us"] > 0 and roof["measured_ceiling"] > 0
    # the prefill half of the metric, in the same line
    p = d["prefill"]
    assert p["unit"] == "TFLOP/s" and p["value"] > 0 and p["T"] == 2048 and p["K"] == 3
    assert p["roofline"]["bound"] == "mfma" and p["roofline"]["peak"] == 2500.0
    assert p["cpu_baseline"]["kind"] == "oracle" and p["cpu_baseline"]["unit"] == "TFLOP/s"
    assert set(d["mlp_decode"]) == {"gate_proj", "down_proj"}
    # the few-token half of row a3: the whole MLP step at 4 and 16 tokens
    assert set(d["few_token"]) == {"T4", "T16"}
    for key, f in d["few_token"].items():
        assert f["T"] == int(key[1:]) and f["K"] == 3 and f["unit"] == "GB/s"
        assert f["value"] > 0 and f["tokens_per_s"] == pytest.approx(f["T"] * 1e3 / f["ms_per_step"])
