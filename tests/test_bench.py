"""The benchmark script's contract.

CPU: more than one GPU is refused with a message; the CPU baseline leg
returns the fields the JSON line carries; committed HBM counters were taken
on the current kernel sources.  GPU: the headline JSON line
has every field, with a roofline block whose figures agree with each other.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from dense_fp32_matrix_03_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_fields():
    w = inputs.WORKLOADS[0]
    cb = bench.cpu_baseline(w, target_s=0.05)
    assert set(cb) == {"value", "unit", "cores", "kind", "sample"}
    assert cb["unit"] == "TFLOP/s" and cb["kind"] == "oracle"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert "rows of C" in cb["sample"]


def test_committed_counters_follow_the_kernel_sources():
    with open(bench.COUNTERS) as f:
        c = json.load(f)
    assert c["workload"] == bench.HEADLINE
    t = bench.measured_traffic(bench.HEADLINE)
    assert bench.measured_traffic(bench.SECONDARY) is None
    # Counters are re-taken with every change to the hot kernel's sources
    # (bench.py --write-hbm-counters); a stale summary fails here.
    assert c.get("source_sha256") == bench.kernel_source_digest(), (
        "hot kernel sources changed since the HBM counters were taken: re-take them")
    # HBM bytes per launch: at least the algorithmic bytes of the workload.
    assert t == c["hbm_bytes_per_launch"]
    assert t >= inputs.BY_NAME[bench.HEADLINE].min_bytes


@pytest.mark.gpu
def test_headline_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2",
                        "--warmup", "1", "--no-cpu-baseline", "--no-secondary"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    out = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in out, k
    assert out["n_gpus"] == 1 and out["steps"] == 2 and out["warmup"] == 1
    assert out["unit"] == "TFLOP/s" and out["higher_is_better"] is True
    assert out["config"]["workload"] == bench.HEADLINE
    assert out["output_finite"] is True
    w = inputs.BY_NAME[bench.HEADLINE]
    assert abs(out["value"] - w.flops / (out["ms_per_step"] * 1e-3) / 1e12) < 0.01 * out["value"]
    rf = out["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == bench.PEAK_TFLOPS
    assert rf["achieved"] == out["value"]
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert 0.5 < rf["frac"] < 1.0
