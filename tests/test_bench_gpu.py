"""bench.py on the GPU at a reduced size: one JSON line with the contract's
fields, the roofline of the dominant call computed from its algorithmic
bytes and average launch time, the single-pass encode schedule, and the
discrepancy of guided rounding below RTN's on every layer."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_small():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--layers", "2", "--chunks", "2", "--steps", "2",
           "--warmup", "1", "--no-cpu-baseline", "--no-variants", "--no-record", "--no-diag"]
    print("bench:", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "kernels"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["cpu_baseline"] is None
    n = d["config"]["elements_per_side_per_step"]
    assert n == 2 * 2 * 8192 * 2048
    assert abs(d["value"] - n / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"]
    assert d["config"]["encode_schedule"] == "single-pass"
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["kernel"] == "guided_fake_quant_stats"
    achieved = roof["algorithmic_bytes_per_launch"] / (roof["avg_launch_us"] * 1e-6) / 1e9
    assert abs(roof["achieved"] - achieved) <= 0.002 * achieved
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) <= 1e-3
    assert roof["algorithmic_bytes_per_launch"] == int(2 * 8192 * 2048 * (2 + 2 + 1 / 8 + 1 / 16 + 2))
    k = d["kernels"]
    assert k["encode_guidance"]["calls_per_pass"] == 1 and k["encode_guidance"]["elements_per_call"] == n
    assert k["guided_fake_quant_stats"]["calls_per_pass"] == 2
    assert k["encode_guidance_per_layer"]["calls_per_pass"] == 2
    # guided rounding removes the train-rollout FP4 discrepancy on this data
    assert all(x < 0 for x in d["rel_excess_mse_guided_per_layer"])
    # no bounded wait of the single-pass encode gave up; a measured copy rate
    assert d["encode_wait_failures"] == 0
    c = d["copy_ceiling"]
    for r in (c, c["two_in_one_out"], c["torch_copy"]):
        assert 0 < r["frac_of_peak"] < 1 and abs(r["GB_s"] - r["bytes_read_plus_written"] / (r["avg_us"] * 1e3)) \
            <= 0.01 * r["GB_s"]
    assert c["two_in_one_out"]["bytes_read_plus_written"] == 3 * c["bytes_read_plus_written"] // 2


@pytest.mark.parametrize("config,n_layer", [("kv", 2 * 65536 * 256), ("mxfp4", 65536 * 2048),
                                            ("moe", 65536 * 2048), ("moe_expert", 65536 * 2048)])
def test_bench_other_workloads(config, n_layer):
    """--config selects the other workloads: one JSON line of the same
    contract for a one-layer step of each."""
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--config", config, "--layers", "1", "--steps", "2",
           "--warmup", "1", "--no-cpu-baseline"]
    print("bench:", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    assert d["config"]["elements_per_side_per_step"] == n_layer
    assert d["value"] > 0 and d["roofline"]["frac"] > 0 and d["encode_wait_failures"] == 0
    assert abs(d["value"] - n_layer / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"]
    assert all(x < 0 for x in d["rel_excess_mse_guided_per_layer"])
