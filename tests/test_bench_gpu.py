"""bench.py end to end on the GPU: one short run of a small workload prints
one JSON line with the fields the benchmark contract names, consistent with
each other."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def test_bench_prints_one_consistent_json_line(gpu):
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "2",
           "--no-per-config", "--cpu-seconds", "0.2", "--steps", "200", "--warmup", "5"]
    print("bench.py workload 2, 200 steps", flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 200 and d["warmup"] == 5
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["dtype"] == "bf16" and "workload" in d["config"]
    bytes_per_step = d["config"]["algorithmic_bytes_per_step"]
    assert bytes_per_step == 2113664
    # value is algorithmic bytes / step time
    assert abs(d["value"] - bytes_per_step / (d["ms_per_step"] * 1e-3) / 1e9) < 0.01 * d["value"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["bytes_per_launch"] == bytes_per_step
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
    assert c["single_thread"]["value"] > 0
    # median and min of the timed regions; the read ceiling beside the kernel
    assert d["reps"] == 5 and 0 < d["us_min"] <= d["us_per_step"]
    # device-clock region times exclude the graph launches the events include
    assert 0 < d["us_per_step"] <= 1.02 * d["us_per_step_events"]
    assert r["read_ceiling_us"] > 0 and r["read_ceiling_bytes"] >= bytes_per_step
    assert abs(r["frac_of_read_ceiling"] - r["read_ceiling_us"] / r["avg_launch_us"]) < 1e-3


def test_bench_case_option_reports_its_launch(gpu):
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--case",
           "2,300,32,8,128,16,f16", "--partitions", "3", "--cpu-seconds", "0",
           "--steps", "50", "--warmup", "3"]
    print("bench.py --case 2,300,32,8,128,16,f16 --partitions 3", flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout
    d = json.loads(lines[0])
    c = d["config"]
    assert d["dtype"] == "f16" and c["batch"] == 2 and c["context_len"] == 300
    assert c["num_heads"] == 32 and c["num_kv_heads"] == 8 and c["block_size"] == 16
    # 16 units x 3 partitions fill at most a quarter of the CUs: V split in two
    assert c["num_partitions"] == 3 and c["v_slices"] == 2
    assert d["per_config"] == [] and d["cpu_baseline"] is None
    assert d["roofline"]["traffic"] is None   # counters were taken on another workload
