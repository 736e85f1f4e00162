"""bench.py end to end on the GPU: one short run of a small workload prints
one JSON line with the fields the benchmark contract names, consistent with
each other."""
import ctypes
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import pa_inputs as pi
from gpu_util import DeviceCase, say

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
    # and the kernel's own gather, with no arithmetic and no merge
    assert r["gather_ceiling_us"] > 0 and r["gather_ceiling_us_min"] <= r["gather_ceiling_us"]
    assert abs(r["frac_of_gather_ceiling"] - r["gather_ceiling_us"] / r["avg_launch_us"]) < 1e-3


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


def live_words_xor(case, with_k=True):
    """The xor of every 32-bit word of every live K (if with_k) and V row
    (t < context length, table entry >= 0) of every (sequence, kv head), on
    the host."""
    k = case.k_cache if case.dtype == "f32" else case.k_bits
    v = case.v_cache if case.dtype == "f32" else case.v_bits
    kw = np.ascontiguousarray(k).view(np.uint32)
    vw = np.ascontiguousarray(v).view(np.uint32)
    acc = np.uint32(0)
    for b in range(case.batch):
        n = int(case.context_lens[b])
        t = np.arange(n)
        blk = case.block_tables[b, t // case.block_size]
        keep = blk >= 0
        rows = (blk[keep], (t % case.block_size)[keep])
        for w in ((kw, vw) if with_k else (vw,)):
            sel = w[rows[0], rows[1]]          # [live][Hkv][words]
            if sel.size:
                acc ^= np.bitwise_xor.reduce(sel.reshape(-1))
    return int(acc)


@pytest.mark.parametrize("dtype,d,bs", [("bf16", 128, 16), ("bf16", 64, 64), ("f16", 256, 16),
                                        ("f32", 128, 32)])
@pytest.mark.parametrize("vs", [1, 2])
def test_gather_probe_reads_every_live_row_once(gpu, dtype, d, bs, vs):
    # the gather ceiling's probe reads what a decode step reads: the xor of
    # its whole sink is the xor of every live K and V row, each once (a row
    # read twice or skipped changes it), for any partition count; with V
    # split in two, every K row is read twice (and cancels) and each half of
    # every V row once
    from paged_attention_decode_pa_amd import build as hip_build
    lib = ctypes.CDLL(hip_build.PROBE_LIB)
    V, I = ctypes.c_void_p, ctypes.c_int
    lib.pa_probe_gather.argtypes = [V, V, V, V, I, I, I, I, I, I, I, V, V]
    case = pi.make_case(5, [3000, 0, 1, 777, 64], 32, 8, d, bs, dtype=dtype, seed=43,
                        holes=[(0, 2), (3, 1)], max_blocks=200)
    dc = DeviceCase(case, gpu)
    want = live_words_xor(case, with_k=vs == 1)
    elem = 4 if dtype == "f32" else 2
    for P in (1, 3, 32, 200):
        say(f"gather probe {dtype} d={d} bs={bs} P={P} V slices {vs}")
        sink = torch.zeros(case.batch * case.num_kv_heads * P * vs, dtype=torch.int32,
                           device=gpu)
        rc = lib.pa_probe_gather(dc.k.data_ptr(), dc.v.data_ptr(), dc.table.data_ptr(),
                                 dc.lens.data_ptr(), case.batch, case.num_kv_heads, d * elem,
                                 bs, case.max_blocks, P, vs, sink.data_ptr(), None)
        assert rc == 0
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert int(got) == want, f"P={P}: {int(got):#x} != {want:#x}"
