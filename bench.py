"""Benchmark of the paged-attention decode step on one MI355X.

A step is one pa_decode call: the whole decode (split kernel + merge kernel,
or the single-pass kernel) over one batch of synthetic, seeded inputs.  The
headline workload is the largest one, bf16 B=1, context 16384, 32 query / 8 kv
heads, head_dim 128, block_size 16, with the partition count chosen by the
library's heuristic.

Timing: inputs are resident in HBM before the timed region.  Each step uses
the next of N distinct copies of (K/V pool, q, table, lengths, out), N chosen
so the copies span >= 1 GiB, so the 256 MB Infinity Cache cannot serve a
step's K/V reads from the previous visit.  W warm-up steps, then REPS (5)
timed regions of exactly K steps each.  Each region's K steps are captured in
a HIP graph of their own (--eager times plain launches) together with a
one-thread kernel at each end that writes the device clock (s_memrealtime,
libpa_read_probe.so), so a region's time is what its K steps took on the
device, without the graph's launch overhead; HIP events recorded around each
replay on the same stream are reported beside it (us_per_step_events).  An
untimed region is enqueued first and the regions follow back to back with no
host synchronisation between them, and the rotation runs on across them.
value is the median region; the minimum is reported beside it.

Output: one JSON line (rank 0, N = 1).  value = algorithmic bytes per step /
step time (GB/s); algorithmic bytes = every live K and V row once per kv head
+ q + out + block table.  A step of the headline workload is one launch of
the split kernel with its fused merge, so "roofline" (the dominant kernel)
uses the same timed regions: algorithmic bytes per launch / average launch
time.  Beside it the roofline reports the read ceiling: a plain streaming
read of the same bytes with the kernel's load shape (libpa_read_probe.so),
timed the same way.  "cpu_baseline" times the fp64 C oracle on the host's
cores (and on one) on the same workload.  "per_config" adds the other
workloads and the single-pass runs, each measured in a child process of its
own, so that a fault in one is reported as that configuration's CRASH.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode step μs and achieved HBM GB/s (% of MI355X peak) per config"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
ROTATION_BYTES = 1 << 30       # distinct bytes the copies must span
MAX_COPIES = 64
REPS = 5                       # timed regions of K steps; the median is reported
VARIANT = None                 # ablation library to time instead (--variant)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--eager", action="store_true", help="time plain launches, no HIP graph")
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU work budget of the oracle baseline (0 = skip)")
    ap.add_argument("--case", default=None, metavar="B,CTX,H,HKV,D,BS,DTYPE",
                    help="time this shape instead of a named workload (uniform context "
                         "length CTX, a scattered table over exactly the blocks needed, "
                         "DTYPE bf16|f16|f32); implies --no-per-config")
    ap.add_argument("--partitions", type=int, default=0,
                    help="partition count for the timed workload (0 = the heuristic, "
                         "-1 = the heuristic told that all lengths are equal)")
    ap.add_argument("--variant", default=None,
                    choices=["valu_qk", "no_vsplit", "ordered", "timeline", "breakdown"],
                    help="time an ablation build instead of the library: valu_qk runs the "
                         "q.K product on the vector ALUs instead of the matrix cores; "
                         "no_vsplit never splits V's head dim over two workgroups; ordered "
                         "orders the fused merge by release / acquire; timeline writes "
                         "per-workgroup stamps")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain elementwise copy of this many MiB (counter scale)")
    ap.add_argument("--reps", type=int, default=REPS,
                    help="timed regions of --steps steps each (median reported)")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the plain streaming-read and gather legs")
    ap.add_argument("--timeline", action="store_true",
                    help="instead of the bench line, the per-workgroup timeline of the timed "
                         "workload's last graph-replayed step (libpa_decode_timeline.so)")
    ap.add_argument("--breakdown", action="store_true",
                    help="instead of the bench line, what a fused split adds to its own gather: "
                         "the step, the step stopped after its partial sums and after its "
                         "stream (libpa_decode_breakdown.so, timing only), and the gather "
                         "probe, timed interleaved")
    ap.add_argument("--timeline-runs", type=int, default=1, metavar="N",
                    help="with --timeline: measure N times in one process (the XCD that runs "
                         "each kv head's units moves from one measurement to the next) and add "
                         "every run's per-kv-head and per-XCD medians")
    ap.add_argument("--leg", default=None, metavar="WORKLOAD:PARTITIONS",
                    help=argparse.SUPPRESS)   # one per-config leg, run as a child process
    ap.add_argument("--sweep", nargs="?", const="design-note", default=None,
                    choices=["design-note", "ragged", "script", "shapes", "uniform", "read"],
                    help="instead of the headline, a sweep: design-note (single pass vs split "
                         "over batch 1/4 and KV 512..16384), ragged (long-tailed batches), "
                         "script (the benchmark script's default grid), shapes (the headline "
                         "problem at other head dims, dtypes and block sizes), uniform "
                         "(uniform batches covering the device: heuristic, uniform-lengths "
                         "hint, single pass), read (the plain read of the headline's bytes at "
                         "other launch shapes)")
    return ap.parse_args()


TORCH_DTYPES = {"bf16": "bfloat16", "f16": "float16", "f32": "float32"}
# parity tolerances: |gpu - oracle| <= atol + rtol * |oracle| (fp32: max abs)
TOLERANCE = {"f32": (1e-5, 0.0), "bf16": (2e-3, 1e-2), "f16": (5e-5, 2.0 ** -10)}


def rotation_copies(step_bytes):
    """Distinct input copies one workload rotates over: enough to span
    ROTATION_BYTES, at most MAX_COPIES, at least 2."""
    return max(2, min(MAX_COPIES, math.ceil(ROTATION_BYTES / step_bytes)))


class Workload:
    """N rotation copies of one workload's inputs on the device."""

    def __init__(self, case, dev, num_partitions=0):
        import torch
        import paged_attention_decode_pa_amd as pa

        self.case = case
        c = self.case
        self.bytes = c.algorithmic_bytes()
        self.ncopies = rotation_copies(self.bytes)
        if c.dtype != "f32":
            tdt = getattr(torch, TORCH_DTYPES[c.dtype])
            conv = lambda b: torch.from_numpy(b.view(np.int16)).to(dev).view(tdt)
            q0, k0, v0 = conv(c.q_bits), conv(c.k_bits), conv(c.v_bits)
        else:
            q0, k0, v0 = (torch.from_numpy(x).to(dev) for x in (c.q, c.k_cache, c.v_cache))
        t0 = torch.from_numpy(c.block_tables).to(dev)
        n0 = torch.from_numpy(c.context_lens).to(dev)
        self.copies = []
        for i in range(self.ncopies):
            if i == 0:
                q, k, v, t, n = q0, k0, v0, t0, n0
            else:
                q, k, v, t, n = (x.clone() for x in (q0, k0, v0, t0, n0))
            self.copies.append(dict(q=q, k=k, v=v, t=t, n=n, out=torch.empty_like(q0)))
        self.dtype = pa.dtype_code(q0.dtype)
        self.cus = pa.pa_device_num_cus(dev.index or 0)
        # the launch the library makes: partitions, and V slices per partition
        self.P, self.v_slices = pa.pa_plan(c.batch, c.num_kv_heads, c.head_dim, c.max_blocks,
                                           c.block_size, self.cus, num_partitions,
                                           H=c.num_heads, dtype=self.dtype)
        self.num_partitions = num_partitions
        # every step here uses the library-owned workspace (no caller workspace)
        self.caller_workspace = False
        self.lib = pa.load_variant(VARIANT) if VARIANT else pa.load()

    def step(self, i, stream):
        """One whole decode step on copy i % N (pa_decode / pa_decode_ex)."""
        c, x = self.case, self.copies[i % self.ncopies]
        if self.num_partitions == 0:
            rc = self.lib.pa_decode(x["out"].data_ptr(), x["q"].data_ptr(), x["k"].data_ptr(),
                                    x["v"].data_ptr(), x["t"].data_ptr(), x["n"].data_ptr(),
                                    c.batch, c.num_heads, c.num_kv_heads, c.head_dim,
                                    c.block_size, c.max_blocks, float(c.scale), self.dtype,
                                    stream)
        else:
            rc = self.lib.pa_decode_ex(x["out"].data_ptr(), x["q"].data_ptr(), x["k"].data_ptr(),
                                       x["v"].data_ptr(), x["t"].data_ptr(), x["n"].data_ptr(),
                                       c.batch, c.num_heads, c.num_kv_heads, c.head_dim,
                                       c.block_size, c.max_blocks, float(c.scale), self.dtype,
                                       stream, self.num_partitions, 0, None, 0)
        if rc != 0:
            raise RuntimeError(f"pa_decode failed: {rc}")

    def launches_per_step(self):
        """Kernel launches of one step, from the plan: the single pass is one;
        a split is one with the library workspace (fused merge), two with a
        caller workspace (split kernel, then merge kernel)."""
        if self.P == 1 or not self.caller_workspace:
            return 1
        return 2

    def single_launch(self):
        return self.launches_per_step() == 1

    def kernel_name(self):
        v = ", V split in two" if self.v_slices > 1 else ""
        if self.P == 1:
            return f"pa_decode_kernel (single pass{v})"
        return f"pa_decode_kernel (split, fused merge{v})"


_PROBE = None


def probe_lib():
    """libpa_read_probe.so: the plain read and the device-clock stamp."""
    global _PROBE
    if _PROBE is None:
        import ctypes
        from paged_attention_decode_pa_amd import build as hip_build
        if not os.path.exists(hip_build.PROBE_LIB):
            raise RuntimeError(f"{hip_build.PROBE_LIB} not found: build the package first")
        lib = ctypes.CDLL(hip_build.PROBE_LIB)
        lib.pa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.pa_probe_read.restype = ctypes.c_int
        lib.pa_probe_stamp.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.pa_probe_stamp.restype = ctypes.c_int
        V, I = ctypes.c_void_p, ctypes.c_int
        lib.pa_probe_gather.argtypes = [V, V, V, V, I, I, I, I, I, I, I, V, V]
        lib.pa_probe_gather.restype = ctypes.c_int
        _PROBE = lib
    return _PROBE


STAMP_HZ = 100e6  # s_memrealtime


def time_region(fn, steps, warmup, use_graph, ncopies, reps=REPS):
    """Seconds per call of fn(i, stream) in each of `reps` regions of exactly
    `steps` calls, as (device-clock times, event times).  Call i uses rotation
    copy i % ncopies; an untimed region goes first and the timed ones follow
    back to back on one stream with no host synchronisation in between, and
    the call index runs on across them, so every region starts on a busy GPU
    and continues the rotation.  Each timed region is bracketed twice: by a
    device-clock stamp kernel at each end, in the same graph as its steps (so
    the graph's launch overhead falls outside), and by HIP events around the
    graph replay on the same stream."""
    import torch
    probe = probe_lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    stamps = torch.zeros(2 * reps, dtype=torch.int64, device="cuda")
    slot = lambda j: stamps.data_ptr() + 8 * j

    def stamp(j, s):
        if probe.pa_probe_stamp(slot(j), s) != 0:
            raise RuntimeError("pa_probe_stamp failed")

    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
    if use_graph:
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        # warm up on the capture stream itself: the library keeps its split
        # workspace per stream and must not allocate while capturing
        with torch.cuda.stream(cap):
            for i in range(warmup):
                fn(i, cap.cuda_stream)
        torch.cuda.synchronize()
        for r in range(reps + 1):        # region 0 is the untimed lead
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cap):
                g.capture_begin()
                if r > 0:
                    stamp(2 * (r - 1), cap.cuda_stream)
                for i in range(steps):
                    fn(r * steps + i, cap.cuda_stream)
                if r > 0:
                    stamp(2 * (r - 1) + 1, cap.cuda_stream)
                g.capture_end()
            graphs.append(g)
        torch.cuda.synchronize()
        graphs[0].replay()
        for r, (start, end) in enumerate(events):
            start.record(stream)
            graphs[r + 1].replay()
            end.record(stream)
        torch.cuda.synchronize()
        del graphs
    else:
        for i in range(warmup):
            fn(i, sh)
        torch.cuda.synchronize()
        for i in range(steps):             # untimed region 0
            fn(i, sh)
        for r, (start, end) in enumerate(events):
            start.record(stream)
            stamp(2 * r, sh)
            for i in range(steps):
                fn((r + 1) * steps + i, sh)
            stamp(2 * r + 1, sh)
            end.record(stream)
        torch.cuda.synchronize()
    st = stamps.cpu().tolist()
    dev = [(st[2 * r + 1] - st[2 * r]) / STAMP_HZ / steps for r in range(reps)]
    ev = [a.elapsed_time(b) * 1e-3 / steps for a, b in events]
    return dev, ev


def summarize(times):
    """(median, min) of per-region seconds per step."""
    t = sorted(times)
    n = len(t)
    med = t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])
    return med, t[0]


def parity_gate(w):
    """Copy 0 against the oracle at the stated tolerance, every copy bitwise equal."""
    import torch
    import oracle
    torch.cuda.synchronize()
    ref = oracle.decode_case(w.case)
    got = w.copies[0]["out"].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    atol, rtol = TOLERANCE[w.case.dtype]
    ok = bool((err <= atol + rtol * np.abs(ref)).all())
    same = all(torch.equal(x["out"], w.copies[0]["out"]) for x in w.copies)
    return ok and same, float(err.max())


def measure(case, dev, steps, warmup, use_graph, num_partitions=0, reps=REPS):
    """The workload's parity gate, then its timed regions: (Workload, median
    seconds per step, min seconds per step, max abs error)."""
    w = Workload(case, dev, num_partitions)
    for i in range(w.ncopies):
        w.step(i, None)
    ok, max_err = parity_gate(w)
    if not ok:
        raise SystemExit(f"{case.name}: parity gate FAILED (max err {max_err:.3e}); "
                         "timing would be meaningless")
    dev, ev = time_region(w.step, steps, warmup, use_graph, w.ncopies, reps)
    med, best = summarize(dev)
    w.event_median = summarize(ev)[0]
    return w, med, best, max_err


def sweep_read(dev, steps, warmup, use_graph):
    """The plain streaming read (libpa_read_probe.so) of the headline's bytes
    at other launch shapes: 256 / 512 / 1024 workgroups of 4 waves, 8 / 16 /
    32 KB in flight per wave; then the decode kernel's own gather of the
    headline's K and V rows (pa_probe_gather) at the launch's partition count
    and at twice it; and an empty launch (the one-thread clock kernel), the
    floor under any step."""
    import pa_inputs as pi
    nbytes = pi.make_config_case(5).algorithmic_bytes()
    points = []
    for wgs in (256, 512, 1024):
        for depth in (8, 16, 32):
            med, best, nb = read_ceiling(dev, nbytes, wgs, steps, warmup, use_graph, depth=depth)
            points.append(dict(kind="read", workgroups=wgs, kb_in_flight_per_wave=depth, bytes=nb,
                               us=round(med * 1e6, 3), us_min=round(best * 1e6, 3),
                               GBps=round(nb / med / 1e9, 1)))
            log(f"read {nb} bytes, {wgs} workgroups, {depth} KB per wave: {med * 1e6:.2f} us "
                f"({nb / med / 1e9:.0f} GB/s)")
    # the decode kernel's own gather of the headline's K and V rows (no
    # arithmetic, no merge) at its partition count and at twice it
    w = Workload(pi.make_config_case(5), dev, 0)
    for P in (w.P, 2 * w.P):
        med, best = gather_ceiling(w, steps, warmup, use_graph, partitions=P)
        nb = w.case.algorithmic_bytes()
        points.append(dict(kind="gather", partitions=P, workgroups=w.case.num_kv_heads * P,
                           kb_in_flight_per_wave=16, bytes=nb, us=round(med * 1e6, 3),
                           us_min=round(best * 1e6, 3), GBps=round(nb / med / 1e9, 1)))
        log(f"gather of the headline's rows, {P} partitions: {med * 1e6:.2f} us")
    del w
    # the floor under any step: a launch of a one-thread kernel that only
    # writes the clock, replayed back to back like the decode steps
    import torch
    lib = probe_lib()
    slot = torch.zeros(1, dtype=torch.int64, device=dev)

    def empty(i, stream):
        if lib.pa_probe_stamp(slot.data_ptr(), stream) != 0:
            raise RuntimeError("pa_probe_stamp failed")

    med, best = summarize(time_region(empty, steps, warmup, use_graph, 1)[0])
    points.append(dict(kind="empty", workgroups=1, us=round(med * 1e6, 3),
                       us_min=round(best * 1e6, 3)))
    log(f"empty launch: {med * 1e6:.2f} us")
    return dict(metric="plain streaming read us of the headline's bytes by launch shape",
                unit="us", higher_is_better=False, n_gpus=1, steps=steps, warmup=warmup,
                data="synthetic", points=points)


def read_ceiling(dev, nbytes, workgroups, steps, warmup, use_graph, reps=REPS, depth=16):
    """Seconds per launch of a plain streaming read of nbytes (rounded up to
    16 bytes) with the decode kernel's load shape: `workgroups` workgroups of 4
    waves, `depth` KB of non-temporal 16-byte loads in flight per wave, over a
    rotation of copies spanning >= 1 GiB like the decode step's (depth: 16-byte
    loads in flight per lane, i.e. KB per wave)."""
    import torch
    lib = probe_lib()
    nbytes = (nbytes + 15) // 16 * 16
    ncopies = rotation_copies(nbytes)
    bufs = [torch.zeros(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(ncopies)]
    sink = torch.zeros(workgroups, dtype=torch.int32, device=dev)

    def fn(i, stream):
        rc = lib.pa_probe_read(bufs[i % ncopies].data_ptr(), nbytes, workgroups, depth,
                               sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"pa_probe_read failed: {rc}")

    med, best = summarize(time_region(fn, steps, warmup, use_graph, ncopies, reps)[0])
    del bufs
    torch.cuda.empty_cache()
    return med, best, nbytes


def gather_ceiling(w, steps, warmup, use_graph, reps=REPS, partitions=None):
    """Seconds per launch (median, min) of pa_probe_gather over the
    workload's rotation copies: the decode kernel's own gather of the K and V
    rows -- its grid of (kv head, sequence, partition[, V slice]) workgroups
    at the launch's partition count and V slices, the same tiles, table reads
    and loads -- with no arithmetic and no merge.  None where the probe does
    not take the shape (rows of 1 KB, more than 65535 sequences)."""
    import torch
    c = w.case
    P = partitions or w.P
    row = c.head_dim * (4 if c.dtype == "f32" else 2)
    lib = probe_lib()
    x0 = w.copies[0]
    vs = w.v_slices
    sink = torch.zeros(c.batch * c.num_kv_heads * P * vs, dtype=torch.int32,
                       device=x0["k"].device)
    args = lambda x: (x["k"].data_ptr(), x["v"].data_ptr(), x["t"].data_ptr(), x["n"].data_ptr(),
                      c.batch, c.num_kv_heads, row, c.block_size, c.max_blocks, P, vs,
                      sink.data_ptr())
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.pa_probe_gather(*args(x0), stream)
    if rc == -3:
        return None
    if rc != 0:
        raise RuntimeError(f"pa_probe_gather failed: {rc}")

    def fn(i, s):
        if lib.pa_probe_gather(*args(w.copies[i % w.ncopies]), s) != 0:
            raise RuntimeError("pa_probe_gather failed")

    return summarize(time_region(fn, steps, warmup, use_graph, w.ncopies, reps)[0])


def strip_c_comments(text):
    """C/C++ source without its comments and with each run of whitespace made
    one space (string and character literals are kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_sha256():
    """One digest over the library's code: every file under csrc/ but the
    probes' (sorted by name, each name followed by its text) and the C
    header, with comments and whitespace runs removed, so that edits to
    comments alone keep it."""
    import hashlib
    csrc = os.path.join(ROOT, "paged_attention_decode_pa_amd", "csrc")
    # (the probes' source builds a library of its own, not this one)
    files = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc)) if f != "pa_read_probe.hip"]
    files.append(os.path.join(ROOT, "include", "pa_decode.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode() + b"\0")
        h.update(strip_c_comments(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()


def recorded_traffic(workload_name):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the kernel sources as they are now and on this workload; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
        sha = kernel_source_sha256()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha or rec.get("workload") != workload_name:
        return None
    return int(rec["traffic_bytes_per_launch"])


def cpu_description():
    """The host's CPU model and core counts, from /proc/cpuinfo and the
    process's affinity mask."""
    model, cores = None, set()
    phys = core = None
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8", errors="replace"):
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key == "model name" and model is None:
                model = val
            elif key == "physical id":
                phys = val
            elif key == "core id":
                core = val
            elif not key:
                if core is not None:
                    cores.add((phys, core))
                phys = core = None
        if core is not None:
            cores.add((phys, core))
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return dict(cpu_model=model, physical_cores=len(cores) or None,
                logical_cpus=os.cpu_count(), usable_cpus=usable)


def time_oracle(case, threads, budget_s):
    """Median seconds per full step of the oracle on `threads` OpenMP threads
    over repetitions filling about budget_s (at least 5, or 1 if one alone
    takes longer than the budget), and the repetition count."""
    import oracle
    times = []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.decode_case(case, threads=threads)
        times.append(time.perf_counter() - t0)
        el = time.perf_counter() - t_all
        if len(times) >= 5 and el >= budget_s:
            break
        if el * (len(times) + 1) / len(times) > 3 * budget_s:
            break
    med, _ = summarize(times)
    return med, len(times)


def cpu_baseline(case, budget_s):
    """The fp64 C oracle on the same workload: on all the threads OpenMP
    takes (the reported value) and on one thread."""
    import oracle
    threads = oracle.max_threads()
    oracle.decode_case(case, threads=threads)  # load, first touch
    per, reps = time_oracle(case, threads, budget_s)
    one, reps1 = time_oracle(case, 1, budget_s)
    gbs = lambda t: round(case.algorithmic_bytes() / t / 1e9, 4)
    return dict(value=gbs(per), unit="GB/s", cores=threads, kind="oracle",
                sample=f"the full step of {case.name}: median of {reps} repetitions "
                       f"({per * 1e3:.1f} ms each) on {threads} threads, and of {reps1} "
                       f"({one * 1e3:.1f} ms each) on one; fp64 C oracle, OpenMP over (b, h)",
                ms_per_step=round(per * 1e3, 3),
                single_thread=dict(value=gbs(one), unit="GB/s", ms_per_step=round(one * 1e3, 3),
                                   reps=reps1),
                reps=reps, **cpu_description())


# The flash-decoding-bench design note's sweep: decode steps (one query token)
# at batch sizes 1 and 4 over KV lengths 512 .. 16384, fused single pass
# against the KV-parallel split.  The note models plain multi-head attention
# (no grouped-query heads) and gives no head count; 32 heads of 128 in fp16 are
# used here, in 16-token blocks of a scattered table over a pool of exactly the
# blocks needed.
SWEEP_BATCHES = (1, 4)
SWEEP_KV = (512, 1024, 2048, 4096, 8192, 16384)
SWEEP_SHAPE = dict(H=32, Hkv=32, d=128, bs=16, dtype="f16")


def point(case, dev, steps, warmup, use_graph, parts):
    """One measured configuration: partition count, µs per step, live GB/s."""
    import torch
    w, ts, tmin, err = measure(case, dev, steps, warmup, use_graph, parts)
    row = dict(partitions=w.P, v_slices=w.v_slices, us=round(ts * 1e6, 3),
               us_min=round(tmin * 1e6, 3), GBps=round(w.bytes / ts / 1e9, 1),
               max_abs_err=err, algorithmic_bytes=w.bytes)
    del w
    torch.cuda.empty_cache()
    return row


def skewed_lens(B, seed):
    """A long-tailed batch: most lengths uniform in 128..2048, one in ten in
    8192..16384, the first one 16384."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(128, 2049, size=B)
    long = rng.random(B) < 0.1
    lens[long] = rng.integers(8192, 16385, size=int(long.sum()))
    lens[0] = 16384
    return [int(x) for x in lens]


def sweep_ragged(dev, steps, warmup, use_graph):
    """Batches of unequal lengths in a table wide enough for the longest
    (16384 tokens), bf16, 32 query / 8 kv heads, d 128, 16-token blocks; one
    with -1 holes.  Heuristic partitions against a single pass; GB/s counts
    live tokens only."""
    import pa_inputs as pi
    cases = []
    for B, seed in ((8, 2), (32, 1), (64, 3)):
        cases.append((f"B={B} long-tailed", pi.make_case(
            B, skewed_lens(B, seed), 32, 8, 128, 16, dtype="bf16", seed=seed, max_blocks=1024,
            name=f"bf16 B={B} long-tailed lengths H=32 Hkv=8 d=128 bs=16 width=1024")))
    lens = skewed_lens(32, 4)
    holes = [(b, (n // 16) // 2) for b, n in enumerate(lens) if n >= 64][:16]
    cases.append(("B=32 long-tailed, 16 holes", pi.make_case(
        32, lens, 32, 8, 128, 16, dtype="bf16", seed=4, max_blocks=1024, holes=holes,
        name="bf16 B=32 long-tailed lengths with -1 holes H=32 Hkv=8 d=128 bs=16 width=1024")))
    cases.append(("B=32 uniform 2048", pi.make_case(
        32, 2048, 32, 8, 128, 16, dtype="bf16", seed=5, max_blocks=1024,
        name="bf16 B=32 ctx=2048 H=32 Hkv=8 d=128 bs=16 width=1024")))
    points = []
    for label, case in cases:
        row = dict(case=label, lens_sum=int(case.context_lens.sum()),
                   lens_max=int(case.context_lens.max()))
        for tag, parts in (("heuristic", 0), ("single", 1)):
            r = point(case, dev, steps, warmup, use_graph, parts)
            row.update({f"{tag}_{k}": v for k, v in r.items() if k != "algorithmic_bytes"})
            row["algorithmic_bytes"] = r["algorithmic_bytes"]
        log(f"{label}: heuristic P={row['heuristic_partitions']} {row['heuristic_us']:.1f} us "
            f"({row['heuristic_GBps']:.0f} GB/s), single {row['single_us']:.1f} us")
        points.append(row)
    return dict(metric="decode step us and live-token GB/s, batches of unequal lengths",
                unit="us", higher_is_better=False, n_gpus=1, steps=steps, warmup=warmup,
                dtype="bf16", data="synthetic", points=points)


def sweep_script(dev, steps, warmup, use_graph):
    """benchmark_decoding.py's default grid: batch 1/8/32 x sequence length
    128/512/2048, 16 query / 8 kv heads, d 128, block size 256, fp16, a
    scattered table over a pool of exactly the blocks needed."""
    import pa_inputs as pi
    points = []
    for B in (1, 8, 32):
        for seq in (128, 512, 2048):
            case = pi.make_case(B, seq, 16, 8, 128, 256, dtype="f16", seed=B * 10000 + seq,
                                name=f"f16 B={B} ctx={seq} H=16 Hkv=8 d=128 bs=256")
            r = point(case, dev, steps, warmup, use_graph, 0)
            log(f"script grid B={B} seq={seq}: P={r['partitions']} {r['us']:.2f} us "
                f"({r['GBps']:.0f} GB/s)")
            points.append(dict(batch=B, seq_len=seq, **r))
    return dict(metric="decode step us and GB/s, the benchmark script's default grid",
                unit="us", higher_is_better=False, n_gpus=1, steps=steps, warmup=warmup,
                dtype="f16", data="synthetic", points=points)


def sweep_shapes(dev, steps, warmup, use_graph):
    """The headline problem (B=1, 16384 tokens, 32 query / 8 kv heads) at the
    other built head dims, element types and block sizes."""
    import pa_inputs as pi
    points = []
    for dtype, d, bs in (("bf16", 128, 16), ("bf16", 64, 16), ("bf16", 256, 16),
                         ("f16", 128, 16), ("f32", 128, 16), ("bf16", 128, 256),
                         ("f16", 256, 256)):
        case = pi.make_case(1, 16384, 32, 8, d, bs, dtype=dtype, seed=d + bs,
                            pool=2 * 16384 // bs,
                            name=f"{dtype} B=1 ctx=16384 H=32 Hkv=8 d={d} bs={bs}")
        r = point(case, dev, steps, warmup, use_graph, 0)
        log(f"{case.name}: P={r['partitions']} {r['us']:.2f} us ({r['GBps']:.0f} GB/s)")
        points.append(dict(dtype=dtype, head_dim=d, block_size=bs, **r))
    return dict(metric="decode step us and GB/s at other shapes of the headline problem",
                unit="us", higher_is_better=False, n_gpus=1, steps=steps, warmup=warmup,
                data="synthetic", points=points)


def sweep_uniform(dev, steps, warmup, use_graph):
    """Uniform batches that cover the device (bf16, 32 query / 8 kv heads,
    d 128, 16-token blocks): the heuristic (which splits sequences longer than
    2048 tokens), the heuristic told that the lengths are equal
    (PA_PARTITIONS_UNIFORM) and a forced single pass."""
    import pa_inputs as pi
    points = []
    for B, ctx in ((32, 4096), (32, 8192), (64, 4096), (64, 8192), (128, 4096)):
        case = pi.make_case(B, ctx, 32, 8, 128, 16, dtype="bf16", seed=B * 7 + ctx,
                            name=f"bf16 B={B} ctx={ctx} H=32 Hkv=8 d=128 bs=16")
        row = dict(batch=B, context_len=ctx)
        for tag, parts in (("heuristic", 0), ("uniform_hint", -1), ("single", 1)):
            r = point(case, dev, steps, warmup, use_graph, parts)
            row.update({f"{tag}_{k}": v for k, v in r.items() if k != "algorithmic_bytes"})
            row["algorithmic_bytes"] = r["algorithmic_bytes"]
        log(f"uniform B={B} x {ctx}: heuristic P={row['heuristic_partitions']} "
            f"{row['heuristic_us']:.1f} us, hint {row['uniform_hint_us']:.1f} us, single "
            f"{row['single_us']:.1f} us")
        points.append(row)
    return dict(metric="decode step us, uniform batches covering the device", unit="us",
                higher_is_better=False, n_gpus=1, steps=steps, warmup=warmup, dtype="bf16",
                data="synthetic", points=points)


def sweep(dev, steps, warmup, use_graph):
    import torch
    import pa_inputs as pi
    sh = SWEEP_SHAPE
    points = []
    for batch in SWEEP_BATCHES:
        for kv in SWEEP_KV:
            case = pi.make_case(batch, kv, sh["H"], sh["Hkv"], sh["d"], sh["bs"],
                                dtype=sh["dtype"], seed=batch * 100000 + kv,
                                name=f"{sh['dtype']} B={batch} ctx={kv} H={sh['H']} "
                                     f"Hkv={sh['Hkv']} d={sh['d']} bs={sh['bs']}")
            row = dict(batch=batch, kv_len=kv, algorithmic_bytes=case.algorithmic_bytes())
            for label, parts in (("single", 1), ("split", 0)):
                w, ts, tmin, err = measure(case, dev, steps, warmup, use_graph, parts)
                row[f"{label}_partitions"] = w.P
                row[f"{label}_v_slices"] = w.v_slices
                row[f"{label}_us"] = round(ts * 1e6, 3)
                row[f"{label}_us_min"] = round(tmin * 1e6, 3)
                row[f"{label}_GBps"] = round(w.bytes / ts / 1e9, 1)
                row[f"{label}_max_abs_err"] = err
                del w
                torch.cuda.empty_cache()
            row["split_speedup"] = round(row["single_us"] / row["split_us"], 3)
            log(f"B={batch} kv={kv}: single {row['single_us']:.2f} us, split "
                f"(P={row['split_partitions']}) {row['split_us']:.2f} us, "
                f"speedup {row['split_speedup']:.2f}x")
            points.append(row)
    crossover = {}
    for batch in SWEEP_BATCHES:
        # (a point where the heuristic itself runs one partition is the single
        # pass twice, not a win of the split)
        wins = [p["kv_len"] for p in points if p["batch"] == batch and p["split_speedup"] > 1
                and p["split_partitions"] > 1]
        crossover[str(batch)] = min(wins) if wins else None
    return dict(
        metric="decode step us, fused single pass vs split-KV (Flash-Decoding) with fused merge",
        unit="us", higher_is_better=False, n_gpus=1, steps=steps, warmup=warmup,
        dtype=sh["dtype"], data="synthetic",
        config=dict(workload="design-note sweep: batch 1 and 4, KV 512..16384, one query "
                             "token, multi-head", num_heads=sh["H"], num_kv_heads=sh["Hkv"],
                    head_dim=sh["d"], block_size=sh["bs"],
                    timing="HIP graph replay of K steps" if use_graph else "eager launches"),
        crossover_kv_len=crossover, points=points)


def pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]


def breakdown(case, dev, steps, warmup, use_graph, parts, rounds=3):
    """What a fused split adds to its own gather.  The library's step (behind
    the parity gate), the breakdown library (include/pa_breakdown.h) at stage
    0 (the whole step), stopped after the partial sums are stored (no ticket,
    no merge), after the waves' sums are combined (nothing stored) and after
    the stream (no epilogue), and pa_probe_gather (the same rows
    gathered the same way, no arithmetic), timed interleaved over the same
    rotation copies, `rounds` times each; medians in microseconds.  The
    stopped launches write no output, so only the library is checked."""
    import ctypes
    import torch
    import paged_attention_decode_pa_amd as pa
    w, _, _, err = measure(case, dev, steps, warmup, use_graph, parts)
    if w.P == 1:
        raise SystemExit(f"{case.name}: a single pass (P = 1) has no split to break down")
    main = w.lib
    bd = pa.load_variant("breakdown")
    bd.pa_breakdown_stop_after.argtypes = [ctypes.c_int]
    keys = ("step", "step_breakdown_build", "stop_after_partials", "stop_after_combine",
            "stop_after_stream", "gather")
    times = {k: [] for k in keys}
    region = lambda: summarize(time_region(w.step, steps, warmup, use_graph, w.ncopies)[0])[0]
    try:
        for _ in range(rounds):
            w.lib = main
            times["step"].append(region())
            w.lib = bd
            for stage, key in ((0, "step_breakdown_build"), (3, "stop_after_partials"),
                               (2, "stop_after_combine"), (1, "stop_after_stream")):
                if bd.pa_breakdown_stop_after(stage) != 0:
                    raise RuntimeError("pa_breakdown_stop_after failed")
                times[key].append(region())
            bd.pa_breakdown_stop_after(0)
            g = gather_ceiling(w, steps, warmup, use_graph)
            times["gather"].append(g[0] if g else float("nan"))
    finally:
        bd.pa_breakdown_stop_after(0)
    us = {k: round(float(np.median(v)) * 1e6, 3) for k, v in times.items()}
    log("breakdown (us): " + ", ".join(f"{k} {v}" for k, v in us.items()))
    out = dict(workload=case.name, partitions=w.P, v_slices=w.v_slices, rounds=rounds,
               steps=steps, max_abs_err=err, us=us,
               merge_us=round(us["step"] - us["stop_after_partials"], 3),
               epilogue_us=round(us["stop_after_partials"] - us["stop_after_stream"], 3),
               store_us=round(us["stop_after_partials"] - us["stop_after_combine"], 3),
               combine_us=round(us["stop_after_combine"] - us["stop_after_stream"], 3),
               stream_over_gather=round(us["stop_after_stream"] / us["gather"], 4),
               step_over_gather=round(us["step"] / us["gather"], 4))
    del w
    return out


def timeline(case, dev, steps, warmup, use_graph, parts):
    """The per-workgroup stamps of the last step of the timed regions, from
    the timeline library (include/pa_timeline.h), summarised in microseconds
    from the first workgroup's entry."""
    import ctypes
    import torch
    import paged_attention_decode_pa_amd as pa
    lib = pa.load_variant("timeline")
    lib.pa_timeline_enable.argtypes = [ctypes.c_int]
    lib.pa_timeline_copy.argtypes = [ctypes.c_void_p, ctypes.c_int]
    cap = 1 << 16
    if lib.pa_timeline_enable(cap) != 0:
        raise RuntimeError("pa_timeline_enable failed")
    w, med, best, err = measure(case, dev, steps, warmup, use_graph, parts, reps=1)
    torch.cuda.synchronize()
    c = w.case
    nwg = c.num_kv_heads * c.batch * w.P * w.v_slices
    if nwg > cap:
        raise SystemExit(f"{nwg} workgroups: more than the timeline keeps")
    st = np.zeros(nwg * 16, dtype=np.uint64)
    if lib.pa_timeline_copy(st.ctypes.data, nwg) != 0:
        raise RuntimeError("pa_timeline_copy failed")
    st = st.reshape(nwg, 16).astype(np.int64)
    t0 = st[:, 0].min()
    us = lambda x: (x - t0) * 0.01
    loop_end = us(st[:, 1:5].max(axis=1))
    kind = st[:, 12]
    pub = kind == 2
    role = st[:, 8] & 0xFF
    merger = role > 0
    xcc = st[:, 10] & 0xF
    q = lambda xs: dict(min=round(float(min(xs)), 2), median=round(float(pct(xs, 0.5)), 2),
                        p90=round(float(pct(xs, 0.9)), 2), max=round(float(max(xs)), 2))
    out = dict(workload=c.name, partitions=w.P, v_slices=w.v_slices, workgroups=nwg,
               us_per_step_timeline_build=round(med * 1e6, 3), max_abs_err=err,
               entry=q(us(st[:, 0])), loop_end=q(loop_end),
               per_xcd_loop_end_median={int(x): round(float(pct(loop_end[xcc == x], 0.5)), 2)
                                        for x in sorted(set(xcc.tolist()))},
               # kv head fastest in the grid: workgroup i serves kv head i mod Hkv
               per_kv_head_loop_end_median={
                   h: round(float(pct(loop_end[np.arange(nwg) % c.num_kv_heads == h], 0.5)), 2)
                   for h in range(c.num_kv_heads)},
               # workgroups dealt to the 8 XCDs round-robin by linear id, from an
               # XCD that need not be 0: the share of workgroups on XCD
               # (linear id + the most common offset) mod 8, and that offset
               xcd_round_robin=round(float(np.bincount((xcc - np.arange(nwg)) % 8,
                                                        minlength=8).max() / nwg), 4),
               xcd_offset=int(np.bincount((xcc - np.arange(nwg)) % 8, minlength=8).argmax()))
    if pub.any():
        w0_end = us(st[pub, 1])
        out["wave0_loop_end_to_rows_merged"] = q((us(st[pub, 13]) - w0_end).tolist())
        out["loop_end_to_waves_in_lds"] = q((us(st[pub, 14]) - loop_end[pub]).tolist())
        out["waves_in_lds_to_published"] = q((us(st[pub, 6]) - us(st[pub, 14])).tolist())
        out["loop_end_to_published"] = q((us(st[pub, 6]) - loop_end[pub]).tolist())
        out["published_to_acknowledged"] = q((us(st[pub, 15]) - us(st[pub, 6])).tolist())
        out["acknowledged_to_ticket"] = q((us(st[pub, 7]) - us(st[pub, 15])).tolist())
    if merger.any():
        # per (sequence, kv head) unit: from its last record issued to the end
        # of its last merger, the part of the step no streaming overlaps
        unit = np.arange(nwg) % (c.num_kv_heads * c.batch)
        tails, last_issue = [], []
        for u in sorted(set(unit[merger].tolist())):
            m = unit == u
            li = us(st[m & pub, 6]).max()
            last_issue.append(li)
            tails.append(us(st[m & merger, 9]).max() - li)
        out["mergers"] = int(merger.sum())
        out["merge_ways"] = int(((st[merger, 8] >> 40) & 0xFF).max())
        out["merge"] = q((us(st[merger, 9]) - us(st[merger, 7])).tolist())
        out["unit_last_record"] = q(last_issue)
        out["unit_last_record_to_merged"] = q(tails)
        out["step_end"] = round(float(us(st[merger, 9]).max()), 2)
    else:
        out["step_end"] = round(float(loop_end.max()), 2)
    del w
    return out


def leg_row(cid, parts, dev, steps, warmup, use_graph, reps):
    """One per-config leg: workload cid at partition count parts (0 = the
    heuristic), parity-gated and timed like the headline."""
    import pa_inputs as pi
    w, ts, tmin, err = measure(pi.make_config_case(cid), dev, steps, warmup, use_graph, parts,
                               reps)
    row = dict(
        workload=cid, name=w.case.name, status="ok", partitions=w.P, v_slices=w.v_slices,
        path=("single-pass" if w.P == 1 else "split-KV + fused merge")
             + (", V split in two" if w.v_slices > 1 else ""),
        us_per_step=round(ts * 1e6, 3), us_min=round(tmin * 1e6, 3),
        GBps=round(w.bytes / ts / 1e9, 1),
        pct_of_peak=round(100 * w.bytes / ts / 1e9 / HBM_PEAK_GBS, 1),
        launches_per_step=w.launches_per_step(), max_abs_err=err,
        rotation_copies=w.ncopies, algorithmic_bytes=w.bytes)
    # the same rows gathered the same way (the launch's partitions and V
    # slices) with no arithmetic
    g = gather_ceiling(w, steps, warmup, use_graph, reps)
    if g is not None:
        row.update(gather_us=round(g[0] * 1e6, 3), frac_of_gather=round(g[0] / ts, 4))
    return row


# A child that ends on a signal or an abort has faulted or crashed: its
# device state is gone, and nothing more is run on the GPU after it.
CRASH_CODES = (134, 137, 139)


def child_legs(args, plan, python=None):
    """Each (workload, partitions) leg of `plan` in a fresh child process (a
    subprocess, not an exec of this one).  Returns (rows, crashed): a leg
    whose child faulted, crashed or hung is reported as CRASH and ends the
    run, as a fault that poisons the device context would; one that failed
    normally (e.g. its parity gate) is reported as FAILED."""
    import subprocess
    rows = []
    for cid, parts in plan:
        cmd = [python or sys.executable, "-u", os.path.abspath(__file__), "--leg", f"{cid}:{parts}",
               "--steps", str(min(args.steps, 1000)), "--warmup", str(args.warmup),
               "--reps", str(args.reps)]
        if args.eager:
            cmd.append("--eager")
        if args.variant:
            cmd += ["--variant", args.variant]
        try:
            res = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
            rc, out, err = res.returncode, res.stdout, res.stderr
        except subprocess.TimeoutExpired as e:
            rc, out, err = -9, "", (e.stderr or b"").decode(errors="replace") \
                if isinstance(e.stderr, bytes) else (e.stderr or "")
        sys.stderr.write(err)
        lines = [l for l in out.splitlines() if l.strip()]
        if rc == 0 and lines:
            row = json.loads(lines[-1])
            log(f"workload {cid} P={row['partitions']}: {row['us_per_step']:.2f} us/step "
                f"(min {row['us_min']:.2f}) {row['GBps']:.0f} GB/s")
            rows.append(row)
            continue
        crashed = rc < 0 or rc in CRASH_CODES
        status = "CRASH" if crashed else "FAILED"
        log(f"workload {cid} partitions={parts}: {status} (child exit status {rc})")
        rows.append(dict(workload=cid, requested_partitions=parts, status=status, rc=rc,
                         stderr_tail=err[-400:]))
        if crashed:
            return rows, True
    return rows, False


def main():
    global VARIANT
    args = parse()
    if args.timeline and args.breakdown:
        sys.exit("--timeline and --breakdown are separate runs")
    VARIANT = "timeline" if args.timeline else args.variant
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the decode step has no multi-GPU path in this library)", file=sys.stderr)
        sys.exit(2)
    if args.reps < 1:
        sys.exit("--reps must be at least 1")
    use_graph = not args.eager

    if args.leg:                          # a child: one per-config leg, one JSON row
        import torch
        import paged_attention_decode_pa_amd as pa
        if not torch.cuda.is_available():
            sys.exit("bench.py needs a GPU")
        pa.load()
        if VARIANT:
            pa.load_variant(VARIANT)
        cid, parts = (int(x) for x in args.leg.split(":"))
        print(json.dumps(leg_row(cid, parts, torch.device("cuda:0"), args.steps, args.warmup,
                                 use_graph, args.reps)), flush=True)
        return

    # the per-config legs first, each in its own process, before this process
    # touches the GPU
    per_config = []
    if (not args.no_per_config and not args.case and not args.sweep and not args.timeline
            and not args.breakdown):
        plan = [(c, 0) for c in (1, 2, 3, 4, 5) if c != args.workload] + [(4, 1), (5, 1)]
        per_config, crashed = child_legs(args, plan)
        if crashed:
            print(json.dumps({"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1,
                              "steps": args.steps, "warmup": args.warmup,
                              "status": "CRASH in a per-config leg; nothing more was run",
                              "per_config": per_config}), flush=True)
            sys.exit(3)

    import torch
    import pa_inputs as pi
    import paged_attention_decode_pa_amd as pa
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    pa.load()
    if VARIANT:
        pa.load_variant(VARIANT)
    dev = torch.device("cuda:0")
    if args.sweep:
        fn = {"design-note": sweep, "ragged": sweep_ragged, "script": sweep_script,
              "shapes": sweep_shapes, "uniform": sweep_uniform, "read": sweep_read}[args.sweep]
        print(json.dumps(fn(dev, min(args.steps, 500), args.warmup, use_graph)), flush=True)
        return

    if args.case:
        B, ctx, H, Hkv, d, bs, dt = args.case.split(",")
        B, ctx, H, Hkv, d, bs = (int(x) for x in (B, ctx, H, Hkv, d, bs))
        headline = pi.make_case(B, ctx, H, Hkv, d, bs, dtype=dt, seed=B * 1000 + ctx,
                                name=f"{dt} B={B} ctx={ctx} H={H} Hkv={Hkv} d={d} bs={bs}")
    else:
        headline = pi.make_config_case(args.workload)

    if args.breakdown:
        print(json.dumps(breakdown(headline, dev, min(args.steps, 1000), args.warmup, use_graph,
                                   args.partitions)), flush=True)
        return

    if args.timeline:
        runs = [timeline(headline, dev, min(args.steps, 200), args.warmup, use_graph,
                         args.partitions) for _ in range(max(1, args.timeline_runs))]
        out = runs[0]
        if len(runs) > 1:
            keep = ("xcd_offset", "per_kv_head_loop_end_median", "per_xcd_loop_end_median",
                    "step_end")
            out["runs"] = [{k: r[k] for k in keep} for r in runs]
        print(json.dumps(out), flush=True)
        return

    w, t_step, t_min, err = measure(headline, dev, args.steps, args.warmup, use_graph,
                                    args.partitions, args.reps)
    gbs = w.bytes / t_step / 1e9
    log(f"timed workload {headline.name} P={w.P}: {t_step * 1e6:.2f} us/step (median of "
        f"{args.reps} regions of {args.steps} steps; min {t_min * 1e6:.2f}) {gbs:.0f} GB/s")
    if not w.single_launch():
        raise SystemExit("the headline step must be a single kernel launch")
    # the step is one launch of the dominant kernel: its timed regions are the step's
    t_dom, dom_bytes = t_step, w.bytes
    dom_gbs = dom_bytes / t_dom / 1e9
    c = w.case
    grid = c.num_kv_heads * c.batch * w.P * w.v_slices
    ncopies, P, v_slices, kname = w.ncopies, w.P, w.v_slices, w.kernel_name()
    t_events = w.event_median
    gather = None
    if not args.no_read_ceiling:
        gather = gather_ceiling(w, args.steps, args.warmup, use_graph, args.reps)
        if gather is not None:
            log(f"gather ceiling: the kernel's own K/V gather ({P} partitions, no arithmetic) "
                f"in {gather[0] * 1e6:.2f} us (min {gather[1] * 1e6:.2f})")
    del w
    torch.cuda.empty_cache()

    read = None
    if not args.no_read_ceiling:
        r_med, r_min, r_bytes = read_ceiling(dev, dom_bytes, grid, args.steps, args.warmup,
                                             use_graph, args.reps)
        read = dict(us=r_med * 1e6, us_min=r_min * 1e6, bytes=r_bytes)
        log(f"read ceiling: {r_bytes} bytes by {grid} workgroups in {r_med * 1e6:.2f} us "
            f"(min {r_min * 1e6:.2f}), {r_bytes / r_med / 1e9:.0f} GB/s")

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.randn(n // 2, device=dev).to(torch.bfloat16)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read and {n} bytes written per launch, 5 launches")

    base = None
    if args.cpu_seconds > 0:
        base = cpu_baseline(headline, args.cpu_seconds)

    roofline = {
        "bound": "hbm",
        "kernel": kname,
        "achieved": round(dom_gbs, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
        "traffic": None if VARIANT else recorded_traffic(c.name),
        "avg_launch_us": round(t_dom * 1e6, 3),
        "launches_per_step": 1,
        "bytes_per_launch": dom_bytes,
        "workgroups": grid,
    }
    if read is not None:
        roofline.update({
            "read_ceiling_us": round(read["us"], 3),
            "read_ceiling_us_min": round(read["us_min"], 3),
            "read_ceiling_GBps": round(read["bytes"] / read["us"] / 1e3, 1),
            "read_ceiling_bytes": read["bytes"],
            "frac_of_read_ceiling": round(read["us"] / (t_dom * 1e6), 4),
        })
    if gather is not None:
        roofline.update({
            "gather_ceiling_us": round(gather[0] * 1e6, 3),
            "gather_ceiling_us_min": round(gather[1] * 1e6, 3),
            "frac_of_gather_ceiling": round(gather[0] / t_dom, 4),
        })
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 6),
        "us_per_step": round(t_step * 1e6, 3),
        "us_min": round(t_min * 1e6, 3),
        "us_per_step_events": round(t_events * 1e6, 3),
        "reps": args.reps,
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic",
        "config": {
            "workload": c.name + (" split-KV (Flash-Decoding) + merge" if P > 1
                                  else " single-pass"),
            "batch": c.batch, "context_len": int(c.context_lens[0]),
            "num_heads": c.num_heads, "num_kv_heads": c.num_kv_heads,
            "head_dim": c.head_dim, "block_size": c.block_size,
            "pool_blocks": c.num_pool_blocks, "num_partitions": P, "v_slices": v_slices,
            "algorithmic_bytes_per_step": dom_bytes, "rotation_copies": ncopies,
            "timing": (f"median of {args.reps} regions of {args.steps} steps, each a HIP graph "
                       "replayed back to back with the others and timed by device-clock "
                       "stamps captured at its two ends (HIP events around the replays in "
                       "us_per_step_events)" if use_graph else
                       f"median of {args.reps} regions of {args.steps} eager steps, timed by "
                       "device-clock stamps at their two ends"),
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "cpu_baseline": base,
        "library": (f"ablation build {VARIANT} ({os.path.basename(pa.VARIANT_PATHS[VARIANT])})"
                    if VARIANT else os.path.basename(pa.LIB_PATH)),
        "max_abs_err": err,
        "per_config": per_config,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
