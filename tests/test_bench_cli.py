"""bench.py's host-side contract on the CPU: it refuses more than one GPU
before touching one, and its oracle baseline leg reports what it measured."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_timeline_and_breakdown_are_separate_runs():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--timeline",
                          "--breakdown"], capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "separate runs" in res.stderr
    assert res.stdout == ""


def test_source_digest_leaves_out_the_probes(monkeypatch):
    # the probes build a library of their own: a change to their source keeps
    # the digest that ties counter summaries to the decode library's code,
    # while a change to the library's own sources moves it
    import builtins
    base = bench.kernel_source_sha256()
    real_open = builtins.open

    def edited(name):
        def fake_open(path, *a, **k):
            f = real_open(path, *a, **k)
            if os.path.basename(str(path)) != name:
                return f
            import io
            return io.StringIO(f.read() + "\nint edited_for_the_test = 1;\n")
        return fake_open

    monkeypatch.setattr(builtins, "open", edited("pa_read_probe.hip"))
    assert bench.kernel_source_sha256() == base
    monkeypatch.setattr(builtins, "open", edited("pa_kernels.h"))
    assert bench.kernel_source_sha256() != base


def test_cpu_baseline_fields():
    import pa_inputs as pi
    case = pi.make_config_case(1)
    base = bench.cpu_baseline(case, 0.2)
    assert base["kind"] == "oracle" and base["unit"] == "GB/s"
    assert base["value"] > 0 and base["cores"] >= 1 and base["ms_per_step"] > 0
    assert case.name in base["sample"]


def test_recorded_traffic_needs_matching_workload():
    assert bench.recorded_traffic("no such workload") is None


def test_source_digest_ignores_comments_only():
    code = 'int a = 1; // one\n/* two */ const char *s = "// kept"; int b = 2;'
    same = 'int a = 1;   /* other words */\nconst char *s = "// kept";\n// more\nint b = 2;'
    changed = 'int a = 1; const char *s = "// kept"; int b = 3;'
    literal = 'int a = 1; const char *s = "/ / kept"; int b = 2;'
    strip = bench.strip_c_comments
    assert strip(code) == strip(same)
    assert strip(code) != strip(changed)
    assert strip(code) != strip(literal)


def _args(**kw):
    import argparse
    d = dict(steps=20, warmup=1, reps=5, eager=False, variant=None)
    d.update(kw)
    return argparse.Namespace(**d)


def test_child_leg_failure_is_reported_and_the_run_goes_on():
    # without a GPU each child leg exits with an error of its own: every leg
    # is still tried, and each is reported as FAILED (not a crash)
    import torch
    if torch.cuda.is_available():
        import pytest
        pytest.skip("a GPU is present")
    rows, crashed = bench.child_legs(_args(), [(1, 0), (4, 1)])
    assert not crashed
    assert [r["workload"] for r in rows] == [1, 4]
    assert all(r["status"] == "FAILED" and r["rc"] == 1 for r in rows)
    assert "needs a GPU" in rows[0]["stderr_tail"]


def test_child_leg_crash_ends_the_run(tmp_path):
    # a child that ends on SIGABRT (as after a device fault) is a CRASH, and
    # no later leg is started
    fake = tmp_path / "aborting_python"
    fake.write_text("#!/bin/sh\nkill -ABRT $$\n")
    fake.chmod(0o755)
    rows, crashed = bench.child_legs(_args(), [(2, 0), (3, 0), (5, 1)], python=str(fake))
    assert crashed
    assert len(rows) == 1
    assert rows[0]["workload"] == 2 and rows[0]["status"] == "CRASH" and rows[0]["rc"] < 0


def test_cpu_baseline_reports_one_thread_and_the_host():
    import pa_inputs as pi
    case = pi.make_config_case(1)
    base = bench.cpu_baseline(case, 0.1)
    one = base["single_thread"]
    assert one["value"] > 0 and one["ms_per_step"] > 0 and one["reps"] >= 1
    assert base["reps"] >= 1
    assert base["logical_cpus"] >= 1 and base["usable_cpus"] >= 1
    assert base["physical_cores"] is None or base["physical_cores"] >= 1
    assert "one" in base["sample"]


def test_rotation_and_summary():
    # >= 1 GiB of distinct copies, capped; median of an even count averages
    assert bench.rotation_copies(67129344) == 16
    assert bench.rotation_copies(1 << 20) == bench.MAX_COPIES
    assert bench.rotation_copies(1 << 31) == 2
    assert bench.summarize([3.0, 1.0, 2.0]) == (2.0, 1.0)
    assert bench.summarize([4.0, 1.0, 2.0, 3.0]) == (2.5, 1.0)
