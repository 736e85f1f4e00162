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
