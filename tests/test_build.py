"""The HIP library builds for gfx950 with no kernel using scratch memory (a
spilled or dynamically indexed register array would silently cost a memory
round trip per access)."""
import os
import re
import subprocess
import tempfile

from paged_attention_decode_pa_amd import build as hip_build


def test_no_kernel_uses_scratch():
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [hip_build.HIPCC, *hip_build.FLAGS, "-I", os.path.join(hip_build.ROOT, "include"),
               "-Rpass-analysis=kernel-resource-usage", hip_build.SRC,
               "-o", os.path.join(tmp, "lib.so")]
        res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", res.stderr)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", res.stderr)]
    assert len(names) >= 32 and len(scratch) == len(names)
    bad = [n for n, s in zip(names, scratch) if s != 0]
    assert not bad, f"kernels using scratch: {bad}"
