"""The HIP library builds for gfx950 with no kernel using scratch memory (a
spilled or dynamically indexed register array would silently cost a memory
round trip per access)."""
import re
import subprocess
import tempfile

from paged_attention_decode_pa_amd import build as hip_build


def test_no_kernel_uses_scratch():
    with tempfile.TemporaryDirectory() as tmp:
        results = hip_build.compile_objects(hip_build.KERNEL_SOURCES, tmp,
                                            extra=["-Rpass-analysis=kernel-resource-usage"])
    names, scratch = [], []
    for src, _, rc, err in results:
        assert rc == 0, err[-2000:]
        n = re.findall(r"Function Name: (\S+)", err)
        s = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", err)]
        assert len(n) == len(s) and n, src
        names += n
        scratch += s
    # (d, G) pairs built in the 4 modes without V split: fp32 5 + 5 + 3, bf16
    # and fp16 5 + 5 + 4 (d = 256 with larger groups only splits V); the two
    # V-split modes for every G at d >= 128 (5 + 5 per dtype); and the split
    # kernel with V split for the shapes that always split it (fp32 G = 8,
    # 16 and 16-bit G = 16 at d = 256)
    decode = [n for n in names if "pa_decode_kernel" in n]
    assert len(decode) == (13 + 14 + 14) * 4 + (10 + 10 + 10) * 2 + (2 + 1 + 1)
    assert sum("pa_merge_kernel" in n for n in names) == 3
    bad = [n for n, s in zip(names, scratch) if s != 0]
    assert not bad, f"kernels using scratch: {bad}"


def test_ablation_kernels_use_no_scratch():
    """The ablation builds' changed kernels also keep to registers (the
    vector-ALU q.K build changes only the 16-bit kernels).  All variants'
    objects compile in one parallel batch."""
    import os
    with tempfile.TemporaryDirectory() as tmp:
        pending = []
        for variant in ("valu_qk", "ordered", "timeline", "breakdown"):
            _, flags, _ = hip_build.VARIANTS[variant]
            srcs = [x for x in hip_build.KERNEL_SOURCES if variant != "valu_qk" or "f32" not in x]
            out = os.path.join(tmp, variant)
            os.mkdir(out)
            pending.append((variant, hip_build.compile_objects_async(
                srcs, out, extra=[*flags, "-Rpass-analysis=kernel-resource-usage"])))
        for variant, procs in pending:
            for src, _, proc in procs:
                _, err = proc.communicate()
                assert proc.returncode == 0, err[-2000:]
                n = re.findall(r"Function Name: (\S+)", err)
                sc = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", err)]
                assert len(n) == len(sc) and n, (variant, src)
                bad = [a for a, b in zip(n, sc) if b != 0]
                assert not bad, f"{variant}: kernels using scratch: {bad}"


def test_probe_kernels_use_no_scratch():
    """The measuring kernels of libpa_read_probe.so keep to registers too: a
    spill would slow the ceilings they set."""
    with tempfile.TemporaryDirectory() as tmp:
        results = hip_build.compile_objects(hip_build.PROBE_SOURCES, tmp,
                                            extra=["-Rpass-analysis=kernel-resource-usage"])
    for src, _, rc, err in results:
        assert rc == 0, err[-2000:]
        n = re.findall(r"Function Name: (\S+)", err)
        s = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", err)]
        assert len(n) == len(s) and n, src
        assert sum("gather_kernel" in x for x in n) == 6 and sum("read_kernel" in x for x in n) == 3
        bad = [a for a, b in zip(n, s) if b != 0]
        assert not bad, f"probe kernels using scratch: {bad}"
