"""Compile the HIP library for gfx950 into this package directory.

The kernels of each element type are a translation unit of their own
(csrc/pa_kernels_<dtype>.hip) and compile in parallel with the host launcher
(csrc/pa_decode.hip); the objects are then linked into libpa_decode.so.
"""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in
           ("pa_decode.hip", "pa_kernels_f32.hip", "pa_kernels_bf16.hip", "pa_kernels_f16.hip")]
KERNEL_SOURCES = SOURCES[1:]
LIB = os.path.join(HERE, "libpa_decode.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
INCLUDES = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
_NOISE = "is not a recognized feature for this target"


def _clean(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if _NOISE not in l)


def compile_objects(sources, outdir, extra=()):
    """Compile each source to an object in outdir, all at once.  Returns
    [(source, object, returncode, stderr)]."""
    procs = []
    for src in sources:
        obj = os.path.join(outdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, *INCLUDES, *extra, "-c", src, "-o", obj]
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.PIPE, text=True)))
    results = []
    for src, obj, p in procs:
        _, err = p.communicate()
        results.append((src, obj, p.returncode, err))
    return results


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory() as tmp:
        if verbose:
            print(f"{HIPCC} {' '.join(FLAGS)} -c <each of {len(SOURCES)} sources>", flush=True)
        results = compile_objects(SOURCES, tmp)
        for src, _, rc, err in results:
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{_clean(err)}")
            if verbose and _clean(err).strip():
                print(_clean(err), file=sys.stderr)
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
               *[obj for _, obj, _, _ in results], "-o", LIB + ".tmp"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{_clean(res.stderr)}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
