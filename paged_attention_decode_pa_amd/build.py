"""Compile the HIP library for gfx950 into this package directory.

The kernels of each element type are a translation unit of their own
(csrc/pa_kernels_<dtype>.hip) and compile in parallel with the host launcher
(csrc/pa_decode.hip); the objects are then linked into libpa_decode.so.

Ablation libraries are built beside it, each only to measure what one
design choice brings; the package never loads them by itself:
libpa_decode_valu_qk.so (PA_QK_VALU=1: the q.K product of the 16-bit,
head-dim-128, 4-heads-per-kv-head kernels on the vector ALUs instead of the
matrix cores; bench.py --variant valu_qk) and libpa_decode_no_vsplit.so
(PA_SPLIT_V=0 in the launcher: never split V's head dim over two workgroups
where it need not, i.e. except for the d = 256 shapes built only with the
split; bench.py --variant no_vsplit).  A third, libpa_decode_ordered.so
(PA_ORDERED_TICKET=1), orders the fused merge's exchange of partial sums by
release / acquire in the memory model instead of by cache policy (bench.py
--variant ordered); it computes the same bits.  libpa_decode_timeline.so
(PA_TIMELINE=1) writes per-workgroup time stamps (include/pa_timeline.h;
bench.py --timeline), and libpa_decode_breakdown.so (PA_BREAKDOWN=1) can stop
a fused split after its partial sums or after its stream, for timing only
(include/pa_breakdown.h; bench.py --breakdown).  All else is identical.

libpa_read_probe.so (csrc/pa_read_probe.hip, include/pa_read_probe.h) holds
a plain streaming read with the decode kernel's load shape and the decode
kernel's own gather of the K and V rows with no arithmetic, the ceilings
bench.py measures the decode kernel against; nothing else loads it.
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
PROBE_SOURCES = [os.path.join(CSRC, "pa_read_probe.hip")]
PROBE_LIB = os.path.join(HERE, "libpa_read_probe.so")
# name -> (library file, extra compiler flags, sources compiled with them; the
# other sources' objects are the main library's)
VARIANTS = {
    "valu_qk": (os.path.join(HERE, "libpa_decode_valu_qk.so"), ["-DPA_QK_VALU=1"], SOURCES),
    "no_vsplit": (os.path.join(HERE, "libpa_decode_no_vsplit.so"), ["-DPA_SPLIT_V=0"],
                  SOURCES[:1]),
    "ordered": (os.path.join(HERE, "libpa_decode_ordered.so"), ["-DPA_ORDERED_TICKET=1"],
                KERNEL_SOURCES),
    "timeline": (os.path.join(HERE, "libpa_decode_timeline.so"), ["-DPA_TIMELINE=1"], SOURCES),
    "breakdown": (os.path.join(HERE, "libpa_decode_breakdown.so"), ["-DPA_BREAKDOWN=1"], SOURCES),
}
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


def compile_objects_async(sources, outdir, extra=()):
    """Start compiling each source to an object in outdir.  Returns
    [(source, object, Popen)]."""
    procs = []
    for src in sources:
        obj = os.path.join(outdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, *INCLUDES, *extra, "-c", src, "-o", obj]
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.PIPE, text=True)))
    return procs


def compile_objects(sources, outdir, extra=()):
    """Compile each source to an object in outdir, all at once.  Returns
    [(source, object, returncode, stderr)]."""
    results = []
    for src, obj, p in compile_objects_async(sources, outdir, extra):
        _, err = p.communicate()
        results.append((src, obj, p.returncode, err))
    return results


def build(verbose: bool = False, variants=tuple(VARIANTS)) -> str:
    """Compile and link libpa_decode.so, the named ablation libraries and the
    read probe (all objects compile in parallel).  Returns the path of
    libpa_decode.so."""
    jobs = [(LIB, [], SOURCES)] + [VARIANTS[v] for v in variants]
    jobs.append((PROBE_LIB, [], PROBE_SOURCES))
    with tempfile.TemporaryDirectory() as tmp:
        if verbose:
            print(f"{HIPCC} {' '.join(FLAGS)} -c <each of {len(SOURCES)} sources>"
                  + "".join(f", again with {' '.join(f)} for {os.path.basename(l)}"
                            for l, f, _ in jobs[1:-1])
                  + f"; {os.path.basename(PROBE_LIB)} from "
                  + ", ".join(os.path.basename(x) for x in PROBE_SOURCES), flush=True)
        procs = []
        for n, (lib, extra, sources) in enumerate(jobs):
            outdir = os.path.join(tmp, str(n))
            os.mkdir(outdir)
            procs.append((lib, compile_objects_async(sources, outdir, extra)))
        main_objs = {}
        for lib, pending in procs:
            objs = {}
            for src, obj, p in pending:
                _, err = p.communicate()
                if p.returncode != 0:
                    raise RuntimeError(f"hipcc failed on {src} for {os.path.basename(lib)} "
                                       f"({p.returncode}):\n{_clean(err)}")
                if verbose and _clean(err).strip():
                    print(_clean(err), file=sys.stderr)
                objs[src] = obj
            if lib == LIB:
                main_objs = dict(objs)
            elif lib != PROBE_LIB:
                # a variant that recompiles only some sources links the rest
                # from the main library's objects
                objs = {src: objs.get(src, main_objs[src]) for src in SOURCES}
            objs = list(objs.values())
            cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib + ".tmp"]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError(f"link failed ({res.returncode}):\n{_clean(res.stderr)}")
            os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
