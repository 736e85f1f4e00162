"""The allocation-free entry point, pa_decode_noalloc, through the C ABI on the
GPU: it launches what pa_decode launches with the tickets and partials in the
library's fixed device array, so its output must equal pa_decode's bit for
bit (same kernels, same partition count, same reduction order), and match the
oracle at the stated tolerance.  Two calls in a row, the second smaller, so
the array is reused with the previous call's contents in it; a covering batch
(late-query fused split) and a single pass; a split too large for the
array is refused before anything is launched; and the call captured in a HIP
graph and replayed, with other calls on the array in between."""
import numpy as np
import pytest
import torch

import oracle
import pa_inputs as pi
import paged_attention_decode_pa_amd as pa

from gpu_util import DeviceCase, assert_close, check_host_preconditions, say, to_f64

pytestmark = pytest.mark.gpu


def both(case, dev):
    """(pa_decode output, pa_decode_noalloc output) for one case."""
    check_host_preconditions(case)
    d = DeviceCase(case, dev)
    ref = torch.empty_like(d.q)
    got = torch.full_like(d.q, float("nan"))
    pa.pa_decode(ref, *d.args(), None)
    pa.pa_decode_noalloc(got, *d.args(), None)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("first,second", [
    # (larger, then smaller): the headline split, then the 512-token split
    ((1, 16384), (1, 512)),
    # a covering batch whose long sequences split (late-query fused), then a
    # batch of 4 x 2048 (fused split)
    ((40, [2200, 300] * 20), (4, 2048)),
])
def test_noalloc_equals_pa_decode_twice_in_a_row(gpu, first, second):
    for i, (B, lens) in enumerate((first, second)):
        pool = None
        case = pi.make_case(B, lens, 32, 8, 128, 16, dtype="bf16", seed=100 + i + B, pool=pool)
        P, vs = pa.pa_plan(B, 8, 128, case.max_blocks, 16, pa.pa_device_num_cus(0))
        say(f"noalloc call {i + 1}: B={B} max ctx={int(case.context_lens.max())} P={P} "
            f"v_slices={vs}")
        ref, got = both(case, gpu)
        assert torch.equal(got, ref), f"call {i + 1}: noalloc differs from pa_decode"
        assert_close(to_f64(got), oracle.decode_case(case), "bf16", f"noalloc call {i + 1}")


def test_noalloc_small_split_then_more_units(gpu):
    # a split of few (sequence, kv head) units, then one of many: the second
    # call's tickets must not land where the first call left its partials
    for i, (B, lens) in enumerate(((1, 512), (40, [2200, 300] * 20), (2, 900))):
        case = pi.make_case(B, lens, 32, 8, 128, 16, dtype="bf16", seed=300 + i)
        say(f"noalloc sequence call {i + 1}: B={B}")
        ref, got = both(case, gpu)
        assert torch.equal(got, ref), f"call {i + 1}: noalloc differs from pa_decode"
        assert_close(to_f64(got), oracle.decode_case(case), "bf16", f"sequence call {i + 1}")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_noalloc_other_dtypes_and_the_single_pass(gpu, dtype):
    # a split (fp32 / fp16) and a short context that runs as a single pass
    for B, lens in ((2, [3000, 777]), (3, [60, 1, 0])):
        case = pi.make_case(B, lens, 32, 8, 128, 16, dtype=dtype, seed=7 + B)
        say(f"noalloc {dtype} B={B} lens={lens}")
        ref, got = both(case, gpu)
        assert torch.equal(got, ref)
        assert_close(to_f64(got), oracle.decode_case(case), dtype, f"noalloc {dtype}")


def test_noalloc_refuses_a_split_beyond_its_array(gpu):
    # 256 sequences x 8 kv heads covering the device, table of 1024 blocks:
    # 16 partitions, 256 * 32 * 16 * (128 + 2) * 4 bytes of partials > 64 MiB.
    # Refused before any launch, so the pool can be a few blocks here.
    B, H, Hkv, d, bs, W = 256, 32, 8, 128, 16, 1024
    assert pa.pa_plan(B, Hkv, d, W, bs, pa.pa_device_num_cus(0))[0] == 16
    q = torch.zeros(B, H, d, dtype=torch.bfloat16, device=gpu)
    out = torch.full_like(q, 7.0)
    k = torch.zeros(4, bs, Hkv, d, dtype=torch.bfloat16, device=gpu)
    table = torch.zeros(B, W, dtype=torch.int32, device=gpu)
    lens = torch.full((B,), W * bs, dtype=torch.int32, device=gpu)
    say("noalloc beyond the array: refused")
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode_noalloc(out, q, k, k, table, lens, B, H, Hkv, d, bs, W, 0.088,
                             pa.PA_DTYPE_BF16)
    assert e.value.code == pa.PA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())   # nothing was launched


@pytest.mark.parametrize("B,lens", [(1, 16384), (4, 2048), (40, [2200, 300] * 20)])
def test_noalloc_replayed_from_a_captured_graph(gpu, B, lens):
    # the callers it is for capture it: the call records its kernels (and
    # nothing that allocates) on a fresh stream, and every replay, with other
    # calls on the device array in between, equals pa_decode bit for bit
    case = pi.make_case(B, lens, 32, 8, 128, 16, dtype="bf16", seed=700 + B)
    check_host_preconditions(case)
    d = DeviceCase(case, gpu)
    ref = torch.empty_like(d.q)
    pa.pa_decode(ref, *d.args(), None)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    out = torch.empty_like(d.q)
    say(f"noalloc under graph capture: B={B}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.capture_begin()
        pa.pa_decode_noalloc(out, *d.args(), s)
        g.capture_end()
    torch.cuda.synchronize()
    other = pi.make_case(1, 3000, 32, 8, 128, 16, dtype="bf16", seed=701)
    od = DeviceCase(other, gpu)
    oo = torch.empty_like(od.q)
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        pa.pa_decode_noalloc(oo, *od.args(), None)   # the array in between
        torch.cuda.synchronize()
    assert_close(to_f64(out), oracle.decode_case(case), "bf16", f"noalloc graph B={B}")


FIRST_CALL_UNDER_CAPTURE = r"""
import sys, torch
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + '/tests')
import pa_inputs as pi, paged_attention_decode_pa_amd as pa
from gpu_util import DeviceCase
case = pi.make_case(1, 16384, 32, 8, 128, 16, dtype='bf16', seed=707)
d = DeviceCase(case, torch.device('cuda:0'))
out = torch.empty_like(d.q)
s = torch.cuda.Stream()
g = torch.cuda.CUDAGraph()
with torch.cuda.stream(s):
    g.capture_begin()
    pa.pa_decode_noalloc(out, *d.args(), s)   # the process's first decode call
    g.capture_end()
torch.cuda.synchronize()
ref = torch.empty_like(d.q)
pa.pa_decode(ref, *d.args(), None)
torch.cuda.synchronize()
for i in range(3):
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, ref), f'replay {i}'
print('ok', flush=True)
"""


def test_first_call_of_a_process_under_capture(gpu):
    # a caller whose very first decode call is inside a graph capture: the
    # launcher's one-time setup (the device array's address, its ticket
    # clear, the kernel's occupancy for the shared merge) happens during the
    # capture, and every replay still equals pa_decode bit for bit
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    say("noalloc: first call of a fresh process under graph capture")
    res = subprocess.run([sys.executable, "-c", FIRST_CALL_UNDER_CAPTURE, root],
                         capture_output=True, text=True, timeout=110)
    assert res.returncode == 0, res.stderr[-2000:]
    assert res.stdout.strip().endswith("ok")
