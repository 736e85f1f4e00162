"""Parity of the ablation builds with the fp64 oracle, through their C ABI.

libpa_decode_valu_qk.so (q.K on the vector ALUs for 16-bit elements, head dim
128, 4 query heads per kv head): every kernel mode that build changes --
single pass, fused split, fused split with the late query (a batch covering
the device), and the split kernel with the separate merge kernel.

libpa_decode_ordered.so (the fused merge ordered by release / acquire):
every fused mode, and bit for bit the library's output, since it does the
same arithmetic in the same order.

libpa_decode_no_vsplit.so (never splits V's head dim): the launches whose V
split it removes.

libpa_decode_timeline.so (per-workgroup time stamps): the library's exact
bits, and stamps in causal order.

libpa_decode_breakdown.so (a fused split stopped early, for timing): at stage
0 the library's exact bits; its stopped launches write no output and leave
the tickets as they were, so the next whole step is exact again.

Their timings only mean something if they compute the same decode step."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import pa_inputs as pi
import paged_attention_decode_pa_amd as pa

from gpu_util import DeviceCase, assert_close, check_host_preconditions, say, to_f64

pytestmark = pytest.mark.gpu


def run_variant(case, dev, parts, workspace=False, variant="valu_qk"):
    check_host_preconditions(case)
    lib = pa.load() if variant is None else pa.load_variant(variant)
    d = DeviceCase(case, dev)
    out = torch.empty_like(d.q)
    c = case
    ws, ws_bytes = None, 0
    if workspace:
        P = max(1, min(parts, c.max_blocks * c.block_size // 16, 4096))
        ws_bytes = pa.pa_workspace_bytes(c.batch, c.num_heads, c.head_dim, P)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    rc = lib.pa_decode_ex(out.data_ptr(), d.q.data_ptr(), d.k.data_ptr(), d.v.data_ptr(),
                          d.table.data_ptr(), d.lens.data_ptr(), c.batch, c.num_heads,
                          c.num_kv_heads, c.head_dim, c.block_size, c.max_blocks, float(c.scale),
                          d.dtype, torch.cuda.current_stream().cuda_stream, parts,
                          c.num_pool_blocks, None if ws is None else ws.data_ptr(), ws_bytes)
    assert rc == 0, pa.strerror(rc)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
@pytest.mark.parametrize("parts", [0, 1])
def test_valu_qk_workloads(gpu, cid, parts):
    case = pi.make_config_case(cid)
    say(f"valu_qk workload {cid} P={parts}")
    out = run_variant(case, gpu, parts)
    assert_close(to_f64(out), oracle.decode_case(case), case.dtype, f"valu_qk w{cid} P={parts}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("parts,workspace", [(0, False), (1, False), (3, False), (5, True)])
def test_valu_qk_ragged_with_holes(gpu, dtype, parts, workspace):
    case = pi.make_case(5, [0, 1, 17, 300, 1000], 32, 8, 128, 16, dtype=dtype, seed=21,
                        holes=[(3, 4), (4, 0), (4, 30)])
    say(f"valu_qk ragged {dtype} P={parts} workspace={workspace}")
    out = run_variant(case, gpu, parts, workspace)
    assert_close(to_f64(out), oracle.decode_case(case), dtype,
                 f"valu_qk ragged {dtype} P={parts}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_valu_qk_covering_batch(gpu, dtype):
    # 40 x 8 units cover the device: the fused mode with the late query load
    lens = [3000, 17, 0, 2048] + [int(x) for x in np.random.default_rng(22).integers(1, 400, 36)]
    need = sum(math.ceil(n / 16) for n in lens)
    case = pi.make_case(40, lens, 32, 8, 128, 16, dtype=dtype, seed=22, pool=need + 3)
    say(f"valu_qk covering batch {dtype}")
    out = run_variant(case, gpu, 0)
    assert_close(to_f64(out), oracle.decode_case(case), dtype, f"valu_qk covering {dtype}")


ORDERED_CASES = [
    # (B, lens, H, Hkv, d, dtype, forced partitions (0 = heuristic))
    (1, [16384], 32, 8, 128, "bf16", 0),     # fused split, 32 partitions
    (4, [2048] * 4, 32, 8, 128, "bf16", 0),  # fused split, 8 partitions
    (1, [512], 32, 8, 128, "bf16", 0),       # fused split with V split
    (5, [0, 1, 17, 300, 1000], 32, 8, 128, "f32", 7),
    (3, [700, 90, 2500], 16, 16, 64, "f16", 0),
    (40, [2200, 300] * 20, 32, 8, 128, "bf16", 0),   # late-query fused split
]


@pytest.mark.parametrize("shape", ORDERED_CASES, ids=lambda s: f"B{s[0]}_{s[5]}_P{s[6]}")
def test_ordered_ticket_build(gpu, shape):
    B, lens, H, Hkv, d, dtype, parts = shape
    case = pi.make_case(B, lens, H, Hkv, d, 16, dtype=dtype, seed=sum(lens) % 1000 + 5)
    say(f"ordered ticket B={B} {dtype} P={parts}")
    out = run_variant(case, gpu, parts, variant="ordered")
    assert_close(to_f64(out), oracle.decode_case(case), dtype, f"ordered B={B}")
    ref = run_variant(case, gpu, parts, variant=None)
    assert torch.equal(out, ref), "the ordered build must compute the library's bits"


@pytest.mark.parametrize("B,lens", [(1, [512]), (16, [256] * 16), (2, [60, 60])])
def test_no_vsplit_build(gpu, B, lens):
    case = pi.make_case(B, lens, 32, 8, 128, 16, dtype="bf16", seed=B + 31)
    say(f"no_vsplit B={B}")
    out = run_variant(case, gpu, 0, variant="no_vsplit")
    assert_close(to_f64(out), oracle.decode_case(case), "bf16", f"no_vsplit B={B}")


def test_timeline_build(gpu):
    # the stamps change no arithmetic, and they come in causal order: entry
    # <= end of streaming <= rows merged <= waves in LDS <= record issued <=
    # stores acknowledged <= ticket <= end of merge, with the last `ways`
    # arrivals of every (sequence, kv head) merging, the last one last
    tl = pa.load_variant("timeline")
    tl.pa_timeline_enable.argtypes = [ctypes.c_int]
    tl.pa_timeline_copy.argtypes = [ctypes.c_void_p, ctypes.c_int]
    case = pi.make_config_case(5)
    assert tl.pa_timeline_enable(4096) == 0
    say("timeline build, workload 5")
    out = run_variant(case, gpu, 0, variant="timeline")
    ref = run_variant(case, gpu, 0, variant=None)
    assert torch.equal(out, ref)
    P, vs = pa.pa_plan(1, 8, 128, case.max_blocks, 16, pa.pa_device_num_cus(0))
    n = 8 * P * vs
    st = np.zeros(16 * n, dtype=np.uint64)
    assert tl.pa_timeline_copy(st.ctypes.data, n) == 0
    st = st.reshape(n, 16).astype(np.int64)
    loop_end = st[:, 1:5].max(axis=1)
    assert (st[:, 0] > 0).all() and (st[:, 0] <= st[:, 1:5].min(axis=1)).all()
    assert (st[:, 12] == 2).all()                      # every partition publishes
    assert (st[:, 1] <= st[:, 13]).all() and (loop_end <= st[:, 14]).all()
    assert (st[:, 14] <= st[:, 6]).all() and (st[:, 6] <= st[:, 15]).all()
    assert (st[:, 15] <= st[:, 7]).all()
    role = st[:, 8] & 0xFF
    ways = (st[:, 8] >> 40) & 0xFF
    count = (st[:, 8] >> 8) & 0xFFFFFFFF
    merger = role > 0
    assert (st[merger, 7] <= st[merger, 9]).all()
    kvh = np.arange(n) % 8
    for h in range(8):
        u = kvh == h
        assert sorted(count[u].tolist()) == list(range(P * vs))  # one ticket each
        assert merger[u].sum() == ways[u][0]                     # the last `ways` arrivals
        assert role[u & (count == P * vs - 1)][0] == ways[u][0]  # the last one among them


@pytest.mark.parametrize("cid", [2, 4, 5])
def test_breakdown_build(gpu, cid):
    # workload 2 is a fused split with V split, 4 and 5 fused splits; every
    # partition of them publishes partial sums, so none writes out directly
    bd = pa.load_variant("breakdown")
    bd.pa_breakdown_stop_after.argtypes = [ctypes.c_int]
    case = pi.make_config_case(cid)
    c = case
    d = DeviceCase(case, gpu)
    ref = run_variant(case, gpu, 0, variant=None)
    try:
        for stage in (0, 1, 2, 3, 0, 3, 2, 1, 0):
            assert bd.pa_breakdown_stop_after(stage) == 0
            say(f"breakdown build, workload {cid}, stage {stage}")
            out = torch.full_like(d.q, 7.0)
            rc = bd.pa_decode(out.data_ptr(), d.q.data_ptr(), d.k.data_ptr(), d.v.data_ptr(),
                              d.table.data_ptr(), d.lens.data_ptr(), c.batch, c.num_heads,
                              c.num_kv_heads, c.head_dim, c.block_size, c.max_blocks,
                              float(c.scale), d.dtype, torch.cuda.current_stream().cuda_stream)
            assert rc == 0, pa.strerror(rc)
            torch.cuda.synchronize()
            if stage == 0:
                assert torch.equal(out, ref), "stage 0 differs from the library"
            else:
                assert (out == 7.0).all(), f"stage {stage} wrote output"
    finally:
        bd.pa_breakdown_stop_after(0)
