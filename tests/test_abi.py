"""The C-ABI library on the CPU: it loads, exports what include/pa_decode.h
declares, and rejects invalid arguments before any HIP call.  No compute call
is made here (there is no GPU); the fake device addresses below are never
dereferenced because validation fails first."""
import math
import os
import re

import pytest

import paged_attention_decode_pa_amd as pa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "pa_decode.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = pa.load()
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(pa.EXPORTS)


@pytest.mark.parametrize("variant", ["valu_qk", "no_vsplit", "ordered", "timeline", "breakdown"])
def test_ablation_library_exports_the_same_functions(variant):
    lib = pa.load_variant(variant)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror_covers_codes():
    for code in range(0, -11, -1):
        s = pa.strerror(code)
        assert s and s != "unknown error code", code
    assert pa.strerror(-99) == "unknown error code"


@pytest.mark.parametrize("B,Hkv,max_blocks,bs,cus,expect", [
    (2, 8, 4, 16, 256, 1),        # 60 tokens: too short to split (needs 8 tiles/partition)
    (1, 8, 32, 16, 256, 4),       # 512 tokens: capped at 32 / 8 partitions
    (16, 8, 16, 16, 256, 1),      # 128 units, 16 tiles: two rounds of loads beat a split
    (16, 8, 17, 16, 256, 2),      # 17 tiles: 2 partitions
    (4, 8, 128, 16, 256, 8),      # 32 units -> 8 partitions of 16 tiles
    (1, 8, 1024, 16, 256, 32),    # 8 units -> 32 partitions of 32 tiles
    (32, 8, 1024, 16, 256, 16),   # units fill the CUs: split long rows, 64 tiles each, <= 16
    (32, 8, 64, 16, 256, 1),      # ... a row of 64 tiles does not split
    (32, 8, 128, 16, 256, 1),     # ... nor one of 128 (2048 tokens)
    (64, 8, 300, 16, 256, 5),     # ... 300 tiles -> 5
    (64, 8, 100000, 16, 256, 16),  # ... at most 16
    (1, 1, 100, 16, 256, 12),     # capped at 100 // 8 = 12 (runs of 8 or 9 tiles)
    (1, 8, 7, 16, 256, 1),
    (0, 8, 10, 16, 256, 1),
    (3, 8, 1000, 16, 0, 1),
    (1, 8, 64, 256, 256, 32),     # 16384 tokens in 256-token blocks: same as 1024 x 16
    (8, 8, 2, 256, 256, 4),       # 512 tokens, 64 units -> 4 partitions of 8 tiles
    (1, 8, 16, 32, 256, 4),       # 512 tokens in 32-token blocks
    (1, 8, 10, 8, 256, 1),        # block_size below 16
    (12, 8, 64, 16, 256, 2),      # 96 units: floor(256 / 96) = 2, not 3 (no CU holds two)
    (6, 8, 128, 16, 256, 5),      # 48 units: 5 partitions, 240 workgroups
    (20, 8, 64, 16, 256, 1),      # 160 units: one partition each
])
def test_choose_partitions(B, Hkv, max_blocks, bs, cus, expect):
    assert pa.pa_choose_partitions(B, Hkv, max_blocks, bs, cus) == expect


def test_choose_partitions_properties():
    for B in (1, 2, 3, 5, 8, 31):
        for Hkv in (1, 2, 8):
            for mb in (1, 7, 8, 9, 64, 129, 1000, 4097):
                for cus in (80, 256, 304):
                    P = pa.pa_choose_partitions(B, Hkv, mb, 16, cus)
                    assert 1 <= P <= max(1, mb)
                    if B * Hkv >= cus:
                        # units cover the device: only rows over 128 tiles
                        # split, into partitions of up to 64 tiles, at most 16
                        assert P == (1 if mb <= 128 else min(16, math.ceil(mb / 64)))
                    elif mb <= 16:
                        assert P == 1   # a row of 16 tiles or fewer does not split
                    elif P > 1:
                        # every partition of a full row gets at least 8 tiles
                        assert mb // P >= 8
                        # and never more workgroups than compute units
                        assert B * Hkv * P <= cus
                        # unless the 8-tile floor or the 4096 cap binds, no fewer
                        # than that either: one more partition would exceed them
                        assert B * Hkv * (P + 1) > cus or mb // (P + 1) < 8 or P == 4096


@pytest.mark.parametrize("args,expect", [
    ((1, 8, 128, 1024, 16, 256, 0), (32, 1)),   # 16384 tokens: the fused split fills the CUs
    ((4, 8, 128, 128, 16, 256, 0), (8, 1)),     # 4 x 2048: 256 workgroups
    ((16, 8, 128, 16, 16, 256, 0), (1, 2)),     # 16 x 256: single pass, 128 units -> V split
    ((1, 8, 128, 32, 16, 256, 0), (4, 2)),      # 512 tokens: 32 workgroups -> V split
    ((4, 32, 128, 32, 16, 256, 0), (1, 2)),     # P = 2 on a 32-tile table -> single, V split
    ((4, 32, 64, 32, 16, 256, 0), (2, 1)),      # ... not for d = 64 (no V split there)
    ((4, 32, 128, 64, 16, 256, 0), (2, 1)),     # ... nor for a 64-tile table
    ((40, 8, 128, 256, 16, 256, 0), (4, 1)),    # units cover the device
    ((40, 8, 128, 256, 16, 256, 1), (1, 1)),    # forced single pass, 320 units: no V split
    ((2, 8, 128, 4, 16, 256, 1), (1, 2)),       # forced single pass, 16 units: V split
    ((2, 8, 128, 64, 16, 256, 3), (3, 2)),      # forced split, 48 workgroups: V split
    ((2, 8, 128, 64, 16, 256, 5), (5, 1)),      # forced split, 80 workgroups: no V split
    ((2, 8, 256, 64, 16, 256, 3), (3, 2)),
    ((0, 8, 128, 64, 16, 256, 0), (1, 2)),
])
def test_plan(args, expect):
    assert pa.pa_plan(*args) == expect


@pytest.mark.parametrize("dtype,G,split_only", [
    (pa.PA_DTYPE_BF16, 8, False), (pa.PA_DTYPE_BF16, 16, True), (pa.PA_DTYPE_F16, 16, True),
    (pa.PA_DTYPE_F32, 4, False), (pa.PA_DTYPE_F32, 8, True), (pa.PA_DTYPE_F32, 16, True),
])
def test_plan_of_shapes_that_always_split_v(dtype, G, split_only):
    # d = 256 with the groups whose whole-row accumulators would not fit the
    # register file: V split whatever the launch's size, and half the
    # heuristic's partitions while the units are fewer than the CUs
    for B, Hkv, W, parts in ((1, 8, 1024, 0), (40, 8, 256, 0), (2, 8, 64, 5), (64, 8, 64, 1),
                             (2, 8, 4, 0)):
        got = pa.pa_plan(B, Hkv, 256, W, 16, 256, parts, H=G * Hkv, dtype=dtype)
        ref = pa.pa_plan(B, Hkv, 256, W, 16, 256, parts)      # G = 1: never forced
        if not split_only:
            assert got == ref, (B, W, parts)
            continue
        assert got[1] == 2, (B, W, parts)
        if parts == 0 and B * Hkv < 256 and ref[0] > 1:
            assert got[0] == max(1, ref[0] // 2), (B, W, got, ref)
        elif parts == 0 and B * Hkv < 256:
            assert got[0] == 1
        else:
            assert got[0] == ref[0], (B, W, parts)


def test_plan_rejects_bad_arguments():
    lib = pa.load()
    import ctypes
    P, vs = ctypes.c_int(), ctypes.c_int()
    # (B, H, Hkv, d, dtype, max_blocks, block_size, num_cus, num_partitions)
    assert lib.pa_plan(1, 32, 8, 128, 1, 4, 16, 256, 0, None, ctypes.byref(vs)) == pa.PA_ERR_NULL
    bad = [((1, 32, 0, 128, 1, 4, 16, 256, 0), pa.PA_ERR_SHAPE),
           ((1, 32, 8, 128, 1, 4, 16, 0, 0), pa.PA_ERR_SHAPE),
           ((-1, 32, 8, 128, 1, 4, 16, 256, 0), pa.PA_ERR_SHAPE),
           ((1, 0, 8, 128, 1, 4, 16, 256, 0), pa.PA_ERR_SHAPE),
           ((1, 12, 8, 128, 1, 4, 16, 256, 0), pa.PA_ERR_SHAPE),
           ((1, 32, 8, 128, 7, 4, 16, 256, 0), pa.PA_ERR_DTYPE),
           ((1, 32, 8, 128, 1, 4, 16, 256, -2), pa.PA_ERR_VALUE),
           ((1, 32, 8, 96, 1, 4, 16, 256, 0), pa.PA_ERR_UNSUPPORTED),
           ((1, 32, 8, 128, 1, 4, 8, 256, 0), pa.PA_ERR_UNSUPPORTED),
           ((1, 256, 8, 128, 1, 4, 16, 256, 0), pa.PA_ERR_UNSUPPORTED)]   # G = 32
    for a, code in bad:
        assert lib.pa_plan(*a, ctypes.byref(P), ctypes.byref(vs)) == code, a


def test_workspace_bytes():
    assert pa.pa_workspace_bytes(1, 32, 128, 1) == 0
    assert pa.pa_workspace_bytes(0, 32, 128, 4) == 0
    # (max, sum) pairs padded to 256 bytes, then the fp32 partial sums
    assert pa.pa_workspace_bytes(1, 32, 128, 32) == 8192 + 32 * 32 * 128 * 4
    assert pa.pa_workspace_bytes(4, 32, 128, 3) == 3072 + 4 * 32 * 3 * 128 * 4
    assert pa.pa_workspace_bytes(1, 3, 128, 3) == 256 + 3 * 3 * 128 * 4
    assert pa.pa_workspace_bytes(1, 1, 128, 2) == 256 + 2 * 128 * 4


FAKE = dict(out=0x100000, q=0x200000, k=0x300000, v=0x400000, t=0x500000, n=0x600000)


def call(**kw):
    a = dict(FAKE, B=2, H=32, Hkv=8, d=128, bs=16, mb=4, scale=0.088, dtype=1)
    a.update(kw)
    return pa.load().pa_decode(a["out"], a["q"], a["k"], a["v"], a["t"], a["n"], a["B"], a["H"],
                               a["Hkv"], a["d"], a["bs"], a["mb"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), pa.PA_ERR_UNSUPPORTED),
    (dict(d=32), pa.PA_ERR_UNSUPPORTED),
    (dict(d=256, H=256, Hkv=8), pa.PA_ERR_UNSUPPORTED),          # G = 32
    (dict(Hkv=1 << 20, H=1 << 20), pa.PA_ERR_UNSUPPORTED),      # tile offsets past 2^31
    (dict(B=1 << 26, H=64, Hkv=8), pa.PA_ERR_UNSUPPORTED),      # 2^32 (sequence, head) pairs
    (dict(bs=8), pa.PA_ERR_UNSUPPORTED),
    (dict(bs=48), pa.PA_ERR_UNSUPPORTED),
    (dict(bs=512), pa.PA_ERR_UNSUPPORTED),
    (dict(H=24, Hkv=8), pa.PA_ERR_UNSUPPORTED),   # G = 3
    (dict(H=32, Hkv=6), pa.PA_ERR_SHAPE),         # H % Hkv != 0
    (dict(B=-1), pa.PA_ERR_SHAPE),
    (dict(H=0), pa.PA_ERR_SHAPE),
    (dict(mb=0), pa.PA_ERR_SHAPE),
    (dict(dtype=3), pa.PA_ERR_DTYPE),
    (dict(dtype=-1), pa.PA_ERR_DTYPE),
    (dict(scale=float("nan")), pa.PA_ERR_VALUE),
    (dict(scale=float("inf")), pa.PA_ERR_VALUE),
    (dict(q=0), pa.PA_ERR_NULL),
    (dict(out=0), pa.PA_ERR_NULL),
    (dict(t=0), pa.PA_ERR_NULL),
    (dict(k=0x300008), pa.PA_ERR_ALIGN),
    (dict(out=0x100004), pa.PA_ERR_ALIGN),
    (dict(n=0x600002), pa.PA_ERR_ALIGN),
    (dict(out=0x200000 + 4096), pa.PA_ERR_ALIAS),   # inside q's 2*32*128*2 bytes
    (dict(out=0x300000), pa.PA_ERR_ALIAS),
])
def test_validation_codes(kw, code):
    assert call(**kw) == code


def test_empty_batch_is_a_noop():
    assert call(B=0) == pa.PA_OK
    assert call(B=0, q=0, out=0) == pa.PA_OK


def test_valid_call_without_device_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the launch path is covered by the GPU tests")
    assert call() == pa.PA_ERR_DEVICE
    for bs in (16, 32, 64, 128, 256):  # every supported block size passes validation
        assert call(bs=bs) == pa.PA_ERR_DEVICE
    for dtype in (0, 1, 2):     # every (dtype, d, G) of the supported set is built
        for d in (64, 128, 256):
            for H in (8, 16, 32, 64, 128):
                assert call(dtype=dtype, d=d, H=H, Hkv=8) == pa.PA_ERR_DEVICE, (dtype, d, H)
            assert call(dtype=dtype, d=d, H=256, Hkv=8) == pa.PA_ERR_UNSUPPORTED   # G = 32


def test_ex_and_split_half_validation():
    lib = pa.load()
    args = [FAKE["out"], FAKE["q"], FAKE["k"], FAKE["v"], FAKE["t"], FAKE["n"], 1, 32, 8, 128,
            16, 64, 0.088, 1, None]
    assert lib.pa_decode_ex(*args, -2, 0, None, 0) == pa.PA_ERR_VALUE
    assert lib.pa_decode_ex(*args, 0, -5, None, 0) == pa.PA_ERR_VALUE
    # PA_PARTITIONS_UNIFORM passes validation (and then finds no device here)
    import torch
    if not torch.cuda.is_available():
        assert lib.pa_decode_ex(*args, pa.PA_PARTITIONS_UNIFORM, 0, None, 0) == pa.PA_ERR_DEVICE
    assert lib.pa_decode_partials(FAKE["q"], FAKE["k"], FAKE["v"], FAKE["t"], FAKE["n"], 1, 32,
                                  8, 128, 16, 64, 0.088, 1, -1, 0, 0x700000, 1 << 20,
                                  None) == pa.PA_ERR_VALUE
    assert lib.pa_decode_ex(*args, 4, 0, 0x700004, 1 << 20) == pa.PA_ERR_ALIGN
    # a caller workspace overlapping out or q is refused before any device call
    # (out and q hold 1 * 32 * 128 bf16 = 8 KiB each)
    assert lib.pa_decode_ex(*args, 4, 0, FAKE["out"] + 4096, 1 << 20) == pa.PA_ERR_ALIAS
    assert lib.pa_decode_ex(*args, 4, 0, FAKE["q"] - 4096, 8192) == pa.PA_ERR_ALIAS
    assert lib.pa_decode_ex(*args, 0, 0, FAKE["out"], 256) == pa.PA_ERR_ALIAS
    if not torch.cuda.is_available():   # touching neither passes on to the device
        assert lib.pa_decode_ex(*args, 4, 0, FAKE["q"] - 4096, 4096) == pa.PA_ERR_DEVICE
        assert lib.pa_decode_ex(*args, 4, 0, FAKE["q"] + 8192, 4096) == pa.PA_ERR_DEVICE
    part = [FAKE["q"], FAKE["k"], FAKE["v"], FAKE["t"], FAKE["n"], 1, 32, 8, 128, 16, 64, 0.088,
            1]
    assert lib.pa_decode_partials(*part, 0, 0, 0x700000, 1 << 20, None) == pa.PA_ERR_VALUE
    assert lib.pa_decode_partials(*part, 4, 0, None, 1 << 20, None) == pa.PA_ERR_WORKSPACE
    need = pa.pa_workspace_bytes(1, 32, 128, 4)
    assert lib.pa_decode_partials(*part, 4, 0, 0x700000, need - 1, None) == pa.PA_ERR_WORKSPACE
    assert lib.pa_decode_partials(*part, 5000, 0, 0x700000, 1 << 30, None) == \
        pa.PA_ERR_UNSUPPORTED
    assert lib.pa_decode_partials(*part, 4, 0, FAKE["q"] - 64, need, None) == pa.PA_ERR_ALIAS
    assert lib.pa_merge_partials(FAKE["out"], None, need, 1, 32, 128, 4, 1, None) == \
        pa.PA_ERR_WORKSPACE
    assert lib.pa_merge_partials(FAKE["out"], 0x700000, need - 1, 1, 32, 128, 4, 1, None) == \
        pa.PA_ERR_WORKSPACE
    assert lib.pa_merge_partials(FAKE["out"], 0x700000, need, 1, 32, 96, 4, 1, None) == \
        pa.PA_ERR_UNSUPPORTED
    assert lib.pa_merge_partials(0x700000 + 64, 0x700000, need, 1, 32, 128, 4, 1, None) == \
        pa.PA_ERR_ALIAS
    assert lib.pa_merge_partials(FAKE["out"], 0x700000, need, 0, 32, 128, 4, 1, None) == pa.PA_OK
    assert lib.pa_merge_partials(FAKE["out"], 0x700000, need, 1, 0, 128, 4, 1, None) == \
        pa.PA_ERR_SHAPE


def test_forced_partitions_clamp_rather_than_fail():
    # more partitions than tiles or than 4096 are clamped: the call passes
    # validation and only then finds no device here
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    lib = pa.load()
    args = [FAKE["out"], FAKE["q"], FAKE["k"], FAKE["v"], FAKE["t"], FAKE["n"], 1, 32, 8, 128,
            16, 8192, 0.088, 1, None]
    assert lib.pa_decode_ex(*args, 10 ** 6, 0, None, 0) == pa.PA_ERR_DEVICE
    assert lib.pa_decode_ex(*args, 5000, 0, None, 0) == pa.PA_ERR_DEVICE


def test_binding_rejects_bad_tensors():
    import torch
    q = torch.zeros(2, 32, 128, dtype=torch.float16)
    k = torch.zeros(4, 16, 8, 128, dtype=torch.float16)
    t = torch.zeros(2, 2, dtype=torch.int32)
    n = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(pa.PaError):   # host tensors are never handed to the library
        pa.decode(q, k, k, t, n, 0.1)
    with pytest.raises(pa.PaError):
        pa.decode(q.float(), k.float(), k.float(), t.long(), n, 0.1)
    with pytest.raises(pa.PaError):
        pa.dtype_code(torch.float64)
    assert pa.dtype_code(torch.float16) == pa.PA_DTYPE_F16


def test_decode_helper_refuses_mismatched_tensors_before_any_launch():
    # the C side sees only pointers: a pool of another head dim, a short or
    # mistyped `out` or a strided workspace would be read or written out of
    # bounds, so decode() refuses each of them itself.  On this host every
    # tensor is a CPU tensor, so each refusal below (a shape or dtype code, not
    # PA_ERR_DEVICE) shows that the check runs before the device check and
    # hence before anything is handed to the library.
    import torch
    B, H, Hkv, d, bs = 2, 32, 8, 128, 16
    q = torch.zeros(B, H, d, dtype=torch.bfloat16)
    k = torch.zeros(4, bs, Hkv, d, dtype=torch.bfloat16)
    t = torch.zeros(B, 2, dtype=torch.int32)
    n = torch.zeros(B, dtype=torch.int32)

    def code(**kw):
        args = dict(q=q, k_cache=k, v_cache=k, block_tables=t, context_lens=n)
        extra = {key: kw.pop(key) for key in ("out", "workspace") if key in kw}
        args.update(kw)
        with pytest.raises(pa.PaError) as e:
            pa.decode(args["q"], args["k_cache"], args["v_cache"], args["block_tables"],
                      args["context_lens"], 0.1, **extra)
        return e.value.code

    k64 = torch.zeros(4, bs, Hkv, 64, dtype=torch.bfloat16)
    assert code(k_cache=k64, v_cache=k64) == pa.PA_ERR_SHAPE          # head dim differs
    assert code(v_cache=torch.zeros(5, bs, Hkv, d, dtype=torch.bfloat16)) == pa.PA_ERR_SHAPE
    assert code(q=q[0]) == pa.PA_ERR_SHAPE                             # not [B][H][d]
    assert code(block_tables=torch.zeros(B + 1, 2, dtype=torch.int32)) == pa.PA_ERR_SHAPE
    assert code(context_lens=torch.zeros(B + 1, dtype=torch.int32)) == pa.PA_ERR_SHAPE
    assert code(out=torch.zeros(B, H, d - 2, dtype=torch.bfloat16)) == pa.PA_ERR_SHAPE
    assert code(out=torch.zeros(B - 1, H, d, dtype=torch.bfloat16)) == pa.PA_ERR_SHAPE
    assert code(out=torch.zeros(B, H, d, dtype=torch.float16)) == pa.PA_ERR_DTYPE
    assert code(out=torch.zeros(H, B, d, dtype=torch.bfloat16).transpose(0, 1)) == \
        pa.PA_ERR_SHAPE                                                # not contiguous
    strided_ws = torch.zeros(64, 2, dtype=torch.uint8)[:, 0]
    assert code(workspace=strided_ws) == pa.PA_ERR_SHAPE
    assert code(k_cache=k.float(), v_cache=k.float()) == pa.PA_ERR_DTYPE
    assert code(block_tables=t.long()) == pa.PA_ERR_DTYPE
    # every shape right: only then the device check (host tensors refused)
    assert code() == pa.PA_ERR_DEVICE
    assert code(out=torch.zeros(B, H, d, dtype=torch.bfloat16),
                workspace=torch.zeros(64, dtype=torch.uint8)) == pa.PA_ERR_DEVICE


def test_read_probe_library_exports_its_header():
    # the measuring aid beside the library: what include/pa_read_probe.h declares
    import ctypes
    from paged_attention_decode_pa_amd import build as hip_build
    text = open(os.path.join(os.path.dirname(HEADER), "pa_read_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))
    assert names == ["pa_probe_gather", "pa_probe_read", "pa_probe_stamp"]
    lib = ctypes.CDLL(hip_build.PROBE_LIB)
    fn = lib.pa_probe_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p]
    # argument checks come before any HIP call
    assert fn(None, 1024, 4, 16, 16, None) == -1
    assert fn(16, -1, 4, 16, 16, None) == -2
    assert fn(16, 1024, 0, 16, 16, None) == -2
    assert fn(16, 1024, 4, 12, 16, None) == -3
    lib.pa_probe_stamp.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert lib.pa_probe_stamp(None, None) == -1
    g = lib.pa_probe_gather
    V, I = ctypes.c_void_p, ctypes.c_int
    g.argtypes = [V, V, V, V, I, I, I, I, I, I, I, V, V]
    ok = dict(k=16, v=32, t=48, n=64, B=1, Hkv=8, row=256, bs=16, mb=1024, P=32, vs=1, sink=80)
    gcall = lambda **kw: g(*[dict(ok, **kw)[x] for x in ok], None)
    assert gcall(k=None) == -1 and gcall(sink=None) == -1
    assert gcall(B=-1) == -2 and gcall(Hkv=0) == -2 and gcall(mb=0) == -2 and gcall(P=0) == -2
    assert gcall(row=1024) == -3 and gcall(row=96) == -3 and gcall(bs=8) == -3
    assert gcall(bs=48) == -3 and gcall(P=4097) == -3 and gcall(B=65536) == -3
    assert gcall(vs=0) == -2 and gcall(vs=3) == -3
    assert gcall(mb=1 << 27, bs=16) == -3              # more than 2^30 tokens per row
    assert gcall(B=0) == 0                              # nothing to read: no launch



def test_noalloc_entry_validates_like_pa_decode():
    # the allocation-free entry takes pa_decode's arguments and refuses the
    # same invalid ones before any HIP call
    lib = pa.load()
    base = [FAKE["out"], FAKE["q"], FAKE["k"], FAKE["v"], FAKE["t"], FAKE["n"], 2, 32, 8, 128,
            16, 4, 0.088, 1, None]
    for change, code in ((dict(i=7, v=31), pa.PA_ERR_SHAPE), (dict(i=9, v=96),
                                                              pa.PA_ERR_UNSUPPORTED),
                         (dict(i=13, v=7), pa.PA_ERR_DTYPE), (dict(i=0, v=None), pa.PA_ERR_NULL),
                         (dict(i=12, v=float("nan")), pa.PA_ERR_VALUE)):
        args = list(base)
        args[change["i"]] = change["v"]
        assert lib.pa_decode_noalloc(*args) == code
        assert lib.pa_decode(*args) == code
    args = list(base)
    args[6] = 0
    assert lib.pa_decode_noalloc(*args) == pa.PA_OK   # B == 0: nothing to do


def test_plan_uniform_lengths_hint():
    # PA_PARTITIONS_UNIFORM: a covering batch runs the single pass; below the
    # CU count the hint changes nothing
    cus = 256
    assert pa.pa_plan(64, 8, 128, 512, 16, cus, 0) == (8, 1)
    assert pa.pa_plan(64, 8, 128, 512, 16, cus, pa.PA_PARTITIONS_UNIFORM) == (1, 1)
    for B, W in ((1, 1024), (4, 128), (16, 16), (2, 60)):
        assert pa.pa_plan(B, 8, 128, W, 16, cus, pa.PA_PARTITIONS_UNIFORM) == \
            pa.pa_plan(B, 8, 128, W, 16, cus, 0)
    with pytest.raises(pa.PaError) as e:
        pa.pa_plan(64, 8, 128, 512, 16, cus, -2)
    assert e.value.code == pa.PA_ERR_VALUE
    lib = pa.load()
    args = [FAKE["out"], FAKE["q"], FAKE["k"], FAKE["v"], FAKE["t"], FAKE["n"], 1, 32, 8, 128,
            16, 8, 0.088, 1, None]
    assert lib.pa_decode_ex(*args, -2, 0, None, 0) == pa.PA_ERR_VALUE


def test_no_vsplit_ablation_plans_no_v_split():
    # the ablation build differs only in never splitting V's head dim
    import ctypes
    lib = pa.load_variant("no_vsplit")
    P, vs = ctypes.c_int(0), ctypes.c_int(0)
    for B, W in ((1, 32), (16, 16), (1, 1024), (4, 128)):
        assert lib.pa_plan(B, 32, 8, 128, 1, W, 16, 256, 0, ctypes.byref(P), ctypes.byref(vs)) == 0
        assert vs.value == 1
        ref = pa.pa_plan(B, 8, 128, W, 16, 256, 0)
        if ref[1] == 1:
            assert P.value == ref[0]



def test_timeline_calls_only_in_the_timeline_library():
    text = open(os.path.join(os.path.dirname(HEADER), "pa_timeline.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))
    assert names == ["pa_timeline_copy", "pa_timeline_enable"]
    tl = pa.load_variant("timeline")
    for name in names:
        assert hasattr(tl, name), name
        assert not hasattr(pa.load(), name), name
    import ctypes
    tl.pa_timeline_enable.argtypes = [ctypes.c_int]
    tl.pa_timeline_copy.argtypes = [ctypes.c_void_p, ctypes.c_int]
    assert tl.pa_timeline_enable(0) == pa.PA_ERR_VALUE
    assert tl.pa_timeline_copy(None, 4) == pa.PA_ERR_NULL
    assert tl.pa_timeline_copy(16, 4) == pa.PA_ERR_VALUE   # nothing enabled yet


def test_breakdown_call_only_in_the_breakdown_library():
    import ctypes
    text = open(os.path.join(os.path.dirname(HEADER), "pa_breakdown.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))
    assert names == ["pa_breakdown_stop_after"]
    bd = pa.load_variant("breakdown")
    assert hasattr(bd, names[0]) and not hasattr(pa.load(), names[0])
    for other in ("timeline", "ordered"):
        assert not hasattr(pa.load_variant(other), names[0])
    bd.pa_breakdown_stop_after.argtypes = [ctypes.c_int]
    try:
        assert bd.pa_breakdown_stop_after(4) == pa.PA_ERR_VALUE
        assert bd.pa_breakdown_stop_after(-1) == pa.PA_ERR_VALUE
        for stage in (1, 2, 3, 0):
            assert bd.pa_breakdown_stop_after(stage) == pa.PA_OK
    finally:
        bd.pa_breakdown_stop_after(0)
