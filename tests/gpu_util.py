"""Helpers for the GPU tests: move a pa_inputs.Case to the device, run the HIP
path through the C ABI, compare with the oracle at the stated tolerances."""
import sys

import numpy as np
import torch

import paged_attention_decode_pa_amd as pa

# Tolerances: fp32 max |gpu - oracle| <= 1e-5; bf16 elementwise
# |gpu - oracle| <= 2e-3 + 1e-2 * |oracle| (oracle fed the same bf16 values).
# fp16 elementwise |gpu - oracle| <= 5e-5 + 2^-10 * |oracle|: products of
# binary16 values are exact in fp32, the fp32 path itself stays inside the
# fp32 bar (1e-5), and rounding the result to binary16 adds at most half a
# unit in the last place (2^-11 * |x|); the bound leaves a factor of about two
# on both terms.
F32_ATOL = 1e-5
BF16_ATOL = 2e-3
BF16_RTOL = 1e-2
F16_ATOL = 5e-5
F16_RTOL = 2.0 ** -10
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class DeviceCase:
    def __init__(self, case, dev, extra_pool_blocks=0):
        self.case = case
        if case.dtype != "f32":
            tdt = TORCH_DTYPE[case.dtype]
            conv = lambda bits: torch.from_numpy(bits.view(np.int16)).to(dev).view(tdt)
            self.q = conv(case.q_bits)
            k, v = case.k_bits, case.v_bits
            if extra_pool_blocks:
                pad = np.zeros((extra_pool_blocks,) + k.shape[1:], dtype=np.uint16)
                k = np.concatenate([k, pad]); v = np.concatenate([v, pad])
            self.k = conv(np.ascontiguousarray(k))
            self.v = conv(np.ascontiguousarray(v))
        else:
            self.q = torch.from_numpy(case.q).to(dev)
            k, v = case.k_cache, case.v_cache
            if extra_pool_blocks:
                pad = np.zeros((extra_pool_blocks,) + k.shape[1:], dtype=np.float32)
                k = np.concatenate([k, pad]); v = np.concatenate([v, pad])
            self.k = torch.from_numpy(np.ascontiguousarray(k)).to(dev)
            self.v = torch.from_numpy(np.ascontiguousarray(v)).to(dev)
        self.table = torch.from_numpy(case.block_tables).to(dev)
        self.lens = torch.from_numpy(case.context_lens).to(dev)
        self.dtype = pa.dtype_code(self.q.dtype)

    def args(self):
        c = self.case
        return (self.q, self.k, self.v, self.table, self.lens, c.batch, c.num_heads,
                c.num_kv_heads, c.head_dim, c.block_size, c.max_blocks, float(c.scale),
                self.dtype)


def check_host_preconditions(case):
    """Shapes and table entries the kernels assume, checked before any launch."""
    assert case.block_tables.shape == (case.batch, case.max_blocks)
    assert case.context_lens.shape == (case.batch,)
    assert (case.context_lens >= 0).all()
    assert (case.context_lens <= case.max_blocks * case.block_size).all()
    t = case.block_tables
    assert ((t == -1) | ((t >= 0) & (t < case.num_pool_blocks))).all()


def run_gpu(case, dev, *, num_partitions=None, guard=True, stream=None, workspace=None):
    """One decode step on the GPU.  num_partitions None = pa_decode (heuristic,
    no pool guard); otherwise pa_decode_ex with that count (0 = heuristic)."""
    check_host_preconditions(case)
    d = DeviceCase(case, dev)
    out = torch.empty_like(d.q)
    if num_partitions is None:
        pa.pa_decode(out, *d.args(), stream)
    else:
        ws, ws_bytes = (None, 0) if workspace is None else workspace
        pa.pa_decode_ex(out, *d.args(), stream, num_partitions,
                        case.num_pool_blocks if guard else 0, ws, ws_bytes)
    torch.cuda.synchronize()
    return out


def to_f64(out):
    return out.float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if dtype == "f32":
        worst = err.max() if err.size else 0.0
        assert worst <= F32_ATOL, f"{what}: max abs err {worst:.3e} > {F32_ATOL}"
    else:
        atol, rtol = (BF16_ATOL, BF16_RTOL) if dtype == "bf16" else (F16_ATOL, F16_RTOL)
        bound = atol + rtol * np.abs(ref)
        bad = err > bound
        assert not bad.any(), (f"{what}: {bad.sum()} elements out of tolerance, worst excess "
                               f"{(err - bound).max():.3e}, max abs err {err.max():.3e}")
