"""fp64 CPU oracle for the paged-attention decode step (ctypes wrapper).

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, loads or calls it, and it
shares no code with them.

The arithmetic lives in ``pa_oracle.c`` (plain C, double precision); see that
file's header for what is computed and which passages of the pages each step
follows.  This module only compiles it (``build()``), loads it and marshals
numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "libpa_oracle.so")

ERRORS = {0: "ok", -1: "null pointer", -2: "bad shape", -3: "context length out of range",
          -4: "block-table entry out of range", -5: "out of memory"}


class OracleError(RuntimeError):
    pass


def build(src: str = _SRC, out: str = _LIB, extra: tuple = ()) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", src, "-o", out, "-lm",
           *extra]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load(path: Optional[str] = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    common = [P, P, P, P, P, P, I, I, I, I, I, I, ctypes.c_longlong, ctypes.c_double]
    lib.pa_oracle_decode.argtypes = common + [I]
    lib.pa_oracle_decode_online.argtypes = common + [I, I]
    lib.pa_oracle_decode_split.argtypes = common + [I, I]
    for f in (lib.pa_oracle_decode, lib.pa_oracle_decode_online, lib.pa_oracle_decode_split):
        f.restype = I
    lib.pa_oracle_max_threads.restype = I
    return lib


def max_threads() -> int:
    return int(load().pa_oracle_max_threads())


def _args(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads, block_size, scale,
          num_pool_blocks):
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k_cache, dtype=np.float32)
    v = np.ascontiguousarray(v_cache, dtype=np.float32)
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    n = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, H, d = q.shape
    if k.ndim != 4 or k.shape[1] != block_size or k.shape[2] != num_kv_heads or k.shape[3] != d:
        raise OracleError(f"k_cache shape {k.shape} does not match [pool][{block_size}]"
                          f"[{num_kv_heads}][{d}]")
    if v.shape != k.shape:
        raise OracleError("v_cache shape differs from k_cache")
    if t.ndim != 2 or t.shape[0] != B or n.shape != (B,):
        raise OracleError("block_tables must be [B][max_blocks], context_lens [B]")
    pool = k.shape[0] if num_pool_blocks is None else int(num_pool_blocks)
    out = np.zeros((B, H, d), dtype=np.float64)
    keep = (q, k, v, t, n, out)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    args = [ptr(out), ptr(q), ptr(k), ptr(v), ptr(t), ptr(n), B, H, num_kv_heads, d,
            block_size, t.shape[1], pool, float(scale)]
    return out, keep, args


def _call(fn, args, extra):
    rc = fn(*args, *extra)
    if rc != 0:
        raise OracleError(f"oracle rejected the input: {ERRORS.get(rc, rc)}")


def decode(q, k_cache, v_cache, block_tables, context_lens, *, num_kv_heads, block_size, scale,
           num_pool_blocks=None, threads: int = 0, lib=None) -> np.ndarray:
    """Gather-then-dense two-pass softmax in fp64; returns float64 [B][H][d]."""
    out, keep, args = _args(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
                            block_size, scale, num_pool_blocks)
    _call((lib or load()).pa_oracle_decode, args, [threads])
    return out


def decode_online(q, k_cache, v_cache, block_tables, context_lens, *, num_kv_heads, block_size,
                  scale, tile: int, num_pool_blocks=None, threads: int = 0,
                  lib=None) -> np.ndarray:
    """One-pass running-max softmax over tiles of ``tile`` logical tokens."""
    out, keep, args = _args(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
                            block_size, scale, num_pool_blocks)
    _call((lib or load()).pa_oracle_decode_online, args, [tile, threads])
    return out


def decode_split(q, k_cache, v_cache, block_tables, context_lens, *, num_kv_heads, block_size,
                 scale, num_partitions: int, num_pool_blocks=None,
                 threads: int = 0, lib=None) -> np.ndarray:
    """Partition the table into ``num_partitions`` block ranges, reduce each to
    (max, sum, weighted values), then merge."""
    out, keep, args = _args(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
                            block_size, scale, num_pool_blocks)
    _call((lib or load()).pa_oracle_decode_split, args, [num_partitions, threads])
    return out


def _case_kwargs(case):
    return dict(num_kv_heads=case.num_kv_heads, block_size=case.block_size,
                scale=float(case.scale))


def decode_case(case, threads: int = 0, lib=None) -> np.ndarray:
    """The oracle on a ``pa_inputs.Case``."""
    return decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                  threads=threads, lib=lib, **_case_kwargs(case))


def decode_case_online(case, tile: int, threads: int = 0, lib=None) -> np.ndarray:
    return decode_online(case.q, case.k_cache, case.v_cache, case.block_tables,
                         case.context_lens, tile=tile, threads=threads, lib=lib,
                         **_case_kwargs(case))


def decode_case_split(case, num_partitions: int, threads: int = 0, lib=None) -> np.ndarray:
    return decode_split(case.q, case.k_cache, case.v_cache, case.block_tables,
                        case.context_lens, num_partitions=num_partitions, threads=threads,
                        lib=lib, **_case_kwargs(case))
