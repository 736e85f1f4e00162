"""Python binding of the paged-attention decode C ABI (include/pa_decode.h).

Argument marshalling only: every step of the decode runs in the HIP kernels of
``libpa_decode.so``.  The functions keep the C names and argument order; tensor
arguments may be torch tensors (their ``data_ptr()`` is passed) or raw device
addresses, and ``stream`` may be a ``torch.cuda.Stream``, a raw hipStream_t
value or None (torch's current stream).  A non-zero return code raises
``PaError``.  There is no CPU fallback: if the library is missing, ``load()``
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa_decode.so")
# Ablation builds of the same sources (see build.py), loaded only on request.
VARIANT_PATHS = {"valu_qk": os.path.join(HERE, "libpa_decode_valu_qk.so"),
                 "no_vsplit": os.path.join(HERE, "libpa_decode_no_vsplit.so"),
                 "ordered": os.path.join(HERE, "libpa_decode_ordered.so"),
                 "timeline": os.path.join(HERE, "libpa_decode_timeline.so"),
                 "breakdown": os.path.join(HERE, "libpa_decode_breakdown.so")}

PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1
PA_DTYPE_F16 = 2

PA_OK = 0
PA_ERR_NULL = -1
PA_ERR_SHAPE = -2
PA_ERR_UNSUPPORTED = -3
PA_ERR_DTYPE = -4
PA_ERR_ALIGN = -5
PA_ERR_WORKSPACE = -6
PA_ERR_HIP = -7
PA_ERR_DEVICE = -8
PA_ERR_ALIAS = -9
PA_ERR_VALUE = -10

PA_PARTITIONS_UNIFORM = -1   # num_partitions: heuristic for equal context lengths

EXPORTS = ("pa_decode", "pa_decode_ex", "pa_decode_noalloc", "pa_decode_partials",
           "pa_merge_partials",
           "pa_workspace_bytes", "pa_choose_partitions", "pa_plan", "pa_device_num_cus",
           "pa_strerror", "pa_release")


class PaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


_lib = None


def load(path: Optional[str] = None):
    """Load libpa_decode.so (built by ``build.build()``); raises if absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library {p} not found: run "
                           "`python -m paged_attention_decode_pa_amd.build` first")
    lib = ctypes.CDLL(p)
    V, I, F, LL, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_longlong, ctypes.c_size_t
    core = [V, V, V, V, V, V, I, I, I, I, I, I, F, I, V]
    lib.pa_decode.argtypes = core
    lib.pa_decode_ex.argtypes = core + [I, LL, V, SZ]
    lib.pa_decode_noalloc.argtypes = core
    lib.pa_decode_partials.argtypes = [V, V, V, V, V, I, I, I, I, I, I, F, I, I, LL, V, SZ, V]
    lib.pa_merge_partials.argtypes = [V, V, SZ, I, I, I, I, I, V]
    lib.pa_workspace_bytes.argtypes = [I, I, I, I]
    lib.pa_workspace_bytes.restype = SZ
    lib.pa_choose_partitions.argtypes = [I, I, I, I, I]
    IP = ctypes.POINTER(ctypes.c_int)
    lib.pa_plan.argtypes = [I, I, I, I, I, I, I, I, I, IP, IP]
    lib.pa_device_num_cus.argtypes = [I]
    lib.pa_strerror.argtypes = [I]
    lib.pa_strerror.restype = ctypes.c_char_p
    lib.pa_release.argtypes = []
    lib.pa_release.restype = None
    for name in ("pa_decode", "pa_decode_ex", "pa_decode_noalloc", "pa_decode_partials",
                 "pa_merge_partials",
                 "pa_choose_partitions", "pa_plan", "pa_device_num_cus"):
        getattr(lib, name).restype = I
    if path is None:
        _lib = lib
    return lib


def load_variant(name: str):
    """Load an ablation build by name (raises if it is not built)."""
    if name not in VARIANT_PATHS:
        raise ValueError(f"unknown library variant {name!r}; known: {sorted(VARIANT_PATHS)}")
    return load(VARIANT_PATHS[name])


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc: int, where: str) -> None:
    if rc != PA_OK:
        raise PaError(rc, where)


def strerror(code: int) -> str:
    return load().pa_strerror(code).decode()


def dtype_code(torch_dtype) -> int:
    import torch
    if torch_dtype == torch.float32:
        return PA_DTYPE_F32
    if torch_dtype == torch.bfloat16:
        return PA_DTYPE_BF16
    if torch_dtype == torch.float16:
        return PA_DTYPE_F16
    raise PaError(PA_ERR_DTYPE, f"dtype {torch_dtype}")


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d, block_size,
              max_blocks, scale, dtype, stream=None) -> None:
    rc = load().pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                          _ptr(context_lens), B, H, Hkv, d, block_size, max_blocks, scale, dtype,
                          _stream(stream))
    _check(rc, "pa_decode")


def pa_decode_ex(out, q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d, block_size,
                 max_blocks, scale, dtype, stream=None, num_partitions=0, num_pool_blocks=0,
                 workspace=None, workspace_bytes=0) -> None:
    rc = load().pa_decode_ex(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                             _ptr(block_tables), _ptr(context_lens), B, H, Hkv, d, block_size,
                             max_blocks, scale, dtype, _stream(stream), num_partitions,
                             num_pool_blocks, _ptr(workspace), workspace_bytes)
    _check(rc, "pa_decode_ex")


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d,
                      block_size, max_blocks, scale, dtype, stream=None) -> None:
    rc = load().pa_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(block_tables), _ptr(context_lens), B, H, Hkv, d,
                                  block_size, max_blocks, scale, dtype, _stream(stream))
    _check(rc, "pa_decode_noalloc")


def pa_decode_partials(q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d,
                       block_size, max_blocks, scale, dtype, num_partitions, num_pool_blocks,
                       workspace, workspace_bytes, stream=None) -> None:
    rc = load().pa_decode_partials(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                   _ptr(context_lens), B, H, Hkv, d, block_size, max_blocks,
                                   scale, dtype, num_partitions, num_pool_blocks,
                                   _ptr(workspace), workspace_bytes, _stream(stream))
    _check(rc, "pa_decode_partials")


def pa_merge_partials(out, workspace, workspace_bytes, B, H, d, num_partitions, dtype,
                      stream=None) -> None:
    rc = load().pa_merge_partials(_ptr(out), _ptr(workspace), workspace_bytes, B, H, d,
                                  num_partitions, dtype, _stream(stream))
    _check(rc, "pa_merge_partials")


def pa_workspace_bytes(B, H, d, num_partitions) -> int:
    return int(load().pa_workspace_bytes(B, H, d, num_partitions))


def pa_choose_partitions(B, Hkv, max_blocks, block_size, num_cus) -> int:
    return int(load().pa_choose_partitions(B, Hkv, max_blocks, block_size, num_cus))


def pa_plan(B, Hkv, d, max_blocks, block_size, num_cus, num_partitions=0, H=None,
            dtype=PA_DTYPE_BF16):
    """(partitions, v_slices) of the launch pa_decode_ex makes without a caller
    workspace.  H (default Hkv) and dtype matter only for the shapes that
    always split V's head dim (d = 256 with large groups)."""
    P, vs = ctypes.c_int(0), ctypes.c_int(0)
    _check(load().pa_plan(B, Hkv if H is None else H, Hkv, d, dtype, max_blocks, block_size,
                          num_cus, num_partitions, ctypes.byref(P), ctypes.byref(vs)),
           "pa_plan")
    return P.value, vs.value


def pa_device_num_cus(device: int = 0) -> int:
    n = int(load().pa_device_num_cus(device))
    _check(n if n < 0 else PA_OK, "pa_device_num_cus")
    return n


def pa_strerror(code: int) -> str:
    return strerror(code)


def pa_release() -> None:
    load().pa_release()


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, *, out=None, stream=None,
           num_partitions=0, num_pool_blocks=None, workspace=None):
    """Tensor-level convenience: shapes are read from the tensors, ``out`` is
    allocated with torch when not given, and the call goes to pa_decode_ex.
    ``num_pool_blocks`` defaults to ``k_cache.shape[0]``, so table entries past
    the pool are skipped like -1 instead of being read.  Every check below runs
    before anything is launched: the C side sees only pointers, so a pool of
    another head dim or a short ``out`` would otherwise be read or written out
    of bounds."""
    import torch
    if q.dim() != 3 or k_cache.dim() != 4:
        raise PaError(PA_ERR_SHAPE, "q must be [B][H][d] and k_cache [pool][block_size][Hkv][d]")
    B, H, d = q.shape
    _, block_size, Hkv, kd = k_cache.shape
    if kd != d:
        raise PaError(PA_ERR_SHAPE, f"k_cache head dim {kd} != q head dim {d}")
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise PaError(PA_ERR_SHAPE, "v_cache must have k_cache's shape")
    if (block_tables.dim() != 2 or block_tables.shape[0] != B
            or tuple(context_lens.shape) != (B,)):
        raise PaError(PA_ERR_SHAPE, "block_tables must be [B][max_blocks], context_lens [B]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise PaError(PA_ERR_DTYPE, "q, k_cache and v_cache must share a dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise PaError(PA_ERR_DTYPE, "block_tables and context_lens must be int32")
    if out is not None:
        if tuple(out.shape) != tuple(q.shape):
            raise PaError(PA_ERR_SHAPE, f"out has shape {tuple(out.shape)}, q {tuple(q.shape)}")
        if out.dtype != q.dtype:
            raise PaError(PA_ERR_DTYPE, "out must have q's dtype")
    tensors = [("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
               ("block_tables", block_tables), ("context_lens", context_lens)]
    if out is not None:
        tensors.append(("out", out))
    if workspace is not None:
        tensors.append(("workspace", workspace))
    for name, t in tensors:
        if not t.is_contiguous():
            raise PaError(PA_ERR_SHAPE, f"{name} must be contiguous")
    for name, t in tensors:
        if not t.is_cuda or t.device != q.device:
            raise PaError(PA_ERR_DEVICE, f"{name} must be on q's GPU")
    max_blocks = block_tables.shape[1]
    if num_pool_blocks is None:
        num_pool_blocks = k_cache.shape[0]
    if out is None:
        out = torch.empty_like(q)
    ws_bytes = 0
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    # (the library launches on the current device and sizes its buffers for it)
    with torch.cuda.device(q.device):
        pa_decode_ex(out, q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d,
                     block_size, max_blocks, float(scale), dtype_code(q.dtype), stream,
                     num_partitions, num_pool_blocks, workspace, ws_bytes)
    return out
