"""Seeded synthetic inputs for the paged-attention decode step.

This module is shared by the HIP path's tests, the CPU oracle's tests and the
benchmark.  It holds no attention arithmetic: it only draws random numbers,
rounds them to the storage type and lays them out the way the paged KV cache
stores them.

What the inputs look like follows the pages:

* "Decoding Benchmark" (MinivLLM docs), section "What paged attention decode
  does": q has shape (batch_size, num_heads, head_dim); K/V live in a pool of
  fixed-size physical blocks of shape (num_blocks, block_size, num_kv_heads,
  head_dim); the block table has shape (batch_size, max_num_blocks) and -1
  marks a slot that was never allocated (section "Block table lookup
  mechanics").
* ``benchmark_decoding.py``, function ``setup_test_data``: values are standard
  normal draws, the table is a random permutation of the pool (an identity
  table would let a kernel that ignores the table pass), every sequence has the
  same context length, and scale = 1/sqrt(head_dim).
* The five workloads (``CONFIGS``) use the docs page's shapes (section
  "Benchmark configurations": heads 32, kv heads 8, head_dim 128, block_size
  16) and add a 16384-token single-sequence case from the long end of the
  flash-decoding-bench design note's KV-length sweep.

Draw order for a seed (numpy ``default_rng``): q, then the K pool, then the V
pool (all float32 standard normal), then the pool permutation.  bf16 and fp16
cases round every float32 draw to bfloat16 or IEEE half with
round-to-nearest-even; both the GPU and the oracle then see exactly those
rounded values.  fp16 is the element type ``setup_test_data`` draws in.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Union

import numpy as np

__all__ = [
    "Case", "CONFIGS", "make_case", "make_config_case", "bf16_round_bits",
    "bf16_bits_to_f32", "f16_round_bits", "f16_bits_to_f32", "poison_unused",
    "BF16_NAN_BITS", "F16_NAN_BITS", "DTYPES",
]

BF16_NAN_BITS = 0x7FC0
F16_NAN_BITS = 0x7E00
DTYPES = ("f32", "bf16", "f16")


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), round to nearest even.

    NaN inputs map to the canonical quiet NaN; finite values that overflow
    round to +-inf as IEEE RNE prescribes.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    # In 32-bit arithmetic: for every finite value and +-inf, u + 0x7FFF + lsb
    # stays below 2^32 (the largest, -FLT_MAX = 0xFF7FFFFF, reaches 0xFF807FFF);
    # NaNs are replaced below.
    u = x.view(np.uint32)
    t = (u >> 16) & 1
    t += u
    t += 0x7FFF
    t >>= 16
    rounded = t.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = BF16_NAN_BITS
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> the float32 values they encode (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> IEEE binary16 bit patterns (uint16), round to nearest
    even (numpy's float32 -> float16 conversion rounds that way)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):   # overflow to +-inf is the rounding rule
        return x.astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns (uint16) -> the float32 values they encode (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float32)


_ROUND = {"bf16": (bf16_round_bits, bf16_bits_to_f32, BF16_NAN_BITS),
          "f16": (f16_round_bits, f16_bits_to_f32, F16_NAN_BITS)}


@dataclasses.dataclass
class Case:
    """One decode step's inputs, as host arrays.

    ``q``, ``k_cache`` and ``v_cache`` are float32 arrays holding the exact
    values the GPU sees (for bf16 and fp16 cases, values already rounded);
    ``*_bits`` hold the 16-bit patterns (uint16) for bf16 and fp16 cases,
    else None.
    """

    dtype: str                      # "f32", "bf16" or "f16"
    q: np.ndarray                   # [B][H][d] float32
    k_cache: np.ndarray             # [pool][block_size][Hkv][d] float32
    v_cache: np.ndarray             # [pool][block_size][Hkv][d] float32
    block_tables: np.ndarray        # [B][max_blocks] int32, -1 = unallocated
    context_lens: np.ndarray        # [B] int32
    scale: np.float32
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None
    seed: Optional[int] = None
    name: str = ""

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def num_pool_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def storage(self, which: str) -> np.ndarray:
        """The array in its storage type: uint16 bits for bf16 and fp16,
        float32 else."""
        if self.dtype != "f32":
            return {"q": self.q_bits, "k": self.k_bits, "v": self.v_bits}[which]
        return {"q": self.q, "k": self.k_cache, "v": self.v_cache}[which]

    def algorithmic_bytes(self) -> int:
        """Bytes one decode step must move: every live K and V row once per
        kv head, q, out and the block table (context_lens excluded)."""
        live = 0
        bs = self.block_size
        for b in range(self.batch):
            n = int(self.context_lens[b])
            for t in range(0, n, bs):
                if self.block_tables[b, t // bs] >= 0:
                    live += min(bs, n - t)
        e = self.elem_bytes
        d = self.head_dim
        return (live * self.num_kv_heads * d * e * 2
                + 2 * self.batch * self.num_heads * d * e
                + self.block_tables.size * 4)


# The five workloads.  Shapes from the docs page's configuration table; pool
# oversizing: 1x for the smallest, 2x for the others (the two largest pools'
# size is not stated anywhere; 2x is this module's choice).
CONFIGS = {
    1: dict(dtype="f32", B=2, ctx=60, H=32, Hkv=8, d=128, bs=16, pool=8),
    2: dict(dtype="bf16", B=1, ctx=512, H=32, Hkv=8, d=128, bs=16, pool=64),
    3: dict(dtype="bf16", B=16, ctx=256, H=32, Hkv=8, d=128, bs=16, pool=512),
    4: dict(dtype="bf16", B=4, ctx=2048, H=32, Hkv=8, d=128, bs=16, pool=1024),
    5: dict(dtype="bf16", B=1, ctx=16384, H=32, Hkv=8, d=128, bs=16, pool=2048),
}

CONFIG_NAMES = {
    1: "fp32 B=2 ctx=60 H=32 Hkv=8 d=128 bs=16",
    2: "bf16 B=1 ctx=512 H=32 Hkv=8 d=128 bs=16",
    3: "bf16 B=16 ctx=256 H=32 Hkv=8 d=128 bs=16",
    4: "bf16 B=4 ctx=2048 H=32 Hkv=8 d=128 bs=16",
    5: "bf16 B=1 ctx=16384 H=32 Hkv=8 d=128 bs=16",
}


def make_case(
    B: int,
    ctx: Union[int, Sequence[int]],
    H: int,
    Hkv: int,
    d: int,
    bs: int,
    *,
    dtype: str = "bf16",
    seed: int = 0,
    max_blocks: Optional[int] = None,
    pool: Optional[int] = None,
    table: str = "perm",
    holes: Optional[Sequence[tuple]] = None,
    name: str = "",
) -> Case:
    """Draw one decode step's inputs.

    ctx: one context length for every sequence, or one per sequence.
    max_blocks: table width; defaults to ceil(max(ctx)/bs) (at least 1).
    pool: number of physical blocks; defaults to the blocks the table needs.
    table: "perm" scatters each sequence's blocks over the pool through a
      seeded permutation; "identity" hands them out in order (the docs page's
      arange table).
    holes: (b, logical_block) pairs whose table entry is set to -1 after the
      assignment, i.e. unallocated slots inside a sequence's context.
    """
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {DTYPES}, got {dtype!r}")
    lens = [int(ctx)] * B if np.isscalar(ctx) else [int(c) for c in ctx]
    if len(lens) != B:
        raise ValueError("one context length per sequence expected")
    need = [max(0, math.ceil(n / bs)) for n in lens]
    if max_blocks is None:
        max_blocks = max([1] + need)
    if any(nb > max_blocks for nb in need):
        raise ValueError("a context does not fit in max_blocks * block_size")
    total = sum(need)
    if pool is None:
        pool = max(total, 1)
    if pool < total:
        raise ValueError(f"pool of {pool} blocks cannot hold {total} blocks")

    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, d), dtype=np.float32)
    k = rng.standard_normal((pool, bs, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((pool, bs, Hkv, d), dtype=np.float32)
    if table == "perm":
        order = rng.permutation(pool).astype(np.int32)
    elif table == "identity":
        order = np.arange(pool, dtype=np.int32)
    else:
        raise ValueError(f"unknown table kind {table!r}")

    # sequence b takes the next need[b] entries of `order`, in sequence order
    tables = np.full((B, max_blocks), -1, dtype=np.int32)
    counts = np.asarray(need, dtype=np.int64)
    rows = np.repeat(np.arange(B), counts)
    cols = np.arange(total) - np.repeat(np.cumsum(counts) - counts, counts)
    tables[rows, cols] = order[:total]
    for (b, j) in holes or ():
        tables[b, j] = -1

    case = Case(
        dtype=dtype, q=q, k_cache=k, v_cache=v, block_tables=tables,
        context_lens=np.asarray(lens, dtype=np.int32),
        scale=np.float32(1.0 / math.sqrt(d)), num_heads=H, num_kv_heads=Hkv,
        head_dim=d, block_size=bs, seed=seed, name=name,
    )
    if dtype in _ROUND:
        to_bits, to_f32, _ = _ROUND[dtype]
        case.q_bits = to_bits(q)
        case.k_bits = to_bits(k)
        case.v_bits = to_bits(v)
        case.q = to_f32(case.q_bits)
        case.k_cache = to_f32(case.k_bits)
        case.v_cache = to_f32(case.v_bits)
    return case


def make_config_case(config_id: int, seed: Optional[int] = None) -> Case:
    """Inputs of one of the five named workloads; seed defaults to its id."""
    c = CONFIGS[config_id]
    return make_case(
        c["B"], c["ctx"], c["H"], c["Hkv"], c["d"], c["bs"], dtype=c["dtype"],
        seed=config_id if seed is None else seed, pool=c["pool"],
        name=CONFIG_NAMES[config_id],
    )


def poison_unused(case: Case) -> Case:
    """Copy of ``case`` with NaN in every K/V slot that holds no live token.

    Live tokens are t < context_lens[b] whose table entry is >= 0.  Slots past
    the end of a sequence's last block, blocks no table entry references and
    blocks behind -1 holes are all overwritten.  Table entries at or past
    ceil(context_len / block_size) are set to -1.
    """
    bs = case.block_size
    live = np.zeros((case.num_pool_blocks, bs), dtype=bool)
    tables = case.block_tables.copy()
    for b in range(case.batch):
        n = int(case.context_lens[b])
        nb = math.ceil(n / bs) if n > 0 else 0
        tables[b, nb:] = -1
        for j in range(nb):
            blk = tables[b, j]
            if blk >= 0:
                live[blk, :min(bs, n - j * bs)] = True
    out = dataclasses.replace(case, block_tables=tables)
    dead = ~live
    if case.dtype in _ROUND:
        _, to_f32, nan_bits = _ROUND[case.dtype]
        kb = case.k_bits.copy(); vb = case.v_bits.copy()
        kb[dead] = nan_bits; vb[dead] = nan_bits
        out.k_bits, out.v_bits = kb, vb
        out.k_cache = to_f32(kb); out.v_cache = to_f32(vb)
    else:
        k = case.k_cache.copy(); v = case.v_cache.copy()
        k[dead] = np.nan; v[dead] = np.nan
        out.k_cache, out.v_cache = k, v
    return out
