"""Pins of the fp64 oracle to things other than itself.

The pages print no worked-example values, so the oracle is pinned by:
  * a library routine: torch's scaled_dot_product_attention in float64 on the
    CPU, applied to a contiguous copy obtained by a plain reshape of an
    identity-mapped pool (the docs page's arange block table), with the
    library's own grouped-query head expansion;
  * invariants that hold for the paged lookup: permuting physical blocks with
    the table remapped, NaN in slots that hold no live token, -1 holes equal to
    removing those tokens;
  * closed forms: context length 1, two tokens, scale 0, identical keys, a
    dominant key, per-kv-head constant V, convexity;
  * agreement of the one-pass (running max / normaliser) and split-and-merge
    routes with the two-pass definition.
Each plausible mistake (wrong head mapping, wrong slot, missing scale, flipped
softmax sign, missing normalisation, dropped token, V read from K) fails at
least one of these; test_oracle_mutants.py plants them and checks.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import pa_inputs as pi


def run(oracle_mod, case, **kw):
    return oracle_mod.decode_case(case, **kw)


def sdpa_identity(case):
    """torch SDPA (float64, CPU) on the contiguous sequences of an identity-table
    case: sequence b's tokens are pool blocks [b*nb, (b+1)*nb) in order."""
    B, H, d = case.q.shape
    nb = case.max_blocks
    bs, Hkv = case.block_size, case.num_kv_heads
    outs = np.zeros((B, H, d))
    for b in range(B):
        n = int(case.context_lens[b])
        if n == 0:
            continue
        k = case.k_cache[b * nb:(b + 1) * nb].reshape(nb * bs, Hkv, d)[:n]
        v = case.v_cache[b * nb:(b + 1) * nb].reshape(nb * bs, Hkv, d)[:n]
        qt = torch.from_numpy(case.q[b].astype(np.float64)).reshape(1, H, 1, d)
        kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
        vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
        o = F.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(),
                                           scale=float(case.scale), enable_gqa=(H != Hkv))
        outs[b] = o.reshape(H, d).numpy()
    return outs


SHAPES = [
    # B, ctx, H, Hkv, d, bs
    (1, 1, 1, 1, 1, 1),
    (2, 7, 2, 1, 4, 2),
    (2, [13, 5], 4, 2, 8, 4),
    (3, [40, 16, 1], 4, 2, 8, 16),
    (2, [33, 31], 8, 2, 8, 1),
    (1, 37, 4, 4, 6, 4),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_table_equals_library_sdpa(oracle_mod, shape, dtype):
    B, ctx, H, Hkv, d, bs = shape
    lens = [ctx] * B if np.isscalar(ctx) else ctx
    nb = max(math.ceil(n / bs) for n in lens)
    # identity table needs every sequence to own nb consecutive blocks
    case = pi.make_case(B, lens, H, Hkv, d, bs, dtype=dtype, seed=11, table="identity",
                        max_blocks=nb, pool=B * nb)
    tables = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    for b, n in enumerate(lens):
        tables[b, math.ceil(n / bs):] = -1
    case.block_tables = tables
    got = run(oracle_mod, case)
    ref = sdpa_identity(case)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def permuted(case, perm):
    """Move physical block j to perm[j] and remap the table accordingly."""
    out = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    out.k_cache = case.k_cache[inv]
    out.v_cache = case.v_cache[inv]
    t = case.block_tables.copy()
    t[t >= 0] = perm[t[t >= 0]]
    out.block_tables = t
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_block_permutation_invariance(oracle_mod, seed):
    case = pi.make_case(3, [50, 17, 64], 8, 2, 16, 16, seed=seed, pool=12)
    ref = run(oracle_mod, case)
    perm = np.random.default_rng(100 + seed).permutation(12).astype(np.int32)
    got = run(oracle_mod, permuted(case, perm))
    assert np.array_equal(got, ref)


def test_all_permutations_of_four_block_pool(oracle_mod):
    case = pi.make_case(1, 61, 4, 2, 8, 16, seed=5, pool=4, table="identity")
    ref = run(oracle_mod, case)
    sd = sdpa_identity(case)
    assert np.abs(ref - sd).max() <= 1e-12
    for perm in itertools.permutations(range(4)):
        got = run(oracle_mod, permuted(case, np.array(perm, dtype=np.int32)))
        assert np.array_equal(got, ref)


def test_context_len_one_returns_v_row(oracle_mod):
    case = pi.make_case(3, [1, 1, 1], 8, 4, 16, 16, seed=2, pool=9, max_blocks=3)
    out = run(oracle_mod, case)
    for b in range(3):
        blk = case.block_tables[b, 0]
        for h in range(8):
            assert np.array_equal(out[b, h], case.v_cache[blk, 0, h // 2].astype(np.float64))


def test_two_tokens_closed_form(oracle_mod):
    # d = 2, one head: q = (1, 0), K0 = (2, 0), K1 = (0, 0), scale 1
    # s = (2, 0): out = sigma(2) V0 + sigma(-2) V1
    case = pi.make_case(1, 2, 1, 1, 2, 2, dtype="f32", seed=0, pool=1)
    case.q[:] = [[[1.0, 0.0]]]
    case.k_cache[:] = 0.0
    case.k_cache[0, 0, 0] = [2.0, 0.0]
    case.v_cache[0, 0, 0] = [1.0, -3.0]
    case.v_cache[0, 1, 0] = [5.0, 7.0]
    case.scale = np.float32(1.0)
    out = run(oracle_mod, case)
    w0 = math.exp(2) / (math.exp(2) + 1.0)
    w1 = 1.0 / (math.exp(2) + 1.0)
    expect = [w0 * 1.0 + w1 * 5.0, w0 * -3.0 + w1 * 7.0]
    assert np.abs(out[0, 0] - expect).max() <= 1e-15


def live_rows(case, b, kvh, which):
    """Rows of the live tokens of sequence b (positions via the lookup rule)."""
    cache = case.k_cache if which == "k" else case.v_cache
    rows = []
    for t in range(int(case.context_lens[b])):
        blk = case.block_tables[b, t // case.block_size]
        if blk >= 0:
            rows.append(cache[blk, t % case.block_size, kvh].astype(np.float64))
    return np.array(rows)


def test_scale_zero_gives_mean_of_v(oracle_mod):
    case = pi.make_case(2, [45, 9], 4, 2, 8, 16, seed=4, pool=6)
    case.scale = np.float32(0.0)
    out = run(oracle_mod, case)
    for b in range(2):
        for h in range(4):
            mean = live_rows(case, b, h // 2, "v").mean(axis=0)
            assert np.abs(out[b, h] - mean).max() <= 1e-14


def test_identical_keys_give_mean_of_v(oracle_mod):
    case = pi.make_case(1, 70, 4, 1, 8, 16, seed=6, pool=5)
    case.k_cache[:] = case.k_cache[0, 0, 0]
    out = run(oracle_mod, case)
    mean = live_rows(case, 0, 0, "v").mean(axis=0)
    for h in range(4):
        assert np.abs(out[0, h] - mean).max() <= 1e-14


def test_dominant_key_selects_its_value(oracle_mod):
    case = pi.make_case(1, 48, 2, 1, 8, 16, seed=8, pool=3, dtype="f32")
    j = 29
    blk = case.block_tables[0, j // 16]
    kj = case.k_cache[blk, j % 16, 0]
    case.q[0, :] = 60.0 * kj / np.linalg.norm(kj)
    case.k_cache[:] *= 0.01
    case.k_cache[blk, j % 16, 0] = kj / np.linalg.norm(kj) * 10.0
    out = run(oracle_mod, case)
    vj = case.v_cache[blk, j % 16, 0]
    assert np.abs(out[0] - vj).max() <= 1e-9


def test_gqa_mapping_constant_v(oracle_mod):
    # V = kv-head index everywhere: every output element equals h // (H / Hkv)
    # (up to the rounding of the softmax weights' sum)
    for H, Hkv in [(8, 2), (8, 4), (8, 8), (6, 3), (8, 1)]:
        case = pi.make_case(2, [20, 7], H, Hkv, 4, 4, seed=9, pool=8)
        for kvh in range(Hkv):
            case.v_cache[:, :, kvh, :] = kvh
        out = run(oracle_mod, case)
        for h in range(H):
            assert np.abs(out[:, h] - h // (H // Hkv)).max() <= 1e-14, (H, Hkv, h)


def test_nan_in_dead_slots_is_never_read(oracle_mod):
    case = pi.make_case(3, [37, 16, 3], 4, 2, 8, 16, seed=12, pool=9, max_blocks=3)
    ref = run(oracle_mod, case)
    got = run(oracle_mod, pi.poison_unused(case))
    assert np.array_equal(ref, got)


def test_hole_equals_removed_tokens(oracle_mod):
    # a -1 entry inside the context removes that block's tokens from the softmax:
    # the same result as a sequence that never had them
    case = pi.make_case(1, 64, 4, 2, 8, 16, seed=13, pool=4, holes=[(0, 1)])
    got = run(oracle_mod, case)
    compact = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
    t = case.block_tables[0]
    compact.block_tables = np.array([[t[0], t[2], t[3]]], dtype=np.int32)
    compact.context_lens = np.array([48], dtype=np.int32)
    ref = run(oracle_mod, compact)
    assert np.array_equal(got, ref)


def test_empty_live_set_gives_zeros(oracle_mod):
    case = pi.make_case(3, [0, 20, 16], 4, 2, 8, 16, seed=14, pool=4, max_blocks=2,
                        holes=[(2, 0)])
    out = run(oracle_mod, case)
    assert np.all(out[0] == 0.0) and np.all(out[2] == 0.0)
    assert np.all(np.isfinite(out[1])) and np.any(out[1] != 0.0)


def test_convexity(oracle_mod):
    case = pi.make_case(2, [100, 35], 8, 2, 16, 16, seed=15, pool=12)
    out = run(oracle_mod, case)
    for b in range(2):
        for h in range(8):
            v = live_rows(case, b, h // 4, "v")
            assert np.all(out[b, h] >= v.min(axis=0) - 1e-15)
            assert np.all(out[b, h] <= v.max(axis=0) + 1e-15)


def test_common_key_offset_cancels(oracle_mod):
    # adding the same vector u to every key adds scale*q.u to every score of a
    # head, which the softmax cancels
    case = pi.make_case(1, 40, 4, 2, 8, 16, seed=16, pool=3, dtype="f32")
    ref = run(oracle_mod, case)
    shifted = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
    u = np.random.default_rng(0).standard_normal(8).astype(np.float32)
    shifted.k_cache = (case.k_cache + np.float32(0.5) * u).astype(np.float32)
    got = run(oracle_mod, shifted)
    assert np.abs(got - ref).max() <= 1e-5  # the shifted keys were rounded to f32


def test_sequences_are_independent(oracle_mod):
    case = pi.make_case(2, [30, 30], 4, 2, 8, 16, seed=17, pool=4)
    ref = run(oracle_mod, case)
    other = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
    other.q = case.q.copy()
    other.q[1] *= -3.0
    got = run(oracle_mod, other)
    assert np.array_equal(got[0], ref[0]) and not np.array_equal(got[1], ref[1])


@pytest.mark.parametrize("tile", [1, 3, 16, 64, 1000])
def test_one_pass_agrees_with_two_pass(oracle_mod, tile):
    case = pi.make_case(3, [130, 16, 1], 8, 2, 16, 16, seed=18, pool=14,
                        holes=[(0, 3)])
    ref = run(oracle_mod, case)
    got = oracle_mod.decode_case_online(case, tile)
    assert np.abs(got - ref).max() <= 1e-12


@pytest.mark.parametrize("parts", [1, 2, 3, 5, 9, 20])
def test_split_merge_agrees_with_two_pass(oracle_mod, parts):
    case = pi.make_case(3, [130, 16, 0], 8, 2, 16, 16, seed=19, pool=14, max_blocks=9,
                        holes=[(0, 3)])
    ref = run(oracle_mod, case)
    got = oracle_mod.decode_case_split(case, parts)
    assert np.abs(got - ref).max() <= 1e-12


def test_threads_do_not_change_result(oracle_mod):
    case = pi.make_case(4, [99, 3, 64, 17], 8, 4, 16, 16, seed=20, pool=16)
    a = oracle_mod.decode_case(case, threads=1)
    b = oracle_mod.decode_case(case, threads=4)
    assert np.array_equal(a, b)


def test_rejects_invalid_input(oracle_mod):
    case = pi.make_case(1, 20, 4, 2, 8, 16, seed=0, pool=2)
    bad = pi.Case(**{f: getattr(case, f) for f in case.__dataclass_fields__})
    bad.context_lens = np.array([33], dtype=np.int32)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.decode_case(bad)
    bad.context_lens = np.array([20], dtype=np.int32)
    bad.block_tables = np.array([[0, 2]], dtype=np.int32)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.decode_case(bad)
    bad.block_tables = np.array([[0, -2]], dtype=np.int32)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.decode_case(bad)
