"""The seeded generator: determinism, bf16 and fp16 rounding, table structure,
poisoning."""
import math

import numpy as np
import pytest
import torch

import pa_inputs as pi


def test_same_seed_same_bytes():
    a = pi.make_case(2, [30, 17], 4, 2, 8, 4, seed=7, pool=20)
    b = pi.make_case(2, [30, 17], 4, 2, 8, 4, seed=7, pool=20)
    for x, y in [(a.q_bits, b.q_bits), (a.k_bits, b.k_bits), (a.v_bits, b.v_bits),
                 (a.block_tables, b.block_tables), (a.context_lens, b.context_lens)]:
        assert np.array_equal(x, y)
    c = pi.make_case(2, [30, 17], 4, 2, 8, 4, seed=8, pool=20)
    assert not np.array_equal(a.k_bits, c.k_bits)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.0e38, -3.0e38, 1e-40,
                                  np.inf, -np.inf], dtype=np.float32)])
    # ties: values whose low 16 bits are exactly 0x8000
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ours = pi.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = pi.bf16_bits_to_f32(ours)
    ref_back = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(back.view(np.uint32), ref_back.view(np.uint32))


def test_f16_rounding_is_nearest_even():
    # IEEE binary16 keeps 10 fraction bits: the spacing just above 1 is 2^-10.
    # 1 + 2^-11 lies halfway between 1 and 1 + 2^-10 and goes to the even 1;
    # 1 + 3 * 2^-11 lies halfway between 1 + 2^-10 and 1 + 2^-9 and goes to the
    # even 1 + 2^-9; just above a halfway point goes up.
    x = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -20,
                  65504.0, 65520.0, 2.0 ** -24, 2.0 ** -26], dtype=np.float32)
    bits = pi.f16_round_bits(x)
    assert bits.tolist() == [0x3C00, 0x3C02, 0x3C01, 0x7BFF, 0x7C00, 0x0001, 0x0000]
    rng = np.random.default_rng(0)
    y = rng.standard_normal(100000).astype(np.float32) * 10
    ours = pi.f16_round_bits(y)
    ref = torch.from_numpy(y).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = pi.f16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(y).to(torch.float16).float().numpy())
    # the rounded value is a nearest binary16 neighbour: within half a spacing
    spacing = np.spacing(np.abs(back).astype(np.float16)).astype(np.float32)
    assert (np.abs(back - y) <= spacing / 2).all()


def test_f16_case_holds_rounded_values():
    case = pi.make_case(2, [20, 5], 4, 2, 8, 16, dtype="f16", seed=3, pool=4)
    assert case.elem_bytes == 2 and case.storage("k") is case.k_bits
    assert np.array_equal(case.k_cache, pi.f16_bits_to_f32(case.k_bits))
    ref = pi.make_case(2, [20, 5], 4, 2, 8, 16, dtype="f32", seed=3, pool=4)
    assert np.array_equal(case.k_bits, pi.f16_round_bits(ref.k_cache))
    assert np.array_equal(case.block_tables, ref.block_tables)
    p = pi.poison_unused(case)
    assert (p.k_bits == pi.F16_NAN_BITS).any() and np.isnan(p.k_cache).any()


def test_nan_rounds_to_nan():
    bits = pi.bf16_round_bits(np.array([np.nan], dtype=np.float32))
    assert bits[0] == pi.BF16_NAN_BITS
    assert np.isnan(pi.bf16_bits_to_f32(bits))[0]


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_config_shapes(cid):
    c = pi.CONFIGS[cid]
    case = pi.make_config_case(cid)
    nb = math.ceil(c["ctx"] / c["bs"])
    assert case.q.shape == (c["B"], c["H"], c["d"])
    assert case.k_cache.shape == (c["pool"], c["bs"], c["Hkv"], c["d"])
    assert case.block_tables.shape == (c["B"], nb)
    assert (case.context_lens == c["ctx"]).all()
    # every referenced block is distinct and inside the pool: a permutation prefix
    used = case.block_tables[case.block_tables >= 0]
    assert len(np.unique(used)) == used.size == c["B"] * nb
    assert used.max() < c["pool"]
    assert case.scale == np.float32(1.0 / math.sqrt(128))
    assert (case.dtype == "f32") == (cid == 1)


def test_table_is_scattered_not_identity():
    case = pi.make_config_case(3)
    flat = case.block_tables.reshape(-1)
    assert not np.array_equal(flat, np.arange(flat.size))


def test_docs_page_block_count():
    # Docs page, "Benchmark configurations": 512 tokens at block_size 16 need 32
    # blocks and the sequence's table row has 32 entries.
    case = pi.make_config_case(2)
    assert case.block_tables.shape == (1, 32)


def test_algorithmic_bytes_per_config():
    # bytes = live rows * Hkv * d * elem * 2 (K and V) + q + out + table
    expect = {1: 1048608, 2: 2113664, 3: 17040384, 4: 33622016, 5: 67129344}
    for cid, val in expect.items():
        assert pi.make_config_case(cid).algorithmic_bytes() == val


def test_ragged_lengths_and_holes():
    case = pi.make_case(3, [0, 1, 33], 4, 2, 8, 16, seed=1, max_blocks=4, pool=10,
                        holes=[(2, 1)])
    assert (case.block_tables[0] == -1).all()
    assert case.block_tables[1, 0] >= 0 and (case.block_tables[1, 1:] == -1).all()
    assert case.block_tables[2, 0] >= 0 and case.block_tables[2, 1] == -1
    assert case.block_tables[2, 2] >= 0 and case.block_tables[2, 3] == -1


def test_poison_marks_only_dead_slots():
    case = pi.make_case(2, [20, 5], 4, 2, 8, 16, seed=3, max_blocks=3, pool=6)
    p = pi.poison_unused(case)
    for b, n in enumerate(case.context_lens):
        for t in range(n):
            blk = case.block_tables[b, t // 16]
            assert not np.isnan(p.k_cache[blk, t % 16]).any()
            assert np.array_equal(p.k_bits[blk, t % 16], case.k_bits[blk, t % 16])
    assert np.isnan(p.k_cache).any() and np.isnan(p.v_cache).any()
    referenced = set(case.block_tables[case.block_tables >= 0].tolist())
    for blk in range(6):
        if blk not in referenced:
            assert np.isnan(p.v_cache[blk]).all()


def test_identity_table_kind():
    case = pi.make_case(2, 32, 4, 2, 8, 16, seed=0, table="identity")
    assert np.array_equal(case.block_tables, np.arange(4, dtype=np.int32).reshape(2, 2))


def test_bad_arguments():
    with pytest.raises(ValueError):
        pi.make_case(1, 100, 4, 2, 8, 16, max_blocks=2)
    with pytest.raises(ValueError):
        pi.make_case(2, 32, 4, 2, 8, 16, pool=3)
    with pytest.raises(ValueError):
        pi.make_case(1, 16, 4, 2, 8, 16, dtype="f64")
