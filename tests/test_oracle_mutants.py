"""Plant plausible mistakes in a copy of the oracle's C source and check that the
pins catch every one of them.

Each mutant is compiled from a text substitution of oracle/pa_oracle.c into a
temporary library and run through a battery of checks that do not use the real
oracle: torch SDPA on identity-table cases, closed forms and invariants, and the
agreement of the three routes (two-pass, one-pass, split).  A mutant passes
unnoticed only if every check passes, which fails this test.  Every mutant keeps
all memory accesses inside the arrays.
"""
import math
import os
import tempfile

import numpy as np
import pytest

import oracle
import pa_inputs as pi

from test_oracle_pins import sdpa_identity, permuted

SRC = os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")

MUTANTS = {
    "kv head h % Hkv": ("int kvh = h / (p->H / p->Hkv);", "int kvh = h % p->Hkv;"),
    "scale dropped": ("return p->scale * dot;", "return dot;"),
    "scale applied twice": ("return p->scale * dot;", "return p->scale * p->scale * dot;"),
    "softmax sign flipped": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "no normalisation": ("double w = s[j] / z;", "double w = s[j];"),
    "q of the kv head": ("const float *qr = p->q + ((size_t)b * p->H + h) * p->d;",
                         "const float *qr = p->q + ((size_t)b * p->H + kvh) * p->d;"),
    "V read from K": ("return row(p, p->v, blk, t % p->bs, kvh);",
                      "return row(p, p->k, blk, t % p->bs, kvh);"),
    "wrong slot": ("const float *kr = row(p, p->k, blk, t % p->bs, kvh);",
                   "const float *kr = row(p, p->k, blk, (t + 1) % p->bs, kvh);"),
    "last token dropped": ("for (int t = 0; t < n; ++t) {\n        int32_t blk",
                           "for (int t = 0; t < n - 1; ++t) {\n        int32_t blk"),
    "logical block index halved": (
        "int32_t blk = p->table[(size_t)b * p->max_blocks + t / p->bs];\n    const float *kr",
        "int32_t blk = p->table[(size_t)b * p->max_blocks + t / p->bs / 2];\n    const float *kr"),
    "online: empty set divides 0/0": ("if (l_i > 0.0)\n        for (int i = 0; i < p->d; ++i) o[i] /= l_i;",
                                      "for (int i = 0; i < p->d; ++i) o[i] /= l_i;"),
    "split: empty set divides 0/0": ("if (M == -INFINITY) return;", ""),
    "online: acc not rescaled": ("for (int i = 0; i < p->d; ++i) o[i] *= alpha;", ""),
    "online: normaliser not rescaled": ("l_i *= alpha;", ""),
    "split: no rescale in merge": ("double f = exp(m_p[q] - M);", "double f = 1.0;"),
    "split: tail partition dropped": ("int bpp = (p->max_blocks + parts - 1) / parts;",
                                      "int bpp = p->max_blocks / parts;"),
}


def identity_case(B, lens, H, Hkv, d, bs, seed, dtype="f32"):
    nb = max(math.ceil(n / bs) for n in lens)
    case = pi.make_case(B, lens, H, Hkv, d, bs, dtype=dtype, seed=seed, table="identity",
                        max_blocks=nb, pool=B * nb)
    t = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    for b, n in enumerate(lens):
        t[b, math.ceil(n / bs):] = -1
    case.block_tables = t
    return case


def battery(lib):
    """Yields (name, passed) for every check."""
    run = lambda c: oracle.decode_case(c, lib=lib)
    for i, (B, lens, H, Hkv, d, bs) in enumerate([
            (2, [37, 20], 8, 2, 8, 16), (1, [9], 4, 4, 4, 4), (3, [5, 16, 33], 4, 1, 8, 8)]):
        c = identity_case(B, lens, H, Hkv, d, bs, seed=30 + i)
        got = run(c)
        yield f"sdpa {i}", bool(np.abs(got - sdpa_identity(c)).max() <= 1e-12)
    c = pi.make_case(2, [20, 7], 8, 2, 4, 4, seed=9, pool=8)
    for kvh in range(2):
        c.v_cache[:, :, kvh, :] = kvh
    out = run(c)
    yield "gqa", all(np.abs(out[:, h] - h // 4).max() <= 1e-14 for h in range(8))
    c = pi.make_case(2, [1, 1], 4, 2, 8, 16, seed=2, pool=4, max_blocks=2)
    out = run(c)
    yield "ctx1", all(np.array_equal(out[b, h], c.v_cache[c.block_tables[b, 0], 0, h // 2])
                      for b in range(2) for h in range(4))
    c = pi.make_case(2, [0, 20], 4, 2, 8, 16, seed=14, pool=4, max_blocks=2)
    out = run(c)
    yield "empty", bool(np.all(out[0] == 0.0))
    c = pi.make_case(2, [50, 17], 4, 2, 8, 16, seed=3, pool=8)
    ref = run(c)
    perm = np.random.default_rng(1).permutation(8).astype(np.int32)
    yield "perm", bool(np.array_equal(run(permuted(c, perm)), ref))
    c = pi.make_case(3, [130, 16, 0], 8, 2, 16, 16, seed=19, pool=14, max_blocks=9)
    ref = run(c)
    for tile in (3, 64):
        got = oracle.decode_case_online(c, tile, lib=lib)
        yield f"online {tile}", bool(np.abs(got - ref).max() <= 1e-12)
    for parts in (2, 4):
        got = oracle.decode_case_split(c, parts, lib=lib)
        yield f"split {parts}", bool(np.abs(got - ref).max() <= 1e-12)


def test_unmutated_source_passes_battery():
    results = dict(battery(oracle.load()))
    assert all(results.values()), results


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    pattern, replacement = MUTANTS[name]
    src = open(SRC).read()
    assert pattern in src, f"mutation site for {name!r} not found"
    mutated = src.replace(pattern, replacement)
    with tempfile.TemporaryDirectory() as tmp:
        c_path = os.path.join(tmp, "mutant.c")
        so_path = os.path.join(tmp, "libmutant.so")
        with open(c_path, "w") as f:
            f.write(mutated)
        oracle.build(c_path, so_path)
        lib = oracle.load(so_path)
        with np.errstate(all="ignore"):
            results = dict(battery(lib))
    caught = [k for k, ok in results.items() if not ok]
    assert caught, f"mutant {name!r} passed every check"
