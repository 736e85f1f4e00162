"""Numbers the pages print, checked against the workloads and the generator."""
import math
import os

import pa_inputs as pi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "docs_page_configs.txt")


def read_golden():
    rows, shared, blocks = [], None, None
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].split()
        if not line:
            continue
        if line[0] == "shared":
            shared = [int(x) for x in line[1:]]
        elif line[0] == "blocks":
            blocks = [int(x) for x in line[1:]]
        else:
            rows.append([int(x) for x in line])
    return rows, shared, blocks


def test_first_four_workloads_are_the_docs_page_table():
    rows, shared, _ = read_golden()
    H, Hkv, d, bs, _warmup = shared
    for cid, (B, seq, _iters) in zip((1, 2, 3, 4), rows):
        c = pi.CONFIGS[cid]
        assert (c["B"], c["ctx"], c["H"], c["Hkv"], c["d"], c["bs"]) == (B, seq, H, Hkv, d, bs)


def test_blocks_per_sequence_example():
    _, _, (seq, bs, nb) = read_golden()
    assert math.ceil(seq / bs) == nb
    case = pi.make_case(1, seq, 4, 2, 8, bs, seed=0)
    assert case.block_tables.shape[1] == nb and (case.block_tables[0] >= 0).sum() == nb
