"""Pins of the work-partition definitions (oracle side, no GPU).

Fixed split rule: hand-worked ranges from the FlashAttention tiling page
(tests/golden/fixed_split_examples.json).  Balanced rule: properties that follow
from its definition - every tile of every request is covered exactly once, parts
differ by at most one tile, a request's chunks are consecutive and in token order,
and a request split in one chunk is flagged to write its final output.
"""
import json
import os

import numpy as np
import pytest

from oracle import plan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_fixed_rule_golden_examples():
    g = json.load(open(os.path.join(GOLDEN, "fixed_split_examples.json")))
    for c in g["cases"]:
        items = plan.fixed_items([c["seq_len"]], c["num_splits"])
        got = []
        for (_b, t0, t1) in items:
            got.append([-(-t0 // 64), -(-t1 // 64)])
        assert got == c["block_ranges"], c


def _check_words(words, seq_lens):
    B = len(seq_lens)
    assert words[0] == plan.MAGIC and words[2] == B
    P, nitems = int(words[3]), int(words[4])
    o = plan.HEADER_WORDS
    part_begin = words[o:o + P + 1]
    chunk_off = words[o + P + 1:o + P + 1 + B + 1]
    items = plan.items_of(words)
    assert part_begin[0] == 0 and part_begin[-1] == nitems
    assert np.all(np.diff(part_begin) >= 0)
    assert chunk_off[0] == 0 and chunk_off[-1] == nitems
    covered = [np.zeros(int(L), np.int32) for L in seq_lens]
    for k, (b, t0, t1, flags) in enumerate(items):
        assert chunk_off[b] <= k < chunk_off[b + 1]
        assert 0 <= t0 <= t1 <= seq_lens[b]
        covered[b][t0:t1] += 1
        n_b = chunk_off[b + 1] - chunk_off[b]
        assert flags == (1 if n_b == 1 else 0)
    for b in range(B):
        assert np.all(covered[b] == 1), b
        ks = range(chunk_off[b], chunk_off[b + 1])
        prev = 0
        for k in ks:                                       # consecutive, in token order
            _bb, t0, t1, _f = items[k]
            assert t0 == prev or t0 == t1 == prev
            prev = t1
    return items, part_begin


@pytest.mark.parametrize("lens,splits", [((100, 257), 1), ((100, 257), 2), ((1536,) * 8, 8),
                                         ((0, 5, 64, 65), 3), ((4096,) * 4, 4)])
def test_fixed_rule_words(lens, splits):
    words = plan.plan_words(lens, splits, 0)
    items, part_begin = _check_words(words, lens)
    assert len(items) == len(lens) * splits
    assert np.array_equal(np.diff(part_begin), np.ones(len(lens) * splits))


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("parts", [1, 7, 64, 300])
def test_balanced_rule_words(seed, parts):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lens = [int(x) for x in rng.integers(0, 5000, size=B)]
    if seed == 0:
        lens[0] = 0
    words = plan.plan_words(lens, 0, parts)
    items, part_begin = _check_words(words, lens)
    # each part's tile count (64-token tiles) is floor or ceil of N / parts
    N = sum(-(-L // 64) for L in lens)
    per_part = []
    for p in range(parts):
        tiles = 0
        for k in range(part_begin[p], part_begin[p + 1]):
            _b, t0, t1, _f = items[k]
            tiles += -(-t1 // 64) - t0 // 64
        per_part.append(tiles)
    assert sum(per_part) == N
    assert max(per_part) - min(per_part) <= 1
    assert len(items) <= parts + B
