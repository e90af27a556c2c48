"""Pins of the packing / batching oracle (oracle/packing.py): the pages'
six-prompt example, round trips, the radix property, row limits, and the
batch rule on a hand-worked queue."""
import json
import os

import numpy as np
import pytest

from oracle import packing as OP


def _parts(rng, n):
    return list(rng.integers(0, 32000, n))


def _example_prompts(rng):
    t, s = _parts(rng, 53), _parts(rng, 120)
    prompts = []
    for _ in range(3):
        q = _parts(rng, 24)
        for _ in range(2):
            prompts.append(t + s + q + _parts(rng, 18))
    return prompts


def test_pages_packing_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "packing_example.json")))
    prompts = _example_prompts(np.random.default_rng(0))
    assert all(len(p) == g["printed_tokens_per_prompt"] for p in prompts)
    assert len(prompts) == g["printed_prompts"]
    parts = [[53, 120, 24, 18]] * 6
    rows, toks, place = OP.pack(prompts, parts)
    assert len(rows) == 1
    assert rows[0] == [(b["parent"], b["len"]) for b in g["blocks"]]
    # without the part boundaries template and state are one block
    assert OP.pack(prompts)[0][0][0] == (-1, 173)
    separate = sum(len(p) for p in prompts)
    packed = OP.request_cost(prompts, cached_prefix=g["cached_prefix_tokens"])
    assert (separate, packed) == (1290, 300)
    assert round(separate / packed, 1) == g["printed_ratio"]
    # each prompt reads out at the last token of its own order block
    assert [b for _, b, _ in place] == [3, 4, 6, 7, 9, 10]


def _path_tokens(rows, toks, r, block):
    starts = np.concatenate([[0], np.cumsum([n for _, n in rows[r]])])
    path = []
    while block >= 0:
        path.append(block)
        block = rows[r][block][0]
    out = []
    for b in reversed(path):
        out += toks[r][starts[b]:starts[b + 1]]
    return out


def _random_prompts(rng, n):
    base = [_parts(rng, int(rng.integers(1, 40))) for _ in range(3)]
    prompts = []
    for _ in range(n):
        p = list(base[int(rng.integers(0, 3))])
        for _ in range(int(rng.integers(0, 4))):
            p += _parts(rng, int(rng.integers(1, 12))) if rng.random() < 0.6 else [7, 7, 7]
        prompts.append(p if p else [1])
    prompts += [list(prompts[int(rng.integers(0, n))]) for _ in range(3)]  # duplicates
    prompts.append(list(prompts[0][:max(1, len(prompts[0]) // 2)]))        # a prefix of another
    return prompts


@pytest.mark.parametrize("seed", range(6))
def test_round_trip_and_radix_property(seed):
    rng = np.random.default_rng(seed)
    prompts = _random_prompts(rng, 20)
    rows, toks, place = OP.pack(prompts)
    ends = set()
    for i, p in enumerate(prompts):
        r, b, last = place[i]
        assert _path_tokens(rows, toks, r, b) == p          # the packed path is the prompt
        starts = np.concatenate([[0], np.cumsum([n for _, n in rows[r]])])
        assert last == starts[b + 1] - 1                      # readout = block's last token
        ends.add((r, b))
    for i, j in [(i, j) for i in range(len(prompts)) for j in range(len(prompts))]:
        if prompts[i] == prompts[j]:
            assert place[i] == place[j]                       # identical prompts share a readout
    for r, row in enumerate(rows):
        kids = [0] * len(row)
        for parent, _ in row:
            if parent >= 0:
                kids[parent] += 1
        for b in range(len(row)):                             # a block ends where something branches or ends
            assert kids[b] != 1 or (r, b) in ends
        for b, (parent, _) in enumerate(row):
            assert parent < b
        firsts = [toks[r][int(np.sum([n for _, n in row[:c]]))] for c in range(len(row)) if row[c][0] == -1]
        assert len(set(firsts)) == len(firsts)               # roots differ in their first token


def test_row_limits():
    rng = np.random.default_rng(9)
    prompts = [_parts(rng, 50) for _ in range(7)]
    rows, _, place = OP.pack(prompts, max_row_tokens=120)
    assert [len(r) for r in rows] == [2, 2, 2, 1]
    assert all(sum(n for _, n in r) <= 120 for r in rows)
    assert [p[0] for p in place] == [0, 0, 1, 1, 2, 2, 3]
    # depth: a chain of prompts, each extending the previous one
    chain = [list(range(k + 1)) for k in range(12)]
    rows, _, _ = OP.pack(chain, max_depth=4)
    for r in rows:
        depth = []
        for parent, _ in r:
            depth.append(1 if parent < 0 else depth[parent] + 1)
        assert max(depth) <= 4
    with pytest.raises(ValueError):
        OP.pack([_parts(rng, 200)], max_row_tokens=120)
    with pytest.raises(ValueError):
        OP.pack([[]])


def test_request_cost_counts_shared_prefixes_once():
    a, b = [1, 2, 3, 4], [1, 2, 9]
    assert OP.request_cost([a]) == 4
    assert OP.request_cost([a, b]) == 5
    assert OP.request_cost([a, b, list(a)]) == 5
    assert OP.request_cost([a, b], cached_prefix=2) == 3


def test_batch_rule_hand_worked():
    """First queued request plus each later one that still fits: with limit
    8192, 5000 takes 3000 and 100 (8100); 4000 cannot take 8000."""
    assert OP.form_batches([5000, 4000, 3000, 100, 8000]) == [0, 1, 0, 0, 2]
    assert OP.form_batches([9000, 10]) == [0, 0 + 1]          # an oversize request forms its own batch
    assert OP.form_batches([]) == []
