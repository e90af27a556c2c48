"""The seeded generators against the oracle where a workload's structure uses a
step of the method: config[2]'s forwards are batches formed by the batch rule
(architecture page, section 01 "Batch and prefix tree" and section 04
`max_batch_tokens`: the first queued request plus each later one that fits in
8,192 tokens). The generator's own copy of that rule must agree with the
oracle's (oracle/packing.py, pinned by the page's example in
test_oracle_packing.py) and with the library's tree_form_batches."""
import numpy as np
import pytest

from oracle import packing as OK
from workloads import configs as W


def _as_index(groups, n):
    out = [-1] * n
    for b, grp in enumerate(groups):
        for r in grp:
            assert out[r] == -1, "request in two batches"
            out[r] = b
    return out


def _cases():
    rng = np.random.default_rng(11)
    cases = []
    for seed in range(5):   # config[2]'s own request costs
        reqs = W._config2_requests(np.random.default_rng(seed))
        cases.append(("cfg2-seed%d" % seed, [doc + sum(a + b + c for a, b, c in qs) for doc, qs in reqs],
                      8192))
    for i in range(20):
        n = int(rng.integers(1, 40))
        limit = int(rng.integers(50, 400))
        cases.append(("random%d" % i, rng.integers(0, limit + 60, n).tolist(), limit))
    cases.append(("exact-fit", [4096, 4096, 1, 8192, 0], 8192))
    cases.append(("over-limit-alone", [9000, 10, 9000, 5], 8192))
    cases.append(("empty", [], 8192))
    return cases


CASES = _cases()


@pytest.mark.parametrize("k", range(len(CASES)), ids=[c[0] for c in CASES])
def test_generator_batches_match_oracle(k):
    name, costs, limit = CASES[k]
    want = OK.form_batches(costs, limit)
    got = _as_index(W.form_batches(costs, limit), len(costs))
    assert got == want


def test_config2_forwards_are_the_oracle_batches():
    """Each of config[2]'s forwards holds exactly the requests of one oracle
    batch, in queue order, and their tokens."""
    for seed in range(3):
        wl = W.make_config(2, seed, tensors=False)
        reqs = W._config2_requests(np.random.default_rng(seed))
        costs = [doc + sum(a + b + c for a, b, c in qs) for doc, qs in reqs]
        idx = OK.form_batches(costs, 8192)
        groups = [[r for r in range(len(costs)) if idx[r] == b] for b in range(max(idx) + 1)]
        assert wl.notes["batches"] == groups
        for f, grp in zip(wl.forwards, groups):
            assert f.tree.num_q_tokens() == sum(costs[r] for r in grp) <= 8192


def test_native_batches_match_oracle():
    P = pytest.importorskip("prefix_tree_packed_amd")
    import os
    from prefix_tree_packed_amd import binding as B
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libtreeattn.so not built")
    for name, costs, limit in CASES:
        if not costs:
            continue
        assert P.tree_form_batches(costs, limit).tolist() == OK.form_batches(costs, limit), name
