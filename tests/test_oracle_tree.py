"""Pins of the tree-index oracle against the architecture page's section 03
("Packing") example and section 01 limits, plus identities that two separate
derivations must satisfy. CPU only."""
import json
import os

import numpy as np
import pytest

from oracle import tree as OT
from workloads import configs as W


def _packing(golden_dir, cached=True):
    with open(os.path.join(golden_dir, "packing_example.json")) as f:
        g = json.load(f)
    rows = [[(b["parent"], b["len"]) for b in g["blocks"]]]
    total = sum(b["len"] for b in g["blocks"])
    qb = g["cached_prefix_tokens"] if cached else 0
    return g, W.desc_from_rows(rows, [(qb, total)])


def test_packing_example_counts(golden_dir):
    g, desc = _packing(golden_dir)
    idx = OT.build_index(desc)
    packed, separate = OT.costs(idx)
    leaves, _ = OT.leaf_readouts(idx)
    assert len(leaves) == g["printed_prompts"]
    assert separate == g["printed_prompts"] * g["printed_tokens_per_prompt"]  # 1290
    assert packed == 300
    assert round(separate / packed, 1) == g["printed_ratio"]


def test_packing_example_positions(golden_dir):
    """Each prompt is 215 tokens; a token's position is its place in its own
    prompt, so Q1 order 2 holds positions 197..214."""
    g, desc = _packing(golden_dir)
    idx = OT.build_index(desc)
    toks = OT.query_tokens(idx)
    names = [b["name"] for b in g["blocks"]]
    q1o2 = names.index("Q1 order 2")
    pos = toks["pos_id"][toks["tok_block"] == q1o2]
    assert list(pos) == list(range(53 + 120 + 24, 215))
    # every leaf's last token sits at position 215 - 1
    _, readout = OT.leaf_readouts(idx)
    assert set(toks["pos_id"][readout].tolist()) == {g["printed_tokens_per_prompt"] - 1}


def test_packing_example_visibility(golden_dir):
    g, desc = _packing(golden_dir)
    idx = OT.build_index(desc)
    toks = OT.query_tokens(idx)
    names = [b["name"] for b in g["blocks"]]
    q = names.index(g["visibility_example"]["query_block"])
    sel = np.nonzero(toks["tok_block"] == q)[0]
    m = OT.dense_mask(idx, toks, sel)
    seen = g["visibility_example"]["printed_sees"] + g["visibility_example"]["reading_also_sees"]
    for bi, name in enumerate(names):
        s = idx.block_start[bi]
        cols = m[:, s:s + idx.block_len[bi]]
        if name == g["visibility_example"]["query_block"]:
            assert np.array_equal(cols, np.tril(np.ones_like(cols)))  # causal in own block
        elif name in seen:
            assert cols.all(), name
        else:
            assert not cols.any(), name


def _random_descs():
    rng = np.random.default_rng(11)
    out = []
    for _ in range(6):
        rows = W.random_tree_rows(rng, int(rng.integers(60, 400)), int(rng.integers(1, 4)),
                                  min_len=1, max_len=60)
        out.append(W.desc_from_rows(rows))
    out.append(W.make_config(0, 0).forwards[0].tree)
    out.append(W.small_doc_questions(0).forwards[0].tree)
    out += [f.tree for f in W.small_long_row(0).forwards]
    out += [f.tree for f in W.small_requests(0).forwards]
    return out


@pytest.mark.parametrize("k", range(len(_random_descs())))
def test_visible_count_equals_position_plus_one(k):
    """Two derivations: positions from ancestor lengths, visibility from the
    mask. A token in its own prompt sees exactly the pos+1 tokens before and at it."""
    desc = _random_descs()[k]
    idx = OT.build_index(desc)
    toks = OT.query_tokens(idx)
    m = OT.dense_mask(idx, toks)
    np.testing.assert_array_equal(m.sum(axis=1), toks["pos_id"].astype(np.int64) + 1)
    # no attention across rows
    for t in range(len(toks["tok_row"])):
        r = toks["tok_row"][t]
        lo, hi = idx.row_base[r], idx.row_base[r + 1]
        assert not m[t, :lo].any() and not m[t, hi:].any()


def test_mask_from_parent_pointers_brute_force():
    """Mask rebuilt by walking parent pointers token by token."""
    desc = _random_descs()[0]
    idx = OT.build_index(desc)
    toks = OT.query_tokens(idx)
    m = OT.dense_mask(idx, toks)
    indptr = desc.row_block_indptr
    for r in range(desc.num_rows):
        a, b = indptr[r], indptr[r + 1]
        owner = []
        for j in range(a, b):
            owner += [j - a] * int(desc.block_len[j])
        base = idx.row_base[r]
        for i in range(desc.row_q_begin[r], desc.row_q_end[r]):
            t = int(np.nonzero(toks["row_pos"] == base + i)[0][0])
            bi = owner[i]
            anc = set()
            p = int(desc.block_parent[a + bi])
            while p >= 0:
                anc.add(p)
                p = int(desc.block_parent[a + p])
            for j in range(len(owner)):
                want = (owner[j] == bi and j <= i) or owner[j] in anc
                assert m[t, base + j] == want


def test_chunk_tables_are_slices_of_full():
    wl = W.small_long_row(1)
    full = wl.forwards[0].tree.with_q_range([0], [int(wl.forwards[0].tree.row_lengths()[0])])
    tf = OT.query_tokens(OT.build_index(full))
    got = {k: [] for k in tf}
    for f in wl.forwards:
        t = OT.query_tokens(OT.build_index(f.tree))
        for k in t:
            got[k].append(t[k])
    for k in tf:
        np.testing.assert_array_equal(np.concatenate(got[k]), tf[k])


def test_limits():
    chain9 = W.desc_from_rows([[(-1, 4)] + [(i, 4) for i in range(8)]])
    assert OT.limit_violations(OT.build_index(chain9)) == ["depth"]
    chain8 = W.desc_from_rows([[(-1, 4)] + [(i, 4) for i in range(7)]])
    assert OT.limit_violations(OT.build_index(chain8)) == []
    long_row = W.desc_from_rows([[(-1, 32769)]], [(32769 - 10, 32769)])
    assert OT.limit_violations(OT.build_index(long_row)) == ["row"]
    ok_row = W.desc_from_rows([[(-1, 32768)]], [(32768 - 8192, 32768)])
    assert OT.limit_violations(OT.build_index(ok_row)) == []
    fwd = W.desc_from_rows([[(-1, 8193)]])
    assert OT.limit_violations(OT.build_index(fwd)) == ["forward"]


def test_workload_shapes():
    """Generator sanity: the 60-request workload splits into the forwards the
    batch rule gives, and config[1]'s forward is 7168 tokens over a 96-token
    cached template."""
    w2 = W.make_config(2, 0, tensors=False)
    assert [f.tree.num_q_tokens() for f in w2.forwards] == [8066, 8057, 6255]
    w1 = W.make_config(1, 0, tensors=False)
    assert w1.forwards[0].tree.num_q_tokens() == 7168
    assert int(w1.forwards[0].tree.row_lengths()[0]) == 7264
    w3 = W.make_config(3, 0, tensors=False)
    assert [f.tree.num_q_tokens() for f in w3.forwards] == [8192, 8192, 8192, 7168]
