"""Pins of the dense-mask attention oracle. The architecture page (section 03,
"Attention over tree blocks") fixes that a packed tree must give every token the
result it gets when its full root-to-leaf prompt runs alone; the rest are
textbook special cases, closed forms and scalar brute force. CPU only."""
import math

import numpy as np
import pytest

from oracle import attention as OA
from oracle import tree as OT
from workloads import configs as W


def _causal(q, k, v, scale):
    """Plain causal attention of one prompt, one head: written independently
    of the oracle with an explicit lower-triangular mask."""
    n = q.shape[0]
    s = scale * (q.astype(np.float64) @ k.astype(np.float64).T)
    s[np.triu(np.ones((n, n), bool), 1)] = -np.inf
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p / p.sum(axis=1, keepdims=True)) @ v.astype(np.float64)


def _prompts(desc):
    """Every root-to-leaf prompt as a list of row-local token indices, found by
    walking parent pointers from each leaf."""
    out = []
    for r in range(desc.num_rows):
        a, b = int(desc.row_block_indptr[r]), int(desc.row_block_indptr[r + 1])
        starts, c = [], 0
        for j in range(a, b):
            starts.append(c)
            c += int(desc.block_len[j])
        parents = [int(x) for x in desc.block_parent[a:b]]
        for leaf in range(b - a):
            if leaf in parents:
                continue
            chain = []
            x = leaf
            while x >= 0:
                chain.append(x)
                x = parents[x]
            toks = []
            for blk in reversed(chain):
                toks += list(range(starts[blk], starts[blk] + int(desc.block_len[a + blk])))
            out.append((r, toks))
    return out


def _small_workloads():
    rng = np.random.default_rng(21)
    out = []
    for _ in range(3):
        rows = W.random_tree_rows(rng, int(rng.integers(80, 260)), int(rng.integers(1, 3)),
                                  min_len=1, max_len=50)
        desc = W.desc_from_rows(rows)
        out.append((desc, W.draw_forward(rng, desc, 4, 2, 16)))
    return out


@pytest.mark.parametrize("k", range(3))
def test_packed_equals_separate_prompts(k):
    desc, f = _small_workloads()[k]
    hq, hkv = f.q.shape[1], f.k_row.shape[1]
    scale = 0.37
    o = OA.tree_attention(desc, f.q, f.k_row, f.v_row, scale)
    base = f.row_base()
    # one-shot forward: query index == row-space index
    for r, toks in _prompts(desc):
        rows = [int(base[r]) + t for t in toks]
        for h in range(hq):
            kv = h // (hq // hkv)
            want = _causal(f.q[rows, h], f.k_row[rows, kv], f.v_row[rows, kv], scale)
            np.testing.assert_allclose(o[rows, h], want, rtol=0, atol=1e-12)


def test_single_chain_is_causal_attention():
    rng = np.random.default_rng(3)
    desc = W.desc_from_rows([[(-1, 7), (0, 30), (1, 1), (2, 19)]])
    f = W.draw_forward(rng, desc, 2, 1, 32)
    o = OA.tree_attention(desc, f.q, f.k_row, f.v_row, 0.2)
    for h in range(2):
        want = _causal(f.q[:, h], f.k_row[:, 0], f.v_row[:, 0], 0.2)
        np.testing.assert_allclose(o[:, h], want, rtol=0, atol=1e-12)


def _brute(desc, q, k, v, scale):
    """Scalar loops: visibility re-derived from parent pointers per pair."""
    hq, d = q.shape[1], q.shape[2]
    hkv = k.shape[1]
    g = hq // hkv
    out = np.zeros(q.shape)
    qi = 0
    base = 0
    for r in range(desc.num_rows):
        a, b = int(desc.row_block_indptr[r]), int(desc.row_block_indptr[r + 1])
        owner = []
        for j in range(a, b):
            owner += [j - a] * int(desc.block_len[j])
        parents = [int(x) for x in desc.block_parent[a:b]]

        def sees(i, j):
            if owner[j] == owner[i]:
                return j <= i
            x = parents[owner[i]]
            while x >= 0:
                if x == owner[j]:
                    return True
                x = parents[x]
            return False

        for i in range(int(desc.row_q_begin[r]), int(desc.row_q_end[r])):
            for h in range(hq):
                kv = h // g
                ws, keys = [], []
                for j in range(len(owner)):
                    if sees(i, j):
                        s = sum(float(q[qi, h, c]) * float(k[base + j, kv, c]) for c in range(d))
                        ws.append(scale * s)
                        keys.append(j)
                mx = max(ws)
                es = [math.exp(w - mx) for w in ws]
                z = sum(es)
                for c in range(d):
                    out[qi, h, c] = sum(e * float(v[base + j, kv, c]) for e, j in zip(es, keys)) / z
            qi += 1
        base += len(owner)
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_tiny_trees_with_gqa_and_cached_prefix(seed):
    rng = np.random.default_rng(100 + seed)
    rows = [[(-1, 5), (0, 4), (1, 3), (1, 2), (0, 3)], [(-1, 2), (0, 6), (-1, 3)]]
    desc = W.desc_from_rows(rows, [(3, 17), (0, 11)])  # row 0 has 3 cached tokens
    f = W.draw_forward(rng, desc, 4, 2, 8)
    o = OA.tree_attention(desc, f.q, f.k_row, f.v_row, 0.5)
    np.testing.assert_allclose(o, _brute(desc, f.q, f.k_row, f.v_row, 0.5), rtol=0, atol=1e-12)


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(5)
    desc = _small_workloads()[0][0]
    f = W.draw_forward(rng, desc, 4, 2, 16)
    v = np.broadcast_to(np.arange(16, dtype=np.float16)[None, None, :] * 0.25,
                        f.v_row.shape).copy()
    o = OA.tree_attention(desc, f.q, f.k_row, v, 1.3)
    np.testing.assert_allclose(o, np.broadcast_to(v[:1, :1].astype(np.float64), o.shape),
                               rtol=0, atol=1e-12)


def test_zero_queries_average_visible_values():
    """Q = 0 makes every visible score equal: O is the mean of the visible V rows,
    and LSE = ln(number of visible keys)."""
    rng = np.random.default_rng(6)
    desc = _small_workloads()[1][0]
    f = W.draw_forward(rng, desc, 4, 2, 16)
    q = np.zeros_like(f.q)
    o, lse = OA.tree_attention(desc, q, f.k_row, f.v_row, 0.9, return_lse=True)
    idx = OT.build_index(desc)
    toks = OT.query_tokens(idx)
    for t in range(q.shape[0]):
        rng_ = OT.visible_ranges(idx, int(toks["tok_block"][t]), int(toks["tok_offset"][t]))
        rows = np.concatenate([np.arange(lo, hi) for lo, hi in rng_])
        for h in range(4):
            want = f.v_row[rows, h // 2].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(o[t, h], want, rtol=0, atol=1e-12)
            assert abs(lse[h, t] - math.log(len(rows))) < 1e-12


def test_chunked_forwards_equal_one_shot():
    wl = W.small_long_row(2, doc=300, nq=3, chunk=128, hq=4, hkv=2, d=16)
    f0 = wl.forwards[0]
    full = f0.tree.with_q_range([0], [int(f0.tree.row_lengths()[0])])
    q_all = np.concatenate([f.q for f in wl.forwards])
    o_full, l_full = OA.tree_attention(full, q_all, f0.k_row, f0.v_row, wl.scale, return_lse=True)
    a = 0
    for f in wl.forwards:
        o, l = OA.tree_attention(f.tree, f.q, f.k_row, f.v_row, wl.scale, return_lse=True)
        n = f.q.shape[0]
        # equal up to the BLAS's summation order for different matrix shapes
        np.testing.assert_allclose(o, o_full[a:a + n], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, l_full[:, a:a + n], rtol=0, atol=1e-13)
        a += n
    assert a == q_all.shape[0]


def test_cached_template_chain_is_causal_with_prefix():
    """A branch-free row whose first 9 tokens are cached: the forward's tokens
    equal causal attention over the whole row, restricted to them."""
    rng = np.random.default_rng(8)
    desc = W.desc_from_rows([[(-1, 9), (0, 25)]], [(9, 34)])
    f = W.draw_forward(rng, desc, 2, 2, 8)
    o = OA.tree_attention(desc, f.q, f.k_row, f.v_row, 0.4)
    q_full = np.concatenate([np.zeros((9, 2, 8), np.float16), f.q])
    for h in range(2):
        want = _causal(q_full[:, h], f.k_row[:, h], f.v_row[:, h], 0.4)[9:]
        np.testing.assert_allclose(o[:, h], want, rtol=0, atol=1e-12)


def test_useful_pairs_is_sum_of_visible_counts():
    desc = W.make_config(1, 0, tensors=False).forwards[0].tree
    # 7168 forward tokens: every token sees pos+1 keys
    idx = OT.build_index(desc)
    toks = OT.query_tokens(idx)
    assert OA.useful_pairs(desc) == int((toks["pos_id"].astype(np.int64) + 1).sum()) == 13_610_496
