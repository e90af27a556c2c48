"""The C-ABI library on the CPU (no GPU calls): exported symbols, the host plan
bit-exact against the oracle's index tables, the block-sparse schedule
expanded back to the oracle's dense mask, and every error path that is decided
before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import tree as OT
from workloads import configs as W

P = pytest.importorskip("prefix_tree_packed_amd")
from prefix_tree_packed_amd import binding as B  # noqa: E402
from prefix_tree_packed_amd.binding import key_tile_rows  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libtreeattn.so not built")
    return B.load_library()


def test_every_declared_symbol_is_exported(lib):
    with open(os.path.join(ROOT, "include", "tree_attn.h")) as f:
        text = f.read()
    declared = set(re.findall(r"^(?:ta_status|const char\*)\s+(\w+)\s*\(", text, re.M))
    assert {"tree_attn_plan", "tree_attn_forward", "tree_attn_forward_chunked",
            "decision_readout"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(B.EXPORTED) == declared


def _descs():
    out = [("cfg%d" % i, W.make_config(i, 0, tensors=False)) for i in (0, 1, 2, 3, 4)]
    out += [("cfg4s%d" % s, W.make_config(4, s, tensors=False)) for s in (1, 2, 3, 4)]
    out += [("cfg2s1", W.make_config(2, 1, tensors=False))]
    descs = []
    for name, wl in out:
        for j, f in enumerate(wl.forwards):
            descs.append((f"{name}.f{j}", f.tree, wl.hq, wl.hkv, wl.d))
    rng = np.random.default_rng(7)
    for i in range(6):
        rows = W.random_tree_rows(rng, int(rng.integers(50, 600)), int(rng.integers(1, 5)),
                                  min_len=1, max_len=90)
        d = W.desc_from_rows(rows)
        # some rows start later (cached prefix) and stop early
        if i % 2:
            lens = d.row_lengths()
            qb = [int(rng.integers(0, n)) for n in lens]
            qe = [int(rng.integers(b, n + 1)) for b, n in zip(qb, lens)]
            d = d.with_q_range(qb, qe)
        g = [1, 2, 4, 8][i % 4]
        descs.append((f"rand{i}", d, 2 * g, 2, [64, 128][i % 2]))
    # several trees in one row, and single-token blocks
    descs.append(("forest", W.desc_from_rows([[(-1, 3), (0, 1), (-1, 5), (2, 1), (2, 70), (-1, 1)]]),
                  8, 2, 128))
    return descs


DESCS = _descs()


@pytest.mark.parametrize("k", range(len(DESCS)), ids=[d[0] for d in DESCS])
def test_plan_tables_bit_exact(lib, k):
    name, desc, hq, hkv, d = DESCS[k]
    plan = P.tree_attn_plan(desc, hq, hkv, d, d ** -0.5)
    info = plan.info
    ex = P.tree_attn_plan_export(plan)
    idx = OT.build_index(desc)
    toks = OT.query_tokens(idx)
    for key in ("pos_id", "tok_row", "tok_block", "tok_offset"):
        np.testing.assert_array_equal(ex[key], toks[key], err_msg=key)
    lb, lt = OT.leaf_readouts(idx)
    np.testing.assert_array_equal(ex["leaf_block"], lb)
    np.testing.assert_array_equal(ex["leaf_readout_tok"], lt)
    packed, separate = OT.costs(idx)
    assert info["cost_packed"] == packed and info["cost_separate"] == separate
    assert info["num_q_tokens"] == idx.num_q_tokens
    assert info["num_kv_tokens"] == idx.num_kv_tokens
    assert info["useful_pairs"] == int((toks["pos_id"].astype(np.int64) + 1).sum())
    assert info["max_depth"] == max(idx.block_depth)
    assert info["num_leaves"] == len(lb)
    one_shot = all(b == 0 and e == n for b, e, n in zip(idx.row_q_begin, idx.row_q_end, idx.row_len))
    assert info["one_shot"] == int(one_shot)


def _variant(group, head_dim):
    """(waves, column groups) of the kernel variant, as the header states."""
    if head_dim == 128:
        return (8, 2) if group >= 4 else (4, 2 if group == 2 else 1)
    return 4, min(group, 4)


def decode_mask_bits(block, n_tok, group, head_dim):
    """[n_tok, 64] visibility of (query token of the tile, key slot) from one
    tile's block of bits in the documented lane layout; every lane holding the
    same (token, slot) must agree, and every (token, slot) is held by a lane."""
    waves, ncg = _variant(group, head_dim)
    wpl = max(1, ncg // 2)
    assert block.size == waves * 64 * wpl
    v, lane, cg, ks, r = (a.ravel() for a in np.meshgrid(
        np.arange(waves), np.arange(64), np.arange(ncg), np.arange(4), np.arange(4), indexing="ij"))
    e = (4 * ks + r) * ncg + cg
    bit = (block[(64 * v + lane) * wpl + e // 32] >> (e % 32).astype(np.uint32)) & 1
    tok = np.minimum((16 * ncg * v + 16 * cg + lane % 16) // group, n_tok - 1)
    cell = tok * 64 + 16 * ks + 4 * (lane // 16) + r
    held = np.bincount(cell, minlength=n_tok * 64)
    ones = np.bincount(cell, weights=bit, minlength=n_tok * 64)
    assert (held > 0).all(), "every (token, slot) held by some lane"
    assert ((ones == 0) | (ones == held)).all(), "lanes holding one (token, slot) agree"
    return (ones > 0).reshape(n_tok, 64)


def _expand_schedule(plan, idx, toks, block=1024):
    """Apply the kernel's rule to the exported schedule: a tile's query tokens
    see all keys of its unmasked key tiles, and on masked tiles the keys the
    tile's visibility bits allow. The bits are first checked against the rule
    they encode (the tile counts for t, lo <= P(t) < hi, and P(u) <= P(t) <
    E(u); slots past the tile's keys never). Yields (t0, t1, cover): the
    coverage count per (t, u) for the query tokens [t0, t1) of consecutive
    query tiles holding about ``block`` tokens, so long forwards stream.
    After the last block, checks that every query token is in exactly one
    tile and every masked tile has its own block of bits."""
    sch = P.tree_attn_plan_schedule(plan)
    info = plan.info
    masks = P.tree_attn_plan_masks(plan)
    assert masks.shape[1] == info["mask_words_per_tile"]
    assert masks.shape[0] == info["num_masked_key_tiles"] + 1 and not masks[0].any()
    group = plan.cfg["num_q_heads"] // plan.cfg["num_kv_heads"]
    nq, nkv = idx.num_q_tokens, idx.num_kv_tokens
    pre, end = sch["tok_anc"][:, 0], sch["tok_anc"][:, 1]
    seen_q = np.zeros(nq, np.int32)
    blocks = []
    qt = sch["q_tiles"]
    order = np.argsort(qt[:, 0], kind="stable")
    i0 = 0
    while i0 < len(order):
        i1 = i0
        t0 = int(qt[order[i0], 0])
        while i1 < len(order) and (i1 == i0 or int(qt[order[i1], 0]) + int(qt[order[i1], 2]) - t0 <= block):
            i1 += 1
        t1 = int(qt[order[i1 - 1], 0] + qt[order[i1 - 1], 2])
        assert t1 > t0
        cover = np.zeros((t1 - t0, nkv), np.int16)
        for j in order[i0:i1]:
            qf, qr, n, kb, ke = qt[j]
            assert t0 <= qf and qf + n <= t1
            seen_q[qf:qf + n] += 1
            trows = np.arange(qr, qr + n)
            for i in range(kb, ke):
                _, nk, masked, lo, hi, _, _, mblk = sch["key_tiles"][i]
                keys = key_tile_rows(sch, i)
                assert len(keys) == nk
                if masked:
                    pt = pre[trows]
                    rule = ((lo <= pt) & (pt < hi))[:, None] & (pre[keys][None, :] <= pt[:, None]) & \
                        (pt[:, None] < end[keys][None, :])
                    bits = decode_mask_bits(masks[mblk], n, group, plan.cfg["head_dim"])
                    np.testing.assert_array_equal(bits[:, :nk], rule)
                    assert not bits[:, nk:].any(), "slots past the tile's keys are never visible"
                    vis = bits[:, :nk]
                    blocks.append(int(mblk))
                else:
                    assert mblk == 0
                    vis = np.ones((n, nk), bool)
                np.add.at(cover, (slice(qf - t0, qf - t0 + n), keys), vis)
        yield t0, t1, cover
        i0 = i1
    assert np.all(seen_q == 1), "every query token in exactly one tile"
    assert sorted(blocks) == list(range(1, len(blocks) + 1)), "one block per masked tile"


# blocks of a row listed parents-first but not in pre-order (C's subtree sits
# between B's children), so row order alone cannot decide visibility
NON_PREORDER = W.desc_from_rows([[(-1, 4), (0, 3), (0, 5), (1, 2), (2, 1), (1, 6)],
                                 [(-1, 2), (0, 1), (0, 3), (1, 2), (2, 2), (3, 1)]])


@pytest.mark.parametrize("k", range(len(DESCS) + 1),
                         ids=[d[0] for d in DESCS] + ["non-preorder"])
def test_token_order_encodes_visibility(lib, k):
    """The exported per-token (P, E) decide visibility for every (query, key)
    pair, keys outside any schedule included: P(u) <= P(t) < E(u) equals the
    oracle's ancestor-or-own-prefix mask."""
    if k < len(DESCS):
        name, desc, hq, hkv, d = DESCS[k]
    else:
        desc, hq, hkv, d = NON_PREORDER, 4, 2, 64
    idx = OT.build_index(desc)
    plan = P.tree_attn_plan(desc, hq, hkv, d, d ** -0.5)
    toks = OT.query_tokens(idx)
    pre, end = P.tree_attn_plan_schedule(plan)["tok_anc"].T
    for a in range(0, idx.num_q_tokens, 1024):   # query blocks: the long rows stream
        part = np.arange(a, min(a + 1024, idx.num_q_tokens))
        tpos = pre[toks["row_pos"][part]]
        enc = (pre[None, :] <= tpos[:, None]) & (tpos[:, None] < end[None, :])
        np.testing.assert_array_equal(enc, OT.dense_mask(idx, toks, part))


@pytest.mark.parametrize("inv", [False, True], ids=["union", "by-position"])
@pytest.mark.parametrize("k", range(len(DESCS)), ids=[d[0] for d in DESCS])
def test_schedule_covers_mask_exactly_once(lib, k, inv):
    name, desc, hq, hkv, d = DESCS[k]
    idx = OT.build_index(desc)
    plan = P.tree_attn_plan(desc, hq, hkv, d, d ** -0.5, batch_invariant=inv)
    toks = OT.query_tokens(idx)
    covered = 0
    for t0, t1, cover in _expand_schedule(plan, idx, toks):
        mask = OT.dense_mask(idx, toks, np.arange(t0, t1))
        np.testing.assert_array_equal(cover, mask.astype(np.int16))
        covered += t1 - t0
    assert covered == idx.num_q_tokens
    sch = P.tree_attn_plan_schedule(plan)
    # unmasked tiles must be full 64-key tiles; tiles never exceed 64 keys
    kt = sch["key_tiles"]
    assert np.all(kt[:, 1] >= 1) and np.all(kt[:, 1] <= 64)
    assert np.all(kt[kt[:, 2] == 0, 1] == 64)
    # the launch order lists every (tile, kv head) once, longest tile first
    w = sch["work"]
    assert sorted(w.tolist()) == list(range(len(sch["q_tiles"]) * hkv))
    assert all(w[i] // hkv == w[i - i % hkv] // hkv for i in range(len(w)))  # heads interleaved
    costs = []
    for x in w[::hkv]:
        kb, ke = sch["q_tiles"][x // hkv][3:5]
        costs.append(float((1.0 + 0.25 * kt[kb:ke, 2]).sum()))  # masked tiles weigh 1.25
    assert costs == sorted(costs, reverse=True)


@pytest.mark.parametrize("k", range(len(DESCS) + 1), ids=[d[0] for d in DESCS] + ["non-preorder"])
def test_tiles_by_prompt_position(lib, k):
    """With batch_invariant the key tiles a query token counts form the same
    sequence whatever shares its forward, row, tree or query tile: tile j holds
    the keys at positions 64j .. 64j+63 of the token's own prompt in that order
    (slot s = position - 64j), one tile per j for j = 0 .. pos // 64, in
    increasing j, and every other tile of its query tile is fully masked for it
    (a fully masked tile adds exact zeros and leaves the running max alone).
    This is what makes the kernel's result depend on the prompt only."""
    if k < len(DESCS):
        name, desc, hq, hkv, d = DESCS[k]
    else:
        desc, hq, hkv, d = NON_PREORDER, 4, 2, 64
    idx = OT.build_index(desc)
    plan = P.tree_attn_plan(desc, hq, hkv, d, d ** -0.5, batch_invariant=True)
    assert plan.info["batch_invariant"] == 1
    sch = P.tree_attn_plan_schedule(plan)
    toks = OT.query_tokens(idx)
    pre, end = sch["tok_anc"][:, 0], sch["tok_anc"][:, 1]
    # prompt position of every row-space key on the path of each block
    nkv = idx.num_kv_tokens
    key_block = np.zeros(nkv, np.int64)
    for g in range(len(idx.block_len)):
        b0 = idx.row_base[idx.block_row[g]] + idx.block_start[g]
        key_block[b0:b0 + idx.block_len[g]] = g
    anc_len = [sum(idx.block_len[a] for a in idx.block_anc[g]) for g in range(len(idx.block_len))]
    rng = np.random.default_rng(k)
    sample = set(rng.choice(idx.num_q_tokens, min(idx.num_q_tokens, 300), replace=False).tolist())
    for qf, qr, n, kb, ke in sch["q_tiles"]:
        for t in range(qf, qf + n):
            if t not in sample:
                continue
            tr = qr + (t - qf)
            blk, pos = int(toks["tok_block"][t]), int(toks["pos_id"][t])
            path = set(idx.block_anc[blk]) | {blk}
            js = []
            for i in range(kb, ke):
                _, nk, masked, lo, hi, _, _, _ = sch["key_tiles"][i]
                keys = key_tile_rows(sch, i)
                counts = not masked or lo <= pre[tr] < hi
                vis = np.ones(nk, bool) if not masked else \
                    (lo <= pre[tr] < hi) & (pre[keys] <= pre[tr]) & (pre[tr] < end[keys])
                if not counts:
                    assert not vis.any()
                    continue
                # a counted tile lies on the token's path at positions 64j + slot
                kbk = key_block[keys]
                assert all(int(g) in path for g in kbk)
                kpos = np.array([anc_len[int(g)] for g in kbk]) + \
                    (keys - np.array([idx.row_base[idx.block_row[int(g)]] + idx.block_start[int(g)] for g in kbk]))
                j = int(kpos[0]) // 64
                np.testing.assert_array_equal(kpos, 64 * j + np.arange(nk))
                np.testing.assert_array_equal(vis, kpos <= pos)
                if vis.any():
                    js.append(j)
            assert js == list(range(pos // 64 + 1)), (t, js)


@pytest.mark.parametrize("k", range(len(DESCS)), ids=[d[0] for d in DESCS])
def test_workgroup_lists(lib, k):
    """The persistent split covers every work item exactly once, keeps the
    longest-first order inside each list, is balanced as longest-processing-
    time packing guarantees (no list exceeds the mean load of its XCD class by
    more than one item; the local search after it only lowers the largest
    load), and keeps each KV head on one XCD class when the counts allow."""
    name, desc, hq, hkv, d = DESCS[k]
    plan = P.tree_attn_plan(desc, hq, hkv, d, d ** -0.5)
    sch = P.tree_attn_plan_schedule(plan)
    work, qt, kt = sch["work"], sch["q_tiles"], sch["key_tiles"]
    cost = {}
    for x in work:
        kb, ke = qt[x // hkv][3:5]
        cost[int(x)] = 1.0 + float((1.0 + 0.25 * kt[kb:ke, 2]).sum())
    rank = {int(x): i for i, x in enumerate(work)}
    for n_wg in sorted({1, 3, 8, 64, 256, len(work), len(work) + 5}):
        wg = P.tree_attn_plan_workgroups(plan, n_wg)
        ptr, items = wg["wg_ptr"], wg["wg_items"]
        assert ptr[0] == 0 and ptr[-1] == len(work) and np.all(np.diff(ptr) >= 0)
        assert sorted(items.tolist()) == sorted(work.tolist())
        loads = []
        for w in range(n_wg):
            lst = [int(x) for x in items[ptr[w]:ptr[w + 1]]]
            assert [rank[x] for x in lst] == sorted(rank[x] for x in lst)
            loads.append(sum(cost[x] for x in lst))
            if hkv % 8 == 0 and n_wg % 8 == 0:
                assert all((x % hkv) % 8 == w % 8 for x in lst)
        if not (hkv % 8 == 0 and n_wg % 8 == 0):
            assert max(loads) <= sum(loads) / n_wg + max(cost.values()) + 1e-9
        else:
            for c in range(8):
                cls = loads[c::8]
                assert max(cls) <= sum(cls) / len(cls) + max(cost.values()) + 1e-9
    # argument checks
    for bad in (0, -1, 8193):
        with pytest.raises(P.TreeAttnError):
            P.tree_attn_plan_workgroups(plan, bad)
    for bad in (-1, 8193):
        with pytest.raises(P.TreeAttnError):
            P.tree_attn_plan_set_max_workgroups(plan, bad)
    P.tree_attn_plan_set_max_workgroups(plan, 0)
    P.tree_attn_plan_set_max_workgroups(plan, 8192)


def test_long_row_chunks_schedule_rows(lib):
    """For the 32k-token row's chunks check coverage on sampled query tokens."""
    wl = W.make_config(3, 0, tensors=False)
    rng = np.random.default_rng(0)
    for f in wl.forwards:
        desc = f.tree
        idx = OT.build_index(desc)
        toks = OT.query_tokens(idx)
        plan = P.tree_attn_plan(desc, wl.hq, wl.hkv, wl.d, wl.d ** -0.5)
        sch = P.tree_attn_plan_schedule(plan)
        pre, end = sch["tok_anc"][:, 0], sch["tok_anc"][:, 1]
        picks = set(rng.integers(0, idx.num_q_tokens, 24).tolist())
        for qf, qr, n, kb, ke in sch["q_tiles"]:
            for t in range(qf, qf + n):
                if t not in picks:
                    continue
                tr = qr + (t - qf)
                row = np.zeros(idx.num_kv_tokens, np.int16)
                for i in range(kb, ke):
                    _, nk, masked, lo, hi, _, _, _ = sch["key_tiles"][i]
                    keys = key_tile_rows(sch, i)
                    if masked:
                        vis = (lo <= pre[tr] < hi) & (pre[keys] <= pre[tr]) & (pre[tr] < end[keys])
                    else:
                        vis = np.ones(nk, bool)
                    np.add.at(row, keys, vis)
                want = OT.dense_mask(idx, toks, [t])[0]
                np.testing.assert_array_equal(row, want.astype(np.int16))


# ---------------------------------------------------------------------------
# error paths (decided on the host before any launch)
# ---------------------------------------------------------------------------

def _err(fn, *a, **kw):
    with pytest.raises(B.TreeAttnError) as ei:
        fn(*a, **kw)
    return ei.value.status


def test_limits_and_invalid_trees(lib):
    ok = W.desc_from_rows([[(-1, 4), (0, 4)]])
    assert P.tree_attn_plan(ok, 4, 1, 64, 0.1).info["num_q_tokens"] == 8
    chain9 = W.desc_from_rows([[(-1, 2)] + [(i, 2) for i in range(8)]])
    assert _err(P.tree_attn_plan, chain9, 4, 1, 64, 0.1) == 3
    chain8 = W.desc_from_rows([[(-1, 2)] + [(i, 2) for i in range(7)]])
    assert P.tree_attn_plan(chain8, 4, 1, 64, 0.1).info["max_depth"] == 8
    row = W.desc_from_rows([[(-1, 32769)]], [(32769 - 8, 32769)])
    assert _err(P.tree_attn_plan, row, 4, 1, 64, 0.1) == 3
    row_ok = W.desc_from_rows([[(-1, 32768)]], [(32768 - 8192, 32768)])
    assert P.tree_attn_plan(row_ok, 4, 1, 64, 0.1).info["num_q_tokens"] == 8192
    fwd = W.desc_from_rows([[(-1, 8193)]])
    assert _err(P.tree_attn_plan, fwd, 4, 1, 64, 0.1) == 3
    two_rows = W.desc_from_rows([[(-1, 4096)], [(-1, 4097)]])
    assert _err(P.tree_attn_plan, two_rows, 4, 1, 64, 0.1) == 3
    bad_parent = W.desc_from_rows([[(-1, 4), (1, 4)]])
    assert _err(P.tree_attn_plan, bad_parent, 4, 1, 64, 0.1) == 2
    bad_parent2 = W.desc_from_rows([[(-1, 4), (-2, 4)]])
    assert _err(P.tree_attn_plan, bad_parent2, 4, 1, 64, 0.1) == 2
    zero_len = W.desc_from_rows([[(-1, 4), (0, 0)]])
    assert _err(P.tree_attn_plan, zero_len, 4, 1, 64, 0.1) == 2
    empty_row = W.TreeDesc(np.array([0, 1, 1], np.int32), np.array([-1], np.int32),
                           np.array([3], np.int32), np.array([0, 0], np.int32),
                           np.array([3, 0], np.int32))
    assert _err(P.tree_attn_plan, empty_row, 4, 1, 64, 0.1) == 2
    bad_span = ok.with_q_range([5], [3])
    assert _err(P.tree_attn_plan, bad_span, 4, 1, 64, 0.1) == 1
    bad_span2 = ok.with_q_range([0], [9])
    assert _err(P.tree_attn_plan, bad_span2, 4, 1, 64, 0.1) == 1
    # the row space (all rows' tokens, cached ones included) stays below 2^26:
    # 2048 full rows reach it, one query token each
    n_rows = (1 << 26) // 32768
    big = W.TreeDesc(np.arange(n_rows + 1, dtype=np.int32), np.full(n_rows, -1, np.int32),
                     np.full(n_rows, 32768, np.int32), np.full(n_rows, 32767, np.int32),
                     np.full(n_rows, 32768, np.int32))
    assert _err(P.tree_attn_plan, big, 4, 1, 64, 0.1) == 3


def test_head_config_errors(lib):
    ok = W.desc_from_rows([[(-1, 4)]])
    assert _err(P.tree_attn_plan, ok, 6, 4, 64, 0.1) == 1      # not a multiple
    assert _err(P.tree_attn_plan, ok, 48, 3, 64, 0.1) == 3     # 16 heads per KV head
    assert _err(P.tree_attn_plan, ok, 3, 1, 64, 0.1) == 3      # 3 heads per KV head
    assert _err(P.tree_attn_plan, ok, 4, 1, 96, 0.1) == 3      # head_dim
    assert _err(P.tree_attn_plan, ok, 4, 1, 64, 0.0) == 1      # scale
    assert _err(P.tree_attn_plan, ok, 4, 1, 64, float("nan")) == 1
    assert _err(P.tree_attn_plan, ok, 0, 1, 64, 0.1) == 1
    # in-row key offsets are 32-bit: num_kv_heads * head_dim * 32768 < 2^31
    assert _err(P.tree_attn_plan, ok, 512, 512, 128, 0.1) == 3
    assert P.tree_attn_plan(ok, 511, 511, 128, 0.1).info["num_q_tokens"] == 4


def test_binding_rejects_short_tree_arrays(lib):
    """The C planner indexes the block arrays up to row_block_indptr[-1] and the
    per-row arrays up to num_rows; the binding refuses shorter arrays."""
    ok = W.desc_from_rows([[(-1, 4), (0, 4)], [(-1, 3)]])
    short_parent = W.TreeDesc(ok.row_block_indptr, ok.block_parent[:-1], ok.block_len,
                              ok.row_q_begin, ok.row_q_end)
    short_len = W.TreeDesc(ok.row_block_indptr, ok.block_parent, ok.block_len[:-1],
                           ok.row_q_begin, ok.row_q_end)
    short_qb = W.TreeDesc(ok.row_block_indptr, ok.block_parent, ok.block_len,
                          ok.row_q_begin[:-1], ok.row_q_end)
    short_qe = W.TreeDesc(ok.row_block_indptr, ok.block_parent, ok.block_len,
                          ok.row_q_begin, ok.row_q_end[:-1])
    decreasing = W.TreeDesc(np.array([0, 2, 1], np.int32), ok.block_parent[:1], ok.block_len[:1],
                            ok.row_q_begin, ok.row_q_end)
    for bad in (short_parent, short_len, short_qb, short_qe, decreasing):
        with pytest.raises(ValueError):
            P.tree_attn_plan(bad, 4, 1, 64, 0.1)
    assert P.tree_attn_plan(ok, 4, 1, 64, 0.1).info["num_q_tokens"] == 11


def test_forward_needs_upload_and_checks_pointers(lib):
    """Argument errors return before anything touches a device."""
    desc = W.desc_from_rows([[(-1, 40), (0, 9)]])
    plan = P.tree_attn_plan(desc, 4, 2, 64, 0.125)
    fake = ctypes.c_void_p(4096)
    st = lib.tree_attn_forward(plan.handle, fake, fake, fake, fake, None, None)
    assert st == 5  # not uploaded
    st = lib.tree_attn_forward_chunked(plan.handle, fake, fake, fake, fake, fake, 49, fake, None, None)
    assert st == 5
    assert lib.tree_attn_plan_upload(plan.handle, None, 1 << 20, None) == 1
    assert lib.tree_attn_plan_upload(plan.handle, ctypes.c_void_p(4096), 16, None) == 5
    assert lib.tree_attn_plan_upload(plan.handle, ctypes.c_void_p(4096 + 8), 1 << 20, None) == 5
    assert "aligned" in P.tree_attn_last_error()
    assert lib.decision_readout(fake, 4, 1, fake, fake, fake, fake, 2, fake, fake, None) == 1
    assert lib.decision_readout(None, 4, 4, fake, fake, fake, fake, 2, fake, fake, None) == 1
    assert lib.decision_readout(fake, 0, 4, fake, fake, fake, fake, 2, fake, fake, None) == 1
    assert lib.decision_readout(fake, 4, 4, fake, fake, fake, fake, -1, fake, fake, None) == 1
    assert lib.decision_readout(None, 0, 0, None, None, None, None, 0, None, None, None) == 0


def test_empty_forward(lib):
    desc = W.desc_from_rows([[(-1, 40)]], [(40, 40)])
    plan = P.tree_attn_plan(desc, 4, 2, 64, 0.125)
    assert plan.info["num_q_tokens"] == 0 and plan.info["num_work_items"] == 0
    # nothing to compute: returns OK without touching the (null) buffers
    assert lib.tree_attn_forward_chunked(plan.handle, None, None, None, None, None, 0, None, None,
                                         None) == 0
    empty = W.TreeDesc(np.array([0], np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32),
                       np.zeros(0, np.int32), np.zeros(0, np.int32))
    plan0 = P.tree_attn_plan(empty, 4, 2, 64, 0.125)
    assert plan0.info["num_q_tokens"] == 0 and plan0.info["num_kv_tokens"] == 0
