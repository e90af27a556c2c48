"""The native packer (tree_pack, tree_request_cost, tree_form_batches) against
the oracle (oracle/packing.py): exact rows, tokens and readouts; then the
packed rows planned and checked against the prompts they came from."""
import numpy as np
import pytest

from oracle import packing as OP
from oracle import tree as OT
from workloads import configs as W

P = pytest.importorskip("prefix_tree_packed_amd")
from prefix_tree_packed_amd import binding as B  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libtreeattn.so not built")
    return B.load_library()


def _flat(rows, toks, place):
    """Oracle output in the native export's layout."""
    indptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    parent = np.array([p for r in rows for p, _ in r], np.int32)
    length = np.array([n for r in rows for _, n in r], np.int32)
    return indptr, parent, length, np.array([t for r in toks for t in r], np.int32), \
        np.array(place, np.int32).reshape(-1, 3)


def _check_same(native, prompts, parts=None, **kw):
    rows, toks, place = OP.pack(prompts, parts, **kw)
    indptr, parent, length, rt, pl = _flat(rows, toks, place)
    np.testing.assert_array_equal(native["row_block_indptr"], indptr)
    np.testing.assert_array_equal(native["block_parent"], parent)
    np.testing.assert_array_equal(native["block_len"], length)
    np.testing.assert_array_equal(native["row_tokens"], rt)
    np.testing.assert_array_equal(np.stack([native["prompt_row"], native["prompt_block"],
                                            native["prompt_readout"]], 1), pl)
    assert native["separate_tokens"] == sum(len(p) for p in prompts)


def _example(rng):
    parts = lambda n: list(rng.integers(0, 32000, n))  # noqa: E731
    t, s = parts(53), parts(120)
    prompts = []
    for _ in range(3):
        q = parts(24)
        for _ in range(2):
            prompts.append(t + s + q + parts(18))
    return prompts


def test_pages_example(lib):
    prompts = _example(np.random.default_rng(0))
    parts = [[53, 120, 24, 18]] * 6
    native = P.tree_pack(prompts, parts)
    _check_same(native, prompts, parts)
    assert list(native["block_len"]) == [53, 120, 24, 18, 18, 24, 18, 18, 24, 18, 18]
    assert P.tree_request_cost(prompts, cached_prefix=53) == 300
    assert P.tree_request_cost(prompts) == 353


def _random(rng, n, with_parts):
    base = [list(rng.integers(0, 50, int(rng.integers(1, 30)))) for _ in range(4)]
    prompts, parts = [], []
    for _ in range(n):
        p = list(base[int(rng.integers(0, 4))])
        q = [len(p)]
        for _ in range(int(rng.integers(0, 4))):
            ext = list(rng.integers(0, 6, int(rng.integers(1, 9))))  # small alphabet: many shared runs
            p += ext
            q.append(len(ext))
        prompts.append(p)
        parts.append(q)
    for _ in range(3):
        k = int(rng.integers(0, n))
        prompts.append(list(prompts[k]))
        parts.append(list(parts[k]))
    return prompts, (parts if with_parts else None)


@pytest.mark.parametrize("with_parts", [False, True])
@pytest.mark.parametrize("seed", range(8))
def test_random_prompt_sets(lib, seed, with_parts):
    rng = np.random.default_rng(seed)
    prompts, parts = _random(rng, 40, with_parts)
    _check_same(P.tree_pack(prompts, parts), prompts, parts)
    # tight limits: several rows, shallow trees
    kw = dict(max_row_tokens=int(rng.integers(60, 150)), max_depth=int(rng.integers(2, 5)))
    ok = True
    try:
        OP.pack(prompts, parts, **kw)
    except ValueError:
        ok = False
    if ok:
        _check_same(P.tree_pack(prompts, parts, **kw), prompts, parts, **kw)
    else:
        with pytest.raises(P.TreeAttnError):
            P.tree_pack(prompts, parts, **kw)
    for cp in (0, 3):
        assert P.tree_request_cost(prompts, cp) == OP.request_cost(prompts, cp)


def test_batches(lib):
    rng = np.random.default_rng(3)
    for _ in range(20):
        costs = list(rng.integers(1, 5000, int(rng.integers(0, 30))))
        np.testing.assert_array_equal(P.tree_form_batches(costs, 8192), OP.form_batches(costs, 8192))
    assert list(P.tree_form_batches([5000, 4000, 3000, 100, 8000])) == [0, 1, 0, 0, 2]
    with pytest.raises(P.TreeAttnError):
        P.tree_form_batches([1, -2])


def test_errors(lib):
    with pytest.raises(P.TreeAttnError):
        P.tree_pack([[1, 2], []])
    with pytest.raises(P.TreeAttnError):
        P.tree_pack([[1, 2, 3]], [[1, 1]])          # parts do not split the prompt
    with pytest.raises(P.TreeAttnError):
        P.tree_pack([list(range(100))], max_row_tokens=50)
    with pytest.raises(P.TreeAttnError):
        P.tree_pack([[1]], max_depth=0)


def test_packed_rows_plan_like_the_prompts(lib):
    """The packed description plans cleanly; every prompt's root-to-readout path
    holds its tokens; its readout's position id is its length - 1 and it sees
    exactly its own tokens (the oracle's mask over the packed rows)."""
    rng = np.random.default_rng(11)
    prompts, parts = _random(rng, 30, True)
    pk = P.tree_pack(prompts, parts, max_row_tokens=400)
    rows = []
    ip = pk["row_block_indptr"]
    for r in range(len(ip) - 1):
        rows.append([(int(pk["block_parent"][b]), int(pk["block_len"][b])) for b in range(ip[r], ip[r + 1])])
    desc = W.desc_from_rows(rows)
    plan = P.tree_attn_plan(desc, 4, 2, 64, 0.125)
    ex = P.tree_attn_plan_export(plan)
    idx = OT.build_index(desc)
    toks = OT.query_tokens(idx)
    base = np.concatenate([[0], np.cumsum(desc.row_lengths())])
    mask = OT.dense_mask(idx, toks)
    for i, p in enumerate(prompts):
        r, ro = int(pk["prompt_row"][i]), int(pk["prompt_readout"][i])
        t = base[r] + ro                         # one-shot: forward index == row-space index
        assert ex["pos_id"][t] == len(p) - 1
        seen = np.nonzero(mask[t])[0]
        assert len(seen) == len(p)
        np.testing.assert_array_equal(pk["row_tokens"][seen], np.asarray(p, np.int32))


@pytest.mark.parametrize("order", ["grow", "shrink", "mixed"])
@pytest.mark.parametrize("max_depth", [1, 3, 8])
def test_nested_prompts_depth_limit(lib, order, max_depth):
    """Prompts that are prefixes of one another: each either extends the
    deepest path or ends inside an existing block (splitting it), so the depth
    grows by one per prompt and rows close exactly at the depth limit."""
    rng = np.random.default_rng(17)
    seq = list(rng.integers(0, 1000, 120))
    lens = list(range(6, 121, 6))
    if order == "shrink":
        lens = lens[::-1]
    elif order == "mixed":
        lens = list(rng.permutation(lens))
    prompts = [seq[:n] for n in lens]
    parts = [[n // 2, n - n // 2] for n in lens]
    for pp in (None, parts):
        if pp is not None and max_depth < 2:  # two parts: every prompt alone is 2 blocks deep
            with pytest.raises(ValueError):
                OP.pack(prompts, pp, max_depth=max_depth)
            with pytest.raises(P.TreeAttnError):
                P.tree_pack(prompts, pp, max_depth=max_depth)
            continue
        _check_same(P.tree_pack(prompts, pp, max_depth=max_depth), prompts, pp, max_depth=max_depth)

