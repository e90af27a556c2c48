"""Rotary embedding at tree positions fused with the cache write
(tree_attn_rope_cache_write) against the oracle (oracle/rope.py).

Bar: rotated Q and K within one f16 unit in the last place of the float64
rotation of the same f16 inputs and f32 table, plus the f32 rounding of the
two products and their sum (2^-22 of the pair's magnitude; the kernel rounds
one f32 result to f16); V copied bit-exactly; cache rows outside this forward left
untouched; attention over the rotated Q/K within the attention parity bar.
"""
import numpy as np
import pytest

from oracle import attention as OA
from oracle import rope as OR
from oracle import tree as OT
from workloads import configs as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefix_tree_packed_amd as P
    P.load_library()
    return P


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _ulp16(x):
    """Spacing of f16 numbers at |x| (normal range; subnormal spacing below)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def _bound(x, want, style):
    """One f16 ulp of the exact result plus the f32 rounding of its two
    products and difference, at most 2^-23 (|a| + |b|) for pair (a, b) (taken
    as 2^-22): near a zero result the latter dominates."""
    x = np.abs(np.asarray(x, np.float64))
    f, s = OR.pair_index(x.shape[-1], style)
    mag = np.empty_like(x)
    mag[..., f] = mag[..., s] = x[..., f] + x[..., s]
    return _ulp16(want) + 2.0 ** -22 * mag


def _cases():
    return [
        ("cfg0", lambda: W.make_config(0, 0)),
        ("doc-questions", lambda: W.small_doc_questions(1)),
        ("long-row-chunks", lambda: W.small_long_row(2)),
        ("random-g8", lambda: W.small_random(3, hq=16, hkv=2)),
        ("random-g4-d64", lambda: W.small_random(4, hq=8, hkv=2, d=64)),
    ]


def _rope_forward(P, wl, f, style, tab, in_place=False):
    plan = P.tree_attn_plan(f.tree, wl.hq, wl.hkv, wl.d, wl.scale)
    P.tree_attn_plan_upload(plan)
    kn, vn = f.kv_new()
    kc0, vc0 = f.cache_before()
    q_in = _dev(f.q)
    q_out = q_in if in_place else torch.empty_like(q_in)
    kc, vc = _dev(kc0), _dev(vc0)
    P.tree_attn_rope_cache_write(plan, q_in, q_out, _dev(kn), _dev(vn), _dev(tab), kc, vc, style=style)
    torch.cuda.synchronize()
    return plan, q_out.cpu().numpy(), kc.cpu().numpy(), vc.cpu().numpy()


@pytest.mark.parametrize("style", OR.STYLES)
@pytest.mark.parametrize("case", range(len(_cases())), ids=[c[0] for c in _cases()])
def test_rope_cache_write_matches_oracle(P, case, style):
    name, make = _cases()[case]
    wl = make()
    print(f"[rope] {name} {style}", flush=True)
    for fi, f in enumerate(wl.forwards):
        idx = OT.build_index(f.tree)
        toks = OT.query_tokens(idx)
        tab = OR.table(int(toks["pos_id"].max()) + 1 + 7 * fi, wl.d)
        plan, q_got, kc, vc = _rope_forward(P, wl, f, style, tab, in_place=(fi % 2 == 1))
        kn, vn = f.kv_new()
        q_want = OR.apply(f.q, toks["pos_id"], tab, style)
        k_want = OR.apply(kn, toks["pos_id"], tab, style)
        rows = toks["row_pos"]
        assert np.all(np.abs(q_got.astype(np.float64) - q_want) <= _bound(f.q, q_want, style)), \
            "Q off by more than 1 ulp + f32 rounding"
        assert np.all(np.abs(kc[rows].astype(np.float64) - k_want) <= _bound(kn, k_want, style)), \
            "K off by more than 1 ulp + f32 rounding"
        assert np.array_equal(vc[rows], vn), "V not copied exactly"
        kc0, vc0 = f.cache_before()
        other = np.setdiff1d(np.arange(kc.shape[0]), rows)
        assert np.array_equal(kc[other], kc0[other]) and np.array_equal(vc[other], vc0[other])


@pytest.mark.parametrize("style", OR.STYLES)
def test_tree_positions_equal_separate_prompts(P, style):
    """Rotating a packed tree gives bitwise the same rows as rotating each
    root-to-leaf prompt alone at positions 0 .. len-1 (architecture page,
    section 03: a token's position is its place in its own prompt)."""
    rows = [[(-1, 40), (0, 25), (1, 9), (1, 30), (0, 17), (4, 3)]]
    desc = W.desc_from_rows(rows)
    rng = np.random.default_rng(5)
    hq, hkv, d = 8, 2, 128
    f = W.draw_forward(rng, desc, hq, hkv, d)
    wl = W.Workload("tree", hq, hkv, d, [f], None)
    tab = OR.table(128, d)
    _, q_tree, k_tree, _ = _rope_forward(P, wl, f, style, tab)
    idx = OT.build_index(desc)
    for g in range(len(idx.block_len)):
        if not idx.block_is_leaf[g]:
            continue
        path = idx.block_anc[g] + [g]
        sel = np.concatenate([idx.block_start[b] + np.arange(idx.block_len[b]) for b in path])
        alone = W.desc_from_rows([[(-1, len(sel))]])
        fa = W.Forward(alone, f.q[sel], f.k_row[sel], f.v_row[sel])
        _, q_a, k_a, _ = _rope_forward(P, W.Workload("alone", hq, hkv, d, [fa], None), fa, style, tab)
        assert np.array_equal(q_tree[sel], q_a) and np.array_equal(k_tree[sel], k_a)


@pytest.mark.parametrize("style", OR.STYLES)
def test_attention_after_rope(P, style):
    """rope + cache write, then attention over the cache, against the oracle
    attention of the oracle-rotated Q and K (rounded to f16 as the kernel stores
    them)."""
    wl = W.small_doc_questions(6)
    f = wl.forwards[0]
    idx = OT.build_index(f.tree)
    toks = OT.query_tokens(idx)
    tab = OR.table(int(toks["pos_id"].max()) + 1, wl.d)
    plan = P.tree_attn_plan(f.tree, wl.hq, wl.hkv, wl.d, wl.scale, out_dtype="f32")
    P.tree_attn_plan_upload(plan)
    kn, vn = f.kv_new()
    kc0, vc0 = f.cache_before()
    q = _dev(f.q)
    kc, vc = _dev(kc0), _dev(vc0)
    P.tree_attn_rope_cache_write(plan, q, q, _dev(kn), _dev(vn), _dev(tab), kc, vc, style=style)
    o = torch.empty((plan.info["num_q_tokens"], wl.hq, wl.d), dtype=torch.float32, device="cuda")
    P.tree_attn_forward_cached(plan, q, kc, vc, o)
    torch.cuda.synchronize()
    # oracle: rotate every row-space token at its own prompt position
    pos_all = np.zeros(idx.num_kv_tokens, np.int64)
    for g in range(len(idx.block_len)):
        b0 = idx.row_base[idx.block_row[g]] + idx.block_start[g]
        pa = sum(idx.block_len[a] for a in idx.block_anc[g])
        pos_all[b0:b0 + idx.block_len[g]] = pa + np.arange(idx.block_len[g])
    k_rot = OR.apply(f.k_row, pos_all, tab, style).astype(np.float16)
    q_rot = OR.apply(f.q, toks["pos_id"], tab, style).astype(np.float16)
    # rows cached before this forward hold whatever earlier forwards wrote (here
    # the generator's K as given); this forward's rows hold the rotated K
    pre = np.setdiff1d(np.arange(idx.num_kv_tokens), toks["row_pos"])
    k_mixed = k_rot.copy()
    k_mixed[pre] = kc0[pre]
    want = OA.tree_attention(f.tree, q_rot, k_mixed, f.v_row, wl.scale)
    got = o.double().cpu().numpy()
    assert np.abs(got - want).max() <= 2e-3
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel <= 1e-3


def test_rope_argument_errors(P):
    wl = W.make_config(0, 0)
    f = wl.forwards[0]
    plan = P.tree_attn_plan(f.tree, wl.hq, wl.hkv, wl.d, wl.scale)
    P.tree_attn_plan_upload(plan)
    kn, vn = f.kv_new()
    q = _dev(f.q)
    kc, vc = _dev(f.k_row), _dev(f.v_row)
    max_pos = int(P.tree_attn_plan_export(plan)["pos_id"].max())
    short = _dev(OR.table(max_pos, wl.d))  # one position short
    with pytest.raises(P.TreeAttnError):
        P.tree_attn_rope_cache_write(plan, q, q, _dev(kn), _dev(vn), short, kc, vc)
    with pytest.raises(ValueError):
        P.tree_attn_rope_cache_write(plan, q, q, _dev(kn), _dev(vn), _dev(OR.table(200, wl.d)), kc, vc,
                                     style="sideways")
    with pytest.raises(ValueError):  # wrong table width
        P.tree_attn_rope_cache_write(plan, q, q, _dev(kn), _dev(vn), _dev(OR.table(200, wl.d * 2)), kc, vc)
