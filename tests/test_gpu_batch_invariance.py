"""Batch invariance of tree attention (section 05 "Reproducibility": attention
tiled by position; tree-block attention gives the same result alone, in a batch
and in a tree).

One prompt (template -> document -> question -> leaf) is computed in several
contexts: alone as a chain of blocks, alone as one block, as one leaf of a tree
with sibling questions and leaves, as one row of a batch of rows, and as the
same tree computed in chunks over a row-space cache. With batch_invariant the
outputs (O in f16 and f32, and LSE) of every token of the prompt must be
bitwise identical across all of them; they must also match the oracle.
"""
import numpy as np
import pytest

from lse_bound import lse_atol
from oracle import attention as OA
from workloads import configs as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

HQ, HKV, D = 8, 2, 128
# lengths chosen so that key windows of 64 straddle every block boundary
PROMPT = [96, 300, 40, 21]


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefix_tree_packed_amd as P
    P.load_library()
    return P


def _f16(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def _prompt_values(seed):
    rng = np.random.default_rng(seed)
    n = sum(PROMPT)
    return _f16(rng, (n, HQ, D)), _f16(rng, (n, HKV, D)), _f16(rng, (n, HKV, D))


def _context(kind, vals, seed):
    """Rows, the row-space index of each prompt token, and row-space Q/K/V
    with the prompt's values in place (random values elsewhere)."""
    L = PROMPT
    chain = [(-1, L[0]), (0, L[1]), (1, L[2]), (2, L[3])]
    if kind == "alone":
        rows, ours = [chain], (0, [0, 1, 2, 3])
    elif kind == "one-block":
        rows, ours = [[(-1, sum(L))]], None
    elif kind in ("tree", "chunked"):
        # siblings laid out before ours, so the row is not in pre-order
        row = [(-1, L[0]), (0, L[1]), (1, 55), (1, L[2]), (2, 25), (3, 17), (3, L[3]), (3, 30)]
        rows, ours = [row], (0, [0, 1, 3, 6])
    elif kind == "batch":
        rows = [[(-1, 70), (0, 33), (0, 41)], chain, [(-1, 150), (0, 64), (1, 12)]]
        ours = (1, [0, 1, 2, 3])
    else:
        raise ValueError(kind)
    desc = W.desc_from_rows(rows)
    lens = desc.row_lengths()
    base = np.concatenate([[0], np.cumsum(lens)])
    n_kv = int(base[-1])
    rng = np.random.default_rng(seed)
    q, k, v = _f16(rng, (n_kv, HQ, D)), _f16(rng, (n_kv, HKV, D)), _f16(rng, (n_kv, HKV, D))
    if ours is None:
        pos = np.arange(sum(L))
    else:
        r, blocks = ours
        starts = np.concatenate([[0], np.cumsum([n for _, n in rows[r]])])
        pos = np.concatenate([base[r] + starts[b] + np.arange(rows[r][b][1]) for b in blocks])
    q[pos], k[pos], v[pos] = vals
    return desc, pos, q, k, v


def _run(P, kind, vals, out_dtype, inv, seed=11):
    """O and LSE of the prompt's tokens in context `kind` (one-shot forward, or
    three chunked forwards over one row-space cache for "chunked")."""
    desc, pos, q, k, v = _context(kind, vals, seed)
    odt = torch.float16 if out_dtype == "f16" else torch.float32
    kd = torch.from_numpy(k).cuda()
    vd = torch.from_numpy(v).cuda()
    n_kv = q.shape[0]
    o_all = np.zeros((n_kv, HQ, D), np.float64)
    l_all = np.zeros((HQ, n_kv), np.float64)
    if kind == "chunked":
        cuts = [0, 200, 450, n_kv]
        kc = torch.zeros_like(kd)
        vc = torch.zeros_like(vd)
        for a, b in zip(cuts[:-1], cuts[1:]):
            d = desc.with_q_range([a], [b])
            plan = P.tree_attn_plan(d, HQ, HKV, D, D ** -0.5, out_dtype=out_dtype, write_lse=True,
                                    batch_invariant=inv)
            P.tree_attn_plan_upload(plan)
            o = torch.empty((b - a, HQ, D), dtype=odt, device="cuda")
            l = torch.empty((HQ, b - a), dtype=torch.float32, device="cuda")
            P.tree_attn_forward_chunked(plan, torch.from_numpy(q[a:b]).cuda(), kd[a:b].contiguous(),
                                        vd[a:b].contiguous(), kc, vc, o, l)
            torch.cuda.synchronize()
            o_all[a:b] = o.double().cpu().numpy()
            l_all[:, a:b] = l.double().cpu().numpy()
    else:
        plan = P.tree_attn_plan(desc, HQ, HKV, D, D ** -0.5, out_dtype=out_dtype, write_lse=True,
                                batch_invariant=inv)
        P.tree_attn_plan_upload(plan)
        o = torch.empty((n_kv, HQ, D), dtype=odt, device="cuda")
        l = torch.empty((HQ, n_kv), dtype=torch.float32, device="cuda")
        P.tree_attn_forward(plan, torch.from_numpy(q).cuda(), kd, vd, o, l)
        torch.cuda.synchronize()
        o_all[:] = o.double().cpu().numpy()
        l_all[:] = l.double().cpu().numpy()
    return o_all[pos], l_all[:, pos], (desc, q, k, v)


@pytest.mark.parametrize("out_dtype", ["f16", "f32"])
def test_bitwise_identical_across_contexts(P, out_dtype):
    vals = _prompt_values(3)
    print(f"[invariance] {out_dtype}", flush=True)
    ref_o, ref_l, (desc, q, k, v) = _run(P, "tree", vals, out_dtype, True)
    want, want_lse = OA.tree_attention(desc, q, k, v, D ** -0.5, return_lse=True)
    row = _context("tree", vals, 11)[1]
    err = np.abs(ref_o - want[row]).max()
    assert err <= 2e-3, f"tree context vs oracle: max-abs {err:.3g}"
    assert np.all(np.abs(ref_l - want_lse[:, row]) <= lse_atol(q[row], k, D ** -0.5, HQ, HKV))
    for kind in ("alone", "one-block", "batch", "chunked"):
        print(f"[invariance] {out_dtype} {kind}", flush=True)
        o, l, _ = _run(P, kind, vals, out_dtype, True)
        assert np.array_equal(o, ref_o), f"O differs between tree and {kind}"
        assert np.array_equal(l, ref_l), f"LSE differs between tree and {kind}"


def test_union_tiling_agrees_to_rounding(P):
    """Without batch_invariant the contexts agree to rounding only (and the
    invariant tiling agrees with the union tiling to rounding)."""
    vals = _prompt_values(4)
    ref, _, _ = _run(P, "tree", vals, "f32", True)
    for kind in ("tree", "alone", "batch", "chunked"):
        o, _, _ = _run(P, kind, vals, "f32", False)
        assert np.abs(o - ref).max() <= 2e-3
