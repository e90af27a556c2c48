"""Pins of the rotary-embedding oracle (oracle/rope.py) against closed forms,
an independent complex-number formulation and the tree-position rule."""
import numpy as np
import pytest

from oracle import rope as OR
from oracle import tree as OT
from workloads import configs as W


def _x(rng, t, h, d):
    return rng.standard_normal((t, h, d)).astype(np.float16)


def test_table_values():
    tab = OR.table(5, 8, theta=10000.0)
    assert tab.shape == (5, 4, 2) and tab.dtype == np.float32
    assert np.array_equal(tab[0], np.stack([np.ones(4), np.zeros(4)], -1).astype(np.float32))
    # p = 1, i = 0: angle 1; i = 3: angle 10000^(-6/8)
    assert tab[1, 0, 0] == np.float32(np.cos(1.0)) and tab[1, 0, 1] == np.float32(np.sin(1.0))
    a = 10000.0 ** (-0.75)
    assert tab[3, 3, 1] == np.float32(np.sin(3 * a))


@pytest.mark.parametrize("style", OR.STYLES)
def test_position_zero_is_identity_and_norms_are_kept(style):
    rng = np.random.default_rng(0)
    x = _x(rng, 6, 3, 16)
    tab = OR.table(64, 16)
    np.testing.assert_array_equal(OR.apply(x, np.zeros(6, int), tab, style), x.astype(np.float64))
    y = OR.apply(x, rng.integers(0, 64, 6), tab, style)
    f, s = OR.pair_index(16, style)
    xn = x.astype(np.float64)[..., f] ** 2 + x.astype(np.float64)[..., s] ** 2
    yn = y[..., f] ** 2 + y[..., s] ** 2
    np.testing.assert_allclose(yn, xn, rtol=1e-6)  # table in f32: cos^2 + sin^2 = 1 to ~1e-7


def test_interleaved_is_the_complex_multiply():
    """The guide's form: view consecutive pairs as complex numbers and multiply
    by cos + i sin of the token's row of the table."""
    rng = np.random.default_rng(1)
    x = _x(rng, 5, 2, 12)
    tab = OR.table(40, 12)
    pos = np.array([0, 3, 7, 39, 11])
    z = x.astype(np.float64)[..., 0::2] + 1j * x.astype(np.float64)[..., 1::2]
    w = tab[pos, :, 0].astype(np.float64) + 1j * tab[pos, :, 1].astype(np.float64)
    r = z * w[:, None, :]
    want = np.empty(x.shape)
    want[..., 0::2], want[..., 1::2] = r.real, r.imag
    np.testing.assert_allclose(OR.apply(x, pos, tab, "interleaved"), want, rtol=0, atol=1e-12)


def test_half_is_interleaved_up_to_a_permutation():
    rng = np.random.default_rng(2)
    d = 16
    x = _x(rng, 4, 2, d)
    tab = OR.table(30, d)
    pos = np.array([1, 5, 29, 0])
    perm = np.empty(d, int)            # half-split element j -> interleaved slot
    perm[:d // 2] = np.arange(0, d, 2)
    perm[d // 2:] = np.arange(1, d, 2)
    xi = np.empty_like(x)
    xi[..., perm] = x
    yi = OR.apply(xi, pos, tab, "interleaved")
    np.testing.assert_allclose(OR.apply(x, pos, tab, "half"), yi[..., perm], rtol=0, atol=1e-12)


@pytest.mark.parametrize("style", OR.STYLES)
def test_scores_depend_on_relative_position(style):
    """With an exact (float64) table, q.k after rotation depends only on the
    position difference -- the property rotary embedding exists for."""
    rng = np.random.default_rng(3)
    d = 32
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    i = np.arange(d // 2)
    ang = np.arange(200)[:, None] * 10000.0 ** (-2.0 * i / d)
    tab = np.stack([np.cos(ang), np.sin(ang)], -1)
    s = [float((OR.apply(q, [p + 13], tab, style) * OR.apply(k, [p], tab, style)).sum()) for p in (0, 40, 150)]
    np.testing.assert_allclose(s, s[0], rtol=1e-10)


@pytest.mark.parametrize("style", OR.STYLES)
def test_tree_positions_equal_separate_prompts(style):
    """Rotating the packed tree's tokens at the plan's position ids equals
    rotating every root-to-leaf prompt on its own at positions 0 .. len-1
    (architecture page, section 03: a token's position is its place in its own
    prompt)."""
    rng = np.random.default_rng(4)
    rows = [[(-1, 20), (0, 7), (1, 5), (1, 9), (0, 12), (4, 3)]]
    desc = W.desc_from_rows(rows)
    idx = OT.build_index(desc)
    toks = OT.query_tokens(idx)
    n = idx.num_q_tokens
    x = _x(rng, n, 2, 8)
    tab = OR.table(64, 8)
    packed = OR.apply(x, toks["pos_id"], tab, style)
    for g in range(len(idx.block_len)):
        if not idx.block_is_leaf[g]:
            continue
        path = idx.block_anc[g] + [g]
        rows_of = np.concatenate([idx.block_start[b] + np.arange(idx.block_len[b]) for b in path])
        alone = OR.apply(x[rows_of], np.arange(len(rows_of)), tab, style)
        np.testing.assert_array_equal(packed[rows_of], alone)
