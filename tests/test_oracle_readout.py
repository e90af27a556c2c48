"""Pins of the readout-only last layer oracle (oracle/readout.py) to facts
that do not come from the oracle: a hand-worked example (with a float16 tie),
closed forms of the RMS norm and silu, the residual path, and the pages' claim
that computing the last layer only at readout rows and letter columns equals
the ordinary full computation restricted to them."""
import json
import math
import os

import numpy as np
import pytest

from oracle import readout as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "readout_worked_example.json")


def test_worked_example():
    g = json.load(open(GOLDEN))
    st = R.readout_mlp(np.array(g["hidden"]), g["readout_tok"], g["norm_w"], np.array(g["w_gate"]),
                       np.array(g["w_up"]), np.array(g["w_down"]), g["eps"])
    e = g["expect"]
    np.testing.assert_array_equal(st["xn"], e["xn"])
    np.testing.assert_array_equal(st["act"], e["act"])
    np.testing.assert_array_equal(st["h_out"], e["h_out"])
    y, lg = R.letter_logits(st["h_out"], g["final_norm_w"], g["eps"], np.array(g["lm_head"]),
                            np.array(g["letter_ids"]), g["n_letters"], 2)
    np.testing.assert_array_equal(y, e["y"])
    np.testing.assert_array_equal(lg, e["logits"])


def test_rn16_ties_to_even():
    sp = 2.0 ** -9  # float16 spacing in [2, 4)
    assert R.rn16(2 + 0.5 * sp) == 2.0
    assert R.rn16(2 + 1.5 * sp) == 2 + 2 * sp
    assert R.rn16(2 + 0.5 * sp + 1e-9) == 2 + sp


def test_rms_norm_closed_forms():
    x = np.array([3.0, 4.0])
    np.testing.assert_allclose(R.rms_norm(x, [1, 1], 0.0), x / math.sqrt(12.5), rtol=1e-15)
    np.testing.assert_allclose(R.rms_norm(x, [1, 1], 0.5), x / math.sqrt(13.0), rtol=1e-15)
    np.testing.assert_allclose(R.rms_norm(x, [2, -1], 0.0), [6 / math.sqrt(12.5), -4 / math.sqrt(12.5)],
                               rtol=1e-15)
    rng = np.random.default_rng(0)
    v = rng.normal(size=(5, 64))
    y = R.rms_norm(v, np.ones(64), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)   # unit mean square
    np.testing.assert_allclose(R.rms_norm(7.5 * v, np.ones(64), 0.0), y, rtol=1e-13)  # scale-free
    assert np.all(R.rms_norm(np.zeros(8), np.ones(8), 1e-5) == 0)       # eps keeps zeros finite


def test_silu_identities():
    assert R.silu(0.0) == 0.0
    z = np.linspace(-9, 9, 37)
    np.testing.assert_allclose(R.silu(z) - R.silu(-z), z, atol=1e-14)   # z*s(z) + z*s(-z) = z
    assert abs(R.silu(40.0) - 40.0) < 1e-15 * 40
    assert 0 > R.silu(-40.0) > -1e-15
    h = 1e-6
    assert abs((R.silu(h) - R.silu(-h)) / (2 * h) - 0.5) < 1e-9        # slope 1/2 at 0
    np.testing.assert_allclose(R.silu(1.0), 1 / (1 + math.exp(-1)), rtol=1e-15)


def _weights(rng, dm, ff, vocab):
    f16 = lambda a: a.astype(np.float16).astype(np.float64)  # noqa: E731
    return dict(norm_w=f16(1 + 0.1 * rng.normal(size=dm)),
                w_gate=f16(rng.normal(size=(ff, dm)) / math.sqrt(dm)),
                w_up=f16(rng.normal(size=(ff, dm)) / math.sqrt(dm)),
                w_down=f16(rng.normal(size=(dm, ff)) / math.sqrt(ff)),
                final_norm_w=f16(1 + 0.1 * rng.normal(size=dm)),
                lm_head=f16(2 * rng.normal(size=(vocab, dm)) / math.sqrt(dm)))


def test_readout_only_equals_full_layer():
    """The pages' readout-only last layer: rows and letter columns of the
    ordinary computation (every token, whole vocabulary)."""
    rng = np.random.default_rng(1)
    dm, ff, vocab, T, eps = 16, 24, 50, 30, 1e-5
    W = _weights(rng, dm, ff, vocab)
    hidden = rng.normal(size=(T, dm)).astype(np.float16).astype(np.float64)
    readout = np.array([29, 3, 17, 3, 0, 11, 29])          # repeated rows: a shared readout
    n_letters = rng.integers(2, 6, len(readout))
    ids = rng.integers(0, vocab, (len(readout), 5))
    ids[3], n_letters[3] = ids[1], n_letters[1]            # the shared readout's letters
    full = R.last_layer_full(hidden, W["norm_w"], W["w_gate"], W["w_up"], W["w_down"],
                             W["final_norm_w"], eps, W["lm_head"])
    st = R.readout_mlp(hidden, readout, W["norm_w"], W["w_gate"], W["w_up"], W["w_down"], eps)
    _, lg = R.letter_logits(st["h_out"], W["final_norm_w"], eps, W["lm_head"], ids, n_letters, 5)
    for r, t in enumerate(readout):
        for j in range(n_letters[r]):
            assert abs(lg[r, j] - full[t, ids[r, j]]) <= 1e-12
        assert np.all(lg[r, n_letters[r]:] == 0)
    np.testing.assert_array_equal(lg[1], lg[3])            # shared readout, same logits


def test_residual_path_and_zero_branches():
    rng = np.random.default_rng(2)
    dm, ff = 32, 48
    W = _weights(rng, dm, ff, 4)
    h = rng.normal(size=(6, dm)).astype(np.float16).astype(np.float64)
    st = R.mlp_rows(h, W["norm_w"], W["w_gate"], W["w_up"], np.zeros((dm, ff)), 1e-5)
    np.testing.assert_array_equal(st["h_out"], h)          # no down projection: the residual alone
    st = R.mlp_rows(h, W["norm_w"], W["w_gate"], np.zeros((ff, dm)), W["w_down"], 1e-5)
    assert np.all(st["act"] == 0)
    np.testing.assert_array_equal(st["h_out"], h)
    # every stored stage is a float16 value
    st = R.mlp_rows(h, W["norm_w"], W["w_gate"], W["w_up"], W["w_down"], 1e-5)
    for k, v in st.items():
        np.testing.assert_array_equal(R.rn16(v), v, err_msg=k)


def test_hidden_unit_permutation():
    """Reordering the MLP's hidden units (rows of gate and up, columns of down)
    leaves the block's output unchanged."""
    rng = np.random.default_rng(3)
    dm, ff = 32, 40
    W = _weights(rng, dm, ff, 4)
    h = rng.normal(size=(5, dm)).astype(np.float16).astype(np.float64)
    p = rng.permutation(ff)
    a = R.mlp_rows(h, W["norm_w"], W["w_gate"], W["w_up"], W["w_down"], 1e-5)
    b = R.mlp_rows(h, W["norm_w"], W["w_gate"][p], W["w_up"][p], W["w_down"][:, p], 1e-5)
    np.testing.assert_array_equal(a["act"][:, p], b["act"])
    np.testing.assert_array_equal(a["h_out"], b["h_out"])


def test_unit_head_reads_the_normalized_state():
    """Head rows that are unit vectors read coordinates of the final normalized
    state, whose mean square is 1 (norm weight 1, eps 0) up to float16 rounding."""
    rng = np.random.default_rng(4)
    dm = 64
    h = rng.normal(size=(3, dm)).astype(np.float16).astype(np.float64)
    head = np.eye(dm)
    ids = np.array([[5, 0, 63], [1, 2, 3], [63, 62, 61]])
    y, lg = R.letter_logits(h, np.ones(dm), 0.0, head, ids, [3, 3, 3], 3)
    for r in range(3):
        np.testing.assert_array_equal(lg[r], y[r, ids[r]])
    exact = R.rms_norm(h, np.ones(dm), 0.0)
    assert np.all(np.abs(y - exact) <= 2.0 ** -11 * np.abs(exact) + 2.0 ** -25)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=2e-3)
