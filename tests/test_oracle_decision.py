"""Pins of the decision oracle against the architecture page's section 02
("Basal protocol"): the printed worked example, and closed forms / invariants
of its two formulas. CPU only."""
import json
import math
import os

import numpy as np
import pytest

from oracle import decision as D


def _load(golden_dir):
    with open(os.path.join(golden_dir, "decision_worked_example.json")) as f:
        return json.load(f)


def _round2(x):
    return [round(float(v), 2) for v in x]


def test_worked_example_order_probabilities(golden_dir):
    g = _load(golden_dir)
    p1 = D.softmax(g["order1_logits"])
    p2 = D.softmax(g["order2_logits"])
    assert _round2(p1) == g["order1_probs_2dp"]
    assert _round2(p2) == g["order2_probs_2dp"]


def test_worked_example_average_and_calibration(golden_dir):
    g = _load(golden_dir)
    p, p_cal = D.decision(g["order1_logits"], g["order2_logits"], g["T"])
    assert _round2(p) == g["average_2dp"]
    assert _round2(p_cal) == g["calibrated_2dp"]
    # the labels line up: the average is in order-1 option order, and order 2
    # lists the same options reversed
    assert g["order2_labels"][::-1] == g["order1_labels"] == g["average_labels"]
    # "T = 1.00" leaves the average unchanged, exactly (up to rounding)
    np.testing.assert_allclose(p_cal, p, rtol=0, atol=1e-15)


def test_probabilities_sum_to_one():
    rng = np.random.default_rng(1)
    for n in (2, 3, 8, 255):
        l1 = rng.normal(0, 2, n)
        l2 = rng.normal(0, 2, n)
        for T in (0.5, 1.0, 1.7):
            p, c = D.decision(l1, l2, T)
            assert abs(p.sum() - 1) < 1e-12 and abs(c.sum() - 1) < 1e-12
            assert np.all(p > 0) and np.all(c > 0)


def test_calibration_closed_form_power():
    """Without the clamp binding, softmax(ln p / T) = p^(1/T) / sum p^(1/T)."""
    rng = np.random.default_rng(2)
    for _ in range(50):
        n = int(rng.integers(2, 9))
        l1, l2 = rng.normal(0, 2, n), rng.normal(0, 2, n)
        T = float(rng.uniform(0.3, 3.0))
        p, c = D.decision(l1, l2, T)
        assert p.min() >= 1e-12
        w = np.array([math.pow(float(x), 1.0 / T) for x in p])
        np.testing.assert_allclose(c, w / w.sum(), rtol=1e-12, atol=0)


def test_average_closed_form_with_explicit_reversal():
    """p[i] = (softmax(l1)[i] + softmax(l2)[n-1-i]) / 2, written with math.exp."""
    l1 = [1.0, -2.0, 0.5, 3.0]
    l2 = [0.25, 2.0, -1.0, 0.0]
    z1 = sum(math.exp(x) for x in l1)
    z2 = sum(math.exp(x) for x in l2)
    n = len(l1)
    want = [(math.exp(l1[i]) / z1 + math.exp(l2[n - 1 - i]) / z2) / 2 for i in range(n)]
    p, _ = D.decision(l1, l2, 1.0)
    np.testing.assert_allclose(p, want, rtol=1e-14, atol=0)


def test_sharpen_flatten_and_argmax():
    """T < 1 sharpens, T > 1 flattens; the selected option stays the same."""
    rng = np.random.default_rng(3)
    for _ in range(50):
        n = int(rng.integers(2, 9))
        l1, l2 = rng.normal(0, 2, n), rng.normal(0, 2, n)
        p, _ = D.decision(l1, l2, 1.0)
        if np.sort(p)[-1] - np.sort(p)[-2] < 1e-9:
            continue
        _, sharp = D.decision(l1, l2, 0.6)
        _, flat = D.decision(l1, l2, 1.8)
        assert np.argmax(sharp) == np.argmax(p) == np.argmax(flat)
        assert sharp.max() >= p.max() >= flat.max()


def test_clamp_binds_on_tiny_probabilities():
    """With a logit gap of 60 the small letters fall below 1e-12: their
    calibrated weight is 1e-12^(1/T) / Z."""
    l1 = np.array([60.0, 0.0, 0.0])
    l2 = l1[::-1].copy()
    T = 0.7
    p, c = D.decision(l1, l2, T)
    assert p[1] < 1e-12 and p[2] < 1e-12
    w = np.array([p[0] ** (1 / T), 1e-12 ** (1 / T), 1e-12 ** (1 / T)])
    np.testing.assert_allclose(c, w / w.sum(), rtol=1e-12, atol=0)
    # without the clamp the small letters would be far smaller still
    assert c[1] > (p[1] ** (1 / T)) / w.sum()


def test_symmetric_orders_give_plain_softmax():
    """If order 2's logits are order 1's reversed, the average is softmax(l1)."""
    rng = np.random.default_rng(4)
    for n in (2, 5, 17):
        l1 = rng.normal(0, 2, n)
        e = np.exp(l1 - l1.max())
        p, _ = D.decision(l1, l1[::-1], 1.0)
        np.testing.assert_allclose(p, e / e.sum(), rtol=1e-14)


def test_nonpositive_temperature_rejected():
    with pytest.raises(ValueError):
        D.decision([0.0, 1.0], [1.0, 0.0], 0.0)


def test_batched_matches_single():
    rng = np.random.default_rng(5)
    logits = rng.normal(0, 2, (6, 8))
    row1, row2 = [0, 2, 4], [1, 3, 5]
    nl, T = [3, 8, 2], [1.0, 0.7, 1.3]
    pa, pc = D.decisions(logits, row1, row2, nl, T)
    for i in range(3):
        a, c = D.decision(logits[row1[i], :nl[i]], logits[row2[i], :nl[i]], T[i])
        np.testing.assert_array_equal(pa[i, :nl[i]], a)
        np.testing.assert_array_equal(pc[i, :nl[i]], c)
        assert np.all(pa[i, nl[i]:] == 0) and np.all(pc[i, nl[i]:] == 0)
