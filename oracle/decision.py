"""The Basal decision from letter logits (oracle, float64).

TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the bench's CPU
baseline, never by the product path.

Source: the architecture page "How basal-rs computes a decision", section 02
"Basal protocol" (its two formulas and the worked example) and section 01,
stage "Decision and response". A question is asked twice, the second time with
its options in reverse order. Letter logits of each order become probabilities
through a softmax; the second order's probabilities are put back in the
original option order; the two are averaged; calibration divides the log of the
clamped average by the question type's temperature T and applies softmax again.

Readings where the page is silent: "log" is the natural logarithm; the clamp
1e-12 applies elementwise to the average; restoring order 2 is the index
reversal i -> n-1-i of its probabilities; probabilities are returned unrounded.
"""
from __future__ import annotations

import numpy as np

CLAMP = 1e-12


def softmax(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def decision(l_order1, l_order2, T: float):
    """Returns (p, p_cal) for one question: l_order1 are the letter logits with
    the options in the request's order, l_order2 with the options reversed."""
    if not T > 0:
        raise ValueError("temperature must be positive")
    p1 = softmax(l_order1)
    p2 = softmax(l_order2)
    p = (p1 + p2[::-1]) / 2.0
    p_cal = softmax(np.log(np.maximum(p, CLAMP)) / float(T))
    return p, p_cal


def decisions(logits: np.ndarray, row1, row2, n_letters, T):
    """Batched form over a logits matrix [n_rows, ld]: decision i reads rows
    row1[i] and row2[i], first n_letters[i] columns. Outputs [n_dec, ld] float64
    with zeros beyond each decision's letters."""
    logits = np.asarray(logits, dtype=np.float64)
    n_dec = len(row1)
    ld = logits.shape[1]
    p_avg = np.zeros((n_dec, ld))
    p_cal = np.zeros((n_dec, ld))
    for i in range(n_dec):
        n = int(n_letters[i])
        a, c = decision(logits[int(row1[i]), :n], logits[int(row2[i]), :n], float(T[i]))
        p_avg[i, :n] = a
        p_cal[i, :n] = c
    return p_avg, p_cal
