"""Bound on the error of the attention kernel's LSE output, derived from its
arithmetic (used by the GPU parity tests; no GPU or oracle code here).

Two roundings move the kernel's LSE away from the exact one:
- the probabilities are rounded to f16 for the P.V product and the row sum is
  taken over the rounded values: |p~ - p| <= 2^-11 p, so the log of the sum
  moves by at most ln(1 + 2^-11);
- each Q element enters the score products as f16(q * scale * log2 e): its
  error e is at most 2^-11 of the element, or 2^-25 below the f16 normal range.
  A score (log2 units) then moves by e . k, at most ||e||_2 ||k||_2
  (Cauchy-Schwarz), and the LSE (natural log) by at most ln 2 times the largest
  such move over the keys the token sees; every key of the row bounds those.
f32 accumulation and the exponential add far less than the 1e-5 slack.
"""
import math

import numpy as np


def lse_atol(q, k_row, scale, hq, hkv):
    """Per (head, token) bound, shape [hq, n]: q [n, hq, d] the queries
    compared, k_row [n_kv, hkv, d] every key of their rows."""
    d = q.shape[-1]
    c = scale * math.log2(math.e)
    qn = np.linalg.norm(np.asarray(q, np.float64), axis=-1)              # [n, hq]
    e = 2.0 ** -11 * c * qn + 2.0 ** -25 * math.sqrt(d)
    kn = np.linalg.norm(np.asarray(k_row, np.float64), axis=-1).max(axis=0)  # [hkv]
    kmax = np.repeat(kn, hq // hkv)                                       # head h reads KV head h // group
    return (math.log1p(2.0 ** -11) + math.log(2.0) * e * kmax[None, :] + 1e-5).T
