"""Dense-mask tree attention in float64 (oracle).

TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the bench's CPU
baseline, never by the product path.

Source: the architecture page "How basal-rs computes a decision", section 03
"Packing" ("Attention over tree blocks": a token attends to the earlier tokens
of its own block and to its ancestor blocks), and section 01, stage "GPU
forward pass" (the forward runs in f16 with attention accumulated in f32; the
f32 path is the page's reference precision, section 06). The oracle goes one
step further and works in float64 on the exact f16 input values.

Definition computed, per query head h with KV head kv = floor(h / (Hq/Hkv))
(grouped heads are contiguous; the page is silent on grouping):

    S = scale * Q[:, h] K[:, kv]^T,  S[t, u] = -inf where M[t, u] is false
    m = max_u S,  P = exp(S - m),  l = sum_u P
    O[:, h] = P V[:, kv] / l,  LSE[h] = m + ln l

Query rows are independent; they are processed in slices of ``block`` rows only
to bound memory. Every row has at least one visible key (the token itself).
"""
from __future__ import annotations

import numpy as np

from . import tree as _tree


def attention_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                    scale: float, return_lse: bool = False):
    """q [T_q, Hq, D], k/v [T_kv, Hkv, D] (any float dtype, widened to float64),
    mask bool [T_q, T_kv]. Returns O float64 [T_q, Hq, D] (and LSE [Hq, T_q])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0
    g = hq // hkv
    out = np.zeros((tq, hq, d), dtype=np.float64)
    lse = np.zeros((hq, tq), dtype=np.float64)
    for h in range(hq):
        kv = h // g
        s = scale * (q[:, h, :] @ k[:, kv, :].T)
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        out[:, h, :] = (p @ v[:, kv, :]) / l
        lse[h] = (m + np.log(l))[:, 0]
    return (out, lse) if return_lse else out


def tree_attention(desc, q: np.ndarray, k_row: np.ndarray, v_row: np.ndarray, scale: float,
                   block: int = 1024, return_lse: bool = False, sel=None):
    """Tree attention of one forward: ``q`` holds this forward's query tokens (in
    forward order), ``k_row``/``v_row`` the K/V of every row-space token (cached
    prefix included). ``sel`` restricts the output to some query tokens."""
    idx = _tree.build_index(desc)
    toks = _tree.query_tokens(idx)
    n = len(toks["tok_block"])
    sel = np.arange(n) if sel is None else np.asarray(sel)
    hq, d = q.shape[1], q.shape[2]
    out = np.zeros((len(sel), hq, d), dtype=np.float64)
    lse = np.zeros((hq, len(sel)), dtype=np.float64)
    for a in range(0, len(sel), block):
        part = sel[a:a + block]
        m = _tree.dense_mask(idx, toks, part)
        o, l = attention_dense(q[part], k_row, v_row, m, scale, return_lse=True)
        out[a:a + len(part)] = o
        lse[:, a:a + len(part)] = l
    return (out, lse) if return_lse else out


def useful_pairs(desc) -> int:
    """Sum over this forward's query tokens of the number of keys each may see."""
    idx = _tree.build_index(desc)
    toks = _tree.query_tokens(idx)
    total = 0
    for b, o in zip(toks["tok_block"], toks["tok_offset"]):
        total += sum(hi - lo for lo, hi in _tree.visible_ranges(idx, int(b), int(o)))
    return total
