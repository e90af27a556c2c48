"""Rotary position embedding at tree positions (oracle, float64).

TEST INFRASTRUCTURE ONLY: used by tests, never by the product path.

Sources:
* the architecture page "How basal-rs computes a decision", section 03
  "Packing" ("Attention over tree blocks"): a token's position for the
  position encoding is its position in its own prompt (the plan's position id:
  summed lengths of the ancestor blocks plus the offset in its block);
* AstrAI's inference guide ("Inference"), section "Rotary Embedding Backend":
  a table of [cos, sin] pairs of shape [max_len, dim/2, 2] in float32, looked
  up by position id, and a rotation done as a complex multiply of consecutive
  element pairs; section "KV Cache": rotary is applied before K is written to
  the cache.

Rotation of one pair (a, b) by the table entry (c, s) of its position and
frequency index i: (a c - b s, a s + b c), i.e. (a + ib)(c + is).

Pairing (the pages fix the complex-multiply form, not which elements pair up;
both common conventions are provided):
* "interleaved": elements (2i, 2i+1) form pair i (the complex view of the
  guide's [dim/2, 2] layout);
* "half": elements (i, i + dim/2) form pair i (the split-halves convention of
  Llama checkpoints as usually stored).

Readings: the table is an input (the guide stores it precomputed); ``table``
below builds the usual one, angle p * theta^(-2i/dim), and rounds it to
float32 as the guide's table is. The rotation itself is taken in float64 on the
float16 inputs and the float32 table values.
"""
from __future__ import annotations

import numpy as np

STYLES = ("half", "interleaved")


def table(max_pos: int, dim: int, theta: float = 10000.0) -> np.ndarray:
    """[max_pos, dim/2, 2] float32 table of (cos, sin) of p * theta^(-2i/dim)."""
    i = np.arange(dim // 2, dtype=np.float64)
    freq = theta ** (-2.0 * i / dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * freq[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def pair_index(dim: int, style: str):
    """Element indices (first, second) of pair i = 0 .. dim/2 - 1."""
    if style == "interleaved":
        return np.arange(0, dim, 2), np.arange(1, dim, 2)
    if style == "half":
        return np.arange(dim // 2), np.arange(dim // 2, dim)
    raise ValueError(style)


def apply(x: np.ndarray, pos: np.ndarray, tab: np.ndarray, style: str) -> np.ndarray:
    """Rotate x [T, H, dim] (any float type) of tokens at positions pos [T]
    with table tab [max_pos, dim/2, 2]; returns float64 [T, H, dim]."""
    x = np.asarray(x, np.float64)
    out = x.copy()
    first, second = pair_index(x.shape[-1], style)
    for t in range(x.shape[0]):
        c = tab[int(pos[t]), :, 0].astype(np.float64)
        s = tab[int(pos[t]), :, 1].astype(np.float64)
        a = x[t][:, first]
        b = x[t][:, second]
        out[t][:, first] = a * c - b * s
        out[t][:, second] = a * s + b * c
    return out
