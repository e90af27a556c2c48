"""Readout-only last layer: the MLP block and the answer-letter logits computed
only at readout positions (oracle, float64 with float16 storage points).

TEST INFRASTRUCTURE ONLY: used by tests, never by the product path.

Sources: the architecture page "How basal-rs computes a decision":
* section 01, stage "GPU forward pass": in the final layer of the Llama model,
  the MLP block and the logits are computed only for readout positions and
  answer letters;
* section 01, stage "Batch and prefix tree": identical prompts share a single
  readout (so a readout row may serve several prompts);
* section 05 ("Compute precision and decision agreement", f16 default row):
  residual stream, normalizations and MLP blocks are float16, matrix products
  accumulate in float32;
* section 05 ("Batch-independent GEMM table"): letters are read out by a
  custom kernel and letter logits are bitwise identical whatever the batch.

The Llama last-layer MLP (the pages name the model family, not its formulas;
these are the family's published definitions): RMS normalization
x * (mean(x^2) + eps)^(-1/2) * w, a SwiGLU block down(silu(gate(x)) * up(x))
with silu(z) = z / (1 + exp(-z)), a residual add, the final RMS normalization
and the language-model head, whose row for a token id gives that token's logit.

Readings (where the pages fix a precision but not each rounding point):
* every tensor the pages call float16 is rounded to float16 once, after its op
  is computed exactly: the normalized input, the gate and up products, the
  SwiGLU output, the down product, the residual sum, and the final normalized
  state;
* silu(g) * u is one op on the float16 g and u (one rounding);
* the letter logits are the float32-accumulated head products and stay
  unrounded (they leave the model for the decision formula); here they are
  float64;
* ``hidden`` is the residual stream entering the last layer's MLP block (after
  that layer's attention and its residual add), one row per packed token.

Float16 rounding is numpy's float64 -> float16 conversion (round to nearest,
ties to even).
"""
from __future__ import annotations

from typing import Dict, Sequence

import numpy as np


def rn16(x) -> np.ndarray:
    """Round to the nearest float16 (ties to even), returned as float64."""
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x * (mean(x^2) + eps)^(-1/2) * w over the last axis (exact, float64)."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, np.float64)


def silu(z) -> np.ndarray:
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def mlp_rows(h: np.ndarray, norm_w, w_gate, w_up, w_down, eps: float) -> Dict[str, np.ndarray]:
    """The MLP block with its residual on rows h [n, d_model] (float16 values).
    Weights follow the linear-layer convention out = x @ W.T: w_gate, w_up
    [d_ff, d_model], w_down [d_model, d_ff]. Returns every float16 stage."""
    h = np.asarray(h, np.float64)
    xn = rn16(rms_norm(h, norm_w, eps))
    g = rn16(xn @ np.asarray(w_gate, np.float64).T)
    u = rn16(xn @ np.asarray(w_up, np.float64).T)
    act = rn16(silu(g) * u)
    d = rn16(act @ np.asarray(w_down, np.float64).T)
    out = rn16(h + d)
    return {"xn": xn, "g": g, "u": u, "act": act, "d": d, "h_out": out}


def readout_mlp(hidden: np.ndarray, readout_tok: Sequence[int], norm_w, w_gate, w_up, w_down,
                eps: float) -> Dict[str, np.ndarray]:
    """MLP block only at the readout tokens: gather hidden[readout_tok] then
    the block (rows in readout order)."""
    rows = np.asarray(hidden)[np.asarray(readout_tok, np.int64)]
    return mlp_rows(rows, norm_w, w_gate, w_up, w_down, eps)


def letter_logits(h: np.ndarray, final_norm_w, eps: float, lm_head: np.ndarray,
                  letter_ids: np.ndarray, n_letters: Sequence[int], ld: int):
    """Final normalization of readout rows h [n, d_model], then the logits of
    row r's letters letter_ids[r, :n_letters[r]] only. Returns (y, logits
    [n, ld] with zeros beyond each row's letters)."""
    y = rn16(rms_norm(h, final_norm_w, eps))
    n = y.shape[0]
    logits = np.zeros((n, ld))
    head = np.asarray(lm_head)
    for r in range(n):
        for j in range(int(n_letters[r])):
            logits[r, j] = float(np.dot(head[int(letter_ids[r, j])].astype(np.float64), y[r]))
    return y, logits


def last_layer_full(hidden: np.ndarray, norm_w, w_gate, w_up, w_down, final_norm_w, eps: float,
                    lm_head: np.ndarray) -> np.ndarray:
    """The same last layer computed the ordinary way: the MLP block for every
    token and logits over the whole vocabulary, [n_tokens, vocab]. Readout-only
    computation must equal selected rows and columns of this."""
    st = mlp_rows(hidden, norm_w, w_gate, w_up, w_down, eps)
    y = rn16(rms_norm(st["h_out"], final_norm_w, eps))
    return y @ np.asarray(lm_head, np.float64).T
