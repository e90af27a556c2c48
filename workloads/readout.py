"""Seeded synthetic inputs of the readout-only last layer.

Random draws only (``numpy.random.default_rng(seed)``), in this order: the
residual stream rows, the MLP block's weights, the final norm weight, the
letters' head rows, the letter ids and counts. Scales keep every stage of
order 1, like a trained model's: the residual stream ~ N(0, 1); norm weights
1 + 0.1 N(0, 1); gate and up rows N(0, 1/d_model); down rows N(0, 1/d_ff);
head rows N(0, 4/d_model), so letter logits come out with standard deviation
about 2 (the spread the workloads give letter logits). Everything is float16.
Only the head rows of letters that can be drawn are materialised; the full
head is a zero matrix with those rows filled in (the kernels read no others).

Nothing here computes norms, products or logits.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

# the shapes of the two Llama models the workloads name (8B and 70B)
LLAMA_8B = dict(d_model=4096, d_ff=14336, vocab=128256)
LLAMA_70B = dict(d_model=8192, d_ff=28672, vocab=128256)


@dataclass
class ReadoutInputs:
    hidden: np.ndarray        # f16 [n_tokens, d_model]
    readout_tok: np.ndarray   # int32 [n_readout]
    norm_w: np.ndarray        # f16 [d_model]
    w_gate: np.ndarray        # f16 [d_ff, d_model]
    w_up: np.ndarray          # f16 [d_ff, d_model]
    w_down: np.ndarray        # f16 [d_model, d_ff]
    final_norm_w: np.ndarray  # f16 [d_model]
    head_ids: np.ndarray      # int32 [n_head_rows] vocabulary ids with drawn head rows
    head_rows: np.ndarray     # f16 [n_head_rows, d_model]
    vocab: int
    letter_ids: np.ndarray    # int32 [n_readout, ld]
    n_letters: np.ndarray     # int32 [n_readout]
    eps: float = 1e-5

    @property
    def d_model(self) -> int:
        return int(self.hidden.shape[1])

    @property
    def d_ff(self) -> int:
        return int(self.w_gate.shape[0])

    def lm_head(self) -> np.ndarray:
        """The full [vocab, d_model] head: zeros except the drawn rows."""
        h = np.zeros((self.vocab, self.d_model), np.float16)
        h[self.head_ids] = self.head_rows
        return h


def _f16(rng, shape, std: float) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float16)


def draw(seed: int, n_tokens: int, readout_tok: Sequence[int], d_model: int, d_ff: int,
         vocab: int = 1024, letters: int = 4, ld: Optional[int] = None,
         n_letters: Optional[Sequence[int]] = None, n_alphabet: int = 8) -> ReadoutInputs:
    """Inputs for readout rows readout_tok of n_tokens tokens. Letter ids come
    from an alphabet of n_alphabet distinct vocabulary ids (the answer
    letters); row r uses the first n_letters[r] of them (default ``letters``
    for every row), in alphabet order."""
    rng = np.random.default_rng(seed)
    readout_tok = np.asarray(readout_tok, np.int32)
    n = len(readout_tok)
    hidden = _f16(rng, (n_tokens, d_model), 1.0)
    norm_w = (1.0 + 0.1 * rng.standard_normal(d_model)).astype(np.float16)
    w_gate = _f16(rng, (d_ff, d_model), 1.0 / math.sqrt(d_model))
    w_up = _f16(rng, (d_ff, d_model), 1.0 / math.sqrt(d_model))
    w_down = _f16(rng, (d_model, d_ff), 1.0 / math.sqrt(d_ff))
    final_norm_w = (1.0 + 0.1 * rng.standard_normal(d_model)).astype(np.float16)
    alphabet = np.sort(rng.choice(vocab, size=n_alphabet, replace=False)).astype(np.int32)
    head_rows = _f16(rng, (n_alphabet, d_model), 2.0 / math.sqrt(d_model))
    nl = np.full(n, letters, np.int32) if n_letters is None else np.asarray(n_letters, np.int32)
    ld = int(nl.max()) if ld is None else ld
    ids = np.zeros((n, ld), np.int32)
    for r in range(n):
        ids[r, :nl[r]] = alphabet[:nl[r]]
    return ReadoutInputs(hidden, readout_tok, norm_w, w_gate, w_up, w_down, final_norm_w, alphabet,
                         head_rows, vocab, ids, nl)
