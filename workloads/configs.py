"""Seeded synthetic inputs with the shapes of the five prefix-tree workloads.

Conventions (all drawn with ``numpy.random.default_rng(seed)``):

* tree structure first, then, per forward, Q, K and V (float32 draws from N(0, 1)
  rounded to float16), then the decision inputs;
* K and V are drawn for every token of a row in *row space* (cached prefix tokens
  included), Q only for the tokens a forward computes;
* letter logits are float32 draws from N(0, 2) (standard deviation 2).

A tree is described the way the C-ABI takes it: per row, a CSR slice of blocks,
each with a parent index inside its row (-1 for a root) and a length, listed
parent-before-child (these generators use depth-first pre-order), plus the span
``[q_begin, q_end)`` of row tokens this forward computes. Tokens before
``q_begin`` are K/V that an earlier forward (or start-up, for the prompt template)
already put in the cache.

Nothing here computes positions, masks, attention or decisions.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

CONFIG_NAMES = {
    0: "tiny-tree-4x64",
    1: "llama8b-doc2048-32q",
    2: "60-small-requests",
    3: "long-row-32k-4chunks",
    4: "random-depth8-70b",
}

MAX_FORWARD_TOKENS = 8192
TEMPLATE_TOKENS = 96


@dataclass
class TreeDesc:
    row_block_indptr: np.ndarray  # int32 [R+1]
    block_parent: np.ndarray      # int32 [NB], index inside the row, -1 = root
    block_len: np.ndarray         # int32 [NB]
    row_q_begin: np.ndarray       # int32 [R]
    row_q_end: np.ndarray         # int32 [R]

    @property
    def num_rows(self) -> int:
        return int(self.row_block_indptr.shape[0] - 1)

    def row_lengths(self) -> np.ndarray:
        out = np.zeros(self.num_rows, np.int64)
        for r in range(self.num_rows):
            a, b = self.row_block_indptr[r], self.row_block_indptr[r + 1]
            out[r] = int(self.block_len[a:b].sum())
        return out

    def num_q_tokens(self) -> int:
        return int((self.row_q_end.astype(np.int64) - self.row_q_begin).sum())

    def with_q_range(self, q_begin: Sequence[int], q_end: Sequence[int]) -> "TreeDesc":
        return TreeDesc(self.row_block_indptr.copy(), self.block_parent.copy(),
                        self.block_len.copy(), np.asarray(q_begin, np.int32),
                        np.asarray(q_end, np.int32))


@dataclass
class Decisions:
    logits: np.ndarray     # float32 [n_rows, ld]; row i = readout i (leaf order)
    row1: np.ndarray       # int32 [n_dec] option order 1 row
    row2: np.ndarray       # int32 [n_dec] option order 2 row (options reversed)
    n_letters: np.ndarray  # int32 [n_dec]
    T: np.ndarray          # float32 [n_dec]

    @property
    def n_dec(self) -> int:
        return int(self.row1.shape[0])


@dataclass
class Forward:
    tree: TreeDesc
    q: np.ndarray          # float16 [T_q, Hq, D], this forward's query tokens
    k_row: np.ndarray      # float16 [T_rowspace, Hkv, D], K of every row token
    v_row: np.ndarray      # float16 [T_rowspace, Hkv, D]

    def row_base(self) -> np.ndarray:
        lens = self.tree.row_lengths()
        return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)

    def kv_new(self) -> Tuple[np.ndarray, np.ndarray]:
        """K/V of this forward's own tokens, in forward order (what a chunk adds)."""
        base = self.row_base()
        idx = []
        for r in range(self.tree.num_rows):
            idx.append(np.arange(base[r] + self.tree.row_q_begin[r],
                                 base[r] + self.tree.row_q_end[r]))
        idx = np.concatenate(idx) if idx else np.zeros(0, np.int64)
        return self.k_row[idx], self.v_row[idx]

    def cache_before(self) -> Tuple[np.ndarray, np.ndarray]:
        """Row-space K/V cache as it stands before this forward: rows' tokens before
        ``q_begin`` hold their K/V, everything else is zero."""
        base = self.row_base()
        kc = np.zeros_like(self.k_row)
        vc = np.zeros_like(self.v_row)
        for r in range(self.tree.num_rows):
            a = base[r]
            b = base[r] + self.tree.row_q_begin[r]
            kc[a:b] = self.k_row[a:b]
            vc[a:b] = self.v_row[a:b]
        return kc, vc

    @property
    def one_shot(self) -> bool:
        lens = self.tree.row_lengths()
        return bool(np.all(self.tree.row_q_begin == 0) and np.all(self.tree.row_q_end == lens))


@dataclass
class Workload:
    name: str
    hq: int
    hkv: int
    d: int
    forwards: List[Forward]
    decisions: Decisions
    chunked: bool = False          # forwards are consecutive chunks of the same rows
    notes: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# ----------------------------------------------------------------------------
# structure helpers (pure bookkeeping)
# ----------------------------------------------------------------------------

def desc_from_rows(rows: Sequence[Sequence[Tuple[int, int]]],
                   q_ranges: Optional[Sequence[Tuple[int, int]]] = None) -> TreeDesc:
    """rows[r] = list of (parent_index_in_row, length) in parent-before-child order.
    q_ranges[r] = (q_begin, q_end); default: the whole row."""
    indptr = [0]
    parents, lens = [], []
    for row in rows:
        for p, n in row:
            parents.append(p)
            lens.append(n)
        indptr.append(len(parents))
    if q_ranges is None:
        q_ranges = [(0, sum(n for _, n in row)) for row in rows]
    return TreeDesc(np.asarray(indptr, np.int32), np.asarray(parents, np.int32),
                    np.asarray(lens, np.int32),
                    np.asarray([a for a, _ in q_ranges], np.int32),
                    np.asarray([b for _, b in q_ranges], np.int32))


def _f16_normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


_TENSORS = [True]


def draw_forward(rng: np.random.Generator, tree: TreeDesc, hq: int, hkv: int, d: int) -> Forward:
    """Q for this forward's tokens, then K and V for every row-space token."""
    if not _TENSORS[0]:
        return Forward(tree, None, None, None)
    tq = tree.num_q_tokens()
    tkv = int(tree.row_lengths().sum())
    q = _f16_normal(rng, (tq, hq, d))
    k = _f16_normal(rng, (tkv, hkv, d))
    v = _f16_normal(rng, (tkv, hkv, d))
    return Forward(tree, q, k, v)


def _paired_decisions(rng: np.random.Generator, n_pairs: int, n_letters: int,
                      T: float = 1.0) -> Decisions:
    logits = (rng.standard_normal((2 * n_pairs, n_letters), dtype=np.float32) * 2.0)
    row1 = np.arange(0, 2 * n_pairs, 2, dtype=np.int32)
    return Decisions(logits.astype(np.float32), row1, row1 + 1,
                     np.full(n_pairs, n_letters, np.int32), np.full(n_pairs, T, np.float32))


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

def _config0(seed: int) -> Workload:
    rng = np.random.default_rng(seed)
    tree = desc_from_rows([[(-1, 64), (0, 32), (1, 24), (1, 24)]])
    fwd = draw_forward(rng, tree, 4, 4, 64)
    logits = (rng.standard_normal((2, 3), dtype=np.float32) * 2.0).astype(np.float32)
    dec = Decisions(logits, np.array([0, 0], np.int32), np.array([1, 1], np.int32),
                    np.array([3, 3], np.int32), np.array([1.0, 0.7], np.float32))
    return Workload(CONFIG_NAMES[0], 4, 4, 64, [fwd], dec)


def _question_tree(doc_parent: int, blocks: List[Tuple[int, int]], qlen: int,
                   l1: int, l2: int) -> None:
    q = len(blocks)
    blocks.append((doc_parent, qlen))
    blocks.append((q, l1))
    blocks.append((q, l2))


def _config1(seed: int, doc: int = 2048, nq: int = 32, qlen: int = 64, leaf: int = 48,
             template: int = TEMPLATE_TOKENS, hq: int = 32, hkv: int = 8, d: int = 128) -> Workload:
    rng = np.random.default_rng(seed)
    blocks: List[Tuple[int, int]] = [(-1, template), (0, doc)]
    for _ in range(nq):
        _question_tree(1, blocks, qlen, leaf, leaf)
    row_len = sum(n for _, n in blocks)
    tree = desc_from_rows([blocks], [(template, row_len)])
    fwd = draw_forward(rng, tree, hq, hkv, d)
    dec = _paired_decisions(rng, nq, 4)
    return Workload(CONFIG_NAMES[1], hq, hkv, d, [fwd], dec, chunked=True,
                    notes={"cached_template": template})


def _config2_requests(rng: np.random.Generator, n_req: int = 60):
    reqs = []
    for _ in range(n_req):
        doc = int(rng.integers(64, 257))
        nq = int(rng.integers(1, 5))
        qs = []
        for _ in range(nq):
            ql = int(rng.integers(16, 65))
            l1 = int(rng.integers(8, 33))
            l2 = int(rng.integers(8, 33))
            qs.append((ql, l1, l2))
        reqs.append((doc, qs))
    return reqs


def form_batches(costs: Sequence[int], limit: int = MAX_FORWARD_TOKENS) -> List[List[int]]:
    """The batch rule of the architecture page (request path, stage "Batch and
    prefix tree"; scheduling, max_batch_tokens): the first queued request plus
    every later one that still fits within ``limit`` tokens."""
    queue = list(range(len(costs)))
    batches = []
    while queue:
        batch = [queue[0]]
        total = costs[queue[0]]
        for r in queue[1:]:
            if total + costs[r] <= limit:
                batch.append(r)
                total += costs[r]
        taken = set(batch)
        queue = [r for r in queue if r not in taken]
        batches.append(batch)
    return batches


def _config2(seed: int, n_req: int = 60, hq: int = 32, hkv: int = 8, d: int = 128,
             template: int = TEMPLATE_TOKENS, limit: int = MAX_FORWARD_TOKENS) -> Workload:
    rng = np.random.default_rng(seed)
    reqs = _config2_requests(rng, n_req)
    costs = [doc + sum(a + b + c for a, b, c in qs) for doc, qs in reqs]
    batches = form_batches(costs, limit)
    forwards = []
    n_pairs = 0
    for batch in batches:
        blocks: List[Tuple[int, int]] = [(-1, template)]
        for r in batch:
            doc, qs = reqs[r]
            di = len(blocks)
            blocks.append((0, doc))
            for ql, l1, l2 in qs:
                _question_tree(di, blocks, ql, l1, l2)
                n_pairs += 1
        row_len = sum(n for _, n in blocks)
        forwards.append(desc_from_rows([blocks], [(template, row_len)]))
    fwds = [draw_forward(rng, t, hq, hkv, d) for t in forwards]
    dec = _paired_decisions(rng, n_pairs, 4)
    return Workload(CONFIG_NAMES[2], hq, hkv, d, fwds, dec, chunked=True,
                    notes={"cached_template": template, "batches": batches,
                           "requests_per_forward": [len(b) for b in batches]})


def _config3(seed: int, doc: int = 16384, nq: int = 96, qlen: int = 64, leaf: int = 48,
             chunk: int = MAX_FORWARD_TOKENS, hq: int = 32, hkv: int = 8, d: int = 128) -> Workload:
    rng = np.random.default_rng(seed)
    blocks: List[Tuple[int, int]] = [(-1, doc)]
    for _ in range(nq):
        _question_tree(0, blocks, qlen, leaf, leaf)
    row_len = sum(n for _, n in blocks)
    full = desc_from_rows([blocks])
    if _TENSORS[0]:
        q_all = _f16_normal(rng, (row_len, hq, d))
        k = _f16_normal(rng, (row_len, hkv, d))
        v = _f16_normal(rng, (row_len, hkv, d))
    else:
        q_all = k = v = None
    fwds = []
    for a in range(0, row_len, chunk):
        b = min(row_len, a + chunk)
        fwds.append(Forward(full.with_q_range([a], [b]),
                            None if q_all is None else q_all[a:b], k, v))
    dec = _paired_decisions(rng, nq, 4)
    return Workload(CONFIG_NAMES[3], hq, hkv, d, fwds, dec, chunked=True,
                    notes={"row_tokens": row_len, "shared_cache": True})


def random_tree_rows(rng: np.random.Generator, total: int, n_rows: int,
                     max_depth: int = 8, min_len: int = 16, max_len: int = 512,
                     max_children: int = 4) -> List[List[Tuple[int, int]]]:
    """Rows grown depth-first until each row's token budget is spent. A node at
    depth < max_depth draws 1..max_children children; block lengths are
    log-uniform in [min_len, max_len], cut to the remaining budget. Leftover
    budget goes into more depth-2 subtrees under the root."""
    budgets = [total // n_rows] * (n_rows - 1)
    budgets.append(total - sum(budgets))
    lo, hi = math.log(min_len), math.log(max_len)
    rows = []
    for budget0 in budgets:
        blocks: List[Tuple[int, int]] = []
        budget = [budget0]

        def grow(parent: int, depth: int) -> None:
            if budget[0] <= 0:
                return
            n = int(math.floor(math.exp(rng.uniform(lo, hi)) + 0.5))
            n = max(1, min(n, budget[0]))
            budget[0] -= n
            me = len(blocks)
            blocks.append((parent, n))
            if depth < max_depth and budget[0] > 0:
                k = int(rng.integers(1, max_children + 1))
                for _ in range(k):
                    grow(me, depth + 1)

        grow(-1, 1)
        while budget[0] > 0:
            grow(0, 2)
        rows.append(blocks)
    return rows


def _config4(seed: int, total: int = MAX_FORWARD_TOKENS, hq: int = 64, hkv: int = 8,
             d: int = 128) -> Workload:
    rng = np.random.default_rng(seed)
    n_rows = int(rng.integers(2, 7))
    rows = random_tree_rows(rng, total, n_rows)
    tree = desc_from_rows(rows)
    fwd = draw_forward(rng, tree, hq, hkv, d)
    # one decision per leaf (a block nobody names as parent), in block order
    n_leaves = 0
    for row in rows:
        has_child = [False] * len(row)
        for p, _ in row:
            if p >= 0:
                has_child[p] = True
        n_leaves += sum(1 for h in has_child if not h)
    n_letters = rng.integers(2, 9, size=n_leaves).astype(np.int32)
    T = rng.uniform(0.5, 2.0, size=n_leaves).astype(np.float32)
    logits = (rng.standard_normal((2 * n_leaves, 8), dtype=np.float32) * 2.0).astype(np.float32)
    row1 = np.arange(0, 2 * n_leaves, 2, dtype=np.int32)
    dec = Decisions(logits, row1, row1 + 1, n_letters, T)
    return Workload(CONFIG_NAMES[4], hq, hkv, d, [fwd], dec,
                    notes={"rows": n_rows, "blocks": int(tree.block_len.shape[0]),
                           "leaves": n_leaves})


def make_config(index: int, seed: int = 0, tensors: bool = True) -> Workload:
    """The workload of the given configuration index (0-4) for ``seed``. With
    ``tensors=False`` only the tree structure is drawn (Q/K/V are None and the
    decision inputs are not meaningful)."""
    _TENSORS[0] = tensors
    try:
        return {0: _config0, 1: _config1, 2: _config2, 3: _config3, 4: _config4}[index](seed)
    finally:
        _TENSORS[0] = True


# ----------------------------------------------------------------------------
# reduced shapes for parity tests (same structure kinds, oracle-sized)
# ----------------------------------------------------------------------------

def small_doc_questions(seed: int, doc: int = 300, nq: int = 3, qlen: int = 40, leaf: int = 21,
                        template: int = 37, hq: int = 8, hkv: int = 2, d: int = 128) -> Workload:
    """Template (cached) -> document -> questions -> two leaves, like the 8B-shaped
    workload but small enough for the oracle; lengths chosen off tile multiples."""
    return _config1(seed, doc=doc, nq=nq, qlen=qlen, leaf=leaf, template=template,
                    hq=hq, hkv=hkv, d=d)


def small_requests(seed: int, n_req: int = 12, limit: int = 1500, hq: int = 8, hkv: int = 2,
                   d: int = 128) -> Workload:
    return _config2(seed, n_req=n_req, hq=hq, hkv=hkv, d=d, limit=limit)


def small_long_row(seed: int, doc: int = 700, nq: int = 4, chunk: int = 512, hq: int = 8,
                   hkv: int = 2, d: int = 128) -> Workload:
    return _config3(seed, doc=doc, nq=nq, qlen=33, leaf=19, chunk=chunk, hq=hq, hkv=hkv, d=d)


def small_random(seed: int, total: int = 900, n_rows: Optional[int] = None, hq: int = 16,
                 hkv: int = 2, d: int = 128, max_len: int = 200) -> Workload:
    rng = np.random.default_rng(seed)
    if n_rows is None:
        n_rows = int(rng.integers(2, 5))
    rows = random_tree_rows(rng, total, n_rows, max_len=max_len, min_len=4)
    tree = desc_from_rows(rows)
    fwd = draw_forward(rng, tree, hq, hkv, d)
    dec = _paired_decisions(rng, 4, 5)
    return Workload("small-random", hq, hkv, d, [fwd], dec)
