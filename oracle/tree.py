"""Index tables and the dense visibility mask of prefix-tree-packed rows (oracle).

TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the bench's CPU
baseline, never by the product path.

Source: the architecture page "How basal-rs computes a decision", section 03
"Packing" (sub-part "Attention over tree blocks") and section 01 "Request path"
(stage "Batch and prefix tree"). What it fixes:

* the prompts of a batch form rows; each row is a tree of blocks whose shared
  prefixes are computed once; before computation the tree becomes one row of
  tokens;
* a token sees the earlier tokens of its own block and the tokens of its
  ancestor blocks; sibling blocks are masked, so the result equals running each
  full (root-to-leaf) prompt on its own;
* a token's RoPE position is its position inside its own prompt;
* limits: a row holds at most 32,768 tokens, a forward at most 8,192, a tree is
  at most 8 blocks deep; request cost counts shared prefixes once.

Readings where the page is silent (each listed in the design notes):

* blocks are laid out in the order given, which must put a parent before its
  children; a row's token ``i`` lives at row-space index ``row_base[r] + i`` where
  rows are concatenated in order;
* "earlier tokens of its own block" includes the token itself (causal);
* positions are 0-based and count cached prefix tokens;
* there is no attention across rows, nor between separate trees of one row;
* a leaf (a block with no children) is read out at its last token.

Everything here is plain Python loops over the description; NumPy is used only
to hold arrays and to set mask slices.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

ROW_TOKEN_LIMIT = 32768      # section 01, "Batch and prefix tree"
FORWARD_TOKEN_LIMIT = 8192   # same place
DEPTH_LIMIT = 8              # same place ("tree depth of up to 8 blocks")


@dataclass
class TreeIndex:
    num_rows: int
    row_len: List[int]
    row_base: List[int]              # row-space start of each row
    row_q_begin: List[int]
    row_q_end: List[int]
    block_row: List[int]             # global block index -> row
    block_local: List[int]           # global block index -> index inside row
    block_parent: List[int]          # global parent index or -1
    block_len: List[int]
    block_start: List[int]           # row-local first token
    block_depth: List[int]           # blocks on the path root..block, itself included
    block_anc: List[List[int]]       # proper ancestors, root first (global indices)
    block_is_leaf: List[bool]

    @property
    def num_blocks(self) -> int:
        return len(self.block_len)

    @property
    def num_kv_tokens(self) -> int:
        return self.row_base[-1]

    @property
    def num_q_tokens(self) -> int:
        return sum(e - b for b, e in zip(self.row_q_begin, self.row_q_end))


def build_index(desc) -> TreeIndex:
    """Lay each row's blocks out in the given order and record ancestry.

    ``desc`` has the fields of the C-ABI tree description (``row_block_indptr``,
    ``block_parent`` (row-local), ``block_len``, ``row_q_begin``, ``row_q_end``).
    Follows section 03 ("the tree becomes one row of tokens"): block ``b`` of a
    row starts where the previous block of that row ended.
    """
    indptr = [int(x) for x in desc.row_block_indptr]
    parent_local = [int(x) for x in desc.block_parent]
    lens = [int(x) for x in desc.block_len]
    R = len(indptr) - 1
    idx = TreeIndex(R, [], [0], [int(x) for x in desc.row_q_begin],
                    [int(x) for x in desc.row_q_end], [], [], [], [], [], [], [], [])
    for r in range(R):
        a, b = indptr[r], indptr[r + 1]
        cursor = 0
        for g in range(a, b):
            local = g - a
            p_local = parent_local[g]
            p = -1 if p_local < 0 else a + p_local
            idx.block_row.append(r)
            idx.block_local.append(local)
            idx.block_parent.append(p)
            idx.block_len.append(lens[g])
            idx.block_start.append(cursor)
            cursor += lens[g]
            if p < 0:
                idx.block_depth.append(1)
                idx.block_anc.append([])
            else:
                idx.block_depth.append(idx.block_depth[p] + 1)
                idx.block_anc.append(idx.block_anc[p] + [p])
            idx.block_is_leaf.append(True)
            if p >= 0:
                idx.block_is_leaf[p] = False
        idx.row_len.append(cursor)
        idx.row_base.append(idx.row_base[-1] + cursor)
    return idx


def query_tokens(idx: TreeIndex):
    """Per query token of this forward (rows in order, each row's tokens
    ``[q_begin, q_end)``): row, global block, offset in block, position id and
    row-space index.

    Position id = sum of the ancestor blocks' lengths + offset in the own block:
    the token's index inside its own root-to-leaf prompt (section 03, RoPE
    position "is its position in its own prompt").
    """
    tok_row, tok_block, tok_offset, pos_id, row_pos = [], [], [], [], []
    for r in range(idx.num_rows):
        # blocks of a row are laid out one after another, so walking them in
        # order visits the row's tokens in increasing index
        for g in range(idx.num_blocks):
            if idx.block_row[g] != r:
                continue
            prefix = sum(idx.block_len[a] for a in idx.block_anc[g])
            for off in range(idx.block_len[g]):
                i = idx.block_start[g] + off
                if not (idx.row_q_begin[r] <= i < idx.row_q_end[r]):
                    continue
                tok_row.append(r)
                tok_block.append(g)
                tok_offset.append(off)
                pos_id.append(prefix + off)
                row_pos.append(idx.row_base[r] + i)
    as32 = lambda x: np.asarray(x, dtype=np.int32)  # noqa: E731
    return {"tok_row": as32(tok_row), "tok_block": as32(tok_block),
            "tok_offset": as32(tok_offset), "pos_id": as32(pos_id),
            "row_pos": np.asarray(row_pos, dtype=np.int64)}


def visible_ranges(idx: TreeIndex, block: int, offset: int) -> List[Tuple[int, int]]:
    """Row-space key ranges a token (``block``, ``offset``) may attend to: every
    ancestor block in full, and its own block up to and including itself
    (section 03, "Attention over tree blocks")."""
    r = idx.block_row[block]
    base = idx.row_base[r]
    out = []
    for a in idx.block_anc[block]:
        s = base + idx.block_start[a]
        out.append((s, s + idx.block_len[a]))
    s = base + idx.block_start[block]
    out.append((s, s + offset + 1))
    return out


def dense_mask(idx: TreeIndex, toks=None, sel=None) -> np.ndarray:
    """Boolean [n_query, T_kv] with M[t, u] true iff query token t may attend to
    row-space key u. ``sel`` optionally picks a subset of query tokens."""
    if toks is None:
        toks = query_tokens(idx)
    blocks = toks["tok_block"]
    offs = toks["tok_offset"]
    n = len(blocks)
    sel = range(n) if sel is None else list(sel)
    m = np.zeros((len(sel), idx.num_kv_tokens), dtype=bool)
    for j, t in enumerate(sel):
        for lo, hi in visible_ranges(idx, int(blocks[t]), int(offs[t])):
            m[j, lo:hi] = True
    return m


def leaf_readouts(idx: TreeIndex):
    """Leaves (blocks no block names as parent) whose last token is computed by
    this forward, in block order, with that token's index among this forward's
    query tokens. The readout sits at a prompt's last token (section 01, stage
    "GPU forward pass": logits only at readout positions)."""
    # forward index of each row's first query token
    q_off = [0]
    for r in range(idx.num_rows):
        q_off.append(q_off[-1] + idx.row_q_end[r] - idx.row_q_begin[r])
    leaf_block, readout = [], []
    for g in range(idx.num_blocks):
        if not idx.block_is_leaf[g]:
            continue
        r = idx.block_row[g]
        last = idx.block_start[g] + idx.block_len[g] - 1
        if idx.row_q_begin[r] <= last < idx.row_q_end[r]:
            leaf_block.append(g)
            readout.append(q_off[r] + last - idx.row_q_begin[r])
    return np.asarray(leaf_block, np.int32), np.asarray(readout, np.int32)


def costs(idx: TreeIndex):
    """Tokens computed by this forward with shared prefixes counted once (section
    01, stage "Validation and planning": request cost), and the tokens that
    running every root-to-leaf prompt separately would compute (the comparison
    of section 03)."""
    packed = idx.num_q_tokens
    separate = 0
    for g in range(idx.num_blocks):
        if idx.block_is_leaf[g]:
            separate += sum(idx.block_len[a] for a in idx.block_anc[g]) + idx.block_len[g]
    return packed, separate


def limit_violations(idx: TreeIndex) -> List[str]:
    """Which of the section-01 limits (row tokens, forward tokens, depth) the
    description breaks."""
    out = []
    if any(n > ROW_TOKEN_LIMIT for n in idx.row_len):
        out.append("row")
    if idx.num_q_tokens > FORWARD_TOKEN_LIMIT:
        out.append("forward")
    if any(d > DEPTH_LIMIT for d in idx.block_depth):
        out.append("depth")
    return out
