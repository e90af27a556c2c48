"""Packing tokenized prompts into prefix trees, and batch formation (oracle).

TEST INFRASTRUCTURE ONLY: used by tests, never by the product path.

Sources: the architecture page "How basal-rs computes a decision":
* section 01, "Batch and prefix tree": the prompts of a batch are arranged
  into rows; each row is a tree whose shared prompt prefixes are computed once;
  a row holds up to 32,768 tokens; the tree is at most 8 blocks deep;
  identical prompts share a single output readout;
* section 01, "Validation and planning": a request's cost is the number of
  tokens to compute with shared prefixes counted once;
* section 01 "Batch and prefix tree" and section 04 ("max_batch_tokens"): a
  batch is the first queued request plus each later request that fits within
  8,192 tokens;
* section 03 "Packing": the shared prefix tree (template -> state -> question
  -> the two option orders) of the six-prompt example.

Readings (the pages describe the result, not the procedure):
* blocks are the maximal runs of a prefix trie over token ids in which no
  prompt branches off, ends, or ends one of its parts (a compressed trie cut
  at part boundaries too: the example's template, state, question and option
  order are separate blocks even where nothing branches between them, and the
  template must be a block of its own to be computed once); a prompt's
  readout is the last token of its block;
* blocks are laid out depth-first, children in the order their first prompt
  arrived;
* prompts go to rows in queue order: a prompt joins the current row if the
  row then still holds at most max_row_tokens tokens and is at most max_depth
  blocks deep, otherwise it starts a new row;
* a request fits a batch if the batch's summed request costs stay within the
  limit; tokens of a cached prefix (the template, computed once at start-up)
  are not part of a request's cost.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple


class _Trie:
    def __init__(self):
        self.children: List[Dict[int, int]] = [{}]   # node 0: the empty root
        self.order: List[List[int]] = [[]]          # child ids in arrival order
        self.token: List[int] = [-1]
        self.ends: List[int] = [0]                  # prompts ending at the node
        self.cut: List[bool] = [False]              # some prompt's part ends at the node

    def insert(self, seq: Sequence[int], parts: Sequence[int] = ()) -> int:
        cuts = set()
        at = 0
        for n in parts:
            at += n
            cuts.add(at)
        node = 0
        for k, tok in enumerate(seq):
            nxt = self.children[node].get(tok)
            if nxt is None:
                nxt = len(self.token)
                self.children[node][tok] = nxt
                self.order[node].append(nxt)
                self.children.append({})
                self.order.append([])
                self.token.append(tok)
                self.ends.append(0)
                self.cut.append(False)
            node = nxt
            if k + 1 in cuts:
                self.cut[node] = True
        self.ends[node] += 1
        return node

    def blocks(self):
        """Compressed trie in pre-order: list of (parent block, [nodes]) and
        the block holding each node."""
        out: List[Tuple[int, List[int]]] = []
        block_of: Dict[int, int] = {}

        def walk(start: int, parent: int):
            nodes = [start]
            node = start
            while len(self.order[node]) == 1 and self.ends[node] == 0 and not self.cut[node]:
                node = self.order[node][0]
                nodes.append(node)
            b = len(out)
            out.append((parent, nodes))
            for n in nodes:
                block_of[n] = b
            for c in self.order[node]:
                walk(c, b)

        for c in self.order[0]:
            walk(c, -1)
        return out, block_of


def _depths(blocks) -> List[int]:
    d = []
    for parent, _ in blocks:
        d.append(1 if parent < 0 else d[parent] + 1)
    return d


def pack(prompts: Sequence[Sequence[int]], parts=None, max_row_tokens: int = 32768,
         max_depth: int = 8):
    """Rows of packed prefix trees. parts[i] (optional) lists the lengths of
    prompt i's parts (template, state, question, ...), summing to its length.

    Returns (rows, row_tokens, placement): rows[r] = [(parent index in row,
    length), ...] in layout order; row_tokens[r] = the row's token ids in
    layout order; placement[i] = (row, block index in row, row-local index of
    prompt i's last token)."""
    rows_nodes: List[List[int]] = []
    cur: List[int] = []

    parts = [() for _ in prompts] if parts is None else [tuple(x) for x in parts]
    for i, (p, q) in enumerate(zip(prompts, parts)):
        if q and (sum(q) != len(p) or min(q) < 1):
            raise ValueError(f"parts of prompt {i} do not split it")

    def fits(ids):
        t = _Trie()
        for i in ids:
            t.insert(prompts[i], parts[i])
        blocks, _ = t.blocks()
        n_tok = sum(len(nodes) for _, nodes in blocks)
        return n_tok <= max_row_tokens and max(_depths(blocks)) <= max_depth

    for i, p in enumerate(prompts):
        if len(p) == 0:
            raise ValueError(f"prompt {i} is empty")
        if not fits([i]):
            raise ValueError(f"prompt {i} alone exceeds the row limits")
        if cur and not fits(cur + [i]):
            rows_nodes.append(cur)
            cur = []
        cur.append(i)
    if cur:
        rows_nodes.append(cur)

    rows, row_tokens, placement = [], [], [None] * len(prompts)
    for r, ids in enumerate(rows_nodes):
        t = _Trie()
        ends = [t.insert(prompts[i], parts[i]) for i in ids]
        blocks, block_of = t.blocks()
        starts, at = [], 0
        for _, nodes in blocks:
            starts.append(at)
            at += len(nodes)
        rows.append([(parent, len(nodes)) for parent, nodes in blocks])
        row_tokens.append([t.token[n] for _, nodes in blocks for n in nodes])
        local = {}
        for b, (_, nodes) in enumerate(blocks):
            for k, n in enumerate(nodes):
                local[n] = starts[b] + k
        for i, e in zip(ids, ends):
            placement[i] = (r, block_of[e], local[e])
    return rows, row_tokens, placement


def request_cost(prompts: Sequence[Sequence[int]], cached_prefix: int = 0) -> int:
    """Tokens a request's prompts need with shared prefixes counted once,
    not counting the first cached_prefix tokens of each prompt."""
    t = _Trie()
    for p in prompts:
        t.insert(p)
    # a node's depth is its token's position in every prompt through it
    stack = [(c, 0) for c in t.order[0]]
    n = 0
    while stack:
        node, pos = stack.pop()
        n += pos >= cached_prefix
        stack.extend((c, pos + 1) for c in t.order[node])
    return n


def form_batches(costs: Sequence[int], limit: int = 8192) -> List[int]:
    """Batch index of each request in queue order: each batch is the first
    request not yet batched plus every later one that still fits."""
    batch = [-1] * len(costs)
    b = 0
    for i in range(len(costs)):
        if batch[i] >= 0:
            continue
        total = costs[i]
        batch[i] = b
        for j in range(i + 1, len(costs)):
            if batch[j] < 0 and total + costs[j] <= limit:
                batch[j] = b
                total += costs[j]
        b += 1
    return batch
