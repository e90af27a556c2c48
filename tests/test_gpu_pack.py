"""Packing to attention on the GPU: tokenized prompts packed by the native
packer (tree_pack), the packed rows planned and run through tree attention,
and every token of every prompt compared with plain causal attention over that
prompt alone.

What it checks is the page's claim for packing (architecture page "How basal-rs
computes a decision", section 03 "Packing", "Attention over tree blocks": each
token gets what running its full prompt alone gives; section 01 "Batch and
prefix tree": prompts of a batch arranged into rows of trees, identical
prompts sharing one readout). A token's Q/K/V here are drawn per packed row
token, so a prompt's own Q/K/V are those of the row tokens on its
root-to-leaf path: the same values a model would compute, since a token's
vectors depend only on its prefix. The per-prompt reference is the oracle's
dense attention with a lower-triangular mask (the textbook causal case).
"""
import numpy as np
import pytest

from oracle import attention as OA
from oracle import tree as OT
from workloads import configs as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ATOL = 2e-3
RL2 = 1e-3


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefix_tree_packed_amd as P
    P.load_library()
    return P


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _prompts(seed):
    """A batch shaped like the page's example (template -> document -> question
    -> two option orders, with part marks), plus duplicates, a prompt that is a
    prefix of another, and unmarked prompts over a 4-letter alphabet so the trie
    branches at arbitrary tokens."""
    rng = np.random.default_rng(seed)
    ids = lambda n: rng.integers(0, 32000, n).tolist()  # noqa: E731
    template = ids(37)
    prompts, parts = [], []
    for _ in range(3):                       # documents
        doc = ids(int(rng.integers(60, 220)))
        for _ in range(int(rng.integers(1, 4))):   # questions
            q = ids(int(rng.integers(9, 40)))
            for _ in range(2):               # option orders
                opt = ids(int(rng.integers(5, 30)))
                prompts.append(template + doc + q + opt)
                parts.append([len(template), len(doc), len(q), len(opt)])
    prompts.append(list(prompts[1]))         # a duplicate: shares the readout
    parts.append(list(parts[1]))
    cut = len(template) + parts[0][1] + parts[0][2]
    prompts.append(prompts[0][:cut])         # ends inside the tree (not a leaf)
    parts.append(parts[0][:3])
    for _ in range(6):
        n = int(rng.integers(3, 90))
        prompts.append(rng.integers(0, 4, n).tolist())
        parts.append([n])
    return prompts, parts


def _paths(pk, desc):
    """For each prompt: its row and the row-local token indices of its
    root-to-leaf path (ancestor blocks, then its own block up to the readout)."""
    idx = OT.build_index(desc)
    first = desc.row_block_indptr
    out = []
    for r, b, ro in zip(pk["prompt_row"], pk["prompt_block"], pk["prompt_readout"]):
        g = int(first[r]) + int(b)
        toks = []
        for a in idx.block_anc[g] + [g]:
            s = idx.block_start[a]
            toks.extend(range(s, s + idx.block_len[a]))
        assert toks[-1] == ro, "readout at the prompt's last token"
        out.append((int(r), np.asarray(toks)))
    return idx, out


@pytest.mark.parametrize("seed,hq,hkv,d,row_cap,cached", [
    (0, 8, 2, 128, 32768, False),
    (1, 8, 2, 128, 900, False),     # several rows
    (2, 8, 1, 64, 1500, False),
    (3, 16, 2, 128, 32768, True),   # template cached: each row's first block is K/V already
    (4, 4, 4, 64, 700, True),
])
def test_packed_prompts_match_each_prompt_alone(P, seed, hq, hkv, d, row_cap, cached):
    prompts, parts = _prompts(seed)
    print(f"[pack->attention] seed={seed} heads={hq}/{hkv} d={d} row_cap={row_cap} cached={cached}",
          flush=True)
    pk = P.tree_pack(prompts, parts, max_row_tokens=row_cap)
    lens = [int(pk["block_len"][pk["row_block_indptr"][r]:pk["row_block_indptr"][r + 1]].sum())
            for r in range(len(pk["row_block_indptr"]) - 1)]
    first_len = [int(pk["block_len"][pk["row_block_indptr"][r]]) for r in range(len(lens))]
    qb = first_len if cached else [0] * len(lens)
    desc = W.TreeDesc(pk["row_block_indptr"], pk["block_parent"], pk["block_len"],
                      np.asarray(qb, np.int32), np.asarray(lens, np.int32))
    idx, paths = _paths(pk, desc)
    rng = np.random.default_rng(100 + seed)
    nkv = idx.num_kv_tokens
    q_row = rng.standard_normal((nkv, hq, d), dtype=np.float32).astype(np.float16)
    k_row = rng.standard_normal((nkv, hkv, d), dtype=np.float32).astype(np.float16)
    v_row = rng.standard_normal((nkv, hkv, d), dtype=np.float32).astype(np.float16)

    # forward order: each row's span [q_begin, len), rows in order
    fwd_of = {}
    fwd_rows = []
    for r, n in enumerate(lens):
        for i in range(qb[r], n):
            fwd_of[(r, i)] = len(fwd_rows)
            fwd_rows.append(idx.row_base[r] + i)
    fwd_rows = np.asarray(fwd_rows)
    assert len(fwd_rows) <= 8192
    scale = d ** -0.5
    plan = P.tree_attn_plan(desc, hq, hkv, d, scale)
    P.tree_attn_plan_upload(plan)
    q = _dev(q_row[fwd_rows])
    o = torch.empty((len(fwd_rows), hq, d), dtype=torch.float16, device="cuda")
    if cached:
        kc, vc = k_row.copy(), v_row.copy()
        kc[fwd_rows] = 0
        vc[fwd_rows] = 0
        P.tree_attn_forward_chunked(plan, q, _dev(k_row[fwd_rows]), _dev(v_row[fwd_rows]), _dev(kc),
                                    _dev(vc), o)
    else:
        P.tree_attn_forward(plan, q, _dev(k_row), _dev(v_row), o)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()

    # readouts: a prompt that ends at a leaf reads out where the plan says
    ex = P.tree_attn_plan_export(plan)
    leaf_tok = dict(zip(ex["leaf_block"].tolist(), ex["leaf_readout_tok"].tolist()))
    seen = set()
    for i, (r, path) in enumerate(paths):
        assert [int(t) for t in pk["row_tokens"][idx.row_base[r] + path]] == list(prompts[i]), \
            "the path spells the prompt"
        g = int(pk["row_block_indptr"][r]) + int(pk["prompt_block"][i])
        if idx.block_is_leaf[g]:
            assert leaf_tok[g] == fwd_of[(r, int(path[-1]))]
        # every computed token of the prompt against the prompt run alone
        rows = idx.row_base[r] + path
        want = OA.attention_dense(q_row[rows], k_row[rows], v_row[rows],
                                  np.tril(np.ones((len(rows), len(rows)), bool)), scale)
        sel = [j for j, t in enumerate(path) if (r, int(t)) in fwd_of]
        assert len(sel) == len(path) - (qb[r] if path[0] == 0 else 0)
        g_rows = [fwd_of[(r, int(path[j]))] for j in sel]
        seen.update(g_rows)
        if not sel:      # the whole prompt is the cached block
            continue
        diff = got[g_rows] - want[sel]
        err = float(np.abs(diff).max())
        rel = float(np.linalg.norm(diff) / np.linalg.norm(want[sel]))
        assert err <= ATOL and rel <= RL2, f"prompt {i}: max-abs {err:.2e} rel-L2 {rel:.2e}"
    assert seen == set(range(len(fwd_rows))), "every computed token belongs to some prompt"
    # identical prompts in one row share one readout (the duplicate of prompt 1;
    # prompts join rows in queue order, so under a tight row cap it may land in
    # a later row and get a readout of its own there)
    dup = len(prompts) - 8
    if len(lens) == 1 or pk["prompt_row"][dup] == pk["prompt_row"][1]:
        assert (pk["prompt_row"][dup], pk["prompt_block"][dup], pk["prompt_readout"][dup]) == \
            (pk["prompt_row"][1], pk["prompt_block"][1], pk["prompt_readout"][1])
