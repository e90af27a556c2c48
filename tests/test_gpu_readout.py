"""Readout-only last layer on the GPU (readout_mlp, letter_logits) against the
oracle (oracle/readout.py).

Bar, stage by stage, each stage fed the kernel's own output of the stage
before (xn and act are read from the workspace), so every check is element by
element and tight:
* a float16 result is a round-to-nearest of an f32 value; round-to-nearest is
  monotone, so if the f32 value lies within delta of the exact one the result
  lies in [rn16(exact - delta), rn16(exact + delta)];
* delta for a product accumulated in f32 over K terms by MFMA chains:
  (K/16 + 16) * 2^-24 * sum|terms| (products of f16 values are exact in f32;
  a chain of K/32 MFMAs, each adding 32 products, plus the fixed split and
  lane sums, with a factor 2 of margin); for the RMS norms a relative
  2^-18 (sum of squares of positive terms, square root, division, two
  products); for silu(g) * u in f32 a relative 2^-21;
* letter logits: the f64 dot of the head rows with rn16 of the exact final
  state, within the float16 brackets of that state plus the f32 dot bound.
End to end (the oracle run from the residual stream alone): letter logits
within 2e-3 max-abs and 1e-3 relative L2 (the attention output bar).
Batch invariance: a row's xn, act, h_out and logits are bitwise identical
alone, in batches of other sizes and at other positions.
"""
import math

import numpy as np
import pytest

from oracle import decision as OD
from oracle import readout as R
from oracle import tree as OT
from workloads import configs as W
from workloads import readout as WR

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefix_tree_packed_amd as P
    P.load_library()
    return P


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class _Run:
    """Device copies of one input set and the kernels' outputs."""

    def __init__(self, P, inp: WR.ReadoutInputs, lm_head=None):
        self.inp = inp
        n, dm, ff = len(inp.readout_tok), inp.d_model, inp.d_ff
        self.d = {k: _dev(getattr(inp, k)) for k in ("hidden", "readout_tok", "norm_w", "w_down",
                                                      "final_norm_w", "letter_ids", "n_letters")}
        self.d["w_gate_up"] = P.readout_pack_gate_up(_dev(inp.w_gate), _dev(inp.w_up))
        if lm_head is None:  # zeros except the drawn letter rows, built on the device
            lm_head = torch.zeros((inp.vocab, dm), dtype=torch.float16, device="cuda")
            lm_head[_dev(inp.head_ids).long()] = _dev(inp.head_rows)
        self.lm = lm_head
        self.h_out = torch.empty((n, dm), dtype=torch.float16, device="cuda")
        self.logits = torch.empty((n, inp.letter_ids.shape[1]), dtype=torch.float32, device="cuda")
        d = self.d
        ws = P.readout_mlp(d["hidden"], d["readout_tok"], d["norm_w"], d["w_gate_up"], d["w_down"],
                           self.h_out, eps=inp.eps)
        P.letter_logits(self.h_out, d["final_norm_w"], self.lm, d["letter_ids"], d["n_letters"], self.logits,
                        eps=inp.eps)
        torch.cuda.synchronize()
        xn, act = P.readout_workspace_views(ws, n, dm, ff)
        self.xn = xn.cpu().numpy().astype(np.float64)
        self.act = act.cpu().numpy().astype(np.float64)
        self.h = self.h_out.cpu().numpy().astype(np.float64)
        self.lg = self.logits.cpu().numpy().astype(np.float64)


def _inside(got, lo, hi, what):
    bad = ~((got >= lo) & (got <= hi))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside their bracket, first at {tuple(i)}: "
                             f"{got[tuple(i)]!r} not in [{lo[tuple(i)]!r}, {hi[tuple(i)]!r}]")


def _dot_bracket(a, w, k):
    """exact a @ w.T and its f32 accumulation bound."""
    return a @ w.T, (k / 16 + 16) * U * (np.abs(a) @ np.abs(w).T)


def _head_rows(inp, ids):
    """Rows of the full head for vocabulary ids (zero unless drawn)."""
    out = np.zeros((len(ids), inp.d_model), np.float16)
    k = np.searchsorted(inp.head_ids, ids)
    hit = (k < len(inp.head_ids)) & (inp.head_ids[np.minimum(k, len(inp.head_ids) - 1)] == ids)
    out[hit] = inp.head_rows[k[hit]]
    return out


def check_stages(run: _Run, cols=None):
    """Stage-by-stage bar; cols optionally samples the columns of act and h_out."""
    inp = run.inp
    f64 = lambda a: np.asarray(a, np.float64)  # noqa: E731
    dm, ff = inp.d_model, inp.d_ff
    h_r = f64(inp.hidden[inp.readout_tok])
    # 1. xn = rn16(rmsnorm(h) * w)
    e = R.rms_norm(h_r, f64(inp.norm_w), inp.eps)
    t = 2.0 ** -18 * np.abs(e)
    _inside(run.xn, R.rn16(e - t), R.rn16(e + t), "xn")
    # 2. act from the kernel's xn
    jc = np.arange(ff) if cols is None else cols[0]
    g, dg = _dot_bracket(run.xn, f64(inp.w_gate[jc]), dm)
    u, du = _dot_bracket(run.xn, f64(inp.w_up[jc]), dm)
    g_lo, g_hi, u_lo, u_hi = R.rn16(g - dg), R.rn16(g + dg), R.rn16(u - du), R.rn16(u + du)
    corners = [R.silu(a) * b for a in (g_lo, g_hi) for b in (u_lo, u_hi)]
    g_min = -1.2784645427610738  # where silu has its minimum
    mid = (g_lo < g_min) & (g_hi > g_min)
    corners += [np.where(mid, R.silu(g_min) * b, corners[0]) for b in (u_lo, u_hi)]
    f_lo, f_hi = np.minimum.reduce(corners), np.maximum.reduce(corners)
    slack = 2.0 ** -21 * np.maximum(np.abs(f_lo), np.abs(f_hi))
    _inside(run.act[:, jc], R.rn16(f_lo - slack), R.rn16(f_hi + slack), "act")
    # 3. h_out from the kernel's act
    jd = np.arange(dm) if cols is None else cols[1]
    d, dd = _dot_bracket(run.act, f64(inp.w_down[jd]), ff)
    hj = h_r[:, jd]
    lo, hi = hj + R.rn16(d - dd), hj + R.rn16(d + dd)
    _inside(run.h[:, jd], R.rn16(lo - U * np.abs(lo)), R.rn16(hi + U * np.abs(hi)), "h_out")
    # 4. letter logits from the kernel's h_out
    y = R.rms_norm(run.h, f64(inp.final_norm_w), inp.eps)
    t = 2.0 ** -18 * np.abs(y)
    y16 = R.rn16(y)
    wid = np.maximum(np.abs(R.rn16(y + t) - y16), np.abs(y16 - R.rn16(y - t)))
    for r in range(len(inp.readout_tok)):
        n = int(inp.n_letters[r])
        rows = f64(_head_rows(inp, inp.letter_ids[r, :n]))
        want = rows @ y16[r]
        tol = np.abs(rows) @ wid[r] + (dm / 16 + 16) * U * (np.abs(rows) @ np.abs(y16[r]))
        assert np.all(np.abs(run.lg[r, :n] - want) <= tol), f"logits row {r}"
        assert np.all(run.lg[r, n:] == 0), f"logits row {r} beyond its letters"


def check_end_to_end(run: _Run):
    inp = run.inp
    st = R.readout_mlp(inp.hidden, inp.readout_tok, inp.norm_w, inp.w_gate, inp.w_up, inp.w_down, inp.eps)
    _, want = R.letter_logits(st["h_out"], inp.final_norm_w, inp.eps, inp.lm_head(), inp.letter_ids,
                              inp.n_letters, inp.letter_ids.shape[1])
    err = np.abs(run.lg - want)
    rel = np.linalg.norm(run.lg - want) / np.linalg.norm(want)
    assert err.max() <= 2e-3 and rel <= 1e-3, f"end to end: max-abs {err.max():.2e}, rel-L2 {rel:.2e}"
    return want


SMALL = [  # (d_model, d_ff, readout rows)
    (256, 512, [0]),
    (256, 768, [3, 3, 9, 0, 17]),
    (512, 1536, list(range(0, 40, 3))),       # 14 rows, one 16-row fragment
    (512, 2048, list(range(0, 51, 3))),       # 17 rows: two fragments, ragged
    (1024, 1024, list(range(1, 67, 2))),      # 33 rows: the 64-row pass, ragged
    (768, 2560, list(range(64))),             # 64 rows exactly
    (256, 1280, [i % 90 for i in range(0, 300, 3)]),  # 100 rows: two passes, repeats
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_stages(P, case):
    dm, ff, rows = SMALL[case]
    print(f"[readout] d_model={dm} d_ff={ff} rows={len(rows)}", flush=True)
    rng = np.random.default_rng(case)
    nl = rng.integers(2, 9, len(rows))
    inp = WR.draw(10 + case, 96, rows, dm, ff, vocab=512, n_letters=nl, ld=8)
    run = _Run(P, inp)
    check_stages(run)
    check_end_to_end(run)


def test_decisions_from_letter_logits(P):
    """Readout rows at the leaves of the small doc-questions tree, two per
    question (the two option orders), through decision_readout."""
    wl = W.small_doc_questions(3)
    idx = OT.build_index(wl.forwards[0].tree)
    _, readout = OT.leaf_readouts(idx)
    n_tok = idx.num_q_tokens
    inp = WR.draw(7, n_tok, readout, 512, 1024, vocab=256, letters=4)
    run = _Run(P, inp)
    want = check_end_to_end(run)
    n_dec = len(readout) // 2
    row1 = np.arange(0, 2 * n_dec, 2, dtype=np.int32)
    row2 = row1 + 1
    nl = np.full(n_dec, 4, np.int32)
    T = np.linspace(0.5, 2.0, n_dec).astype(np.float32)
    pa = torch.empty((n_dec, 4), dtype=torch.float32, device="cuda")
    pc = torch.empty_like(pa)
    P.decision_readout(run.logits, _dev(row1), _dev(row2), _dev(nl), _dev(T), pa, pc)
    torch.cuda.synchronize()
    # the decision bar on the kernel's logits, and end to end from the oracle's
    pa_k, pc_k = OD.decisions(run.lg, row1, row2, nl, T)
    assert np.abs(pa.cpu().numpy() - pa_k).max() <= 1e-5 and np.abs(pc.cpu().numpy() - pc_k).max() <= 1e-5
    pa_o, pc_o = OD.decisions(want, row1, row2, nl, T)
    # softmax moves a probability by at most half the largest logit change, the
    # calibration by at most 1/T (<= 2) times that again
    assert np.abs(pa.cpu().numpy() - pa_o).max() <= 1e-3
    assert np.abs(pc.cpu().numpy() - pc_o).max() <= 2e-3


def test_batch_invariance(P):
    """A readout row's xn, act, h_out and logits are bitwise the same alone, in
    batches of 16, 40, 64 and 100 rows, at different positions."""
    dm, ff, n_tok = 512, 1536, 128
    target = 77
    results = []
    for n, pos in ((1, 0), (16, 9), (40, 33), (64, 0), (100, 71)):
        rows = [(target if i == pos else (i * 37) % n_tok) for i in range(n)]
        inp = WR.draw(5, n_tok, rows, dm, ff, vocab=256, letters=4)
        run = _Run(P, inp)
        results.append((run.xn[pos], run.act[pos], run.h[pos], run.lg[pos]))
    for r in results[1:]:
        for a, b, what in zip(results[0], r, ("xn", "act", "h_out", "logits")):
            assert np.array_equal(a, b), f"{what} differs with the batch"


def test_batch_invariance_llama8b_shape(P):
    """At the Llama-8B shape the gate/up workgroups run 7 waves (256 units of
    56 outputs; the small shapes above run 8): a row's act and h_out are
    bitwise the same alone, in passes of 16, 32 and 64 rows and in two passes
    of 128 rows, at different positions."""
    dims = WR.LLAMA_8B
    dm, ff, n_tok = dims["d_model"], dims["d_ff"], 256
    print("[readout batch invariance] llama8b", flush=True)
    inp = WR.draw(6, n_tok, [0], dm, ff, vocab=64, letters=2)
    d = {k: _dev(getattr(inp, k)) for k in ("hidden", "norm_w", "w_down")}
    d["w_gate_up"] = P.readout_pack_gate_up(_dev(inp.w_gate), _dev(inp.w_up))

    def mlp(rows):
        tok = torch.tensor(rows, dtype=torch.int32, device="cuda")
        h = torch.empty((len(rows), dm), dtype=torch.float16, device="cuda")
        ws = P.readout_mlp(d["hidden"], tok, d["norm_w"], d["w_gate_up"], d["w_down"], h, eps=inp.eps)
        torch.cuda.synchronize()
        _, act = P.readout_workspace_views(ws, len(rows), dm, ff)
        return act.cpu().numpy(), h.cpu().numpy()

    target = 77
    act0, h0 = mlp([target])
    assert np.isfinite(h0).all()
    for n, pos in ((16, 9), (32, 31), (64, 0), (200, 141)):
        rows = [(target if i == pos else (i * 37) % n_tok) for i in range(n)]
        act, h = mlp(rows)
        assert np.array_equal(act[pos], act0[0]), f"act differs in a batch of {n}"
        assert np.array_equal(h[pos], h0[0]), f"h_out differs in a batch of {n}"


@pytest.mark.parametrize("shape", ["llama8b", "llama70b"])
def test_full_size(P, shape):
    """The Llama-8B shape with 64 readout rows of 4 letters (every column), and
    the 70B shape with 14 rows of 2-8 letters (512 sampled columns per stage):
    the row counts of the readouts the bench times (config[1]'s and
    config[4]'s leaf readouts), so the same pass heights and workgroup
    shapes."""
    if shape == "llama8b":
        dims, rows, nl, cols = WR.LLAMA_8B, 64, None, None
    else:
        dims, rows, nl = WR.LLAMA_70B, 14, np.random.default_rng(1).integers(2, 9, 14)
    print(f"[readout full] {shape}", flush=True)
    rng = np.random.default_rng(2)
    readout = np.sort(rng.choice(7168, rows, replace=False)).astype(np.int32)
    inp = WR.draw(3, 7168, readout, dims["d_model"], dims["d_ff"], vocab=dims["vocab"], n_letters=nl,
                  ld=None if nl is None else 8)
    if shape == "llama70b":
        cols = (np.sort(rng.choice(dims["d_ff"], 512, replace=False)),
                np.sort(rng.choice(dims["d_model"], 512, replace=False)))
    run = _Run(P, inp)
    check_stages(run, cols)


def test_bad_device_values_give_nan(P):
    inp = WR.draw(4, 32, [1, 40, 2, -1], 256, 512, vocab=64, letters=3, ld=4)
    inp.letter_ids[2, 1] = 64                       # outside the vocabulary
    inp.n_letters[0] = 5                            # more than ld
    run = _Run(P, inp)
    assert np.isnan(run.h[1]).all() and np.isnan(run.h[3]).all()   # readout tokens 40, -1
    assert np.isnan(run.lg[0]).all()
    assert np.isnan(run.lg[2, 1]) and np.isfinite(run.lg[2, 0]) and np.isfinite(run.lg[2, 2])
    assert np.isfinite(run.h[[0, 2]]).all()


def test_gate_up_layout(P):
    """readout_pack_gate_up: rows 16i .. 16i+7 are gate rows 8i .. 8i+7, rows
    16i+8 .. 16i+15 the up rows of the same columns (bit-exact copy)."""
    rng = np.random.default_rng(8)
    g = rng.standard_normal((768, 256)).astype(np.float16)
    u = rng.standard_normal((768, 256)).astype(np.float16)
    got = P.readout_pack_gate_up(_dev(g), _dev(u)).cpu().numpy()
    want = np.concatenate([g.reshape(-1, 8, 256), u.reshape(-1, 8, 256)], axis=1).reshape(-1, 256)
    assert np.array_equal(got, want)


def test_argument_errors(P):
    inp = WR.draw(4, 32, [1, 2], 256, 512, vocab=64, letters=3)
    d = {k: _dev(getattr(inp, k)) for k in ("hidden", "readout_tok", "norm_w", "w_down")}
    d["w_gate_up"] = P.readout_pack_gate_up(_dev(inp.w_gate), _dev(inp.w_up))
    h_out = torch.empty((2, 256), dtype=torch.float16, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(P.TreeAttnError):
        P.readout_mlp(d["hidden"], d["readout_tok"], d["norm_w"], d["w_gate_up"], d["w_down"], h_out,
                      workspace=small)
    with pytest.raises(ValueError):  # wrong dtype
        P.readout_mlp(d["hidden"].float(), d["readout_tok"], d["norm_w"], d["w_gate_up"], d["w_down"], h_out)
    bad = torch.empty((3, 200), dtype=torch.float16, device="cuda")
    with pytest.raises(P.TreeAttnError):  # d_model not a multiple of 256
        P.readout_mlp(bad, d["readout_tok"], torch.ones(200, dtype=torch.float16, device="cuda"),
                      torch.empty((1024, 200), dtype=torch.float16, device="cuda"),
                      torch.empty((200, 512), dtype=torch.float16, device="cuda"),
                      torch.empty((2, 200), dtype=torch.float16, device="cuda"))
    with pytest.raises(P.TreeAttnError):  # d_ff not a multiple of 256
        P.readout_pack_gate_up(torch.empty((200, 256), dtype=torch.float16, device="cuda"),
                               torch.empty((200, 256), dtype=torch.float16, device="cuda"))
    lg = torch.empty((2, 300), dtype=torch.float32, device="cuda")
    with pytest.raises(P.TreeAttnError):  # ld > 255
        P.letter_logits(h_out, d["norm_w"], _dev(inp.lm_head()),
                        torch.zeros((2, 300), dtype=torch.int32, device="cuda"),
                        torch.full((2,), 3, dtype=torch.int32, device="cuda"), lg)


def test_letter_logits_narrow_rows(P):
    """letter_logits alone at a width that is a multiple of 8 but not of 256,
    one-letter rows and ld 1 .. 3, against the oracle within the stage bound."""
    rng = np.random.default_rng(12)
    dm, vocab = 264, 40
    h = (rng.standard_normal((5, dm)) * 3).astype(np.float16)
    w = (1 + 0.1 * rng.standard_normal(dm)).astype(np.float16)
    head = (rng.standard_normal((vocab, dm)) / math.sqrt(dm)).astype(np.float16)
    for ld in (1, 3):
        ids = rng.integers(0, vocab, (5, ld)).astype(np.int32)
        nl = np.minimum(rng.integers(1, 4, 5), ld).astype(np.int32)
        lg = torch.empty((5, ld), dtype=torch.float32, device="cuda")
        P.letter_logits(_dev(h), _dev(w), _dev(head), _dev(ids), _dev(nl), lg, eps=1e-5)
        torch.cuda.synchronize()
        got = lg.cpu().numpy().astype(np.float64)
        y = R.rms_norm(h.astype(np.float64), w.astype(np.float64), 1e-5)
        t = 2.0 ** -18 * np.abs(y)
        y16 = R.rn16(y)
        wid = np.maximum(np.abs(R.rn16(y + t) - y16), np.abs(y16 - R.rn16(y - t)))
        for r in range(5):
            rows = head[ids[r, :nl[r]]].astype(np.float64)
            tol = np.abs(rows) @ wid[r] + (dm / 16 + 16) * U * (np.abs(rows) @ np.abs(y16[r]))
            assert np.all(np.abs(got[r, :nl[r]] - rows @ y16[r]) <= tol)
            assert np.all(got[r, nl[r]:] == 0)


def test_no_readout_rows(P):
    """n_readout = 0 launches nothing and leaves the outputs alone."""
    inp = WR.draw(4, 8, [], 256, 512, vocab=16, letters=2, ld=2)
    w_gu = P.readout_pack_gate_up(_dev(inp.w_gate), _dev(inp.w_up))
    h_out = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    P.readout_mlp(_dev(inp.hidden), torch.empty(0, dtype=torch.int32, device="cuda"), _dev(inp.norm_w), w_gu,
                  _dev(inp.w_down), h_out)
    lg = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    P.letter_logits(h_out, _dev(inp.final_norm_w), _dev(inp.lm_head()),
                    torch.empty((0, 2), dtype=torch.int32, device="cuda"),
                    torch.empty(0, dtype=torch.int32, device="cuda"), lg)
    torch.cuda.synchronize()
