"""readout_mlp_noalloc (the readout MLP for callers that cannot allocate: its
intermediates live in the library's fixed per-device scratch) against
readout_mlp with a caller workspace: the same kernels, so h_out must be
bitwise identical; two calls in a row, the second smaller than the first, so
a stale scratch from the first call cannot leak into the second. Sizes past
the scratch are refused with nothing written."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefix_tree_packed_amd as P
    P.load_library()
    return P


def _inputs(seed, n_tokens, n_rows, dm, ff):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    hidden = torch.randn((n_tokens, dm), device="cuda", generator=g).half()
    tok = torch.randint(0, n_tokens, (n_rows,), device="cuda", generator=g, dtype=torch.int32)
    norm_w = (1 + 0.1 * torch.randn(dm, device="cuda", generator=g)).half()
    w_gate_up = (torch.randn((2 * ff, dm), device="cuda", generator=g) / dm ** 0.5).half()
    w_down = (torch.randn((dm, ff), device="cuda", generator=g) / ff ** 0.5).half()
    return hidden, tok, norm_w, w_gate_up, w_down


def _both(P, inp, eps=1e-5):
    hidden, tok, norm_w, w_gate_up, w_down = inp
    n, dm = tok.shape[0], hidden.shape[1]
    want = torch.full((n, dm), float("nan"), dtype=torch.float16, device="cuda")
    got = torch.full((n, dm), float("nan"), dtype=torch.float16, device="cuda")
    P.readout_mlp(hidden, tok, norm_w, w_gate_up, w_down, want, eps=eps)
    P.readout_mlp_noalloc(hidden, tok, norm_w, w_gate_up, w_down, got, eps=eps)
    torch.cuda.synchronize()
    return want, got


def test_noalloc_matches_workspace_two_calls(P):
    print("[noalloc] llama-8b shape, 64 rows, then 1024/2560 with 7 rows", flush=True)
    big = _inputs(0, 300, 64, 4096, 14336)
    want, got = _both(P, big)
    assert torch.isfinite(want.float()).all().item()
    assert torch.equal(want, got), "first call: noalloc differs from the workspace path"
    del big
    small = _inputs(1, 40, 7, 1024, 2560)
    want, got = _both(P, small)
    assert torch.isfinite(want.float()).all().item()
    assert torch.equal(want, got), "second (smaller) call: noalloc differs from the workspace path"
    # and once more at the first shape's row count with the small model
    again = _inputs(2, 90, 64, 1024, 2560)
    want, got = _both(P, again)
    assert torch.equal(want, got)


def test_noalloc_refuses_sizes_beyond_its_scratch(P):
    print("[noalloc] 128 rows at the llama-8b shape: over the fixed scratch", flush=True)
    hidden, tok, norm_w, w_gate_up, w_down = _inputs(3, 200, 128, 4096, 14336)
    assert P.readout_mlp_workspace_size(128, 4096, 14336) > 16 << 20
    h_out = torch.full((128, 4096), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(P.TreeAttnError) as ei:
        P.readout_mlp_noalloc(hidden, tok, norm_w, w_gate_up, w_down, h_out)
    assert ei.value.status == 3 and "scratch" in ei.value.message
    torch.cuda.synchronize()
    assert bool((h_out == 7.0).all().item()), "a refused call writes nothing"
    # the same call with a workspace still works
    P.readout_mlp(hidden, tok, norm_w, w_gate_up, w_down, h_out)
    torch.cuda.synchronize()
    assert torch.isfinite(h_out.float()).all().item()
