"""Host-side checks of the readout-only last layer through the C ABI (no GPU
needed): the documented workspace layout, a K split that depends on the weight
shape only, and the size limits."""
import os

import pytest

P = pytest.importorskip("prefix_tree_packed_amd")
from prefix_tree_packed_amd import binding as B  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libtreeattn.so not built")
    return B.load_library()


def test_readout_host_checks(lib):
    """readout_mlp_workspace_size: xn at byte 0, act at the next 256-byte
    boundary, then f32 partial sums of the down product for a K split that
    depends on the weight shape only; sizes outside the stated ranges fail."""
    def layout(n, dm, ff):
        xn = n * dm * 2
        act = (xn + 255) // 256 * 256
        part = act + (n * ff * 2 + 255) // 256 * 256
        return part, P.readout_mlp_workspace_size(n, dm, ff) - part
    for dm, ff in ((4096, 14336), (8192, 28672), (256, 768), (512, 1280)):
        splits = set()
        for n in (1, 17, 64, 300):
            part, rest = layout(n, dm, ff)
            assert rest % (n * dm * 4) == 0
            splits.add(rest // (n * dm * 4))
        assert len(splits) == 1                      # the same split whatever the row count
        s = splits.pop()
        assert s in (1, 2, 4, 8) and ff % (s * 256) == 0
    assert P.readout_mlp_workspace_size(0, 4096, 14336) == 0
    for bad in ((4, 200, 512), (4, 256, 300), (4, 32768, 512), (-1, 256, 512)):
        with pytest.raises(P.TreeAttnError):
            P.readout_mlp_workspace_size(*bad)
