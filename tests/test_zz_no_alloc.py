"""The transposed-convolution entry point that allocates nothing.

convT2d_pool_htanh_mean_tanh_noalloc runs the same kernels as
convT2d_pool_htanh_mean_tanh on the library's static per-device scratch in
place of a caller-supplied workspace.  Through the C ABI, two calls in a row
(the second smaller, so it runs on the scratch the first left behind) must
give, bit for bit, what the entry point with a workspace gives, and match
the oracle within the 1e-4 + 1e-4 |ref| tolerance.
"""
import numpy as np
import pytest

import oracle as O
from conv_inputs import CONVT, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import channel_convolution_epilogue_amd as m
    m.load()
    return m


def dev(a):
    return torch.from_numpy(a).cuda()


@pytest.mark.parametrize("cases", [
    [(16, 64, 64, 256, 256), (3, 64, 64, 34, 40)],   # the page's layer, then a smaller call
    [(5, 32, 16, 70, 52), (2, 8, 16, 18, 22)],        # other channel counts, ragged tiles
])
def test_noalloc_matches_workspace_entry_point(cce, cases):
    for i, (N, C_in, C_out, H, W) in enumerate(cases):
        p = make_inputs(CONVT, seed=1400 + 10 * i + N, N=N, C_in=C_in, H=H, W=W, C_out=C_out, k=3)
        x, w, b = dev(p["x"]), dev(p["w"]), dev(p["b"])
        ws = torch.full((cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(N, C_in, H, W, C_out),), 255,
                        dtype=torch.uint8, device="cuda")
        want = cce.convT2d_pool_htanh_mean_tanh(x, w, b, workspace=ws)
        out = torch.full((N, C_out, 1, 1), float("nan"), device="cuda")
        got = cce.convT2d_pool_htanh_mean_tanh_noalloc(x, w, b, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        g, r = got.cpu().numpy(), want.cpu().numpy()
        assert np.array_equal(g, r), f"call {i} (N={N}, {C_in}->{C_out}, {H}x{W}) differs from the workspace entry point"
        ref = O.convT2d_pool_htanh_mean_tanh(p["x"], p["w"], p["b"])
        err = np.abs(g[:, :, 0, 0].astype(np.float64) - ref)
        assert np.all(err <= 1e-4 + 1e-4 * np.abs(ref)), f"call {i}: max abs error {err.max():.3e}"
        print(f"noalloc call {i}: N={N} {C_in}->{C_out} {H}x{W}: bitwise equal, max abs err {err.max():.2e}",
              flush=True)


def test_noalloc_rejects_calls_beyond_its_scratch(cce):
    x = torch.empty((252, 64, 256, 256), device="cuda")
    w = torch.empty((64, 64, 3, 3), device="cuda")
    with pytest.raises(cce.CceError) as e:
        cce.convT2d_pool_htanh_mean_tanh_noalloc(x, w)
    assert e.value.status == -8
