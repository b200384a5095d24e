"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: every element within |gpu - ref| <= 1e-4 + 1e-4 * |ref| (the fp32
atol = rtol = 1e-4 tolerance of the l2_p90 problem statement), no NaN/Inf.
Small cases compare every element and cover several tiles, ragged tails,
odd sizes (scalar load/store paths), the minimum sizes and a NULL bias.
Every full-size workload runs in the launch configuration the benchmark
times and is compared with the oracle at every output (the N = 128
transposed-convolution workload is also marked slow), plus properties that
hold at any size (output range, determinism).  At the ABI's size limits the
outputs are sampled and computed one by one by the oracle.
"""
import math

import numpy as np
import pytest

import oracle as O
from conv_inputs import CONV2D, CONV3D, CONVT, TAIL_GELU, TAIL_POOL, make_inputs, workload_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ATOL = RTOL = 1e-4


@pytest.fixture(scope="module")
def cce():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import channel_convolution_epilogue_amd as m
    m.load()
    return m


def dev(a):
    return None if a is None else torch.from_numpy(a).cuda()


def assert_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance; worst at flat "
                             f"{i}: gpu={got.reshape(-1)[i]!r} ref={ref.reshape(-1)[i]!r}")
    print(f"{what}: max abs err {err.max():.3e} over {err.size} values", flush=True)


def sample_indices(total, count, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, total, size=count, dtype=np.int64)
    return np.unique(np.concatenate([idx, [0, 1, total // 2, total - 2, total - 1]]))


# ---------------------------------------------------------------------------
# Conv2d + ReLU + HardSwish
# ---------------------------------------------------------------------------

CONV2D_SMALL = [  # (N, H, W, bias)   covers: strips, ragged row groups and columns, odd sizes, minimum
    (2, 20, 20, True),
    (3, 37, 29, True),   # W % 4 != 0, plane % 4 != 0: scalar loads and stores; odd output height
    (1, 3, 3, True),     # one output pixel
    (5, 128, 128, True),
    (4, 11, 130, False),  # NULL bias, wide rows: 9 strips, the last one ragged
    (7, 64, 66, True),   # 7 images, output rows of 64 (no strip shift)
    (2, 6, 7, True),     # odd output width with plane % 4 == 0: strips shifted by 0..3 columns
    (3, 18, 19, True),   # the same with two strips per row and masked edge lanes
    (1, 6, 1100, True),  # rows wider than 1024: 69 strips, shifted, 16-byte loads
]


@pytest.mark.parametrize("N,H,W,bias", CONV2D_SMALL)
def test_conv2d_small(cce, N, H, W, bias):
    p = make_inputs(CONV2D, seed=100 + N, N=N, C_in=8, H=H, W=W, C_out=64, k=3)
    b = p["b"] if bias else None
    y = cce.conv2d_relu_hswish(dev(p["x"]), dev(p["w"]), dev(b))
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), O.conv2d_relu_hswish(p["x"], p["w"], b), f"conv2d N={N} {H}x{W}")


@pytest.mark.parametrize("H,W", [(19, 23), (20, 24), (21, 24)])
@pytest.mark.parametrize("C_in,C_out,k", [(4, 16, 1), (8, 32, 3), (16, 64, 3), (4, 64, 5), (8, 16, 5),
                                         (16, 32, 1), (8, 64, 1), (4, 32, 3)])
def test_conv2d_other_layer_shapes(cce, C_in, C_out, k, H, W):
    """Layer shapes beyond the page's 8 -> 64, 3 x 3 (other channel counts and
    kernel sizes): 19 x 23 takes the scalar loads and stores and leaves ragged
    strips and row groups; 20 x 24 and 21 x 24 (W and the output plane
    multiples of 4) the 16-byte ones, which for 16 or 32 output channels run
    2-row strips (21 x 24: an odd output height, so the last row pair has
    one row)."""
    p = make_inputs(CONV2D, seed=600 + C_in + C_out + k + W, N=2, C_in=C_in, H=H, W=W, C_out=C_out, k=k)
    y = cce.conv2d_relu_hswish(dev(p["x"]), dev(p["w"]), dev(p["b"]))
    torch.cuda.synchronize()
    assert y.shape == (2, C_out, H - k + 1, W - k + 1)
    assert_close(y.cpu().numpy(), O.conv2d_relu_hswish(p["x"], p["w"], p["b"]),
                 f"conv2d {C_in}->{C_out} k={k}")


def test_conv2d_workload_n8_full(cce):
    shape, p = workload_inputs("conv2d_relu_hswish_n8", seed=0)
    y = cce.conv2d_relu_hswish(dev(p["x"]), dev(p["w"]), dev(p["b"]))
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), O.conv2d_relu_hswish(p["x"], p["w"], p["b"]), "conv2d n8 full")


def test_conv2d_workload_n128_full(cce):
    shape, p = workload_inputs("conv2d_relu_hswish_n128", seed=0)
    y = cce.conv2d_relu_hswish(dev(p["x"]), dev(p["w"]), dev(p["b"]))
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert yh.shape == (128, 64, 126, 126)
    assert np.all(np.isfinite(yh)) and yh.min() >= 0.0  # HardSwish(ReLU(.)) >= 0
    assert_close(yh, O.conv2d_relu_hswish(p["x"], p["w"], p["b"]), "conv2d n128 every output")


# ---------------------------------------------------------------------------
# Conv3d + LeakyReLU + add + clamp + GELU
# ---------------------------------------------------------------------------

# GELU on [-1, 1] spans [min_t t*Phi(t), GELU(1)].
GELU_LO, GELU_HI = -0.16997120748, 0.84134474607


CONV3D_SMALL = [  # (N, D, H, W, bias)
    (2, 5, 12, 10, True),
    (1, 3, 3, 3, True),     # one output voxel
    (2, 6, 21, 19, True),   # ragged row tiles, odd widths: scalar paths
    (3, 4, 22, 64, False),  # NULL bias, 4 row tiles of 8 (last one 4 rows)
    (1, 16, 64, 64, True),  # one image of the Conv3d workload
    (1, 4, 20, 300, True),  # rows too wide for LDS: column tiles of 76, the last one ragged
    (1, 3, 11, 512, False),  # 512-wide rows: 7 column tiles
    (1, 3, 6, 700, True),   # wider still: 10 column tiles, the last ragged
]


@pytest.mark.parametrize("N,D,H,W,bias", CONV3D_SMALL)
def test_conv3d_small(cce, N, D, H, W, bias):
    p = make_inputs(CONV3D, seed=200 + N, N=N, C_in=8, D=D, H=H, W=W, C_out=64, k=3)
    s = p["s"] * 20  # wider than the workload's 0.02 so the add visibly matters
    b = p["b"] if bias else None
    y = cce.conv3d_lrelu_add_clamp_gelu(dev(p["x"]), dev(p["w"]), dev(b), dev(s), 0.2, -1.0, 1.0)
    torch.cuda.synchronize()
    ref = O.conv3d_lrelu_add_clamp_gelu(p["x"], p["w"], b, s, 0.2, -1.0, 1.0)
    assert_close(y.cpu().numpy(), ref, f"conv3d N={N} {D}x{H}x{W}")


@pytest.mark.parametrize("H,W,lo,hi", [(13, 21, -1.0, 1.0), (14, 24, -1.0, 1.0), (14, 24, -2.0, 1.5)])
@pytest.mark.parametrize("C_in,C_out", [(4, 16), (4, 64), (8, 32), (16, 16), (16, 64)])
def test_conv3d_other_layer_shapes(cce, C_in, C_out, H, W, lo, hi):
    """Channel counts beyond the page's 8 -> 64 (3 x 3 x 3).  13 x 21 takes the
    scalar loads and stores, 14 x 24 the 16-byte ones; clamp bounds inside
    [-1, 1] the polynomial GELU, wider ones erff.  16 -> 64 at these widths
    is one launch with 4-row tiles beside its 110 KB weight (wider rows take
    two 32-channel launches, tested below)."""
    p = make_inputs(CONV3D, seed=700 + C_in + C_out + W, N=2, C_in=C_in, D=5, H=H, W=W, C_out=C_out, k=3)
    y = cce.conv3d_lrelu_add_clamp_gelu(dev(p["x"]), dev(p["w"]), dev(p["b"]), dev(p["s"]), 0.2, lo, hi)
    torch.cuda.synchronize()
    assert y.shape == (2, C_out, 3, H - 2, W - 2)
    assert_close(y.cpu().numpy(), O.conv3d_lrelu_add_clamp_gelu(p["x"], p["w"], p["b"], p["s"], 0.2, lo, hi),
                 f"conv3d {C_in}->{C_out} {H}x{W} clamp [{lo}, {hi}]")


@pytest.mark.parametrize("N,D,H,W,lo,hi,bias", [
    (2, 4, 9, 64, -1.0, 1.0, True),    # 16-byte loads and stores, polynomial GELU
    (1, 5, 12, 50, -2.0, 1.5, True),   # scalar path (W % 4 != 0), erff
    (3, 3, 7, 40, -1.0, 1.0, False),   # no bias: both halves start from 0
])
def test_conv3d_16_to_64_wide_rows(cce, N, D, H, W, lo, hi, bias):
    """16 -> 64 on rows too wide for whole-row tiles beside the full weight:
    two launches of the 16 -> 32 kernel, each writing half of every image's
    output channels with its half of the weight, bias and s."""
    p = make_inputs(CONV3D, seed=790 + H + W, N=N, C_in=16, D=D, H=H, W=W, C_out=64, k=3)
    b = dev(p["b"]) if bias else None
    y = cce.conv3d_lrelu_add_clamp_gelu(dev(p["x"]), dev(p["w"]), b, dev(p["s"]), 0.2, lo, hi)
    torch.cuda.synchronize()
    assert y.shape == (N, 64, D - 2, H - 2, W - 2)
    ref = O.conv3d_lrelu_add_clamp_gelu(p["x"], p["w"], p["b"] if bias else None, p["s"], 0.2, lo, hi)
    assert_close(y.cpu().numpy(), ref, f"conv3d 16->64 N={N} {D}x{H}x{W} bias={bias}")


@pytest.mark.parametrize("H,W,lo,hi", [(5, 21, -1.0, 1.0), (6, 24, -1.0, 1.0), (6, 24, -2.0, 1.5)])
@pytest.mark.parametrize("C_in,C_out", [(4, 16), (8, 64), (16, 32), (16, 64)])
def test_conv3d_pointwise_layers(cce, C_in, C_out, H, W, lo, hi):
    """1 x 1 x 1 kernels (a ring of two planes, one K-step per 4 input
    channels): scalar and 16-byte paths, polynomial GELU and erff."""
    p = make_inputs(CONV3D, seed=750 + C_in + C_out + W, N=2, C_in=C_in, D=3, H=H, W=W, C_out=C_out, k=1)
    y = cce.conv3d_lrelu_add_clamp_gelu(dev(p["x"]), dev(p["w"]), dev(p["b"]), dev(p["s"]), 0.2, lo, hi)
    torch.cuda.synchronize()
    assert y.shape == (2, C_out, 3, H, W)
    assert_close(y.cpu().numpy(), O.conv3d_lrelu_add_clamp_gelu(p["x"], p["w"], p["b"], p["s"], 0.2, lo, hi),
                 f"conv3d 1x1x1 {C_in}->{C_out} {H}x{W} clamp [{lo}, {hi}]")


def test_conv3d_other_epilogue_parameters(cce):
    p = make_inputs(CONV3D, seed=7, N=2, C_in=8, D=5, H=10, W=12, C_out=64, k=3)
    x, w, b, s = (dev(p[k]) for k in "xwbs")
    for slope, lo, hi in [(0.01, -0.5, 0.75), (1.0, -3.0, 3.0), (0.2, 0.0, 0.0)]:
        y = cce.conv3d_lrelu_add_clamp_gelu(x, w, b, s, slope, lo, hi)
        torch.cuda.synchronize()
        ref = O.conv3d_lrelu_add_clamp_gelu(p["x"], p["w"], p["b"], p["s"], slope, lo, hi)
        assert_close(y.cpu().numpy(), ref, f"conv3d slope={slope} clamp=[{lo},{hi}]")


@pytest.mark.parametrize("N,D,H,W,lo,hi", [
    (2, 3, 11, 64, -2.0, 1.5),   # one output plane per block: only the last-tile reload
    (1, 7, 66, 64, -1.0, 1.0),   # 8 row blocks, the last of 8 rows; odd depth
    (3, 5, 13, 64, -0.5, 0.75),  # two row blocks, the second of 3 rows
])
def test_conv3d_page_layer_instance_edges(cce, N, D, H, W, lo, hi):
    """The page's layer on 64-wide rows (buffer-staged planes, buffer stores)
    at block and depth edges, with the polynomial GELU and with erff."""
    p = make_inputs(CONV3D, seed=260 + D + H, N=N, C_in=8, D=D, H=H, W=W, C_out=64, k=3)
    y = cce.conv3d_lrelu_add_clamp_gelu(dev(p["x"]), dev(p["w"]), dev(p["b"]), dev(p["s"]), 0.2, lo, hi)
    torch.cuda.synchronize()
    ref = O.conv3d_lrelu_add_clamp_gelu(p["x"], p["w"], p["b"], p["s"], 0.2, lo, hi)
    assert_close(y.cpu().numpy(), ref, f"conv3d N={N} {D}x{H}x{W} clamp [{lo}, {hi}]")


@pytest.mark.parametrize("N,D,H,lo,hi", [
    (4, 9, 16, -1.0, 1.0),    # 14 rows as 7 + 7: the second block starts mid-quad (7 x 62 = 434)
    (4, 9, 16, -2.0, 1.5),    # the same with erff (clamp bounds outside [-1, 1])
    (2, 4, 12, -1.0, 1.0),    # 10 rows as 5 + 5
    (3, 5, 4, -1.0, 1.0),     # one 2-row block per image
    (2, 4, 128, -1.0, 1.0),   # 126 rows in 16 blocks of 7 and 8
    (5, 6, 30, -1.0, 1.0),    # 28 rows as 7, 7, 7, 7
    (40, 3, 64, -1.0, 1.0),   # 320 row blocks: more than one round, so the rotation is not 0
])
def test_conv3d_balanced_row_tiles(cce, N, D, H, lo, hi):
    """The page's layer (64-wide rows) with an even number of output rows:
    balanced row blocks whose first voxel need not be quad-aligned (partial
    first and last quads), one- and two-block passes, rotated block order."""
    p = make_inputs(CONV3D, seed=280 + N + D + H, N=N, C_in=8, D=D, H=H, W=64, C_out=64, k=3)
    y = cce.conv3d_lrelu_add_clamp_gelu(dev(p["x"]), dev(p["w"]), dev(p["b"]), dev(p["s"]), 0.2, lo, hi)
    torch.cuda.synchronize()
    ref = O.conv3d_lrelu_add_clamp_gelu(p["x"], p["w"], p["b"], p["s"], 0.2, lo, hi)
    assert_close(y.cpu().numpy(), ref, f"conv3d N={N} {D}x{H}x64 clamp [{lo}, {hi}]")


def test_conv3d_workload_n128_full(cce):
    """Every one of the 440,860,672 outputs against the oracle, eight images
    at a time (the oracle's double output for the whole batch would be 3.5 GB)."""
    shape, p = workload_inputs("conv3d_lrelu_add_clamp_gelu_n128", seed=0)
    y = cce.conv3d_lrelu_add_clamp_gelu(dev(p["x"]), dev(p["w"]), dev(p["b"]), dev(p["s"]),
                                        shape["slope"], shape["lo"], shape["hi"])
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    del y
    assert yh.shape == (128, 64, 14, 62, 62)
    assert np.all(np.isfinite(yh))
    assert yh.min() >= GELU_LO - 1e-6 and yh.max() <= GELU_HI + 1e-6
    worst = 0.0
    for n0 in range(0, 128, 8):
        ref = O.conv3d_lrelu_add_clamp_gelu(np.ascontiguousarray(p["x"][n0:n0 + 8]), p["w"], p["b"], p["s"],
                                            shape["slope"], shape["lo"], shape["hi"])
        err = np.abs(yh[n0:n0 + 8].astype(np.float64) - ref)
        bad = err > ATOL + RTOL * np.abs(ref)
        assert not bad.any(), f"conv3d n128 images {n0}..{n0 + 7}: {int(bad.sum())} outputs outside tolerance"
        worst = max(worst, float(err.max()))
    print(f"conv3d n128 every output: max abs err {worst:.3e} over {yh.size} values", flush=True)


# ---------------------------------------------------------------------------
# ConvTranspose2d + MaxPool + Hardtanh + mean + tanh
# ---------------------------------------------------------------------------

CONVT_SMALL = [  # (N, H, W, bias)
    (2, 34, 34, True),    # 2 x 2 tiles, ragged
    (3, 37, 23, True),    # odd sizes: floor pooling drops the last row / column
    (2, 2, 2, True),      # one pooling window
    (1, 16, 32, False),   # exactly one tile, NULL bias
    (2, 64, 96, True),
]


@pytest.mark.parametrize("N,H,W,bias", CONVT_SMALL)
def test_convT_small(cce, N, H, W, bias):
    p = make_inputs(CONVT, seed=300 + N, N=N, C_in=64, H=H, W=W, C_out=64, k=3)
    b = p["b"] if bias else None
    y = cce.convT2d_pool_htanh_mean_tanh(dev(p["x"]), dev(p["w"]), dev(b))
    torch.cuda.synchronize()
    ref = O.convT2d_pool_htanh_mean_tanh(p["x"], p["w"], b)
    assert_close(y.cpu().numpy()[:, :, 0, 0], ref, f"convT N={N} {H}x{W}")


CONVT_LAYERS = [  # (C_in, C_out, N, H, W): W % 4 == 0 takes the 16-byte load path
    (8, 16, 2, 35, 42),
    (16, 64, 2, 34, 36),
    (32, 32, 3, 20, 44),
    (64, 16, 2, 33, 30),
    (128, 64, 1, 40, 40),
    (24, 32, 2, 18, 26),
    (64, 32, 1, 16, 32),
]


@pytest.mark.parametrize("C_in,C_out,N,H,W", CONVT_LAYERS)
def test_convT_other_layer_shapes(cce, C_in, C_out, N, H, W):
    """Channel counts beyond the page's 64 -> 64: C_in / 8 K chunks, C_out / 16
    MFMA column blocks, C_out partial sums per tile."""
    p = make_inputs(CONVT, seed=800 + C_in + C_out, N=N, C_in=C_in, H=H, W=W, C_out=C_out, k=3)
    y = cce.convT2d_pool_htanh_mean_tanh(dev(p["x"]), dev(p["w"]), dev(p["b"]))
    torch.cuda.synchronize()
    assert y.shape == (N, C_out, 1, 1)
    ref = O.convT2d_pool_htanh_mean_tanh(p["x"], p["w"], p["b"])
    assert_close(y.cpu().numpy()[:, :, 0, 0], ref, f"convT {C_in}->{C_out} N={N} {H}x{W}")


def garbage_workspace(nbytes):
    """A workspace whose every byte is 0xFF: no call may rely on its contents."""
    return torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")


def test_convT_workspace_shared_between_layer_shapes(cce):
    """One workspace, never cleared, serves calls of different channel counts in turn."""
    shapes = [(64, 64, 3, 36, 40), (8, 16, 5, 22, 18), (32, 32, 2, 48, 20)]
    need = max(cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(N, ci, H, W, co) for ci, co, N, H, W in shapes)
    ws = garbage_workspace(need)
    ins = [make_inputs(CONVT, seed=900 + i, N=N, C_in=ci, H=H, W=W, C_out=co, k=3)
           for i, (ci, co, N, H, W) in enumerate(shapes)]
    for rep in range(2):
        for (ci, co, N, H, W), p in zip(shapes, ins):
            y = cce.convT2d_pool_htanh_mean_tanh(dev(p["x"]), dev(p["w"]), dev(p["b"]), workspace=ws)
            torch.cuda.synchronize()
            assert_close(y.cpu().numpy()[:, :, 0, 0], O.convT2d_pool_htanh_mean_tanh(p["x"], p["w"], p["b"]),
                         f"convT shared workspace {ci}->{co} pass {rep}")


def test_convT_workspace_reused_by_more_images_than_before(cce):
    """Regression: the per-image counters occupy N * 4 bytes (rounded up to
    256) ahead of the prepared weight, so a call with more images than the
    previous user of the workspace finds the previous call's weight where its
    counters lie.  Each call zeroes its own counters first: N = 16 at 256 x 256
    followed by N = 100 at 32 x 32 (and back) on one workspace both match the
    oracle."""
    cases = [(16, 256, 256), (100, 32, 32), (16, 256, 256), (100, 32, 32)]
    need = max(cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(N, 64, H, W, 64) for N, H, W in cases)
    ws = garbage_workspace(need)
    refs = {}
    for i, (N, H, W) in enumerate(cases):
        p = make_inputs(CONVT, seed=1300 + N, N=N, C_in=64, H=H, W=W, C_out=64, k=3)
        if (N, H, W) not in refs:
            refs[(N, H, W)] = O.convT2d_pool_htanh_mean_tanh(p["x"], p["w"], p["b"])
        y = cce.convT2d_pool_htanh_mean_tanh(dev(p["x"]), dev(p["w"]), dev(p["b"]), workspace=ws)
        torch.cuda.synchronize()
        assert_close(y.cpu().numpy()[:, :, 0, 0], refs[(N, H, W)], f"convT reused workspace call {i}: N={N} {H}x{W}")


def test_convT_hardtanh_bounds_and_saturation(cce):
    p = make_inputs(CONVT, seed=9, N=2, C_in=64, H=20, W=18, C_out=64, k=3)
    x, w = dev(p["x"]), dev(p["w"])
    for lo, hi, scale in [(-0.25, 0.5, 1.0), (-1.0, 1.0, 8.0)]:
        b = (p["b"] * scale).astype(np.float32)
        y = cce.convT2d_pool_htanh_mean_tanh(x, w, dev(b), htanh_lo=lo, htanh_hi=hi)
        torch.cuda.synchronize()
        ref = O.convT2d_pool_htanh_mean_tanh(p["x"], p["w"], b, lo=lo, hi=hi)
        assert_close(y.cpu().numpy()[:, :, 0, 0], ref, f"convT hardtanh [{lo},{hi}]")


def test_convT_workspace_reuse_across_shapes_and_determinism(cce):
    p1 = make_inputs(CONVT, seed=11, N=4, C_in=64, H=48, W=40, C_out=64, k=3)
    p2 = make_inputs(CONVT, seed=12, N=2, C_in=64, H=18, W=70, C_out=64, k=3)
    x1, w1, b1 = dev(p1["x"]), dev(p1["w"]), dev(p1["b"])
    x2, w2, b2 = dev(p2["x"]), dev(p2["w"]), dev(p2["b"])
    need = max(cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(4, 64, 48, 40, 64),
               cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(2, 64, 18, 70, 64))
    ws = garbage_workspace(need)
    outs1, outs2 = [], []
    for _ in range(3):
        outs1.append(cce.convT2d_pool_htanh_mean_tanh(x1, w1, b1, workspace=ws).cpu().numpy())
        outs2.append(cce.convT2d_pool_htanh_mean_tanh(x2, w2, b2, workspace=ws).cpu().numpy())
    for o in outs1[1:]:
        assert np.array_equal(o, outs1[0]), "convT result not bitwise reproducible"
    for o in outs2[1:]:
        assert np.array_equal(o, outs2[0]), "convT result not bitwise reproducible"
    assert_close(outs1[0][:, :, 0, 0], O.convT2d_pool_htanh_mean_tanh(p1["x"], p1["w"], p1["b"]), "convT reuse A")
    assert_close(outs2[0][:, :, 0, 0], O.convT2d_pool_htanh_mean_tanh(p2["x"], p2["w"], p2["b"]), "convT reuse B")


def test_conv3d_alternating_tile_sizes(cce):
    """One kernel instance launched with a different LDS size on each call
    (rows of 20 and 44 floats give different plane rings), back and forth,
    with a 64-wide call of another instance in between: every call matches
    the oracle, so the cached launch set-up follows the LDS size."""
    shapes = [(4, 12, 20), (4, 12, 44), (3, 10, 64), (4, 12, 20), (4, 12, 44)]
    ins = {}
    for i, (D, H, W) in enumerate(shapes):
        if (D, H, W) not in ins:
            p = make_inputs(CONV3D, seed=1100 + i, N=2, C_in=8, D=D, H=H, W=W, C_out=64, k=3)
            ins[(D, H, W)] = (p, O.conv3d_lrelu_add_clamp_gelu(p["x"], p["w"], p["b"], p["s"]))
    for D, H, W in shapes:
        p, ref = ins[(D, H, W)]
        y = cce.conv3d_lrelu_add_clamp_gelu(dev(p["x"]), dev(p["w"]), dev(p["b"]), dev(p["s"]), 0.2, -1.0, 1.0)
        torch.cuda.synchronize()
        assert_close(y.cpu().numpy(), ref, f"conv3d alternating W={W}")


def test_calls_on_two_streams_at_once(cce):
    """Work enqueued on two streams runs concurrently; each stream's results
    are bit-identical to the same calls made one after another (none of the
    kernels reorders its arithmetic from run to run), and those match the
    oracle.  Each stream's transposed-convolution call uses its own
    workspace."""
    p2 = make_inputs(CONV2D, seed=1201, N=3, C_in=8, H=40, W=36, C_out=64, k=3)
    p3 = make_inputs(CONV3D, seed=1202, N=1, C_in=8, D=6, H=20, W=24, C_out=64, k=3)
    pt = [make_inputs(CONVT, seed=1203 + i, N=2, C_in=64, H=32, W=34, C_out=64, k=3) for i in range(2)]
    x2, w2, b2 = dev(p2["x"]), dev(p2["w"]), dev(p2["b"])
    x3, w3, b3, s3 = dev(p3["x"]), dev(p3["w"]), dev(p3["b"]), dev(p3["s"])
    xt = [(dev(p["x"]), dev(p["w"]), dev(p["b"])) for p in pt]
    need = cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(2, 64, 32, 34, 64)
    wss = [garbage_workspace(need) for _ in range(2)]

    def run_a():
        return (cce.conv2d_relu_hswish(x2, w2, b2),
                cce.convT2d_pool_htanh_mean_tanh(*xt[0], workspace=wss[0]))

    def run_b():
        return (cce.conv3d_lrelu_add_clamp_gelu(x3, w3, b3, s3, 0.2, -1.0, 1.0),
                cce.convT2d_pool_htanh_mean_tanh(*xt[1], workspace=wss[1]))

    torch.cuda.synchronize()
    serial = [t.cpu().numpy() for t in run_a() + run_b()]
    assert_close(serial[0], O.conv2d_relu_hswish(p2["x"], p2["w"], p2["b"]), "two streams: conv2d")
    assert_close(serial[2], O.conv3d_lrelu_add_clamp_gelu(p3["x"], p3["w"], p3["b"], p3["s"]),
                 "two streams: conv3d")
    for i, k in ((1, 0), (3, 1)):
        assert_close(serial[i][:, :, 0, 0], O.convT2d_pool_htanh_mean_tanh(pt[k]["x"], pt[k]["w"], pt[k]["b"]),
                     f"two streams: convT {k}")

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        with torch.cuda.stream(s1):
            a = run_a()
        with torch.cuda.stream(s2):
            b = run_b()
        torch.cuda.synchronize()
        for got, want, what in zip(a + b, serial, ("conv2d", "convT 0", "conv3d", "convT 1")):
            assert np.array_equal(got.cpu().numpy(), want), f"two streams, pass {rep}: {what} differs from serial"


def check_convT_workload_full(cce, name):
    """Every output of a full-size workload against the oracle, in the launch
    configuration the benchmark times, plus bitwise determinism and range."""
    shape, p = workload_inputs(name, seed=0)
    x, w, b = dev(p["x"]), dev(p["w"]), dev(p["b"])
    need = cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(shape["N"], 64, 256, 256, 64)
    ws = garbage_workspace(need)
    y = cce.convT2d_pool_htanh_mean_tanh(x, w, b, workspace=ws)
    y2 = cce.convT2d_pool_htanh_mean_tanh(x, w, b, workspace=ws)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()[:, :, 0, 0]
    assert np.array_equal(yh, y2.cpu().numpy()[:, :, 0, 0]), "not bitwise reproducible"
    assert np.all(np.abs(yh) <= math.tanh(1.0) + 1e-6)
    del x, w, b, y, y2, ws
    ref = O.convT2d_pool_htanh_mean_tanh(p["x"], p["w"], p["b"])
    assert_close(yh, ref, f"{name} every output")


def test_convT_workload_n16_full(cce):
    check_convT_workload_full(cce, "convT2d_pool_htanh_mean_tanh_n16")


@pytest.mark.slow
def test_convT_workload_n128_full(cce):
    check_convT_workload_full(cce, "convT2d_pool_htanh_mean_tanh_n128")


# ---------------------------------------------------------------------------
# Epilogue-only operators over a precomputed convolution output
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,C,H,W", [(2, 3, 256, 256), (3, 2, 37, 23), (1, 1, 2, 2), (2, 5, 20, 30),
                                     (4, 64, 64, 64)])
def test_pool_tail_small(cce, N, C, H, W):
    p = make_inputs(TAIL_POOL, seed=400 + N * C, N=N, C=C, H=H, W=W)
    z = p["z"] * np.float32(0.7)
    y = cce.pool_htanh_mean_tanh(dev(z))
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy()[:, :, 0, 0], O.pool_htanh_mean_tanh(z), f"pool tail N={N} C={C} {H}x{W}")


@pytest.mark.parametrize("pk,ps,H,W", [(3, 2, 37, 23), (2, 3, 20, 31), (1, 1, 9, 7), (3, 1, 12, 12),
                                       (4, 4, 64, 64), (5, 3, 17, 40), (2, 2, 9, 14)])
def test_pool_tail_general_window_and_stride(cce, pk, ps, H, W):
    """General MaxPool2d(k, s): overlapping, gapped and degenerate windows (the
    general path), and 2/2 on a width that is not a multiple of 4 (scalar path)."""
    p = make_inputs(TAIL_POOL, seed=450 + 10 * pk + ps, N=2, C=5, H=H, W=W)
    z = p["z"] * np.float32(0.7)
    y = cce.pool_htanh_mean_tanh(dev(z), pk, ps)
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy()[:, :, 0, 0], O.pool_htanh_mean_tanh(z, pk, ps),
                 f"pool tail k={pk} s={ps} {H}x{W}")


def test_pool_tail_workload_full(cce):
    shape, p = workload_inputs("pool_htanh_mean_tanh_n128", seed=0)
    y = cce.pool_htanh_mean_tanh(dev(p["z"]))
    y2 = cce.pool_htanh_mean_tanh(dev(p["z"]))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y2.cpu().numpy())
    assert_close(y.cpu().numpy()[:, :, 0, 0], O.pool_htanh_mean_tanh(p["z"]), "pool tail n128 full")


@pytest.mark.parametrize("N,C,D,H,W", [(2, 64, 3, 10, 12), (1, 3, 1, 1, 7), (3, 5, 2, 9, 11),
                                       (1, 64, 14, 62, 62),
                                       (3, 5, 1, 1, 4),    # one quad per plane, odd channel count
                                       (2, 1, 1, 2, 8),    # one channel
                                       (5, 7, 2, 3, 12)])  # ragged last one-wave workgroup
def test_elementwise_tail_small(cce, N, C, D, H, W):
    p = make_inputs(TAIL_GELU, seed=500 + N * C, N=N, C=C, D=D, H=H, W=W)
    s = p["s"] * 20
    for slope, lo, hi in [(0.2, -1.0, 1.0), (0.1, -2.0, 3.0)]:
        y = cce.lrelu_add_clamp_gelu(dev(p["z"]), dev(s), slope, lo, hi)
        torch.cuda.synchronize()
        assert_close(y.cpu().numpy(), O.lrelu_add_clamp_gelu_array(p["z"], s, slope, lo, hi),
                     f"elementwise tail {N}x{C}x{D}x{H}x{W} clamp [{lo},{hi}]")


@pytest.mark.parametrize("slope,lo,hi", [(0.2, -1.0, 1.0), (1.0, -1.0, 1.0), (1.5, -0.5, 0.25),
                                          (-0.3, -1.0, 1.0), (0.2, -3.0, 4.0)])
def test_epilogue_fp32_accuracy(cce, slope, lo, hi):
    """The LeakyReLU/add/clamp/GELU chain on a dense sweep of inputs, held to
    fp32 accuracy (2e-7 + 2e-7 |ref|: a few roundings of the fp32 chain)
    rather than the operators' 1e-4: covers the polynomial GELU (clamp inside
    [-1, 1]), erff (clamp outside), slopes above 1 and below 0 (the median
    form of LeakyReLU)."""
    z = np.linspace(-6.0, 6.0, 1 << 20).astype(np.float32).reshape(1, 4, -1)
    s = np.array([0.0, 0.37, -0.81, 1.9], np.float32)
    y = cce.lrelu_add_clamp_gelu(dev(z), dev(s), slope, lo, hi)
    torch.cuda.synchronize()
    ref = O.lrelu_add_clamp_gelu_array(z, s, slope, lo, hi)
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref) - 2e-7 * np.abs(ref)
    assert err.max() < 2e-7, f"max excess error {err.max():.3e} (slope {slope}, clamp [{lo}, {hi}])"


@pytest.mark.parametrize("S", [4096 * 3 + 12, 999])
def test_elementwise_tail_in_place(cce, S):
    """y may be z: the in-place call matches the out-of-place one bit for bit
    (16-byte path with a ragged last chunk, and the scalar path)."""
    p = make_inputs(TAIL_GELU, seed=520 + S, N=2, C=3, D=1, H=1, W=S)
    z = dev(p["z"])
    ref = cce.lrelu_add_clamp_gelu(z, dev(p["s"]), 0.2, -1.0, 1.0)
    zz = z.clone()
    out = cce.lrelu_add_clamp_gelu(zz, dev(p["s"]), 0.2, -1.0, 1.0, out=zz)
    torch.cuda.synchronize()
    assert out.data_ptr() == zz.data_ptr()
    assert torch.equal(zz, ref)


def test_elementwise_tail_workload_full(cce):
    """Every element of the [128, 64, 14, 62, 62] workload, eight images at a time."""
    shape, p = workload_inputs("lrelu_add_clamp_gelu_n128", seed=0)
    y = cce.lrelu_add_clamp_gelu(dev(p["z"]), dev(p["s"]), shape["slope"], shape["lo"], shape["hi"])
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    del y
    assert np.all(np.isfinite(yh)) and yh.min() >= GELU_LO - 1e-6 and yh.max() <= GELU_HI + 1e-6
    worst = 0.0
    for n0 in range(0, shape["N"], 8):
        ref = O.lrelu_add_clamp_gelu_array(p["z"][n0:n0 + 8], p["s"], shape["slope"], shape["lo"], shape["hi"])
        err = np.abs(yh[n0:n0 + 8].astype(np.float64) - ref)
        bad = err > ATOL + RTOL * np.abs(ref)
        assert not bad.any(), f"elementwise tail images {n0}..{n0 + 7}: {int(bad.sum())} outside tolerance"
        worst = max(worst, float(err.max()))
    print(f"elementwise tail n128 every element: max abs err {worst:.3e} over {yh.size} values", flush=True)


# ---------------------------------------------------------------------------
# HIP graph capture
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# Sizes at the ABI's limits
# ---------------------------------------------------------------------------

def gather(y, idx):
    """y.flatten()[idx] computed on the GPU, returned to the host."""
    return y.reshape(-1)[torch.from_numpy(idx).cuda()].cpu().numpy()


def test_conv2d_output_near_index_limit(cce):
    """One 5790 x 5788 image: N * C_out * Ho * Wo = 2,143,319,552, within 0.2 %
    of the 2^31 output limit (W and the plane are multiples of 4: 16-byte
    window loads; the 8.6 GB output plane set is past the 2^31-byte range of
    the buffer stores, so results leave through the scalar store path);
    checked at sampled outputs including the last ones."""
    p = make_inputs(CONV2D, seed=81, N=1, C_in=8, H=5790, W=5788, C_out=64, k=3)
    y = cce.conv2d_relu_hswish(dev(p["x"]), dev(p["w"]), dev(p["b"]))
    torch.cuda.synchronize()
    total = y.numel()
    assert total == 64 * 5788 * 5786 and total < 2 ** 31
    idx = np.unique(np.concatenate([sample_indices(total, 3000, 81), np.arange(total - 300, total),
                                    63 * 5788 * 5786 + np.arange(200)]))
    got = gather(y, idx)
    del y
    torch.cuda.empty_cache()
    assert_close(got, O.conv2d_relu_hswish_at(p["x"], p["w"], p["b"], idx), "conv2d near 2^31 outputs")


@pytest.mark.parametrize("C_in,C_out,k,H,W", [
    (8, 64, 3, 2896, 2900),   # output 2,147,023,872 bytes: 16-byte loads and stores
    (16, 16, 1, 5800, 5800),  # input 2,152,960,000 bytes: past the buffer loads' range
])
def test_conv2d_buffer_range_limits(cce, C_in, C_out, k, H, W):
    """The 16-byte paths address one image through 32-bit buffer offsets and
    take images below 2^31 bytes; at and just past that size (sampled outputs,
    the last ones included) the results still match the oracle."""
    p = make_inputs(CONV2D, seed=83, N=1, C_in=C_in, H=H, W=W, C_out=C_out, k=k)
    y = cce.conv2d_relu_hswish(dev(p["x"]), dev(p["w"]), dev(p["b"]))
    torch.cuda.synchronize()
    total = y.numel()
    idx = np.unique(np.concatenate([sample_indices(total, 3000, 83), np.arange(total - 300, total),
                                    np.arange(200)]))
    got = gather(y, idx)
    del y
    torch.cuda.empty_cache()
    assert_close(got, O.conv2d_relu_hswish_at(p["x"], p["w"], p["b"], idx), "conv2d buffer range limits")


def test_conv3d_output_near_index_limit(cce):
    """N * C_out * Do * Ho * Wo = 2,111,864,832 (1 x 64 x 128 x 4158 x 62) on the
    tuned instance for 64-wide rows; sampled outputs including the last ones."""
    p = make_inputs(CONV3D, seed=82, N=1, C_in=8, D=130, H=4160, W=64, C_out=64, k=3)
    y = cce.conv3d_lrelu_add_clamp_gelu(dev(p["x"]), dev(p["w"]), dev(p["b"]), dev(p["s"]), 0.2, -1.0, 1.0)
    torch.cuda.synchronize()
    total = y.numel()
    assert total == 64 * 128 * 4158 * 62 and total < 2 ** 31
    idx = np.unique(np.concatenate([sample_indices(total, 3000, 82), np.arange(total - 300, total)]))
    got = gather(y, idx)
    del y
    torch.cuda.empty_cache()
    assert_close(got, O.conv3d_lrelu_add_clamp_gelu_at(p["x"], p["w"], p["b"], p["s"], idx),
                 "conv3d near 2^31 outputs")


def test_elementwise_tail_plane_longer_than_2_31(cce):
    """One (n, c) plane of 2^31 + 2^20 + 6 elements (offsets past 32 bits inside
    a plane), built by tiling a seeded 2^24-element draw on the GPU; the
    expected value of each sampled element is the oracle's on that element."""
    C, S = 2, 2 ** 31 + 2 ** 20 + 6
    small = make_inputs(TAIL_GELU, seed=83, N=1, C=C, D=1, H=1, W=2 ** 23)
    zs = dev(small["z"]).reshape(-1)
    z = zs.repeat((C * S + zs.numel() - 1) // zs.numel())[:C * S].reshape(1, C, S)
    y = cce.lrelu_add_clamp_gelu(z, dev(small["s"]), 0.2, -1.0, 1.0)
    torch.cuda.synchronize()
    idx = np.unique(np.concatenate([sample_indices(C * S, 4000, 83), np.arange(S - 64, S + 64),
                                    np.arange(2 ** 31 - 64, 2 ** 31 + 64), np.arange(C * S - 64, C * S)]))
    zg, got = gather(z, idx), gather(y, idx)
    del z, y
    torch.cuda.empty_cache()
    ch = idx // S
    ref = np.empty(idx.shape[0])
    for c in range(C):
        m = ch == c
        ref[m] = O.lrelu_add_clamp_gelu_array(zg[m].reshape(1, 1, -1), small["s"][c:c + 1])[0, 0]
    assert_close(got, ref, "elementwise tail, plane longer than 2^31")


@pytest.mark.parametrize("quads", [2 ** 31 - 4, 2 ** 31 + 4])
def test_elementwise_tail_flat_path_limit(cce, quads):
    """The flat 16-byte path of the elementwise tail takes arrays of fewer than
    2^31 quads; from 2^31 on, the per-plane path does.  Both sides of that
    limit, in place (y = z), on two planes of 2 * quads floats (34 GB), built
    by tiling a seeded draw on the GPU; sampled elements (both ends, the
    plane boundary, the 2^31-quad boundary) against the oracle."""
    C, S = 2, 2 * quads
    small = make_inputs(TAIL_GELU, seed=84, N=1, C=C, D=1, H=1, W=2 ** 23)
    zs = dev(small["z"]).reshape(-1)
    z = zs.repeat((C * S + zs.numel() - 1) // zs.numel())[:C * S].reshape(1, C, S)
    del zs
    total = C * S
    idx = np.unique(np.concatenate([sample_indices(total, 4000, 84), np.arange(S - 64, S + 64),
                                    np.arange(min(4 * 2 ** 31, total) - 64, min(4 * 2 ** 31, total)),
                                    np.arange(total - 64, total)]))
    zg = gather(z, idx)
    y = cce.lrelu_add_clamp_gelu(z, dev(small["s"]), 0.2, -1.0, 1.0, out=z)
    torch.cuda.synchronize()
    got = gather(y, idx)
    del z, y
    torch.cuda.empty_cache()
    ch = idx // S
    ref = np.empty(idx.shape[0])
    for c in range(C):
        m = ch == c
        ref[m] = O.lrelu_add_clamp_gelu_array(zg[m].reshape(1, 1, -1), small["s"][c:c + 1])[0, 0]
    assert_close(got, ref, f"elementwise tail in place, {quads} quads")


def off(a=None, shape=None):
    """A GPU tensor (a copy of `a`, or zeros of `shape`) whose data pointer is
    4 bytes past a 16-byte boundary: 4-byte aligned, as the ABI requires, but
    not 16-byte aligned, so every kernel takes its scalar load/store paths."""
    shape = a.shape if a is not None else shape
    n = int(np.prod(shape))
    flat = torch.zeros(n + 4, dtype=torch.float32, device="cuda")
    k = ((4 - flat.data_ptr() % 16) % 16) // 4
    t = flat[k:k + n].view(shape)
    if a is not None:
        t.copy_(torch.from_numpy(np.ascontiguousarray(a)))
    assert t.data_ptr() % 16 == 4
    return t


@pytest.mark.parametrize("op", [CONV2D, CONV3D, CONVT, TAIL_POOL, TAIL_GELU])
def test_pointers_not_16_byte_aligned(cce, op):
    """Every tensor offset by one float from a 16-byte boundary: the weight
    staging's scalar branch and the scalar load/store instances, at shapes
    whose sizes would otherwise take the 16-byte paths."""
    if op == CONV2D:
        p = make_inputs(CONV2D, seed=61, N=2, C_in=8, H=20, W=24, C_out=64, k=3)
        y = off(shape=(2, 64, 18, 22))
        cce.conv2d_relu_hswish(off(p["x"]), off(p["w"]), off(p["b"]), out=y)
        ref = O.conv2d_relu_hswish(p["x"], p["w"], p["b"])
    elif op == CONV3D:
        p = make_inputs(CONV3D, seed=62, N=1, C_in=8, D=5, H=10, W=12, C_out=64, k=3)
        y = off(shape=(1, 64, 3, 8, 10))
        cce.conv3d_lrelu_add_clamp_gelu(off(p["x"]), off(p["w"]), off(p["b"]), off(p["s"]), 0.2, -1.0, 1.0,
                                        out=y)
        ref = O.conv3d_lrelu_add_clamp_gelu(p["x"], p["w"], p["b"], p["s"])
    elif op == CONVT:
        p = make_inputs(CONVT, seed=63, N=2, C_in=64, H=32, W=36, C_out=64, k=3)
        y = off(shape=(2, 64, 1, 1))
        cce.convT2d_pool_htanh_mean_tanh(off(p["x"]), off(p["w"]), off(p["b"]), out=y)
        ref = O.convT2d_pool_htanh_mean_tanh(p["x"], p["w"], p["b"])[:, :, None, None]
    elif op == TAIL_POOL:
        p = make_inputs(TAIL_POOL, seed=64, N=2, C=5, H=16, W=24)
        y = off(shape=(2, 5, 1, 1))
        cce.pool_htanh_mean_tanh(off(p["z"]), out=y)
        ref = O.pool_htanh_mean_tanh(p["z"])[:, :, None, None]
    else:
        p = make_inputs(TAIL_GELU, seed=65, N=2, C=6, D=3, H=4, W=8)
        y = off(shape=p["z"].shape)
        cce.lrelu_add_clamp_gelu(off(p["z"]), off(p["s"]), 0.2, -1.0, 1.0, out=y)
        ref = O.lrelu_add_clamp_gelu_array(p["z"], p["s"])
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), ref, f"{op} with 4-byte-offset pointers")


def test_graph_capture_replays_match_eager(cce):
    """All five operators captured in one HIP graph (torch.cuda.graph) and
    replayed three times, with eager work and a synchronisation between the
    replays: every replay matches the eager results bit for bit.  The calls
    allocate nothing and issue no memset, so they are capturable; the ConvT
    workspace is passed in, and each call's preparation kernel (captured with
    it) zeroes the workspace's counters."""
    p2 = make_inputs(CONV2D, seed=801, N=2, C_in=8, H=21, W=30, C_out=64, k=3)
    p3 = make_inputs(CONV3D, seed=802, N=1, C_in=8, D=5, H=12, W=16, C_out=64, k=3)
    pt = make_inputs(CONVT, seed=803, N=2, C_in=64, H=18, W=20, C_out=64, k=3)
    pp = make_inputs(TAIL_POOL, seed=804, N=2, C=3, H=16, W=20)
    pg = make_inputs(TAIL_GELU, seed=805, N=2, C=4, D=2, H=5, W=8)
    d2 = {k: dev(v) for k, v in p2.items()}
    d3 = {k: dev(v) for k, v in p3.items()}
    dt = {k: dev(v) for k, v in pt.items()}
    zp, zg, sg = dev(pp["z"]), dev(pg["z"]), dev(pg["s"])
    ws = torch.zeros(cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(2, 64, 18, 20, 64),
                     dtype=torch.uint8, device="cuda")

    def run(outs):
        cce.conv2d_relu_hswish(d2["x"], d2["w"], d2["b"], out=outs[0])
        cce.conv3d_lrelu_add_clamp_gelu(d3["x"], d3["w"], d3["b"], d3["s"], 0.2, -1.0, 1.0, out=outs[1])
        cce.convT2d_pool_htanh_mean_tanh(dt["x"], dt["w"], dt["b"], out=outs[2], workspace=ws)
        cce.pool_htanh_mean_tanh(zp, out=outs[3])
        cce.lrelu_add_clamp_gelu(zg, sg, 0.2, -1.0, 1.0, out=outs[4])

    shapes = [(2, 64, 19, 28), (1, 64, 3, 10, 14), (2, 64, 1, 1), (2, 3, 1, 1), tuple(zg.shape)]
    eager = [torch.empty(sh, device="cuda") for sh in shapes]
    run(eager)
    torch.cuda.synchronize()
    outs = [torch.empty(sh, device="cuda") for sh in shapes]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(outs)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), f"replay {rep}, operator {i}"
    assert_close(eager[0].cpu().numpy(), O.conv2d_relu_hswish(p2["x"], p2["w"], p2["b"]), "graph conv2d")


def test_library_loaded_before_torch_in_a_fresh_process():
    """Loading libcce before anything imports torch (as a build step that
    ends by loading the library does) still leaves one HIP runtime in the
    process: a call then succeeds and matches the oracle."""
    import subprocess
    import sys
    from pathlib import Path
    root = Path(__file__).resolve().parents[1]
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import channel_convolution_epilogue_amd as cce\n"
        "cce.load()\n"
        "import numpy as np, torch\n"
        "import oracle as O\n"
        "from conv_inputs import CONV2D, make_inputs\n"
        "p = make_inputs(CONV2D, seed=5, N=2, C_in=8, H=30, W=26, C_out=64, k=3)\n"
        "t = lambda a: torch.from_numpy(a).cuda()\n"
        "y = cce.conv2d_relu_hswish(t(p['x']), t(p['w']), t(p['b'])).cpu().numpy()\n"
        "ref = O.conv2d_relu_hswish(p['x'], p['w'], p['b'])\n"
        "assert np.all(np.abs(y - ref) <= 1e-4 + 1e-4 * np.abs(ref))\n"
        "print('ok', flush=True)\n" % str(root))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=110)
    assert res.returncode == 0 and "ok" in res.stdout, res.stdout + res.stderr


# ---------------------------------------------------------------------------
# Seeded sweep of random shapes: every operator, supported layer shapes,
# ragged / odd / minimal sizes, 16-byte and scalar paths, both GELU forms.
# ---------------------------------------------------------------------------

def _sweep_cases(seed, count, draw):
    rng = np.random.default_rng(seed)
    return [draw(rng) for _ in range(count)]


def test_random_shape_sweep_conv2d(cce):
    def draw(rng):
        C_in = int(rng.choice([4, 8, 16]))
        C_out = int(rng.choice([16, 32, 64]))
        k = int(rng.choice([1, 3, 5] if C_in <= 8 else [1, 3]))
        return dict(N=int(rng.integers(1, 4)), C_in=C_in, C_out=C_out, k=k,
                    H=int(rng.integers(k, 41)), W=int(rng.integers(k, 41)), bias=bool(rng.random() < 0.8))
    for i, c in enumerate(_sweep_cases(2024, 24, draw)):
        print(f"sweep conv2d case {i}: {c}", flush=True)
        p = make_inputs(CONV2D, seed=3000 + i, N=c["N"], C_in=c["C_in"], H=c["H"], W=c["W"], C_out=c["C_out"], k=c["k"])
        b = p["b"] if c["bias"] else None
        y = cce.conv2d_relu_hswish(dev(p["x"]), dev(p["w"]), dev(b))
        torch.cuda.synchronize()
        assert_close(y.cpu().numpy(), O.conv2d_relu_hswish(p["x"], p["w"], b), f"sweep conv2d {c}")


def test_random_shape_sweep_conv3d(cce):
    def draw(rng):
        k = int(rng.choice([1, 3]))
        lo, hi = [(-1.0, 1.0), (-1.0, 1.0), (-2.0, 1.5)][int(rng.integers(0, 3))]
        return dict(N=int(rng.integers(1, 3)), C_in=int(rng.choice([4, 8, 16])), C_out=int(rng.choice([16, 32, 64])),
                    k=k, D=int(rng.integers(k, 7)), H=int(rng.integers(k, 25)), W=int(rng.integers(k, 25)),
                    slope=float(rng.choice([0.2, 0.05])), lo=lo, hi=hi)
    for i, c in enumerate(_sweep_cases(2025, 16, draw)):
        print(f"sweep conv3d case {i}: {c}", flush=True)
        p = make_inputs(CONV3D, seed=3100 + i, N=c["N"], C_in=c["C_in"], D=c["D"], H=c["H"], W=c["W"],
                        C_out=c["C_out"], k=c["k"])
        s = (p["s"] * 20).astype(np.float32)
        y = cce.conv3d_lrelu_add_clamp_gelu(dev(p["x"]), dev(p["w"]), dev(p["b"]), dev(s), c["slope"], c["lo"], c["hi"])
        torch.cuda.synchronize()
        ref = O.conv3d_lrelu_add_clamp_gelu(p["x"], p["w"], p["b"], s, slope=c["slope"], lo=c["lo"], hi=c["hi"])
        assert_close(y.cpu().numpy(), ref, f"sweep conv3d {c}")


def test_random_shape_sweep_conv3d_wide_rows(cce):
    """Rows of 36-68 floats: the page's layer on 64-wide rows (balanced row
    blocks), 16 -> 64 as two 32-channel launches, whole-row tiles of fewer
    rows, even and odd output heights."""
    def draw(rng):
        lo, hi = [(-1.0, 1.0), (-2.0, 1.5)][int(rng.integers(0, 2))]
        return dict(N=int(rng.integers(1, 3)), C_in=int(rng.choice([4, 8, 16])), C_out=int(rng.choice([16, 32, 64])),
                    D=int(rng.integers(3, 6)), H=int(rng.integers(3, 21)), W=int(rng.choice([36, 40, 50, 64, 64, 68])),
                    lo=lo, hi=hi)
    for i, c in enumerate(_sweep_cases(2027, 14, draw)):
        print(f"sweep conv3d wide case {i}: {c}", flush=True)
        p = make_inputs(CONV3D, seed=3300 + i, N=c["N"], C_in=c["C_in"], D=c["D"], H=c["H"], W=c["W"],
                        C_out=c["C_out"], k=3)
        y = cce.conv3d_lrelu_add_clamp_gelu(dev(p["x"]), dev(p["w"]), dev(p["b"]), dev(p["s"]), 0.2, c["lo"], c["hi"])
        torch.cuda.synchronize()
        ref = O.conv3d_lrelu_add_clamp_gelu(p["x"], p["w"], p["b"], p["s"], 0.2, c["lo"], c["hi"])
        assert_close(y.cpu().numpy(), ref, f"sweep conv3d wide {c}")


def test_random_shape_sweep_convT(cce):
    def draw(rng):
        return dict(N=int(rng.integers(1, 3)), C_in=int(8 * rng.integers(1, 9)), C_out=int(rng.choice([16, 32, 64])),
                    H=int(rng.integers(2, 41)), W=int(rng.integers(2, 41)), bias=bool(rng.random() < 0.8))
    for i, c in enumerate(_sweep_cases(2026, 12, draw)):
        print(f"sweep convT case {i}: {c}", flush=True)
        p = make_inputs(CONVT, seed=3200 + i, N=c["N"], C_in=c["C_in"], H=c["H"], W=c["W"], C_out=c["C_out"], k=3)
        b = p["b"] if c["bias"] else None
        y = cce.convT2d_pool_htanh_mean_tanh(dev(p["x"]), dev(p["w"]), dev(b))
        torch.cuda.synchronize()
        assert_close(y.cpu().numpy()[:, :, 0, 0], O.convT2d_pool_htanh_mean_tanh(p["x"], p["w"], b), f"sweep convT {c}")


def test_random_shape_sweep_tails(cce):
    def draw_pool(rng):
        pk = int(rng.integers(1, 4))
        return dict(N=int(rng.integers(1, 3)), C=int(rng.integers(1, 6)), H=int(rng.integers(pk, 40)),
                    W=int(rng.integers(pk, 40)), pk=pk, ps=int(rng.integers(1, 4)))
    for i, c in enumerate(_sweep_cases(2027, 12, draw_pool)):
        print(f"sweep pool tail case {i}: {c}", flush=True)
        p = make_inputs(TAIL_POOL, seed=3300 + i, N=c["N"], C=c["C"], H=c["H"], W=c["W"])
        y = cce.pool_htanh_mean_tanh(dev(p["z"]), pool_k=c["pk"], pool_s=c["ps"])
        torch.cuda.synchronize()
        assert_close(y.cpu().numpy()[:, :, 0, 0], O.pool_htanh_mean_tanh(p["z"], pk=c["pk"], ps=c["ps"]),
                     f"sweep pool tail {c}")

    def draw_elt(rng):
        return dict(N=int(rng.integers(1, 4)), C=int(rng.integers(1, 9)), D=int(rng.integers(1, 4)),
                    H=int(rng.integers(1, 12)), W=int(rng.integers(1, 20)))
    for i, c in enumerate(_sweep_cases(2028, 12, draw_elt)):
        print(f"sweep elementwise tail case {i}: {c}", flush=True)
        p = make_inputs(TAIL_GELU, seed=3400 + i, **c)
        s = (p["s"] * 20).astype(np.float32)
        y = cce.lrelu_add_clamp_gelu(dev(p["z"]), dev(s), 0.2, -1.0, 1.0)
        torch.cuda.synchronize()
        assert_close(y.cpu().numpy(), O.lrelu_add_clamp_gelu_array(p["z"], s), f"sweep elementwise tail {c}")


def test_debug_mode_makes_calls_synchronous():
    """CCE_DEBUG=1 (read once per process, so in a child process): every
    launch is followed by a synchronisation of its stream, so each call
    returns only after its kernel has run -- a call lasts at least the
    kernel's own GPU time (about 1 ms here, against tens of microseconds for
    an asynchronous launch) -- and the results still match the oracle."""
    import os
    import subprocess
    import sys
    from pathlib import Path
    code = r'''
import sys, time, numpy as np, torch
sys.path.insert(0, ".")
import channel_convolution_epilogue_amd as cce, oracle as O
from conv_inputs import CONVT, make_inputs
cce.load()
p = make_inputs(CONVT, seed=77, N=24, C_in=64, H=256, W=256, C_out=64, k=3)
x, w, b = (torch.from_numpy(p[k]).cuda() for k in ("x", "w", "b"))
y = cce.convT2d_pool_htanh_mean_tanh(x, w, b)
torch.cuda.synchronize()
e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
ratios = []
for _ in range(3):
    e0.record()
    t0 = time.perf_counter()
    y = cce.convT2d_pool_htanh_mean_tanh(x, w, b)
    call_ms = (time.perf_counter() - t0) * 1e3
    e1.record()
    torch.cuda.synchronize()
    ratios.append(call_ms / e0.elapsed_time(e1))
idx = np.arange(0, 24 * 64, 97)
ref = O.convT2d_pool_htanh_mean_tanh_at(p["x"], p["w"], p["b"], idx)
got = y.cpu().numpy().reshape(-1)[idx]
ok = np.all(np.abs(got - ref) <= 1e-4 + 1e-4 * np.abs(ref))
print("RATIOS", " ".join("%.3f" % r for r in ratios), "OK", bool(ok), flush=True)
'''
    root = Path(__file__).resolve().parents[1]
    res = subprocess.run([sys.executable, "-c", code], cwd=str(root), env=dict(os.environ, CCE_DEBUG="1"),
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-3000:]
    line = [l for l in res.stdout.splitlines() if l.startswith("RATIOS")]
    assert line, res.stdout + res.stderr[-2000:]
    parts = line[0].split()
    ratios = [float(v) for v in parts[1:4]]
    assert parts[-1] == "True", line[0]
    # the call spans (almost all of) the event-timed GPU work
    assert min(ratios) > 0.8, line[0]
