"""Pins for the CPU oracle: each check compares it with something other than
itself -- values the pages print (tests/golden/page_values.json), closed
forms, invariants, an independent im2col + matrix-product formulation, and
torch's float64 CPU convolutions as an outside library routine.

The checks are chosen so that a plausible slip anywhere in the oracle (a
dropped tap or bias, a wrong sign or offset, an unflipped or transposed
kernel, a wrong pooling window or divisor, epilogue steps out of order)
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.optimize import minimize_scalar
from scipy.special import ndtr

import oracle as O
from conv_inputs import CONV2D, CONV3D, CONVT, make_inputs

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))

# Minimum of GELU(t) = t * Phi(t), from the normal CDF by numeric minimisation
# (about -0.16997 at t = -0.7518); every clamped-GELU output lies in
# [GELU_MIN, GELU(1)].
_GELU_MIN = minimize_scalar(lambda t: t * ndtr(t), bounds=(-1, 0), method="bounded",
                            options={"xatol": 1e-12})
GELU_MIN, GELU_ARGMIN = float(_GELU_MIN.fun), float(_GELU_MIN.x)


def _rand(rng, *shape, scale=1.0):
    return np.ascontiguousarray((rng.standard_normal(shape) * scale).astype(np.float32))


def _t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# ---------------------------------------------------------------------------
# independent formulation: explicit patch matrix (im2col) times weight matrix
# ---------------------------------------------------------------------------

def im2col_conv2d(x, w, b):
    x = x.astype(np.float64)
    N, C, H, W = x.shape
    Co, _, k, _ = w.shape
    Ho, Wo = H - k + 1, W - k + 1
    cols = np.empty((N, Ho, Wo, C, k, k))
    for kh in range(k):
        for kw in range(k):
            cols[..., kh, kw] = x[:, :, kh:kh + Ho, kw:kw + Wo].transpose(0, 2, 3, 1)
    out = cols.reshape(N * Ho * Wo, C * k * k) @ w.reshape(Co, -1).astype(np.float64).T
    if b is not None:
        out = out + b.astype(np.float64)
    return out.reshape(N, Ho, Wo, Co).transpose(0, 3, 1, 2)


def im2col_conv3d(x, w, b):
    x = x.astype(np.float64)
    N, C, D, H, W = x.shape
    Co, _, k, _, _ = w.shape
    Do, Ho, Wo = D - k + 1, H - k + 1, W - k + 1
    cols = np.empty((N, Do, Ho, Wo, C, k, k, k))
    for kd in range(k):
        for kh in range(k):
            for kw in range(k):
                cols[..., kd, kh, kw] = x[:, :, kd:kd + Do, kh:kh + Ho, kw:kw + Wo].transpose(0, 2, 3, 4, 1)
    out = cols.reshape(N * Do * Ho * Wo, C * k ** 3) @ w.reshape(Co, -1).astype(np.float64).T
    if b is not None:
        out = out + b.astype(np.float64)
    return out.reshape(N, Do, Ho, Wo, Co).transpose(0, 4, 1, 2, 3)


# ---------------------------------------------------------------------------
# Conv2d
# ---------------------------------------------------------------------------

CONV2D_SHAPES = [  # (N, C_in, H, W, C_out, k)
    (1, 1, 3, 3, 1, 3),
    (2, 8, 7, 9, 5, 3),
    (1, 3, 6, 5, 4, 2),
    (2, 2, 4, 4, 3, 1),
    (1, 8, 11, 10, 64, 3),
]


@pytest.mark.parametrize("shape", CONV2D_SHAPES)
def test_conv2d_matches_im2col(shape):
    N, C, H, W, Co, k = shape
    rng = np.random.default_rng(hash(shape) % 2**32)
    x, w, b = _rand(rng, N, C, H, W), _rand(rng, Co, C, k, k), _rand(rng, Co)
    np.testing.assert_allclose(O.conv2d(x, w, b), im2col_conv2d(x, w, b), rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", CONV2D_SHAPES)
def test_conv2d_matches_torch_float64(shape):
    N, C, H, W, Co, k = shape
    rng = np.random.default_rng(1 + hash(shape) % 2**32)
    x, w, b = _rand(rng, N, C, H, W), _rand(rng, Co, C, k, k), _rand(rng, Co)
    ref = F.conv2d(_t64(x), _t64(w), _t64(b)).numpy()
    np.testing.assert_allclose(O.conv2d(x, w, b), ref, rtol=0, atol=1e-12)


def test_conv2d_impulse_response_is_flipped_kernel():
    # Correlation: a one-hot input at (i, h0, w0) shows up at output (h, w)
    # through tap (h0 - h, w0 - w), i.e. the kernel appears flipped in space.
    rng = np.random.default_rng(7)
    C, Co, k, H, W = 3, 4, 3, 7, 8
    w = _rand(rng, Co, C, k, k)
    i, h0, w0 = 1, 3, 4
    x = np.zeros((1, C, H, W), np.float32)
    x[0, i, h0, w0] = 1.0
    z = O.conv2d(x, w, None)[0]
    expect = np.zeros_like(z)
    for h in range(H - k + 1):
        for ww in range(W - k + 1):
            dh, dw = h0 - h, w0 - ww
            if 0 <= dh < k and 0 <= dw < k:
                expect[:, h, ww] = w[:, i, dh, dw]
    np.testing.assert_array_equal(z, expect)


def test_conv2d_onehot_centre_weight_picks_offset_input():
    # W[o, i, 1, 1] = 1 selects x[i, h+1, w+1]: pins padding 0 and the +kh offset.
    rng = np.random.default_rng(8)
    N, C, H, W, Co = 2, 3, 6, 7, 2
    x, b = _rand(rng, N, C, H, W), _rand(rng, Co)
    w = np.zeros((Co, C, 3, 3), np.float32)
    w[1, 2, 1, 1] = 1.0
    z = O.conv2d(x, w, b)
    np.testing.assert_array_equal(z[:, 1], x[:, 2, 1:H - 1, 1:W - 1].astype(np.float64) + np.float64(b[1]))
    np.testing.assert_array_equal(z[:, 0], np.full_like(z[:, 0], np.float64(b[0])))


def test_conv2d_linearity_and_translation():
    rng = np.random.default_rng(9)
    x1, x2 = _rand(rng, 1, 2, 8, 8), _rand(rng, 1, 2, 8, 8)
    w = _rand(rng, 3, 2, 3, 3)
    z12 = O.conv2d(np.ascontiguousarray(x1 + 2 * x2), w)
    np.testing.assert_allclose(z12, O.conv2d(x1, w) + 2 * O.conv2d(x2, w), atol=1e-5)
    xs = np.ascontiguousarray(np.roll(x1, 1, axis=3))
    np.testing.assert_allclose(O.conv2d(xs, w)[..., 1:], O.conv2d(x1, w)[..., :-1], atol=1e-12)


def test_conv2d_null_bias_is_zero_bias():
    rng = np.random.default_rng(10)
    x, w = _rand(rng, 1, 2, 5, 5), _rand(rng, 3, 2, 3, 3)
    np.testing.assert_array_equal(O.conv2d(x, w, None), O.conv2d(x, w, np.zeros(3, np.float32)))


def test_conv2d_relu_hswish_matches_torch_and_sampling():
    x, w, b = (make_inputs(CONV2D, seed=3, N=2, C_in=8, H=13, W=11, C_out=64, k=3)[k] for k in "xwb")
    y = O.conv2d_relu_hswish(x, w, b)
    ref = F.hardswish(F.relu(F.conv2d(_t64(x), _t64(w), _t64(b)))).numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)
    # every output, in shuffled order: a handful of indices does not pin the
    # index decoding (the last index decodes the same in any order, and many
    # outputs are zero after the ReLU)
    idx = np.random.default_rng(3).permutation(y.size)
    np.testing.assert_array_equal(O.conv2d_relu_hswish_at(x, w, b, idx), y.reshape(-1)[idx])


def test_conv2d_bad_args_rejected():
    x = np.zeros((1, 1, 2, 2), np.float32)
    w = np.zeros((1, 1, 3, 3), np.float32)
    with pytest.raises(ValueError):
        O.conv2d(x, w)  # output would be empty


# ---------------------------------------------------------------------------
# scalar epilogues
# ---------------------------------------------------------------------------

def test_hardswish_page_points():
    g = GOLDEN["hardswish"]
    for v, expect in g["points"]:
        assert O.hardswish(O.relu(v)) == expect


def test_relu_hardswish_closed_forms():
    assert O.hardswish(O.relu(-1.0)) == 0.0
    assert O.hardswish(O.relu(1.0)) == pytest.approx(2.0 / 3.0, abs=1e-15)
    assert O.hardswish(-1.0) == pytest.approx(-1.0 / 3.0, abs=1e-15)  # HardSwish alone is not 0 below 0
    assert O.hardswish(-4.0) == 0.0
    assert O.hardswish(2.0) == pytest.approx(2.0 * 5.0 / 6.0, abs=1e-15)
    v = np.linspace(-8, 8, 321)
    ref = F.hardswish(_t64(v)).numpy()
    np.testing.assert_allclose([O.hardswish(t) for t in v], ref, rtol=0, atol=1e-15)


def test_gelu_page_value_and_closed_forms():
    g = GOLDEN["gelu_exact_at_1"]
    assert round(O.gelu(g["x"]), g["printed_decimals"]) == g["value"]
    e = GOLDEN["erf_at_inv_sqrt2"]
    # GELU(x) = 0.5 x (1 + erf(x/sqrt 2)) at x = 1 gives erf(1/sqrt 2) = 2 GELU(1) - 1
    assert round(2.0 * O.gelu(1.0) - 1.0, e["printed_decimals"]) == e["value"]
    assert O.gelu(-1.0) == pytest.approx(-0.15865525393145707, abs=1e-15)
    t = np.linspace(-3, 3, 601)
    # GELU(t) = t * Phi(t) with Phi the standard normal CDF (an independent routine)
    np.testing.assert_allclose([O.gelu(v) for v in t], t * ndtr(t), rtol=0, atol=1e-15)
    # odd-part invariant: GELU(t) - GELU(-t) = t
    np.testing.assert_allclose([O.gelu(v) - O.gelu(-v) for v in t], t, rtol=0, atol=1e-15)
    np.testing.assert_allclose([O.gelu(v) for v in t], F.gelu(_t64(t)).numpy(), rtol=0, atol=1e-15)


def test_gelu_range_on_clamped_interval():
    t = np.linspace(-1, 1, 200001)
    vals = np.array([O.gelu(v) for v in t[::100]])
    assert vals.min() == pytest.approx(GELU_MIN, abs=1e-7)  # grid step 1e-3 near the minimum
    assert O.gelu(GELU_ARGMIN) == pytest.approx(GELU_MIN, abs=1e-13)
    assert GELU_MIN == pytest.approx(-0.1699712, abs=1e-7)
    assert O.gelu(1.0) == pytest.approx(0.8413447460685429, abs=1e-15)
    assert t[::100][vals.argmin()] == pytest.approx(GELU_ARGMIN, abs=2e-3)


def test_leaky_relu_and_clamp():
    assert O.leaky_relu(-1.0, 0.2) == pytest.approx(-0.2, abs=1e-16)
    assert O.leaky_relu(2.5, 0.2) == 2.5
    assert O.leaky_relu(0.0, 0.2) == 0.0
    assert O.clamp(-3.0, -1.0, 1.0) == -1.0
    assert O.clamp(3.0, -1.0, 1.0) == 1.0
    assert O.clamp(0.25, -1.0, 1.0) == 0.25


def test_conv3d_epilogue_order():
    # LeakyReLU, then + s, then clamp, then GELU (l2_p90's step order).
    assert O.lrelu_add_clamp_gelu(-10.0, 0.5) == pytest.approx(O.gelu(-1.0), abs=1e-15)
    assert O.lrelu_add_clamp_gelu(3.0, -0.5) == pytest.approx(O.gelu(1.0), abs=1e-15)
    assert O.lrelu_add_clamp_gelu(-1.0, 0.1) == pytest.approx(O.gelu(-0.1), abs=1e-15)
    rng = np.random.default_rng(11)
    v, s = rng.standard_normal(500) * 3, rng.standard_normal(500) * 0.5
    ref = F.gelu(torch.clamp(F.leaky_relu(_t64(v), 0.2) + _t64(s), -1, 1)).numpy()
    np.testing.assert_allclose([O.lrelu_add_clamp_gelu(a, c) for a, c in zip(v, s)], ref, rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# Conv3d
# ---------------------------------------------------------------------------

CONV3D_SHAPES = [  # (N, C_in, D, H, W, C_out, k)
    (1, 1, 3, 3, 3, 1, 3),
    (2, 8, 5, 6, 7, 4, 3),
    (1, 2, 4, 3, 5, 3, 2),
    (2, 4, 3, 4, 5, 16, 1),
]


@pytest.mark.parametrize("shape", CONV3D_SHAPES)
def test_conv3d_matches_im2col_and_torch(shape):
    N, C, D, H, W, Co, k = shape
    rng = np.random.default_rng(2 + hash(shape) % 2**32)
    x, w, b = _rand(rng, N, C, D, H, W), _rand(rng, Co, C, k, k, k), _rand(rng, Co)
    z = O.conv3d(x, w, b)
    np.testing.assert_allclose(z, im2col_conv3d(x, w, b), rtol=0, atol=1e-12)
    np.testing.assert_allclose(z, F.conv3d(_t64(x), _t64(w), _t64(b)).numpy(), rtol=0, atol=1e-12)


def test_conv3d_pointwise_is_a_channel_contraction():
    """A 1 x 1 x 1 convolution is, at every voxel, the matrix product of the
    [C_out, C_in] weight with the voxel's channel vector, plus the bias."""
    rng = np.random.default_rng(31)
    x, w, b = _rand(rng, 2, 16, 3, 4, 5), _rand(rng, 32, 16, 1, 1, 1), _rand(rng, 32)
    ref = np.einsum("oi,nidhw->nodhw", w[:, :, 0, 0, 0].astype(np.float64), x.astype(np.float64))
    ref += b.astype(np.float64)[None, :, None, None, None]
    np.testing.assert_allclose(O.conv3d(x, w, b), ref, rtol=0, atol=1e-12)


def test_conv3d_impulse_and_onehot_weight():
    rng = np.random.default_rng(12)
    C, Co, k, D, H, W = 2, 3, 3, 5, 6, 7
    w = _rand(rng, Co, C, k, k, k)
    x = np.zeros((1, C, D, H, W), np.float32)
    x[0, 1, 2, 3, 4] = 1.0
    z = O.conv3d(x, w)[0]
    for d in range(D - 2):
        for h in range(H - 2):
            for ww in range(W - 2):
                dd, dh, dw = 2 - d, 3 - h, 4 - ww
                inside = 0 <= dd < 3 and 0 <= dh < 3 and 0 <= dw < 3
                expect = w[:, 1, dd, dh, dw] if inside else np.zeros(Co)
                np.testing.assert_array_equal(z[:, d, h, ww], expect)
    x2, b = _rand(rng, 2, C, D, H, W), _rand(rng, Co)
    w1 = np.zeros((Co, C, 3, 3, 3), np.float32)
    w1[2, 0, 1, 1, 1] = 1.0
    z2 = O.conv3d(x2, w1, b)
    np.testing.assert_array_equal(z2[:, 2], x2[:, 0, 1:-1, 1:-1, 1:-1].astype(np.float64) + np.float64(b[2]))


def test_conv3d_model_matches_torch_and_sampling():
    p = make_inputs(CONV3D, seed=4, N=2, C_in=8, D=5, H=7, W=9, C_out=64, k=3)
    x, w, b, s = p["x"], p["w"], p["b"], p["s"]
    s = np.ascontiguousarray(s * 20)  # widen s so the add visibly matters
    y = O.conv3d_lrelu_add_clamp_gelu(x, w, b, s, 0.2, -1.0, 1.0)
    z = F.conv3d(_t64(x), _t64(w), _t64(b))
    ref = F.gelu(torch.clamp(F.leaky_relu(z, 0.2) + _t64(s).view(1, -1, 1, 1, 1), -1, 1)).numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)
    assert y.min() >= GELU_MIN - 1e-12 and y.max() <= 0.8413447460685429 + 1e-12
    idx = np.random.default_rng(4).permutation(y.size)  # every output, shuffled
    np.testing.assert_array_equal(O.conv3d_lrelu_add_clamp_gelu_at(x, w, b, s, idx), y.reshape(-1)[idx])


# ---------------------------------------------------------------------------
# ConvTranspose2d
# ---------------------------------------------------------------------------

CONVT_CASES = [  # (N, C_in, H, W, C_out, k, stride, pad)
    (1, 1, 3, 3, 1, 3, 1, 1),
    (2, 3, 5, 6, 4, 3, 1, 1),
    (1, 4, 4, 4, 2, 3, 1, 0),
    (1, 2, 3, 4, 3, 3, 2, 1),
    (1, 2, 4, 3, 2, 2, 2, 0),
    (1, 64, 6, 6, 64, 3, 1, 1),
]


@pytest.mark.parametrize("case", CONVT_CASES)
def test_convT_scatter_equals_gather_and_torch(case):
    N, C, H, W, Co, k, s, p = case
    rng = np.random.default_rng(3 + hash(case) % 2**32)
    x, w, b = _rand(rng, N, C, H, W), _rand(rng, C, Co, k, k), _rand(rng, Co)
    zs = O.convT2d_scatter(x, w, b, s, p)
    zg = O.convT2d_gather(x, w, b, s, p)
    np.testing.assert_allclose(zs, zg, rtol=0, atol=1e-12)
    ref = F.conv_transpose2d(_t64(x), _t64(w), _t64(b), stride=s, padding=p).numpy()
    assert ref.shape == zs.shape
    np.testing.assert_allclose(zs, ref, rtol=0, atol=1e-12)
    # The model path's tap-major scatter adds each output's terms in the
    # gather form's (i, kh, kw) order: the same doubles, bit for bit.
    np.testing.assert_array_equal(O.convT2d_planes(x, w, b, s, p), zg)


def test_convT_adjoint_identity():
    # <convT(x; W), z> = <x, conv2d(zero-pad(z, p); W viewed as [C_in, C_out, k, k])>
    # for stride 1: the transposed conv is the adjoint of the padded correlation.
    # This fixes the kernel flip and the in/out channel swap at the definition level.
    rng = np.random.default_rng(13)
    C_in, C_out, H, W, k, p = 3, 4, 6, 5, 3, 1
    x, w = _rand(rng, 2, C_in, H, W), _rand(rng, C_in, C_out, k, k)
    y = O.convT2d_gather(x, w, None, 1, p)
    z = _rand(rng, *y.shape)
    zp = np.ascontiguousarray(np.pad(z, ((0, 0), (0, 0), (p, p), (p, p))))
    rhs = float(np.sum(x.astype(np.float64) * O.conv2d(zp, w, None)))
    for yy in (y, O.convT2d_planes(x, w, None, 1, p)):
        lhs = float(np.sum(yy * z.astype(np.float64)))
        assert lhs == pytest.approx(rhs, rel=1e-12, abs=1e-12)


def test_convT_impulse_stamps_unflipped_kernel():
    rng = np.random.default_rng(14)
    C_in, C_out, H, W = 2, 3, 6, 7
    w = _rand(rng, C_in, C_out, 3, 3)
    x = np.zeros((1, C_in, H, W), np.float32)
    h0, w0 = 2, 4
    x[0, 1, h0, w0] = 1.0
    for z in (O.convT2d_scatter(x, w, None, 1, 1)[0], O.convT2d_gather(x, w, None, 1, 1)[0],
              O.convT2d_planes(x, w, None, 1, 1)[0]):
        expect = np.zeros_like(z)
        expect[:, h0 - 1:h0 + 2, w0 - 1:w0 + 2] = w[1]
        np.testing.assert_array_equal(z, expect)


def test_convT_and_pool_output_sizes_golden():
    g = GOLDEN["convT_shapes"]
    assert O.convT_out_size(g["H"], g["k"], g["stride"], g["pad"]) == g["conv_out_hw"]
    assert O.pool_out_size(g["conv_out_hw"], 2, 2) == g["pooled_hw"]
    assert g["pooled_hw"] ** 2 == g["mean_divisor"]
    assert g["N"] * g["C_out"] * g["conv_out_hw"] ** 2 == g["conv_outputs"]
    assert g["conv_outputs"] * g["C_in"] * g["k"] ** 2 == g["macs"]
    for n in (2, 3, 7, 8):  # floor pooling, as torch computes it
        assert O.pool_out_size(n, 2, 2) == F.max_pool2d(torch.zeros(1, 1, n, n), 2, 2).shape[-1]


def test_conv_shapes_and_counts_golden():
    g = GOLDEN["conv2d_shapes"]
    x = np.zeros((1, g["C_in"], g["H"], g["W"]), np.float32)
    w = np.zeros((g["C_out"], g["C_in"], g["k"], g["k"]), np.float32)
    assert O.conv2d(x, w).shape[-2:] == (g["out_hw"], g["out_hw"])
    assert g["N"] * g["C_out"] * g["out_hw"] ** 2 == g["out_elements"]
    assert w.size == g["weight_elements"]
    g = GOLDEN["conv3d_shapes"]
    x = np.zeros((1, g["C_in"], g["D"], g["H"], g["W"]), np.float32)
    w = np.zeros((2, g["C_in"], g["k"], g["k"], g["k"]), np.float32)
    assert list(O.conv3d(x, w).shape[-3:]) == g["out_dhw"]
    assert g["N"] * g["C_out"] * math.prod(g["out_dhw"]) == g["out_elements"]
    assert g["out_elements"] * g["C_in"] * g["k"] ** 3 == g["fmas"]


def test_pool_htanh_mean_tanh_plane_hand_case():
    # 4x4 plane -> 2x2 windows with maxima 5, -0.25, 0.5, -7 -> clamp -> 1, -0.25, 0.5, -1
    z = np.array([[1, 5, -3, -0.25],
                  [0, 2, -1, -0.5],
                  [0.5, 0.1, -7, -8],
                  [-2, 0.2, -9, -7.5]], np.float64)
    expect = math.tanh((1 - 0.25 + 0.5 - 1) / 4)
    assert O.pool_htanh_mean_tanh_plane(z) == pytest.approx(expect, abs=1e-15)
    # odd plane: the last row / column are dropped by the floor in the pool size
    z5 = np.full((5, 5), 0.3)
    z5[4, :] = 100.0
    z5[:, 4] = 100.0
    assert O.pool_htanh_mean_tanh_plane(z5) == pytest.approx(math.tanh(0.3), abs=1e-15)


def test_convT_model_zero_weight_and_saturating_bias():
    N, C_in, C_out, H, W = 2, 3, 4, 6, 8
    rng = np.random.default_rng(15)
    x = _rand(rng, N, C_in, H, W)
    b = np.array([0.3, -0.7, 1.5, -2.0], np.float32)
    w0 = np.zeros((C_in, C_out, 3, 3), np.float32)
    y = O.convT2d_pool_htanh_mean_tanh(x, w0, b)
    np.testing.assert_allclose(y, np.tile(np.tanh(np.clip(b.astype(np.float64), -1, 1)), (N, 1)), atol=1e-15)
    ws = _rand(rng, C_in, C_out, 3, 3, scale=1e-3)
    yb = O.convT2d_pool_htanh_mean_tanh(x, ws, np.array([10, -10, 10, -10], np.float32))
    np.testing.assert_allclose(yb, np.tile([math.tanh(1), -math.tanh(1)] * 2, (N, 1)), atol=1e-15)


@pytest.mark.parametrize("hw", [(8, 8), (6, 10), (7, 9)])
def test_convT_model_matches_torch(hw):
    H, W = hw
    p = make_inputs(CONVT, seed=5, N=2, C_in=64, H=H, W=W, C_out=64, k=3)
    x, w, b = p["x"], p["w"], p["b"]
    y = O.convT2d_pool_htanh_mean_tanh(x, w, b)
    z = F.conv_transpose2d(_t64(x), _t64(w), _t64(b), stride=1, padding=1)
    ref = torch.tanh(F.hardtanh(F.max_pool2d(z, 2, 2), -1, 1).mean(dim=(2, 3), keepdim=True)).numpy()
    assert y.shape == ref.shape[:2]
    np.testing.assert_allclose(y, ref[:, :, 0, 0], rtol=0, atol=1e-13)
    assert np.all(np.abs(y) <= math.tanh(1) + 1e-15)
    idx = np.random.default_rng(5).permutation(y.size)  # every (image, channel), shuffled
    np.testing.assert_array_equal(O.convT2d_pool_htanh_mean_tanh_at(x, w, b, idx), y.reshape(-1)[idx])


def test_input_recipe_distributions():
    # The shared generator draws x ~ N(0,1), W,b ~ U(+-1/sqrt(fan_in)), s ~ 0.02 N(0,1).
    p = make_inputs(CONV3D, seed=0, N=4, C_in=8, D=6, H=16, W=16, C_out=64, k=3)
    assert abs(float(p["x"].mean())) < 0.02 and abs(float(p["x"].std()) - 1) < 0.02
    bound = 1 / math.sqrt(216)
    assert p["w"].min() >= -bound and p["w"].max() <= bound and p["w"].max() > 0.9 * bound
    assert p["s"].shape == (64,) and float(np.abs(p["s"]).max()) < 0.1
    q = make_inputs(CONV3D, seed=0, N=4, C_in=8, D=6, H=16, W=16, C_out=64, k=3)
    assert all(np.array_equal(p[k], q[k]) for k in p)
    t = make_inputs(CONVT, seed=1, N=1, C_in=64, H=4, W=4, C_out=64, k=3)
    assert t["w"].shape == (64, 64, 3, 3) and t["w"].max() <= 1 / 24


# ---------------------------------------------------------------------------
# Epilogue-only operators over a precomputed convolution output
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(2, 3, 8, 8), (1, 2, 7, 9), (2, 1, 2, 2), (1, 4, 5, 12)])
def test_pool_tail_matches_torch_and_plane_function(shape):
    rng = np.random.default_rng(20 + sum(shape))
    z = (rng.standard_normal(shape) * 1.5).astype(np.float32)
    ref = torch.tanh(F.hardtanh(F.max_pool2d(_t64(z), 2, 2), -1, 1).mean(dim=(2, 3))).numpy()
    np.testing.assert_allclose(O.pool_htanh_mean_tanh(z), ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(O.pool_htanh_mean_tanh(z.astype(np.float64)), ref, rtol=0, atol=1e-14)
    n, c = shape[0] - 1, shape[1] - 1
    assert O.pool_htanh_mean_tanh(z)[n, c] == pytest.approx(
        O.pool_htanh_mean_tanh_plane(z[n, c].astype(np.float64)), abs=1e-15)
    # other Hardtanh bounds
    ref2 = torch.tanh(F.hardtanh(F.max_pool2d(_t64(z), 2, 2), -0.3, 0.7).mean(dim=(2, 3))).numpy()
    np.testing.assert_allclose(O.pool_htanh_mean_tanh(z, lo=-0.3, hi=0.7), ref2, rtol=0, atol=1e-14)


@pytest.mark.parametrize("pk,ps", [(3, 2), (2, 3), (1, 1), (3, 1), (4, 4), (5, 3)])
def test_pool_tail_general_window_and_stride(pk, ps):
    """Overlapping (s < k), gapped (s > k) and degenerate windows against torch
    float64 MaxPool2d (floor output size), plus closed forms: k = s = 1 is the
    plain mean of the clamped plane, a window covering the plane is its max."""
    rng = np.random.default_rng(30 + 7 * pk + ps)
    z = (rng.standard_normal((2, 3, 13, 11)) * 1.5).astype(np.float32)
    ref = torch.tanh(F.hardtanh(F.max_pool2d(_t64(z), pk, ps), -1, 1).mean(dim=(2, 3))).numpy()
    np.testing.assert_allclose(O.pool_htanh_mean_tanh(z, pk, ps), ref, rtol=0, atol=1e-14)
    if pk == 1 and ps == 1:
        np.testing.assert_allclose(O.pool_htanh_mean_tanh(z, 1, 1),
                                   np.tanh(np.clip(z.astype(np.float64), -1, 1).mean(axis=(2, 3))),
                                   rtol=0, atol=1e-14)
    sq = z[:, :, :11, :11]
    np.testing.assert_allclose(O.pool_htanh_mean_tanh(np.ascontiguousarray(sq), 11, ps),
                               np.tanh(np.clip(sq.astype(np.float64).max(axis=(2, 3)), -1, 1)),
                               rtol=0, atol=1e-15)


def test_pool_tail_of_convT_equals_fused_model():
    # The tail over the oracle's own transposed-conv output reproduces the fused model.
    p = make_inputs(CONVT, seed=21, N=2, C_in=64, H=6, W=10, C_out=64, k=3)
    z = O.convT2d_gather(p["x"], p["w"], p["b"])
    np.testing.assert_allclose(O.pool_htanh_mean_tanh(z),
                               O.convT2d_pool_htanh_mean_tanh(p["x"], p["w"], p["b"]), rtol=0, atol=1e-15)


def test_elementwise_tail_matches_torch_and_scalar():
    rng = np.random.default_rng(22)
    z = (rng.standard_normal((2, 5, 3, 4, 7)) * 2).astype(np.float32)
    s = (rng.standard_normal(5) * 0.5).astype(np.float32)
    for slope, lo, hi in [(0.2, -1.0, 1.0), (0.05, -0.5, 2.0)]:
        y = O.lrelu_add_clamp_gelu_array(z, s, slope, lo, hi)
        ref = F.gelu(torch.clamp(F.leaky_relu(_t64(z), slope) + _t64(s).view(1, -1, 1, 1, 1), lo, hi)).numpy()
        np.testing.assert_allclose(y, ref, rtol=0, atol=1e-15)
    assert y[1, 3, 2, 1, 6] == O.lrelu_add_clamp_gelu(z[1, 3, 2, 1, 6], s[3], 0.05, -0.5, 2.0)
