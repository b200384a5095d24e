"""The device-side GELU polynomial used on [-1, 1] (csrc/cce_device.hpp,
gelu_small): its coefficients, read from the header, must reproduce
GELU(t) = 0.5 t (1 + erf(t / sqrt 2)) within 2e-8 on [-1, 1] when evaluated
in double, and within fp32 rounding (2e-7) when evaluated in fp32 the way the
kernel does (Horner in u = t^2, then u * r + 0.5 t).  They are the minimax
fit that channel_convolution_epilogue_amd/gelu_poly_fit.py derives from erf,
rounded to fp32: refitting reproduces them."""
import re
from pathlib import Path

import numpy as np
from scipy.special import erf

HDR = Path(__file__).resolve().parents[1] / "channel_convolution_epilogue_amd" / "csrc" / "cce_device.hpp"


def coefficients():
    src = HDR.read_text()
    consts = dict(re.findall(r"(kGeluP\d) = ([-+0-9.eE]+)f", src))
    assert sorted(consts) == [f"kGeluP{k}" for k in range(5)], consts
    body = src[src.index("float gelu_small(float t)"):]
    body = body[:body.index("}")]
    order = [re.search(r"float r = (kGeluP\d);", body).group(1)]
    order += re.findall(r"r = fmaf\(r, u, (kGeluP\d)\);", body)
    assert order == [f"kGeluP{k}" for k in (4, 3, 2, 1, 0)], order
    return [float(consts[k]) for k in order]  # highest degree first


def half_scaled_coefficients():
    """The factors gelu_small_half applies to P's coefficients, highest degree first."""
    src = HDR.read_text()
    body = src[src.index("float gelu_small_half(float h)"):]
    body = body[:body.index("}")]
    first = re.search(r"float r = ([0-9.]+)f \* kGeluP4;", body).group(1)
    rest = re.findall(r"r = fmaf\(r, u, ([0-9.]+)f \* kGeluP(\d)\);", body)
    assert [k for _, k in rest] == ["3", "2", "1", "0"], rest
    return [float(first)] + [float(f) for f, _ in rest]


def test_gelu_polynomial_error_bound():
    c = coefficients()
    assert len(c) == 5
    t = np.linspace(-1.0, 1.0, 400001)
    exact = 0.5 * t * (1.0 + erf(t / np.sqrt(2.0)))
    u = t * t
    r = np.zeros_like(t)
    for ck in c:
        r = r * u + ck
    assert np.abs(0.5 * t + u * r - exact).max() < 2e-8

    t32, u32 = t.astype(np.float32), (t.astype(np.float32) ** 2).astype(np.float32)
    r32 = np.full_like(t32, np.float32(c[0]))
    for ck in c[1:]:
        r32 = (r32 * u32 + np.float32(ck)).astype(np.float32)
    y32 = (u32 * r32 + np.float32(0.5) * t32).astype(np.float32)
    assert np.abs(y32.astype(np.float64) - exact).max() < 2e-7
    # the t -> 0 limit: slope 1/2 and curvature 1/sqrt(2 pi)
    assert abs(c[-1] - 1.0 / np.sqrt(2.0 * np.pi)) < 1e-6


def test_gelu_coefficients_are_the_refit_minimax_polynomial():
    """Refit P from erf (the committed derivation) and compare with the
    header: each coefficient is the fit's value rounded to fp32 (within one
    fp32 ulp, in case the LP solver's last digits differ between platforms),
    and the fit reaches the minimax error the header's comment states."""
    from channel_convolution_epilogue_amd import gelu_poly_fit
    c_fit, err = gelu_poly_fit.fit()
    assert 3e-9 < err < 5e-9
    header = coefficients()
    for got, want in zip(header, c_fit[::-1]):
        ulp = abs(float(np.spacing(np.float32(want))))
        assert abs(float(np.float32(got)) - float(np.float32(want))) <= ulp, (got, want)
        assert abs(got - want) <= 1.5 * ulp


def test_half_scaled_gelu_is_the_same_function_to_the_bit():
    """gelu_small_half(h) evaluates GELU(2 h) with the coefficients of
    Q(x) = 4 P(4 x), i.e. 4^(k+1) p_k: scaling by powers of two commutes with
    each fp32 rounding, so on a dense grid of t in [-1, 1] the fp32
    evaluation from h = t / 2 equals gelu_small's from t bit for bit (both
    emulated here with a rounding after every operation)."""
    c = coefficients()
    f = half_scaled_coefficients()
    assert f == [4.0 ** 5, 4.0 ** 4, 4.0 ** 3, 4.0 ** 2, 4.0], f
    t = np.linspace(-1.0, 1.0, 200001).astype(np.float32)
    f32 = np.float32

    def full(t):
        u = (t * t).astype(f32)
        r = np.full_like(t, f32(c[0]))
        for ck in c[1:]:
            r = ((r * u).astype(f32) + f32(ck)).astype(f32)
        return ((u * r).astype(f32) + (f32(0.5) * t).astype(f32)).astype(f32)

    def half(h):
        u = (h * h).astype(f32)
        r = np.full_like(h, f32(f[0]) * f32(c[0]))
        for fk, ck in zip(f[1:], c[1:]):
            r = ((r * u).astype(f32) + f32(fk) * f32(ck)).astype(f32)
        return ((u * r).astype(f32) + h).astype(f32)

    h = (t * f32(0.5)).astype(f32)
    assert np.array_equal(full(t).view(np.uint32), half(h).view(np.uint32))
