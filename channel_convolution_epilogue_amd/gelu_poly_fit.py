"""Derivation of the GELU polynomial the kernels use on [-1, 1].

    python -m channel_convolution_epilogue_amd.gelu_poly_fit

For |t| <= 1, GELU(t) = 0.5 t (1 + erf(t / sqrt 2)) is written as
0.5 t + u P(u) with u = t^2, where R(u) = (GELU(t) - 0.5 t) / u =
erf(t / sqrt 2) / (2 t) is even in t, so a polynomial in u approximates it.
P (degree 4) is the discrete minimax fit of the error that reaches GELU,
max over u in [0, 1] of |u (P(u) - R(u))|, on 3001 Chebyshev-Lobatto points:
a linear programme (minimise e subject to -e <= u_i (P(u_i) - R(u_i)) <= e)
solved with scipy's HiGHS in double precision.  The error it reaches is
about 4e-9; rounded to fp32, the coefficients err by less than 2e-8, below
the fp32 rounding of the evaluation itself.  The kernel header holds the
fp32-rounded coefficients printed here (highest degree first);
tests/test_gelu_poly_cpu.py refits and compares.
"""
from __future__ import annotations

import numpy as np

DEGREE = 4
POINTS = 3001
SCALE = 1e8  # the LP's feasibility tolerance (1e-10) must sit far below the ~4e-9 error


def fit() -> tuple[np.ndarray, float]:
    """(coefficients c0..c4 of P in increasing degree, in double; max error)."""
    from scipy.optimize import linprog
    from scipy.special import erf
    u = (1.0 - np.cos(np.pi * np.arange(POINTS) / (POINTS - 1))) / 2.0
    t = np.sqrt(u)
    R = np.empty_like(u)
    nz = u > 0
    R[nz] = erf(t[nz] / np.sqrt(2.0)) / (2.0 * t[nz])
    R[~nz] = 1.0 / np.sqrt(2.0 * np.pi)  # the u -> 0 limit
    A = SCALE * u[:, None] * np.vander(u, DEGREE + 1, increasing=True)
    b = SCALE * u * R
    n = DEGREE + 1
    ones = np.ones((len(u), 1))
    res = linprog(np.r_[np.zeros(n), 1.0],
                  A_ub=np.vstack([np.hstack([A, -ones]), np.hstack([-A, -ones])]),
                  b_ub=np.r_[b, -b], bounds=[(None, None)] * n + [(0, None)], method="highs",
                  options=dict(primal_feasibility_tolerance=1e-10, dual_feasibility_tolerance=1e-10))
    if res.status != 0:
        raise RuntimeError(f"minimax fit failed: {res.message}")
    return res.x[:n], float(res.x[-1] / SCALE)


def fp32_coefficients_highest_first() -> list[float]:
    c, _ = fit()
    return [float(np.float32(v)) for v in c[::-1]]


def main() -> None:
    c, err = fit()
    print(f"minimax error of u (P(u) - R(u)) on the grid: {err:.3e}")
    for v in c[::-1]:
        print(f"{np.float32(v)!r:>16}  ({v:.17g})")


if __name__ == "__main__":
    main()
