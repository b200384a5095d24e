"""Seeded synthetic inputs for the three fused convolution workloads.

Shared by the tests, the smoke check and the benchmark.  This module holds
shapes and random-number recipes only -- none of the operators' arithmetic --
so that the CPU oracle and the GPU path see identical inputs while sharing no
computation.

Recipe (the distributions the problem statements use for their modules):
  x     ~ N(0, 1)
  W, b  ~ U(-1/sqrt(fan_in), +1/sqrt(fan_in)), the default initialisation of
          torch conv layers, fan_in = C_in*k*k (Conv2d), C_in*k^3 (Conv3d),
          C_out*k*k (ConvTranspose2d, whose weight is [C_in, C_out, k, k])
  s     ~ 0.02 * N(0, 1), the per-channel sum_tensor of the Conv3d model
  z     ~ N(0, 1), the precomputed convolution output fed to the two
          epilogue-only operators (same shapes as the fused operators'
          intermediate results)
All arrays are C-contiguous float32.  Each tensor draws from its own numpy
PCG64 stream seeded by (seed, tensor index), so the values do not depend on
which other tensors were drawn.
"""
from __future__ import annotations

import math

import numpy as np

CONV2D = "conv2d_relu_hswish"
CONV3D = "conv3d_lrelu_add_clamp_gelu"
CONVT = "convT2d_pool_htanh_mean_tanh"
TAIL_POOL = "pool_htanh_mean_tanh"      # epilogue-only tail over a transposed-conv output
TAIL_GELU = "lrelu_add_clamp_gelu"      # epilogue-only elementwise pass over a Conv3d output

# Named workloads: the pages' problem sizes (and a small one of the same kind).
WORKLOADS = {
    "conv2d_relu_hswish_n8": dict(op=CONV2D, N=8, C_in=8, H=128, W=128, C_out=64, k=3),
    "conv2d_relu_hswish_n128": dict(op=CONV2D, N=128, C_in=8, H=128, W=128, C_out=64, k=3),
    "conv3d_lrelu_add_clamp_gelu_n128": dict(op=CONV3D, N=128, C_in=8, D=16, H=64, W=64, C_out=64,
                                             k=3, slope=0.2, lo=-1.0, hi=1.0),
    "convT2d_pool_htanh_mean_tanh_n16": dict(op=CONVT, N=16, C_in=64, H=256, W=256, C_out=64, k=3,
                                             stride=1, pad=1, pool_k=2, pool_s=2, lo=-1.0, hi=1.0),
    "convT2d_pool_htanh_mean_tanh_n128": dict(op=CONVT, N=128, C_in=64, H=256, W=256, C_out=64,
                                              k=3, stride=1, pad=1, pool_k=2, pool_s=2, lo=-1.0,
                                              hi=1.0),
    # epilogue-only operators over the N = 128 intermediate results
    "pool_htanh_mean_tanh_n128": dict(op=TAIL_POOL, N=128, C=64, H=256, W=256, pool_k=2, pool_s=2,
                                      lo=-1.0, hi=1.0),
    "lrelu_add_clamp_gelu_n128": dict(op=TAIL_GELU, N=128, C=64, D=14, H=62, W=62, slope=0.2,
                                      lo=-1.0, hi=1.0),
}

_X, _W, _B, _S = 0, 1, 2, 3


def _rng(seed: int, which: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), int(which)]))


def _normal(seed, which, shape, scale=1.0):
    a = _rng(seed, which).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return np.ascontiguousarray(a)


def _uniform(seed, which, shape, bound):
    a = _rng(seed, which).uniform(-bound, bound, size=shape).astype(np.float32)
    return np.ascontiguousarray(a)


def fan_in(op: str, C_in: int, C_out: int, k: int) -> int:
    if op == CONV2D:
        return C_in * k * k
    if op == CONV3D:
        return C_in * k ** 3
    if op == CONVT:
        return C_out * k * k
    raise ValueError(op)


def make_inputs(op: str, seed: int = 0, **shape) -> dict:
    """Return {"x", "w", "b"(, "s")} -- or {"z"(, "s")} for the epilogue-only
    operators -- as float32 numpy arrays for `op` at `shape`."""
    if op == TAIL_POOL:
        return {"z": _normal(seed, _X, (shape["N"], shape["C"], shape["H"], shape["W"]))}
    if op == TAIL_GELU:
        z = _normal(seed, _X, (shape["N"], shape["C"], shape["D"], shape["H"], shape["W"]))
        return {"z": z, "s": _normal(seed, _S, (shape["C"],), 0.02)}
    N, C_in, C_out, k = shape["N"], shape["C_in"], shape["C_out"], shape["k"]
    bound = 1.0 / math.sqrt(fan_in(op, C_in, C_out, k))
    if op == CONV2D:
        x = _normal(seed, _X, (N, C_in, shape["H"], shape["W"]))
        w = _uniform(seed, _W, (C_out, C_in, k, k), bound)
    elif op == CONV3D:
        x = _normal(seed, _X, (N, C_in, shape["D"], shape["H"], shape["W"]))
        w = _uniform(seed, _W, (C_out, C_in, k, k, k), bound)
    elif op == CONVT:
        x = _normal(seed, _X, (N, C_in, shape["H"], shape["W"]))
        w = _uniform(seed, _W, (C_in, C_out, k, k), bound)
    else:
        raise ValueError(op)
    out = {"x": x, "w": w, "b": _uniform(seed, _B, (C_out,), bound)}
    if op == CONV3D:
        out["s"] = _normal(seed, _S, (C_out,), 0.02)
    return out


def workload_inputs(name: str, seed: int = 0) -> tuple[dict, dict]:
    """(shape dict, inputs dict) for a named workload."""
    cfg = dict(WORKLOADS[name])
    op = cfg.pop("op")
    return dict(cfg, op=op), make_inputs(op, seed, **cfg)

