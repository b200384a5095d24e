"""ctypes loader for the CPU oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  The GPU library and its Python binding never import
this package.

The oracle is plain C compiled with gcc (-O2, OpenMP, no fast-math); every
function evaluates the operators' definitions in double precision.  The
wrappers below only marshal numpy arrays; all arithmetic happens in the C
loop nests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB = _HERE / "liboracle.so"

_lib = None


def build(force: bool = True) -> Path:
    """Compile oracle.c into liboracle.so with gcc (host code only)."""
    if not force and _LIB.exists() and _LIB.stat().st_mtime >= _SRC.stat().st_mtime:
        return _LIB
    tmp = _LIB.with_suffix(f".so.tmp{os.getpid()}")
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", str(tmp), str(_SRC), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_f = ctypes.POINTER(ctypes.c_float)
_d = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.POINTER(ctypes.c_int64)
_c_int = ctypes.c_int
_c_dbl = ctypes.c_double


def lib() -> ctypes.CDLL:
    """Load liboracle.so, compiling it first if it is missing or stale.

    CCE_ORACLE_LIB, when set, names another build of oracle.c to load instead
    (the mutation test points it at copies with a planted mistake)."""
    global _lib
    if _lib is None:
        override = os.environ.get("CCE_ORACLE_LIB")
        path = Path(override) if override else build(force=False)
        L = ctypes.CDLL(str(path))
        L.oracle_num_threads.restype = _c_int
        L.oracle_set_num_threads.argtypes = [_c_int]
        for name in ("oracle_relu", "oracle_hardswish", "oracle_gelu"):
            getattr(L, name).restype = _c_dbl
            getattr(L, name).argtypes = [_c_dbl]
        L.oracle_leaky_relu.restype = _c_dbl
        L.oracle_leaky_relu.argtypes = [_c_dbl, _c_dbl]
        L.oracle_clamp.restype = _c_dbl
        L.oracle_clamp.argtypes = [_c_dbl, _c_dbl, _c_dbl]
        L.oracle_lrelu_add_clamp_gelu.restype = _c_dbl
        L.oracle_lrelu_add_clamp_gelu.argtypes = [_c_dbl] * 5
        L.oracle_conv2d.argtypes = [_f, _f, _f, _d] + [_c_int] * 6
        L.oracle_conv2d_relu_hswish.argtypes = [_f, _f, _f, _d] + [_c_int] * 6
        L.oracle_conv2d_relu_hswish_at.argtypes = [_f, _f, _f] + [_c_int] * 6 + [_i64, ctypes.c_int64, _d]
        L.oracle_conv3d.argtypes = [_f, _f, _f, _d] + [_c_int] * 7
        L.oracle_conv3d_lrelu_add_clamp_gelu.argtypes = [_f, _f, _f, _f, _d] + [_c_int] * 7 + [_c_dbl] * 3
        L.oracle_conv3d_lrelu_add_clamp_gelu_at.argtypes = (
            [_f, _f, _f, _f] + [_c_int] * 7 + [_c_dbl] * 3 + [_i64, ctypes.c_int64, _d])
        L.oracle_convT_out_size.argtypes = [_c_int] * 4
        L.oracle_pool_out_size.argtypes = [_c_int] * 3
        L.oracle_convT2d_scatter.argtypes = [_f, _f, _f, _d] + [_c_int] * 8
        L.oracle_convT2d_gather.argtypes = [_f, _f, _f, _d] + [_c_int] * 8
        L.oracle_pool_htanh_mean_tanh_plane.restype = _c_dbl
        L.oracle_pool_htanh_mean_tanh_plane.argtypes = [_d] + [_c_int] * 4 + [_c_dbl] * 2
        L.oracle_pool_htanh_mean_tanh.argtypes = [_d, _d] + [_c_int] * 6 + [_c_dbl] * 2
        L.oracle_pool_htanh_mean_tanh_f32.argtypes = [_f, _d] + [_c_int] * 6 + [_c_dbl] * 2 + [_d, ctypes.c_int64]
        L.oracle_convT2d_planes.argtypes = [_f, _f, _f, _d] + [_c_int] * 8
        L.oracle_lrelu_add_clamp_gelu_f32.argtypes = [_f, _f, _d, _c_int, _c_int, ctypes.c_int64] + [_c_dbl] * 3
        L.oracle_convT2d_pool_htanh_mean_tanh_at.argtypes = (
            [_f, _f, _f] + [_c_int] * 10 + [_c_dbl] * 2 + [_i64, ctypes.c_int64, _d, ctypes.c_int64, _d])
        _lib = L
    return _lib


def _fp(a):
    if a is None:
        return None
    assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_f)


def _dp(a):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_d)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad argument (rc={rc})")


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


# -- scalar epilogues ---------------------------------------------------------

def relu(v: float) -> float:
    return lib().oracle_relu(float(v))


def hardswish(v: float) -> float:
    return lib().oracle_hardswish(float(v))


def leaky_relu(v: float, slope: float) -> float:
    return lib().oracle_leaky_relu(float(v), float(slope))


def clamp(v: float, lo: float, hi: float) -> float:
    return lib().oracle_clamp(float(v), float(lo), float(hi))


def gelu(t: float) -> float:
    return lib().oracle_gelu(float(t))


def lrelu_add_clamp_gelu(v, s, slope=0.2, lo=-1.0, hi=1.0) -> float:
    return lib().oracle_lrelu_add_clamp_gelu(float(v), float(s), float(slope), float(lo), float(hi))


# -- conv2d -----------------------------------------------------------------

def conv2d(x, w, b=None):
    N, C_in, H, W = x.shape
    C_out, _, k, _ = w.shape
    z = np.empty((N, C_out, H - k + 1, W - k + 1), np.float64)
    _check(lib().oracle_conv2d(_fp(x), _fp(w), _fp(b), _dp(z), N, C_in, H, W, C_out, k), "conv2d")
    return z


def conv2d_relu_hswish(x, w, b=None):
    N, C_in, H, W = x.shape
    C_out, _, k, _ = w.shape
    y = np.empty((N, C_out, H - k + 1, W - k + 1), np.float64)
    _check(lib().oracle_conv2d_relu_hswish(_fp(x), _fp(w), _fp(b), _dp(y), N, C_in, H, W, C_out, k),
           "conv2d_relu_hswish")
    return y


def conv2d_relu_hswish_at(x, w, b, flat_idx):
    N, C_in, H, W = x.shape
    C_out, _, k, _ = w.shape
    idx = np.ascontiguousarray(flat_idx, dtype=np.int64)
    out = np.empty(idx.shape[0], np.float64)
    _check(lib().oracle_conv2d_relu_hswish_at(_fp(x), _fp(w), _fp(b), N, C_in, H, W, C_out, k,
                                              idx.ctypes.data_as(_i64), idx.shape[0], _dp(out)),
           "conv2d_relu_hswish_at")
    return out


# -- conv3d -----------------------------------------------------------------

def conv3d(x, w, b=None):
    N, C_in, D, H, W = x.shape
    C_out, _, k, _, _ = w.shape
    z = np.empty((N, C_out, D - k + 1, H - k + 1, W - k + 1), np.float64)
    _check(lib().oracle_conv3d(_fp(x), _fp(w), _fp(b), _dp(z), N, C_in, D, H, W, C_out, k), "conv3d")
    return z


def conv3d_lrelu_add_clamp_gelu(x, w, b, s, slope=0.2, lo=-1.0, hi=1.0):
    N, C_in, D, H, W = x.shape
    C_out, _, k, _, _ = w.shape
    y = np.empty((N, C_out, D - k + 1, H - k + 1, W - k + 1), np.float64)
    _check(lib().oracle_conv3d_lrelu_add_clamp_gelu(_fp(x), _fp(w), _fp(b), _fp(s), _dp(y), N, C_in,
                                                    D, H, W, C_out, k, slope, lo, hi),
           "conv3d_lrelu_add_clamp_gelu")
    return y


def conv3d_lrelu_add_clamp_gelu_at(x, w, b, s, flat_idx, slope=0.2, lo=-1.0, hi=1.0):
    N, C_in, D, H, W = x.shape
    C_out, _, k, _, _ = w.shape
    idx = np.ascontiguousarray(flat_idx, dtype=np.int64)
    out = np.empty(idx.shape[0], np.float64)
    _check(lib().oracle_conv3d_lrelu_add_clamp_gelu_at(_fp(x), _fp(w), _fp(b), _fp(s), N, C_in, D, H,
                                                       W, C_out, k, slope, lo, hi,
                                                       idx.ctypes.data_as(_i64), idx.shape[0],
                                                       _dp(out)),
           "conv3d_lrelu_add_clamp_gelu_at")
    return out


# -- transposed conv + pooled mean -------------------------------------------

def convT_out_size(n_in: int, k: int, stride: int, pad: int) -> int:
    return lib().oracle_convT_out_size(n_in, k, stride, pad)


def pool_out_size(n_in: int, pk: int, ps: int) -> int:
    return lib().oracle_pool_out_size(n_in, pk, ps)


def convT2d_scatter(x, w, b=None, stride=1, pad=1):
    N, C_in, H, W = x.shape
    _, C_out, k, _ = w.shape
    Ho, Wo = convT_out_size(H, k, stride, pad), convT_out_size(W, k, stride, pad)
    z = np.empty((N, C_out, Ho, Wo), np.float64)
    _check(lib().oracle_convT2d_scatter(_fp(x), _fp(w), _fp(b), _dp(z), N, C_in, H, W, C_out, k,
                                        stride, pad), "convT2d_scatter")
    return z


def convT2d_gather(x, w, b=None, stride=1, pad=1):
    N, C_in, H, W = x.shape
    _, C_out, k, _ = w.shape
    Ho, Wo = convT_out_size(H, k, stride, pad), convT_out_size(W, k, stride, pad)
    z = np.empty((N, C_out, Ho, Wo), np.float64)
    _check(lib().oracle_convT2d_gather(_fp(x), _fp(w), _fp(b), _dp(z), N, C_in, H, W, C_out, k,
                                       stride, pad), "convT2d_gather")
    return z


def convT2d_planes(x, w, b=None, stride=1, pad=1):
    """The transposed conv as the model path evaluates it (tap-major scatter
    per output plane), [N, C_out, Ho, Wo] in double."""
    N, C_in, H, W = x.shape
    _, C_out, k, _ = w.shape
    Ho, Wo = convT_out_size(H, k, stride, pad), convT_out_size(W, k, stride, pad)
    z = np.empty((N, C_out, Ho, Wo), np.float64)
    _check(lib().oracle_convT2d_planes(_fp(x), _fp(w), _fp(b), _dp(z), N, C_in, H, W, C_out, k,
                                       stride, pad), "convT2d_planes")
    return z


def pool_htanh_mean_tanh_plane(z_plane, pk=2, ps=2, lo=-1.0, hi=1.0) -> float:
    z = np.ascontiguousarray(z_plane, dtype=np.float64)
    Ho, Wo = z.shape
    return lib().oracle_pool_htanh_mean_tanh_plane(_dp(z), Ho, Wo, pk, ps, lo, hi)


def convT2d_pool_htanh_mean_tanh_at(x, w, b, nc_idx, stride=1, pad=1, pk=2, ps=2, lo=-1.0, hi=1.0):
    """Model output y[n, o] at the given flat indices n * C_out + o."""
    N, C_in, H, W = x.shape
    _, C_out, k, _ = w.shape
    Ho, Wo = convT_out_size(H, k, stride, pad), convT_out_size(W, k, stride, pad)
    idx = np.ascontiguousarray(nc_idx, dtype=np.int64)
    scratch = np.empty(max(1, num_threads()) * Ho * Wo, np.float64)
    out = np.empty(idx.shape[0], np.float64)
    _check(lib().oracle_convT2d_pool_htanh_mean_tanh_at(
        _fp(x), _fp(w), _fp(b), N, C_in, H, W, C_out, k, stride, pad, pk, ps, lo, hi,
        idx.ctypes.data_as(_i64), idx.shape[0], _dp(scratch), scratch.shape[0], _dp(out)),
        "convT2d_pool_htanh_mean_tanh_at")
    return out


def convT2d_pool_htanh_mean_tanh(x, w, b=None, stride=1, pad=1, pk=2, ps=2, lo=-1.0, hi=1.0):
    """Whole model output, shape [N, C_out] (the [N, C_out, 1, 1] result)."""
    N = x.shape[0]
    C_out = w.shape[1]
    y = convT2d_pool_htanh_mean_tanh_at(x, w, b, np.arange(N * C_out), stride, pad, pk, ps, lo, hi)
    return y.reshape(N, C_out)


# -- epilogue-only operators over a precomputed convolution output -------------

def pool_htanh_mean_tanh(z, pk=2, ps=2, lo=-1.0, hi=1.0):
    """Tail of the transposed-conv model on z[N, C, H, W] (float32 or float64) -> [N, C]."""
    N, C, H, W = z.shape
    y = np.empty((N, C), np.float64)
    if z.dtype == np.float32:
        scratch = np.empty(max(1, num_threads()) * H * W, np.float64)
        _check(lib().oracle_pool_htanh_mean_tanh_f32(_fp(np.ascontiguousarray(z)), _dp(y), N, C, H, W,
                                                     pk, ps, lo, hi, _dp(scratch), scratch.shape[0]),
               "pool_htanh_mean_tanh")
    else:
        zd = np.ascontiguousarray(z, dtype=np.float64)
        _check(lib().oracle_pool_htanh_mean_tanh(_dp(zd), _dp(y), N, C, H, W, pk, ps, lo, hi),
               "pool_htanh_mean_tanh")
    return y


def lrelu_add_clamp_gelu_array(z, s, slope=0.2, lo=-1.0, hi=1.0):
    """Elementwise epilogue of the Conv3d model on z[N, C, ...] (float32) with s[C]."""
    N, C = z.shape[:2]
    S = int(np.prod(z.shape[2:])) if z.ndim > 2 else 1
    zz = np.ascontiguousarray(z, dtype=np.float32)
    ss = np.ascontiguousarray(np.asarray(s, np.float32).reshape(-1))
    y = np.empty(z.shape, np.float64)
    _check(lib().oracle_lrelu_add_clamp_gelu_f32(_fp(zz), _fp(ss), _dp(y), N, C, S, slope, lo, hi),
           "lrelu_add_clamp_gelu")
    return y
