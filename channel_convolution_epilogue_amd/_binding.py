"""ctypes marshalling for libcce.so.  Same names as the C entry points."""
from __future__ import annotations

import contextlib
import ctypes
import threading
from pathlib import Path

_PKG = Path(__file__).resolve().parent
_LIB_PATH = _PKG / "libcce.so"

EXPORTED_SYMBOLS = (
    "cce_status_string",
    "cce_version",
    "conv2d_relu_hswish",
    "conv3d_lrelu_add_clamp_gelu",
    "convT2d_pool_htanh_mean_tanh",
    "convT2d_pool_htanh_mean_tanh_noalloc",
    "convT2d_pool_htanh_mean_tanh_workspace_bytes",
    "lrelu_add_clamp_gelu",
    "pool_htanh_mean_tanh",
)

_lib = None
_lock = threading.Lock()
_workspaces: dict = {}


class CceError(RuntimeError):
    """A libcce call returned a non-zero cce_status."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


def library_path() -> Path:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libcce.so (raises if it has not been built).

    PyTorch's ROCm wheel carries its own HIP runtime under the same soname
    (libamdhip64.so.7) as the system one libcce.so is linked against, and
    whichever is loaded first serves the whole process.  torch is imported
    first, so libcce binds to the runtime that owns the tensors and streams
    it is handed; loading libcce first put the system runtime under torch
    and made every libcce launch fail."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not _LIB_PATH.exists():
            raise ImportError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m channel_convolution_epilogue_amd.build`")
        import torch  # noqa: F401  (before libcce: one HIP runtime per process)
        L = ctypes.CDLL(str(_LIB_PATH))
        vp, fp, i, f, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.cce_status_string.restype = ctypes.c_char_p
        L.cce_status_string.argtypes = [i]
        L.cce_version.restype = i
        L.conv2d_relu_hswish.restype = i
        L.conv2d_relu_hswish.argtypes = [fp, fp, fp, fp] + [i] * 6 + [vp]
        L.conv3d_lrelu_add_clamp_gelu.restype = i
        L.conv3d_lrelu_add_clamp_gelu.argtypes = [fp] * 5 + [i] * 7 + [f] * 3 + [vp]
        L.convT2d_pool_htanh_mean_tanh.restype = i
        L.convT2d_pool_htanh_mean_tanh.argtypes = [fp] * 4 + [i] * 10 + [f, f, vp, sz, vp]
        L.convT2d_pool_htanh_mean_tanh_noalloc.restype = i
        L.convT2d_pool_htanh_mean_tanh_noalloc.argtypes = [fp] * 4 + [i] * 10 + [f, f, vp]
        L.convT2d_pool_htanh_mean_tanh_workspace_bytes.restype = sz
        L.convT2d_pool_htanh_mean_tanh_workspace_bytes.argtypes = [i] * 10
        L.pool_htanh_mean_tanh.restype = i
        L.pool_htanh_mean_tanh.argtypes = [fp, fp] + [i] * 6 + [f, f, vp]
        L.lrelu_add_clamp_gelu.restype = i
        L.lrelu_add_clamp_gelu.argtypes = [fp, fp, fp, i, i, ctypes.c_longlong, f, f, f, vp]
        _lib = L
        return L


def status_string(status: int) -> str:
    return load().cce_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise CceError(fn, status, status_string(status))


def _dev_ptr(t, name, ndim=None):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a torch tensor on a GPU")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")
    return t.data_ptr()


def _dims(t, ndim, name):
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")


def _expect(t, shape, name):
    """The C ABI takes sizes, not buffers: every tensor handed to it must have
    exactly the shape the sizes imply, or a kernel would read or write past it."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(x, **ts):
    for name, t in ts.items():
        if t is not None and t.device != x.device:
            raise ValueError(f"{name} is on {t.device}, x on {x.device}")


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _on_device(t):
    """The library launches on the current HIP device (and sizes its grids
    for it), so each call runs with the input tensor's device current."""
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError("the input must be a torch tensor on a GPU")
    if t.device.index is None or t.device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(t.device)


def conv2d_relu_hswish(x, w, b=None, out=None):
    """HardSwish(ReLU(conv2d(x, w, b))), stride 1, padding 0.

    x [N, C_in, H, W], w [C_out, C_in, k, k], b [C_out] or None -> [N, C_out, H-k+1, W-k+1]
    """
    import torch
    L = load()
    _dims(x, 4, "x")
    _dims(w, 4, "w")
    N, C_in, H, W = x.shape
    C_out, _, k, _ = w.shape
    _expect(w, (C_out, C_in, k, k), "w")
    _expect(b, (C_out,), "b")
    _expect(out, (N, C_out, H - k + 1, W - k + 1), "out")
    _same_device(x, w=w, b=b, out=out)
    if out is None:
        out = torch.empty((N, C_out, H - k + 1, W - k + 1), device=x.device, dtype=torch.float32)
    with _on_device(x):
        st = L.conv2d_relu_hswish(_dev_ptr(x, "x", 4), _dev_ptr(w, "w", 4), _dev_ptr(b, "b", 1),
                                  _dev_ptr(out, "out", 4), N, C_in, H, W, C_out, k, _stream(x))
    _check("conv2d_relu_hswish", st)
    return out


def conv3d_lrelu_add_clamp_gelu(x, w, b, s, negative_slope=0.2, clamp_lo=-1.0, clamp_hi=1.0,
                                out=None):
    """GELU(clamp(LeakyReLU(conv3d(x, w, b)) + s[c], lo, hi)), stride 1, padding 0.

    x [N, C_in, D, H, W], w [C_out, C_in, k, k, k], b [C_out] or None,
    s [C_out] (or [C_out, 1, 1, 1]) -> [N, C_out, D-k+1, H-k+1, W-k+1]
    """
    import torch
    L = load()
    _dims(x, 5, "x")
    _dims(w, 5, "w")
    N, C_in, D, H, W = x.shape
    C_out, _, k, _, _ = w.shape
    _expect(w, (C_out, C_in, k, k, k), "w")
    _expect(b, (C_out,), "b")
    if s.numel() != C_out:
        raise ValueError("s must hold one value per output channel")
    s = s.reshape(C_out)
    _expect(out, (N, C_out, D - k + 1, H - k + 1, W - k + 1), "out")
    _same_device(x, w=w, b=b, s=s, out=out)
    if out is None:
        out = torch.empty((N, C_out, D - k + 1, H - k + 1, W - k + 1), device=x.device,
                          dtype=torch.float32)
    with _on_device(x):
        st = L.conv3d_lrelu_add_clamp_gelu(_dev_ptr(x, "x", 5), _dev_ptr(w, "w", 5), _dev_ptr(b, "b", 1),
                                           _dev_ptr(s, "s", 1), _dev_ptr(out, "out", 5), N, C_in, D, H,
                                           W, C_out, k, float(negative_slope), float(clamp_lo),
                                           float(clamp_hi), _stream(x))
    _check("conv3d_lrelu_add_clamp_gelu", st)
    return out


def convT2d_pool_htanh_mean_tanh_workspace_bytes(N, C_in, H, W, C_out, k=3, stride=1, pad=1,
                                                 pool_k=2, pool_s=2) -> int:
    return int(load().convT2d_pool_htanh_mean_tanh_workspace_bytes(N, C_in, H, W, C_out, k, stride,
                                                                   pad, pool_k, pool_s))


def _workspace(device, stream: int, nbytes: int):
    """A workspace cached per (device, stream) and grown when a call needs
    more.  The call initialises every workspace byte it reads, so the cached
    buffer serves later calls of any shape without being cleared."""
    import torch
    key = (device.index, stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def convT2d_pool_htanh_mean_tanh(x, w, b=None, stride=1, padding=1, pool_k=2, pool_s=2,
                                 htanh_lo=-1.0, htanh_hi=1.0, out=None, workspace=None):
    """tanh(mean_{H,W}(Hardtanh(MaxPool2d(conv_transpose2d(x, w, b))))) -> [N, C_out, 1, 1].

    x [N, C_in, H, W], w [C_in, C_out, k, k], b [C_out] or None.  `workspace`
    (optional) is a uint8 GPU tensor of at least
    convT2d_pool_htanh_mean_tanh_workspace_bytes(...) bytes, any contents.
    """
    import torch
    L = load()
    _dims(x, 4, "x")
    _dims(w, 4, "w")
    N, C_in, H, W = x.shape
    _, C_out, k, _ = w.shape
    _expect(w, (C_in, C_out, k, k), "w")
    _expect(b, (C_out,), "b")
    _expect(out, (N, C_out, 1, 1), "out")
    _same_device(x, w=w, b=b, out=out, workspace=workspace)
    if out is None:
        out = torch.empty((N, C_out, 1, 1), device=x.device, dtype=torch.float32)
    need = convT2d_pool_htanh_mean_tanh_workspace_bytes(N, C_in, H, W, C_out, k, stride, padding,
                                                        pool_k, pool_s)
    stream = _stream(x)
    if workspace is None:
        workspace = _workspace(x.device, stream, need)
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    with _on_device(x):
        st = L.convT2d_pool_htanh_mean_tanh(_dev_ptr(x, "x", 4), _dev_ptr(w, "w", 4), _dev_ptr(b, "b", 1),
                                            _dev_ptr(out, "out", 4), N, C_in, H, W, C_out, k, stride,
                                            padding, pool_k, pool_s, float(htanh_lo), float(htanh_hi),
                                            workspace.data_ptr(), ws_bytes, stream)
    _check("convT2d_pool_htanh_mean_tanh", st)
    return out


def convT2d_pool_htanh_mean_tanh_noalloc(x, w, b=None, stride=1, padding=1, pool_k=2, pool_s=2,
                                         htanh_lo=-1.0, htanh_hi=1.0, out=None):
    """convT2d_pool_htanh_mean_tanh on the library's static per-device scratch
    instead of a workspace: the C call allocates nothing (pass `out` to keep
    this wrapper from allocating the result).  Calls that overlap in time on
    one GPU race on that scratch."""
    import torch
    L = load()
    _dims(x, 4, "x")
    _dims(w, 4, "w")
    N, C_in, H, W = x.shape
    _, C_out, k, _ = w.shape
    _expect(w, (C_in, C_out, k, k), "w")
    _expect(b, (C_out,), "b")
    _expect(out, (N, C_out, 1, 1), "out")
    _same_device(x, w=w, b=b, out=out)
    if out is None:
        out = torch.empty((N, C_out, 1, 1), device=x.device, dtype=torch.float32)
    with _on_device(x):
        st = L.convT2d_pool_htanh_mean_tanh_noalloc(
            _dev_ptr(x, "x", 4), _dev_ptr(w, "w", 4), _dev_ptr(b, "b", 1), _dev_ptr(out, "out", 4), N, C_in,
            H, W, C_out, k, stride, padding, pool_k, pool_s, float(htanh_lo), float(htanh_hi), _stream(x))
    _check("convT2d_pool_htanh_mean_tanh_noalloc", st)
    return out


def pool_htanh_mean_tanh(z, pool_k=2, pool_s=2, htanh_lo=-1.0, htanh_hi=1.0, out=None):
    """tanh(mean_{H,W}(Hardtanh(MaxPool2d(z)))) over a precomputed z [N, C, H, W] -> [N, C, 1, 1]."""
    import torch
    L = load()
    _dims(z, 4, "z")
    N, C, H, W = z.shape
    _expect(out, (N, C, 1, 1), "out")
    _same_device(z, out=out)
    if out is None:
        out = torch.empty((N, C, 1, 1), device=z.device, dtype=torch.float32)
    with _on_device(z):
        st = L.pool_htanh_mean_tanh(_dev_ptr(z, "z", 4), _dev_ptr(out, "out", 4), N, C, H, W, pool_k,
                                    pool_s, float(htanh_lo), float(htanh_hi), _stream(z))
    _check("pool_htanh_mean_tanh", st)
    return out


def lrelu_add_clamp_gelu(z, s, negative_slope=0.2, clamp_lo=-1.0, clamp_hi=1.0, out=None):
    """GELU(clamp(LeakyReLU(z) + s[c], lo, hi)) elementwise over z [N, C, ...] (s has C values)."""
    import torch
    L = load()
    if z.dim() < 2:
        raise ValueError("z must be [N, C, ...]")
    N, C = z.shape[0], z.shape[1]
    S = z.numel() // (N * C) if z.numel() else 0
    if s.numel() != C:
        raise ValueError("s must hold one value per channel")
    s = s.reshape(C)
    _expect(out, tuple(z.shape), "out")
    _same_device(z, s=s, out=out)
    if out is None:
        out = torch.empty_like(z)
    with _on_device(z):
        st = L.lrelu_add_clamp_gelu(_dev_ptr(z, "z"), _dev_ptr(s, "s", 1), _dev_ptr(out, "out"), N, C, S,
                                    float(negative_slope), float(clamp_lo), float(clamp_hi), _stream(z))
    _check("lrelu_add_clamp_gelu", st)
    return out
