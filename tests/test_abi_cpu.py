"""Host-side checks of the C ABI (no GPU needed, no compute launched).

* libcce.so loads and exports every function include/cce.h declares.
* Argument validation returns the documented status before any HIP call:
  every case here fails validation, so nothing reaches the runtime.
"""
import ctypes
import re
from pathlib import Path

import pytest

import channel_convolution_epilogue_amd as cce

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "cce.h"

OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, ELAUNCH, ETOOBIG, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8
FAKE = 0x10000  # a non-NULL, 16-byte aligned address that is never dereferenced


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"^\s*#.*$", "", text, flags=re.M)  # preprocessor lines (macro constants)
    return sorted(set(re.findall(r"\b([a-zA-Z_][a-zA-Z0-9_]*)\s*\(", text)) -
                  {"if", "defined", "sizeof"})


@pytest.fixture(scope="module")
def lib():
    return cce.load()


def test_header_declares_the_api():
    assert declared_functions() == sorted(cce.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(str(cce.library_path()))
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_status_strings(lib):
    for st in (OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, ELAUNCH, ETOOBIG, ESCRATCH):
        s = cce.status_string(st)
        assert s and s != "unknown status"
    assert cce.status_string(12345) == "unknown status"
    assert lib.cce_version() == 104


def c2(lib, x=FAKE, w=FAKE, b=None, y=FAKE, N=1, C_in=8, H=16, W=16, C_out=64, k=3):
    return lib.conv2d_relu_hswish(x, w, b, y, N, C_in, H, W, C_out, k, None)


def test_conv2d_validation(lib):
    assert c2(lib, x=None) == ENULL
    assert c2(lib, w=None) == ENULL
    assert c2(lib, y=None) == ENULL
    assert c2(lib, N=0) == ESHAPE
    assert c2(lib, H=2) == ESHAPE
    assert c2(lib, W=-5) == ESHAPE
    assert c2(lib, C_in=3) == EUNSUP
    assert c2(lib, C_in=32) == EUNSUP
    assert c2(lib, C_out=48) == EUNSUP
    assert c2(lib, k=2) == EUNSUP
    assert c2(lib, C_in=16, k=5) == EUNSUP  # weights and windows exceed LDS
    assert c2(lib, H=1 << 15, W=1 << 13) == ETOOBIG  # one image of 2^31 floats
    assert c2(lib, x=FAKE + 2) == EALIGN
    assert c2(lib, b=FAKE + 1) == EALIGN
    assert c2(lib, N=1 << 20, H=1024, W=1024) == ETOOBIG


def c3(lib, x=FAKE, w=FAKE, b=None, s=FAKE, y=FAKE, N=1, C_in=8, D=5, H=9, W=9, C_out=64, k=3,
       slope=0.2, lo=-1.0, hi=1.0):
    return lib.conv3d_lrelu_add_clamp_gelu(x, w, b, s, y, N, C_in, D, H, W, C_out, k, slope, lo, hi,
                                           None)


def test_conv3d_validation(lib):
    assert c3(lib, s=None) == ENULL
    assert c3(lib, x=None) == ENULL
    assert c3(lib, D=2) == ESHAPE
    assert c3(lib, C_in=3) == EUNSUP
    assert c3(lib, C_in=32) == EUNSUP
    assert c3(lib, C_out=48) == EUNSUP
    assert c3(lib, k=5) == EUNSUP   # 3 x 3 x 3 and 1 x 1 x 1 only
    assert c3(lib, k=2) == EUNSUP
    assert c3(lib, k=1, N=1 << 16, D=64, H=64, W=64) == ETOOBIG  # k = 1 keeps every voxel
    assert c3(lib, lo=1.0, hi=-1.0) == EUNSUP
    assert c3(lib, slope=float("nan")) == EUNSUP
    assert c3(lib, hi=float("inf")) == EUNSUP
    assert c3(lib, s=FAKE + 2) == EALIGN
    assert c3(lib, N=1 << 16, D=64, H=128, W=128) == ETOOBIG


def ct(lib, x=FAKE, w=FAKE, b=None, y=FAKE, N=2, C_in=64, H=16, W=16, C_out=64, k=3, stride=1,
       pad=1, pk=2, ps=2, lo=-1.0, hi=1.0, ws=FAKE, ws_bytes=1 << 20):
    return lib.convT2d_pool_htanh_mean_tanh(x, w, b, y, N, C_in, H, W, C_out, k, stride, pad, pk, ps,
                                            lo, hi, ws, ws_bytes, None)


def test_convT_validation(lib):
    assert ct(lib, x=None) == ENULL
    assert ct(lib, y=None) == ENULL
    assert ct(lib, H=1) == ESHAPE  # conv output 1 x W is smaller than the 2 x 2 pool
    assert ct(lib, stride=0) == ESHAPE
    assert ct(lib, stride=2) == EUNSUP
    assert ct(lib, pad=0) == EUNSUP
    assert ct(lib, pk=3) == EUNSUP
    assert ct(lib, C_in=12) == EUNSUP   # C_in must be a multiple of 8
    assert ct(lib, C_in=520) == EUNSUP  # and at most 512
    assert ct(lib, C_out=48) == EUNSUP  # C_out in {16, 32, 64}
    assert ct(lib, C_out=128) == EUNSUP
    assert ct(lib, lo=2.0, hi=1.0) == EUNSUP
    assert ct(lib, w=FAKE + 2) == EALIGN
    assert ct(lib, ws=None) == EWS
    assert ct(lib, ws=FAKE + 16) == EWS  # must be 256-byte aligned
    need = cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(2, 64, 16, 16, 64)
    assert ct(lib, ws_bytes=need - 1) == EWS
    assert ct(lib, N=1 << 12, H=1024, W=1024) == ETOOBIG


def test_convT_noalloc_validation(lib):
    """The entry point without a workspace validates like the one with it, and
    rejects calls whose workspace would not fit its static 8 MiB scratch
    before any HIP call: the page's layer at 256 x 256 fits up to N = 251."""
    def nt(N=2, H=16, W=16, C_in=64, C_out=64, x=FAKE, y=FAKE, stride=1, lo=-1.0, hi=1.0):
        return lib.convT2d_pool_htanh_mean_tanh_noalloc(x, FAKE, None, y, N, C_in, H, W, C_out, 3, stride, 1,
                                                        2, 2, lo, hi, None)
    assert nt(x=None) == ENULL
    assert nt(H=1) == ESHAPE
    assert nt(stride=2) == EUNSUP
    assert nt(C_out=48) == EUNSUP
    assert nt(lo=2.0, hi=1.0) == EUNSUP
    assert nt(y=FAKE + 2) == EALIGN
    assert nt(N=252, H=256, W=256) == ESCRATCH
    assert cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(251, 64, 256, 256, 64) <= 8 << 20
    assert cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(252, 64, 256, 256, 64) > 8 << 20
    assert "scratch" in cce.status_string(ESCRATCH)


def test_convT_workspace_size(lib):
    # N counters (padded to 256 bytes) + the prepared 64x64x3x3 weight + N * tiles * 64
    # fp32 partial sums, tiles of 8 x 16 pooling windows.
    wprep = 64 * 64 * 9 * 4
    assert cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(16, 64, 256, 256, 64) == 256 + wprep + 16 * 128 * 256
    assert cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(128, 64, 256, 256, 64) == 512 + wprep + 128 * 128 * 256
    assert cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(1, 64, 2, 2, 64) == 256 + wprep + 256
    assert cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(1, 64, 16, 16, 64, stride=2) == 0
    # other layer shapes: C_in x C_out x 9 prepared weights, C_out partials per tile;
    # tiles of 16 pooling-window columns by 16 rows (C_out = 16) or 8 rows (C_out = 32)
    assert cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(3, 8, 35, 42, 16) == \
        256 + 8 * 16 * 9 * 4 + 3 * (2 * 2) * 16 * 4
    assert cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(300, 128, 64, 64, 32) == \
        1280 + 128 * 32 * 9 * 4 + 300 * (4 * 2) * 32 * 4
    assert cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(1, 24, 16, 16, 48) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 8, 8, 8)
    w = torch.zeros(64, 8, 3, 3)
    with pytest.raises(TypeError):
        cce.conv2d_relu_hswish(x, w, None, out=torch.zeros(1, 64, 6, 6))


def test_binding_checks_shapes_before_any_pointer_reaches_the_abi():
    """The ABI trusts its size arguments, so the binding rejects tensors whose
    shapes disagree with the sizes it passes (here on CPU tensors: the shape
    checks come before the device check)."""
    import torch
    z = torch.zeros
    x = z(1, 8, 8, 8)
    w = z(64, 8, 3, 3)
    with pytest.raises(ValueError, match="out"):
        cce.conv2d_relu_hswish(x, w, None, out=z(1, 64, 6, 5))   # too small an output
    with pytest.raises(ValueError, match="w"):
        cce.conv2d_relu_hswish(x, z(64, 4, 3, 3))                 # C_in disagrees with x
    with pytest.raises(ValueError, match="w"):
        cce.conv2d_relu_hswish(x, z(64, 8, 3, 2))                 # non-square kernel
    with pytest.raises(ValueError, match="b"):
        cce.conv2d_relu_hswish(x, w, z(32))
    with pytest.raises(ValueError, match="x"):
        cce.conv2d_relu_hswish(z(8, 8, 8), w)
    x3, w3 = z(1, 8, 5, 6, 6), z(64, 8, 3, 3, 3)
    with pytest.raises(ValueError, match="out"):
        cce.conv3d_lrelu_add_clamp_gelu(x3, w3, None, z(64), out=z(1, 64, 3, 4, 3))
    with pytest.raises(ValueError, match="s"):
        cce.conv3d_lrelu_add_clamp_gelu(x3, w3, None, z(63))
    xt = z(1, 64, 8, 8)
    with pytest.raises(ValueError, match="w"):
        cce.convT2d_pool_htanh_mean_tanh(xt, z(32, 64, 3, 3))    # [C_out, C_in] order given
    with pytest.raises(ValueError, match="out"):
        cce.convT2d_pool_htanh_mean_tanh(xt, z(64, 64, 3, 3), out=z(1, 32, 1, 1))
    with pytest.raises(ValueError, match="out"):
        cce.pool_htanh_mean_tanh(z(2, 3, 8, 8), out=z(2, 3))
    with pytest.raises(ValueError, match="out"):
        cce.lrelu_add_clamp_gelu(z(2, 3, 4, 4), z(3), out=z(2, 3, 16))


def test_tail_validation(lib):
    def pt(z=FAKE, y=FAKE, N=2, C=3, H=8, W=8, pk=2, ps=2, lo=-1.0, hi=1.0):
        return lib.pool_htanh_mean_tanh(z, y, N, C, H, W, pk, ps, lo, hi, None)
    assert pt(z=None) == ENULL
    assert pt(H=1) == ESHAPE
    assert pt(N=0) == ESHAPE
    assert pt(pk=9) == ESHAPE  # window larger than the plane
    assert pt(ps=0) == ESHAPE
    assert pt(lo=1.0, hi=0.0) == EUNSUP
    assert pt(y=FAKE + 1) == EALIGN
    assert pt(N=1 << 20, C=1 << 12) == ETOOBIG

    def lt(z=FAKE, s=FAKE, y=FAKE, N=2, C=3, S=10, slope=0.2, lo=-1.0, hi=1.0):
        return lib.lrelu_add_clamp_gelu(z, s, y, N, C, S, slope, lo, hi, None)
    assert lt(s=None) == ENULL
    assert lt(S=0) == ESHAPE
    assert lt(hi=float("nan")) == EUNSUP
    assert lt(z=FAKE + 2) == EALIGN
    assert lt(S=1 << 41) == ETOOBIG
