"""Fused small-channel convolution + epilogue operators for AMD MI355X (gfx950).

Thin Python binding over the C ABI in include/cce.h (libcce.so, built in-tree
by ``python -m channel_convolution_epilogue_amd.build``).  The binding only
marshals torch tensors into device pointers, sizes and the current HIP
stream; every step of every operator runs in the library's HIP kernels.
There is no CPU fallback: if the library is missing or the tensors are not
on a GPU, the call raises.
"""
from ._binding import (  # noqa: F401
    CceError,
    conv2d_relu_hswish,
    conv3d_lrelu_add_clamp_gelu,
    convT2d_pool_htanh_mean_tanh,
    convT2d_pool_htanh_mean_tanh_noalloc,
    convT2d_pool_htanh_mean_tanh_workspace_bytes,
    library_path,
    lrelu_add_clamp_gelu,
    pool_htanh_mean_tanh,
    load,
    status_string,
    EXPORTED_SYMBOLS,
)
