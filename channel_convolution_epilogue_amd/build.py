"""Build libcce.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m channel_convolution_epilogue_amd.build [--verbose]

Every source is compiled in one hipcc invocation for --offload-arch=gfx950.
Packed fp32 instructions are switched off for the device code
(-target-feature -packed-fp32-ops); hipcc's host pass warns that it does not
know that feature, which is harmless.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libcce.so"

SOURCES = [
    "cce_api.cpp",
    "conv2d_relu_hswish.hip",
    "conv3d_lrelu_add_clamp_gelu.hip",
    "convT2d_pool_htanh_mean_tanh.hip",
    "pool_htanh_mean_tanh.hip",
    "lrelu_add_clamp_gelu.hip",
]

ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = Path(rocm) / "bin" / "hipcc"
    return str(path) if path.exists() else "hipcc"


def build(verbose: bool = False, extra: list[str] | None = None) -> Path:
    tmp = LIB.with_suffix(f".so.tmp{os.getpid()}")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-I", str(INCLUDE), "-I", str(CSRC), "-o", str(tmp)]
    if verbose:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    cmd += list(extra or [])
    # cce_api.cpp is plain HIP host code; compile it as HIP so one driver call links all.
    for s in SOURCES:
        src = CSRC / s
        cmd += (["-x", "hip", str(src), "-x", "none"] if s.endswith(".cpp") else [str(src)])
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = res.stdout + res.stderr
    noise = "is not a recognized feature for this target"
    shown = "\n".join(l for l in out.splitlines() if noise not in l and "warnings generated" not in l)
    if res.returncode != 0:
        sys.stderr.write(shown + "\n")
        raise RuntimeError(f"hipcc failed (rc={res.returncode})")
    if verbose and shown.strip():
        print(shown)
    os.replace(tmp, LIB)
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--verbose", action="store_true", help="print per-kernel register/LDS usage")
    args = ap.parse_args()
    print(build(verbose=args.verbose))


if __name__ == "__main__":
    main()
