"""Build libcce.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m channel_convolution_epilogue_amd.build [--verbose]

Each source is compiled by its own hipcc process for --offload-arch=gfx950
(in parallel, objects under _build/), then the objects are linked.
Packed fp32 instructions are switched off for the device code
(-target-feature -packed-fp32-ops); hipcc's host pass warns that it does not
know that feature, which is harmless.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
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


NOISE = ("is not a recognized feature for this target", "warnings generated")


def _run(cmd: list[str], verbose: bool) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    shown = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                      if not any(n in l for n in NOISE))
    if res.returncode != 0:
        sys.stderr.write(shown + "\n")
        raise RuntimeError(f"hipcc failed (rc={res.returncode}): {' '.join(cmd[-3:])}")
    return shown if verbose else ""


def build(verbose: bool = False, extra: list[str] | None = None) -> Path:
    """Compile every source to an object in parallel (one hipcc per file),
    then link them into libcce.so."""
    objdir = PKG / "_build"
    objdir.mkdir(exist_ok=True)
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-I", str(INCLUDE), "-I", str(CSRC)]
    if verbose:
        flags += ["-Rpass-analysis=kernel-resource-usage"]
    flags += list(extra or [])
    jobs = []
    for s in SOURCES:
        obj = objdir / (Path(s).stem + ".o")
        # cce_api.cpp is plain HIP host code; compile it as HIP like the kernels.
        lang = ["-x", "hip"] if s.endswith(".cpp") else []
        jobs.append((obj, [hipcc(), *flags, "-c", *lang, str(CSRC / s), "-o", str(obj)]))
    workers = max(1, min(len(jobs), os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        outs = list(pool.map(lambda j: _run(j[1], verbose), jobs))
    tmp = LIB.with_suffix(f".so.tmp{os.getpid()}")
    outs.append(_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp),
                      *[str(o) for o, _ in jobs]], verbose))
    for shown in outs:
        if shown.strip():
            print(shown)
    os.replace(tmp, LIB)
    return LIB


SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build_sanitized_api(outdir: Path) -> Path:
    """A debugging copy of the library whose C-ABI layer (cce_api.cpp: every
    argument check, before any HIP call) is built with clang's
    AddressSanitizer and UndefinedBehaviorSanitizer for the host code only,
    linked with the regular kernel objects (built first if missing).  Load it
    with the sanitizer runtime preloaded (sanitizer_runtime()); it never goes
    to a GPU."""
    outdir = Path(outdir)
    outdir.mkdir(parents=True, exist_ok=True)
    objdir = PKG / "_build"
    kernels = [objdir / (Path(s).stem + ".o") for s in SOURCES if s != "cce_api.cpp"]
    if not all(o.exists() for o in kernels):
        build()
    api = outdir / "cce_api_sanitized.o"
    flags = [f"--offload-arch={ARCH}", "-O1", "-std=c++17", "-fPIC", "-Wall", "-I", str(INCLUDE),
             "-I", str(CSRC), *SANITIZE]
    _run([hipcc(), *flags, "-c", "-x", "hip", str(CSRC / "cce_api.cpp"), "-o", str(api)], False)
    lib = outdir / "libcce_sanitized.so"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan", *SANITIZE[:4],
          "-o", str(lib), str(api), *[str(o) for o in kernels]], False)
    return lib


def sanitizer_runtime() -> str:
    """clang's shared AddressSanitizer runtime (which carries the
    UndefinedBehaviorSanitizer handlers) matching hipcc, for LD_PRELOAD."""
    rocm = Path(os.environ.get("ROCM_PATH", "/opt/rocm"))
    found = sorted(rocm.glob("llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under " + str(rocm / "llvm"))
    return str(found[-1])


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--verbose", action="store_true", help="print per-kernel register/LDS usage")
    ap.add_argument("--sanitize-host", metavar="DIR",
                    help="instead, build DIR/libcce_sanitized.so: the C-ABI layer with host "
                         "AddressSanitizer + UndefinedBehaviorSanitizer (load it with "
                         "LD_PRELOAD of the printed runtime)")
    args = ap.parse_args()
    if args.sanitize_host:
        print(build_sanitized_api(Path(args.sanitize_host)))
        print("runtime:", sanitizer_runtime())
        return
    print(build(verbose=args.verbose))


if __name__ == "__main__":
    main()
