"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer runs (CPU only).

* The oracle built with gcc's sanitizers and loaded into the pin suite
  (tests/test_oracle_pins.py) through LD_PRELOAD of their runtimes passes
  every pin: no out-of-bounds access, use after free or undefined arithmetic
  in its loop nests.
* A control copy of the oracle with a planted out-of-bounds read (one input
  element past the end of x) fails that run with an AddressSanitizer
  report, so the check is live.
* The library's C-ABI layer (every argument check before any HIP call)
  built with clang's sanitizers for host code and loaded by the ABI
  validation tests (tests/test_abi_cpu.py) passes them.

Each run is a subprocess (the sanitizer runtimes must be loaded before the
interpreter starts), with pytest's output capture off so that a sanitizer
report reaches the process's stderr even when the sanitizer ends the run.
"""
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
ORACLE_SRC = ROOT / "oracle" / "oracle.c"
SAN_FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-fopenmp", "-fPIC", "-shared", "-std=c11"]


def gcc_runtime(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build_oracle(tmp: Path, text: str) -> Path:
    src, so = tmp / "oracle_san.c", tmp / "liboracle_san.so"
    src.write_text(text)
    subprocess.run(["gcc", *SAN_FLAGS, "-o", str(so), str(src), "-lm"], check=True, capture_output=True)
    return so


def run_pins(lib: Path, stop_at_first_failure=True):
    env = dict(os.environ, CCE_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2",
               LD_PRELOAD=f"{gcc_runtime('libasan.so')} {gcc_runtime('libubsan.so')}",
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return subprocess.run([sys.executable, "-m", "pytest", str(ROOT / "tests" / "test_oracle_pins.py"),
                           *(["-x"] if stop_at_first_failure else []), "-q",
                           "-s", "-p", "no:cacheprovider", "-m", "not gpu"], cwd=str(ROOT), env=env,
                          capture_output=True, text=True, timeout=600)


def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path):
    res = run_pins(build_oracle(tmp_path, ORACLE_SRC.read_text()))
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr


def test_planted_out_of_bounds_read_is_reported(tmp_path):
    """The transposed conv's plane loop reads one input element further on:
    past the end of x at the last element of the last plane.  Small numpy
    buffers come from numpy's own cache (no redzones), so the run goes on
    past the first failing pins (no -x) until a pin with a large input
    reaches the read and AddressSanitizer stops the process."""
    text = ORACLE_SRC.read_text()
    anchor = "z[(size_t)oh * Wo + ow] += (double)xp[(size_t)ih * W + iw] * wv;"
    assert text.count(anchor) == 1
    bad = text.replace(anchor, "z[(size_t)oh * Wo + ow] += (double)xp[(size_t)ih * W + iw + 1] * wv;")
    res = run_pins(build_oracle(tmp_path, bad), stop_at_first_failure=False)
    assert res.returncode != 0
    assert "AddressSanitizer" in res.stderr and "heap-buffer-overflow" in res.stderr, res.stderr[-3000:]


def test_abi_validation_passes_under_asan_and_ubsan(tmp_path):
    from channel_convolution_epilogue_amd import build
    lib = build.build_sanitized_api(tmp_path)
    code = ("import sys, pathlib\n"
            f"sys.path.insert(0, {str(ROOT)!r})\n"
            "import channel_convolution_epilogue_amd._binding as b\n"
            f"b._LIB_PATH = pathlib.Path({str(lib)!r})\n"
            "import pytest\n"
            f"sys.exit(pytest.main([{str(ROOT / 'tests' / 'test_abi_cpu.py')!r}, '-x', '-q', '-s', "
            "'-p', 'no:cacheprovider', '-m', 'not gpu', '-k', 'not fresh_process']))\n")
    env = dict(os.environ, LD_PRELOAD=build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-c", code], cwd=str(ROOT), env=env, capture_output=True, text=True,
                         timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr
    assert " passed" in res.stdout
