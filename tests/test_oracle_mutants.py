"""The oracle's pins catch plausible mistakes.

Each case plants one slip in a copy of oracle/oracle.c (a dropped bias,
transposed kernel taps, an unflipped transposed convolution, a wrong
HardSwish constant, LeakyReLU sign, GELU scale, epilogue order, pooling
window, output size or mean divisor), compiles it with gcc, and runs the pin
suite (tests/test_oracle_pins.py) against that library in a fresh process:
the suite must fail.  A control copy with no change must pass, so a failure
is the mutant's, not the test's own machinery.  CPU only; the planted mistakes live in
temporary copies and never touch the real oracle.
"""
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SRC = ROOT / "oracle" / "oracle.c"
PINS = ROOT / "tests" / "test_oracle_pins.py"

# name -> list of (text in oracle.c, replacement); each text occurs exactly once.
MUTANTS = {
    "conv2d_bias_dropped": [(
        "int n, int o, int h, int ww) {\n  double acc = bias_of(b, o);",
        "int n, int o, int h, int ww) {\n  double acc = 0.0; (void)b;")],
    "conv2d_input_taps_transposed": [(
        "(h + kh)) * W + (ww + kw)];\n        double wv = w[(((size_t)o * C_in + i) * k + kh) * k + kw];",
        "(h + kw)) * W + (ww + kh)];\n        double wv = w[(((size_t)o * C_in + i) * k + kh) * k + kw];")],
    "conv2d_weight_channels_swapped": [(
        "double wv = w[(((size_t)o * C_in + i) * k + kh) * k + kw];",
        "double wv = w[(((size_t)i * C_in + o % C_in) * k + kh) * k + kw];")],
    "relu_leaks": [("double oracle_relu(double v) { return v > 0.0 ? v : 0.0; }",
                    "double oracle_relu(double v) { return v > 0.0 ? v : 0.01 * v; }")],
    "hardswish_divisor": [("double g = (v + 3.0) / 6.0;", "double g = (v + 3.0) / 5.0;")],
    "leaky_relu_sign": [("return v >= 0.0 ? v : slope * v;", "return v >= 0.0 ? v : -slope * v;")],
    "epilogue_add_before_leaky_relu": [(
        "double t = oracle_leaky_relu(v, slope);\n  t = t + s;",
        "double t = oracle_leaky_relu(v + s, slope);")],
    "gelu_scale": [("erf(t / sqrt(2.0))", "erf(t / 2.0)")],
    "clamp_upper_bound": [("if (v > hi) v = hi;", "if (v >= hi) v = lo;")],
    "conv3d_depth_tap": [("(d + kd)) * H + (h + kh)) * W", "(d + kh)) * H + (h + kd)) * W")],
    "conv3d_bias_dropped": [(
        "int n, int o, int d, int h, int ww) {\n  double acc = bias_of(b, o);",
        "int n, int o, int d, int h, int ww) {\n  double acc = 0.0; (void)b;")],
    "convT_gather_unflipped": [("int th = h + pad - kh;", "int th = h - pad + kh;"),
                               ("int tw = ww + pad - kw;", "int tw = ww - pad + kw;")],
    "convT_scatter_weight_as_c_out_by_c_in": [(
        "xv * (double)w[(((size_t)i * C_out + o) * k + kh) * k + kw];",
        "xv * (double)w[(((size_t)o * C_in + i) * k + kh) * k + kw];")],
    "convT_output_size": [("return (in - 1) * stride - 2 * pad + k;", "return (in - 1) * stride - pad + k;")],
    "pool_window_column_offset": [(
        "double v = z[(size_t)(ph * ps + dh) * Wo + (pw * ps + dw)];",
        "double v = z[(size_t)(ph * ps + dh) * Wo + (pw * ps + dh)];")],
    "pool_ceil_mode": [("return (in - pk) / ps + 1;", "return (in - pk + ps - 1) / ps + 1;")],
    "hardtanh_dropped": [("      sum += oracle_clamp(m, lo, hi);\n    }\n  return tanh",
                          "      sum += m; (void)lo; (void)hi;\n    }\n  return tanh")],
    "mean_divisor": [("return tanh(sum / ((double)PH * (double)PW));",
                      "return tanh(sum / ((double)PH * (double)PW + 1.0));")],
    "f32_tail_widened_off_by_one": [(
        "for (size_t p = 0; p < (size_t)H * W; ++p) plane[p] = (double)zp[p];",
        "for (size_t p = 0; p < (size_t)H * W; ++p) plane[p] = (double)zp[p + (p + 1 < (size_t)H * W)];")],
    "f32_elementwise_channel_of_s": [("(double)z[base + e], (double)s[c]",
                                      "(double)z[base + e], (double)s[(c + 1) % C]")],
    "conv3d_model_channel_of_s": [(
        "* Wo + ww] =\n                oracle_lrelu_add_clamp_gelu(v, (double)s[o],",
        "* Wo + ww] =\n                oracle_lrelu_add_clamp_gelu(v, (double)s[(o + 1) % C_out],")],
    "conv2d_sampled_index_decode": [(
        "    int h = (int)(q % Ho); q /= Ho;\n    int o = (int)(q % C_out); q /= C_out;",
        "    int o = (int)(q % C_out); q /= C_out;\n    int h = (int)(q % Ho); q /= Ho;")],
    "conv3d_sampled_index_decode": [(
        "    int d = (int)(q % Do); q /= Do;\n    int o = (int)(q % C_out); q /= C_out;",
        "    int o = (int)(q % C_out); q /= C_out;\n    int d = (int)(q % Do); q /= Do;")],
    "convT_sampled_image_channel_decode": [(
        "int n = (int)(nc_idx[j] / C_out), o = (int)(nc_idx[j] % C_out);",
        "int n = (int)(nc_idx[j] % N), o = (int)(nc_idx[j] / N);")],
    "clamp_lower_bound": [("if (v < lo) v = lo;", "if (v < lo) v = hi;")],
    "pool_running_max_starts_at_zero": [("      double m = z[(size_t)(ph * ps) * Wo + (pw * ps)];",
                                         "      double m = 0.0;")],
    "mean_over_unpooled_count": [("  return tanh(sum / ((double)PH * (double)PW));",
                                  "  return tanh(sum / ((double)Ho * (double)Wo));")],
    "tanh_dropped": [("  return tanh(sum / ((double)PH * (double)PW));", "  return sum / ((double)PH * (double)PW);")],
    "conv3d_weight_taps_swapped": [("double wv = w[((((size_t)o * C_in + i) * k + kd) * k + kh) * k + kw];",
                                    "double wv = w[((((size_t)o * C_in + i) * k + kh) * k + kd) * k + kw];")],
    "pool_tail_plane_order": [("oracle_pool_htanh_mean_tanh_plane(z + ((size_t)n * C + c) * H * W, H, W, pk, ps, lo, hi);",
                               "oracle_pool_htanh_mean_tanh_plane(z + ((size_t)c * N + n) * H * W, H, W, pk, ps, lo, hi);")],
    "f32_tail_plane_order": [("const float *zp = z + ((size_t)n * C + c) * H * W;",
                              "const float *zp = z + ((size_t)c * N + n) * H * W;")],
    "convT_gather_bias_dropped": [(
        "int ww) {\n  double acc = bias_of(b, o);\n  for (int i = 0; i < C_in; ++i)\n    for (int kh = 0; kh < k; ++kh) {\n      int th",
        "int ww) {\n  double acc = 0.0; (void)b;\n  for (int i = 0; i < C_in; ++i)\n    for (int kh = 0; kh < k; ++kh) {\n      int th")],
    "convT_scatter_flipped_positions": [("int oh = ih * stride - pad + kh, ow = iw * stride - pad + kw;",
                                         "int oh = ih * stride + pad - kh, ow = iw * stride + pad - kw;")],
    "convT_model_plane_flipped_positions": [("int oh = ih * stride - pad + kh;", "int oh = ih * stride + pad - kh;"),
                                            ("int ow = iw * stride - pad + kw;", "int ow = iw * stride + pad - kw;")],
    "convT_model_plane_bias_dropped": [("for (size_t p = 0; p < (size_t)Ho * Wo; ++p) z[p] = bias_of(b, o);",
                                       "for (size_t p = 0; p < (size_t)Ho * Wo; ++p) z[p] = 0.0; (void)b;")],
    "convT_model_plane_weight_as_c_out_by_c_in": [(
        "double wv = (double)w[(((size_t)i * C_out + o) * k + kh) * k + kw];",
        "double wv = (double)w[(((size_t)o * C_in + i) * k + kh) * k + kw];")],
    "convT_model_plane_input_channel": [("const float *xp = x + ((size_t)n * C_in + i) * H * W;",
                                        "const float *xp = x + ((size_t)n * C_in + (i + 1) % C_in) * H * W;")],
}


def _build_and_run_pins(workdir: Path, text: str):
    workdir.mkdir(parents=True, exist_ok=True)
    src = workdir / "oracle_copy.c"
    so = workdir / "liboracle_copy.so"
    src.write_text(text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so), str(src), "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, CCE_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-m", "pytest", str(PINS), "-x", "-q", "-p", "no:cacheprovider",
                           "-m", "not gpu"], cwd=str(ROOT), env=env, capture_output=True, text=True,
                          timeout=600)


def _mutant_text(name):
    text = SRC.read_text()
    for old, new in MUTANTS[name]:
        assert text.count(old) == 1, f"{name}: anchor not found exactly once in oracle.c: {old!r}"
        text = text.replace(old, new)
    return text


@pytest.fixture(scope="module")
def pin_runs(tmp_path_factory):
    """The pin suite run against the control copy and every mutant, four at a
    time (each run is its own process with two OpenMP threads)."""
    from concurrent.futures import ThreadPoolExecutor
    base = tmp_path_factory.mktemp("oracle_copies")
    jobs = [("control", SRC.read_text())] + [(n, _mutant_text(n)) for n in sorted(MUTANTS)]
    with ThreadPoolExecutor(max_workers=4) as pool:
        results = list(pool.map(lambda j: (j[0], _build_and_run_pins(base / j[0], j[1])), jobs))
    return dict(results)


def test_control_copy_passes_the_pins(pin_runs):
    res = pin_runs["control"]
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(pin_runs, name):
    res = pin_runs[name]
    tail = res.stdout.strip().splitlines()[-1] if res.stdout.strip() else ""
    # A pin must fail (an assertion), not the test run itself (collection or import errors).
    assert res.returncode == 1 and " failed" in tail and "error" not in tail, \
        f"{name}: pins did not catch it (rc={res.returncode}): {tail}\n{res.stderr[-2000:]}"
    caught = [l.split(" - ")[0].split("::")[-1] for l in res.stdout.splitlines() if l.startswith("FAILED")]
    print(f"{name}: caught by {', '.join(caught) or '?'} ({tail})")
