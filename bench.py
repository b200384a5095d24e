"""Benchmark of the fused small-channel convolution + epilogue kernels on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--prewarm S] [--workload NAME] [--ops all|none]
                    [--no-cpu-baseline] [--seed S]

One step is one call of the headline workload's fused operator on one batch
of seeded synthetic input already resident in device memory (the default
headline is the largest workload: ConvTranspose2d 3x3 64->64 + MaxPool 2x2 +
Hardtanh + mean + tanh at N = 128, 256 x 256).
S seconds of untimed pre-warm calls (an idle GPU needs a moment of load
before its clocks settle), W untimed warm-up steps, then exactly K timed
steps bracketed by device synchronisations; HIP events on the stream the kernels run on give the
per-launch kernel time.  Rank 0 prints one JSON line with the headline
throughput (GFLOP/s of the convolution's multiply-adds, 2 FLOP each), the
roofline of the dominant kernel, the CPU oracle's throughput (a baseline, not
a target) and, under "ops", the same measurement for every workload.  Every
workload's whole output is also compared with the oracle's
(gpu_error_vs_oracle); --no-cpu-baseline skips the oracle.

Only one GPU exists per box and nothing here is distributed: --gpus above 1
exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

from conv_inputs import (CONV2D, CONV3D, CONVT, TAIL_GELU, TAIL_POOL, WORKLOADS,  # noqa: E402
                         make_inputs, workload_inputs)

METRIC = "fused conv+epilogue ms per call, GFLOP/s & % of fp32/HBM roofline (1 MI355X)"
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak
HEADLINE = "convT2d_pool_htanh_mean_tanh_n128"  # the largest workload that fits one GPU

KERNEL_SOURCES = {
    CONV2D: "conv2d_relu_hswish.hip",
    CONV3D: "conv3d_lrelu_add_clamp_gelu.hip",
    CONVT: "convT2d_pool_htanh_mean_tanh.hip",
    TAIL_POOL: "pool_htanh_mean_tanh.hip",
    TAIL_GELU: "lrelu_add_clamp_gelu.hip",
}
HBM_BOUND = (TAIL_POOL, TAIL_GELU)  # the epilogue-only operators move bytes, not FLOPs


def work_counts(shape: dict) -> dict:
    """Algorithmic work of one call: multiply-adds of the convolution (epilogue
    excluded) and bytes that must cross HBM (read x, w, b, s once; write y once).
    The epilogue-only operators have no convolution: bytes only."""
    op = shape["op"]
    if op == TAIL_POOL:
        n = shape["N"] * shape["C"]
        return {"fma": 0, "flop": 0, "bytes": 4 * (n * shape["H"] * shape["W"] + n)}
    if op == TAIL_GELU:
        n = shape["N"] * shape["C"] * shape["D"] * shape["H"] * shape["W"]
        return {"fma": 0, "flop": 0, "bytes": 4 * (2 * n + shape["C"])}
    N, Ci, Co, k = shape["N"], shape["C_in"], shape["C_out"], shape["k"]
    if op == CONV2D:
        Ho, Wo = shape["H"] - k + 1, shape["W"] - k + 1
        outs = N * Co * Ho * Wo
        fma = outs * Ci * k * k
        nbytes = 4 * (N * Ci * shape["H"] * shape["W"] + Co * Ci * k * k + Co + outs)
    elif op == CONV3D:
        Do, Ho, Wo = shape["D"] - k + 1, shape["H"] - k + 1, shape["W"] - k + 1
        outs = N * Co * Do * Ho * Wo
        fma = outs * Ci * k ** 3
        nbytes = 4 * (N * Ci * shape["D"] * shape["H"] * shape["W"] + Co * Ci * k ** 3 + 2 * Co + outs)
    else:
        Ho, Wo = shape["H"], shape["W"]  # stride 1, padding 1, k = 3
        conv_outs = N * Co * Ho * Wo
        fma = conv_outs * Ci * k * k
        nbytes = 4 * (N * Ci * shape["H"] * shape["W"] + Ci * Co * k * k + Co + N * Co)
    return {"fma": fma, "flop": 2 * fma, "bytes": nbytes}


def source_digest(op: str) -> str:
    """Digest of the operator's kernel source and the device header it includes."""
    csrc = ROOT / "channel_convolution_epilogue_amd" / "csrc"
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES[op], "cce_device.hpp"):
        h.update((csrc / name).read_bytes())
    return h.hexdigest()[:16]


def measured_traffic(op: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    counts, used only while the kernel source still matches the profiled one."""
    f = ROOT / "profiles" / "hbm_traffic.json"
    if not f.exists():
        return None
    try:
        rec = json.loads(f.read_text()).get(workload)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    if rec.get("source_sha256_16") != source_digest(op):
        print(f"# {workload}: the HBM-traffic record was taken on another version of "
              f"{KERNEL_SOURCES[op]}; traffic reported as null", file=sys.stderr)
        return None
    return rec.get("bytes_per_launch")


DOMINANT_KERNEL = {  # substring of the kernel symbol that dominates each operator's time
    CONV2D: "conv2d_relu_hswish_kernel",
    CONV3D: "conv3d_lrelu_add_clamp_gelu_kernel",
    CONVT: "convT2d_pool_htanh_mean_tanh_kernel",
    TAIL_POOL: "::pool_htanh_mean_tanh_kernel",
    TAIL_GELU: "::lrelu_add_clamp_gelu_",  # the flat 16-byte kernel or the per-plane one
}
COPY_KERNEL = "copyBuffer"  # torch's device-to-device copy under ROCm


def _counter_per_dispatch(csv_path: Path, kernel_substr: str, counter: str):
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    return (sum(vals) / len(vals)) if vals else None


def record_traffic(pmc_dir: Path, copy_mib: int, previous: dict | None = None) -> dict:
    """Turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch) into HBM
    bytes per launch of each workload's dominant kernel.  Each counter is
    scaled by the factor that makes it read exactly `copy_mib` MiB for a plain
    device copy of that size.  Expects <dir>/{fetch,write}_<workload>/ and
    <dir>/{fetch,write}_copy/ from `rocprofv3 --pmc ... --output-format csv -o run`.
    Records in `previous` for workloads not measured in this directory are
    kept while their kernel source digest still matches."""
    known = copy_mib * 1024 * 1024
    scale = {}
    for kind, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        kib = _counter_per_dispatch(pmc_dir / f"{kind}_copy" / "run_counter_collection.csv",
                                    COPY_KERNEL, counter)
        scale[kind] = known / (kib * 1024.0)
    out = {"_about": ("HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per "
                      "dispatch), each scaled so that a plain %d MiB device copy reads/writes "
                      "exactly %d MiB; valid while the kernel source digest matches." % (copy_mib, copy_mib)),
           "copy_scale": {k: round(v, 5) for k, v in scale.items()}}
    for name, rec in (previous or {}).items():
        cfg = WORKLOADS.get(name)
        if cfg and isinstance(rec, dict) and rec.get("source_sha256_16") == source_digest(cfg["op"]):
            rec.setdefault("copy_scale", previous.get("copy_scale"))
            out[name] = rec
    for name, cfg in WORKLOADS.items():
        op = cfg["op"]
        f = pmc_dir / f"fetch_{name}" / "run_counter_collection.csv"
        w = pmc_dir / f"write_{name}" / "run_counter_collection.csv"
        if not (f.exists() and w.exists()):
            continue
        fk = _counter_per_dispatch(f, DOMINANT_KERNEL[op], "FETCH_SIZE")
        wk = _counter_per_dispatch(w, DOMINANT_KERNEL[op], "WRITE_SIZE")
        fb, wb = fk * 1024 * scale["fetch"], wk * 1024 * scale["write"]
        out[name] = {"kernel": DOMINANT_KERNEL[op], "source_sha256_16": source_digest(op),
                     "fetch_kib_raw": round(fk, 1), "write_kib_raw": round(wk, 1),
                     "bytes_per_launch": int(fb + wb), "fetch_bytes": int(fb), "write_bytes": int(wb),
                     "copy_scale": out["copy_scale"],
                     "algorithmic_bytes": work_counts(dict(cfg))["bytes"]}
    return out


MFMA_COUNTERS = ("MfmaUtil", "MfmaFlopsF32", "SQ_INSTS_VALU_MFMA_F32", "SQ_INSTS_LDS",
                 "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE")


def record_mfma(pmc_dir: Path, previous: dict | None = None) -> dict:
    """Turn rocprofv3 runs of `--pmc MfmaUtil MfmaFlopsF32 SQ_INSTS_VALU_MFMA_F32
    SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE` into per-launch figures of
    each convolution workload's dominant kernel: the fp32 MFMA FLOPs the
    hardware counted (against the algorithmic FLOPs) and the matrix cores'
    busy share of the kernel's active cycles.  Expects <dir>/mfma_<workload>/
    from `--output-format csv -o run`; keeps records of `previous` whose
    kernel source digest still matches."""
    out = {"_about": ("Per-launch rocprofv3 counters of the dominant kernel: MfmaFlopsF32 = "
                      "512 x SQ_INSTS_VALU_MFMA_MOPS_F32; MfmaUtil = matrix-core busy cycles / "
                      "(active cycles x SIMDs) in percent; GRBM_GUI_ACTIVE summed over the 8 XCDs; "
                      "valid while the kernel source digest matches.")}
    for name, rec in (previous or {}).items():
        cfg = WORKLOADS.get(name)
        if cfg and isinstance(rec, dict) and rec.get("source_sha256_16") == source_digest(cfg["op"]):
            out[name] = rec
    for name, cfg in WORKLOADS.items():
        op = cfg["op"]
        f = pmc_dir / f"mfma_{name}" / "run_counter_collection.csv"
        if not f.exists() or op in (TAIL_POOL, TAIL_GELU):
            continue
        vals = {c: _counter_per_dispatch(f, DOMINANT_KERNEL[op], c) for c in MFMA_COUNTERS}
        if any(v is None for v in vals.values()):
            continue
        alg = work_counts(dict(cfg))["flop"]
        out[name] = {"kernel": DOMINANT_KERNEL[op], "source_sha256_16": source_digest(op),
                     "mfma_flops_per_launch": int(vals["MfmaFlopsF32"]), "algorithmic_flops": int(alg),
                     "mfma_flops_over_algorithmic": round(vals["MfmaFlopsF32"] / alg, 4),
                     "mfma_util_pct": round(vals["MfmaUtil"], 2),
                     "mfma_f32_insts": int(vals["SQ_INSTS_VALU_MFMA_F32"]),
                     "lds_insts": int(vals["SQ_INSTS_LDS"]),
                     "lds_bank_conflict_cycles": int(vals["SQ_LDS_BANK_CONFLICT"]),
                     "gui_active_cycles_all_xcds": int(vals["GRBM_GUI_ACTIVE"])}
    return out


def measured_mfma(op: str, workload: str):
    """The committed MFMA counter record of a workload, while its kernel source
    still matches the profiled one."""
    f = ROOT / "profiles" / "mfma_counters.json"
    if not f.exists():
        return None
    try:
        rec = json.loads(f.read_text()).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_digest(op):
        return None
    return {"mfma_util_pct": rec["mfma_util_pct"],
            "mfma_flops_over_algorithmic": rec["mfma_flops_over_algorithmic"]}


def copy_probe(mib: int, reps: int) -> None:
    """A plain device-to-device copy of `mib` MiB, `reps` times: the known-size
    reference that calibrates the HBM byte counters."""
    import torch
    n = mib * 1024 * 1024 // 4
    a = torch.empty(n, device="cuda")
    b = torch.ones(n, device="cuda")
    for _ in range(reps):
        a.copy_(b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_mib": mib, "reps": reps}))


def run_op(cce, shape, d):
    op = shape["op"]
    if op == TAIL_POOL:
        return lambda: cce.pool_htanh_mean_tanh(d["z"], htanh_lo=shape["lo"], htanh_hi=shape["hi"],
                                                out=d["y"])
    if op == TAIL_GELU:
        return lambda: cce.lrelu_add_clamp_gelu(d["z"], d["s"], shape["slope"], shape["lo"], shape["hi"],
                                                out=d["y"])
    if op == CONV2D:
        return lambda: cce.conv2d_relu_hswish(d["x"], d["w"], d["b"], out=d["y"])
    if op == CONV3D:
        return lambda: cce.conv3d_lrelu_add_clamp_gelu(d["x"], d["w"], d["b"], d["s"], shape["slope"],
                                                       shape["lo"], shape["hi"], out=d["y"])
    return lambda: cce.convT2d_pool_htanh_mean_tanh(d["x"], d["w"], d["b"], out=d["y"],
                                                    htanh_lo=shape["lo"], htanh_hi=shape["hi"],
                                                    workspace=d["ws"])


def device_inputs(torch, cce, shape, p):
    d = {k: torch.from_numpy(v).cuda() for k, v in p.items()}
    if shape["op"] == TAIL_POOL:
        d["y"] = torch.empty((shape["N"], shape["C"], 1, 1), device="cuda")
        return d
    if shape["op"] == TAIL_GELU:
        d["y"] = torch.empty_like(d["z"])
        return d
    N, Co, k = shape["N"], shape["C_out"], shape["k"]
    if shape["op"] == CONV2D:
        d["y"] = torch.empty((N, Co, shape["H"] - k + 1, shape["W"] - k + 1), device="cuda")
    elif shape["op"] == CONV3D:
        d["y"] = torch.empty((N, Co, shape["D"] - k + 1, shape["H"] - k + 1, shape["W"] - k + 1),
                             device="cuda")
    else:
        d["y"] = torch.empty((N, Co, 1, 1), device="cuda")
        nb = cce.convT2d_pool_htanh_mean_tanh_workspace_bytes(N, shape["C_in"], shape["H"], shape["W"], Co)
        d["ws"] = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    return d


# Layer shapes beyond the pages' (each parity-tested against the oracle),
# timed by `--layer-shapes`: (op, sizes).  The first of each group is the
# page's layer at the same size, for comparison.
LAYER_SHAPES = (
    [(CONV2D, dict(N=32, C_in=ci, H=128, W=128, C_out=co, k=k))
     for ci, co, k in [(8, 64, 3), (4, 16, 1), (16, 64, 1), (8, 32, 3), (16, 32, 3), (16, 64, 3),
                       (4, 64, 5), (8, 64, 5)]]
    + [(CONV3D, dict(N=32, C_in=ci, D=16, H=64, W=64, C_out=co, k=k, slope=0.2, lo=-1.0, hi=1.0))
       for ci, co, k in [(8, 64, 3), (4, 16, 3), (8, 32, 3), (16, 64, 3), (8, 64, 1), (16, 64, 1)]]
    + [(CONVT, dict(N=16, C_in=ci, H=256, W=256, C_out=co, k=3, stride=1, pad=1, pool_k=2, pool_s=2,
                    lo=-1.0, hi=1.0))
       for ci, co in [(64, 64), (32, 32), (64, 16), (128, 64)]]
)


def time_layer_shapes(torch, cce, steps, warmup, seed, prewarm_s):
    """Time every entry of LAYER_SHAPES like the main workload (events around
    `steps` back-to-back calls after `warmup`); the roofline bound is whichever
    of the fp32 MFMA and HBM times is longer."""
    rows = []
    for op, sizes in LAYER_SHAPES:
        shape = dict(op=op, **sizes)
        p = make_inputs(op, seed, **{k: v for k, v in sizes.items() if k not in ("slope", "lo", "hi",
                                                                                 "stride", "pad",
                                                                                 "pool_k", "pool_s")})
        d = device_inputs(torch, cce, shape, p)
        fn = run_op(cce, shape, d)
        # Generating the inputs leaves the GPU idle; bring its clocks back up.
        t_end = time.perf_counter() + prewarm_s
        while time.perf_counter() < t_end:
            fn()
            torch.cuda.synchronize()
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(steps):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / steps
        wc = work_counts(shape)
        t_mfma = wc["flop"] / (PEAK_FP32_MFMA_TFLOPS * 1e12) * 1e3
        t_hbm = wc["bytes"] / (PEAK_HBM_GBS * 1e9) * 1e3
        rows.append({"op": op, **{k: v for k, v in sizes.items() if k in ("N", "C_in", "C_out", "k", "D", "H", "W")},
                     "ms_per_call": round(ms, 5), "tflops": round(wc["flop"] / ms / 1e9, 2),
                     "gbs": round(wc["bytes"] / ms / 1e6, 1),
                     "bound": "mfma" if t_mfma >= t_hbm else "hbm",
                     "roofline_frac": round(max(t_mfma, t_hbm) / ms, 4)})
        print(f"# {op} {sizes['C_in']}->{sizes['C_out']} k{sizes['k']} N{sizes['N']}: {ms:.4f} ms, "
              f"{rows[-1]['bound']} roofline fraction {rows[-1]['roofline_frac']:.3f}", file=sys.stderr, flush=True)
        del d
        torch.cuda.empty_cache()
    return rows


# The pages' own back-of-envelope time estimates for the same workloads on
# other GPUs (none of them measured): context only, never a target.
PAGES_ESTIMATE = {
    "conv2d_relu_hswish_n128": {"ms": [0.2, 0.3], "hardware": "H100 (assumed by the page)",
                                "what": "fused Conv2d+ReLU+HardSwish, total estimate"},
    "conv3d_lrelu_add_clamp_gelu_n128": {"ms": [7.5, 13.5], "hardware": "A100 (assumed by the page)",
                                         "what": "fused Conv3d kernel, scenarios"},
    "convT2d_pool_htanh_mean_tanh_n128": {"ms": [1.2, 1.5], "hardware": "H100 (assumed by the page)",
                                          "what": "library ConvTranspose2d + fused tail"},
}


def per_call_times(torch, fn, calls, evict=None):
    """Median and minimum of `calls` individually event-timed calls on the
    current stream.  With `evict`, it runs before every call (outside the
    events) -- a 1 GiB scratch write that flushes the L2s and the 256 MB MALL."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for e0, e1 in evs:
        if evict is not None:
            evict()
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    ts = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    return {"median_ms": round(ts[len(ts) // 2], 5), "min_ms": round(ts[0], 5), "calls": calls}


def time_workload(torch, cce, name, steps, warmup, seed, prewarm_s=0.0, cold_calls=0, keep_output=False):
    """Time one workload; with keep_output, also return its host inputs and
    the last call's result (out["inputs"], out["y"]) for the oracle check."""
    shape, p = workload_inputs(name, seed)
    d = device_inputs(torch, cce, shape, p)
    if not keep_output:
        del p
    fn = run_op(cce, shape, d)
    # Bring the GPU out of its idle clocks first: a freshly idle MI355X needs a
    # fraction of a second of load before kernel times settle.
    t_end = time.perf_counter() + prewarm_s
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The calls run back to back on one stream, so the region's GPU time over K
    # is both the step time and the average duration of the step's kernel(s).
    kernel_ms = ev0.elapsed_time(ev1) / steps
    wc = work_counts(shape)
    out = {
        "ms_per_call": kernel_ms,
        "wall_ms_per_step": 1e3 * wall / steps,
        "gflops": wc["flop"] / (kernel_ms * 1e-3) / 1e9,
        "gbs": wc["bytes"] / (kernel_ms * 1e-3) / 1e9,
        "fma": wc["fma"],
        "algorithmic_bytes": wc["bytes"],
    }
    if shape["op"] in HBM_BOUND:
        out["roofline"] = {"bound": "hbm", "achieved": round(out["gbs"], 1), "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": round(out["gbs"] / PEAK_HBM_GBS, 4),
                           "traffic": measured_traffic(shape["op"], name)}
    else:
        tflops = wc["flop"] / (kernel_ms * 1e-3) / 1e12
        out["roofline"] = {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_FP32_MFMA_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP32_MFMA_TFLOPS, 4),
                           "traffic": measured_traffic(shape["op"], name)}
    out["hbm_frac"] = round(out["gbs"] / PEAK_HBM_GBS, 4)
    # Per-call distributions: hot (back to back, as above) and cold.
    out["hot"] = per_call_times(torch, fn, min(steps, 100))
    if cold_calls:
        scratch = torch.empty(1 << 28, device="cuda")  # 1 GiB
        out["cold"] = per_call_times(torch, fn, cold_calls, evict=lambda: scratch.fill_(1.0))
        del scratch
    if keep_output:  # host copy of the last call's result, for the error check
        fn()
        torch.cuda.synchronize()
        out["y"] = d["y"].cpu().numpy()
        out["inputs"] = p
    del d
    torch.cuda.empty_cache()
    return shape, out


def unfused_torch(torch, name, steps, seed):
    """Context only: the same workload as PyTorch-ROCm's eager sequence of
    separate operators (MIOpen convolution, then each elementwise / pooling /
    reduction op as its own kernel, every intermediate in HBM), fp32."""
    import torch.nn.functional as F
    shape, p = workload_inputs(name, seed)
    op = shape["op"]
    if op not in (CONV2D, CONV3D, CONVT):
        return None
    d = {k: torch.from_numpy(v).cuda() for k, v in p.items()}
    del p
    if op == CONV2D:
        fn = lambda: F.hardswish(F.relu(F.conv2d(d["x"], d["w"], d["b"])))  # noqa: E731
    elif op == CONV3D:
        s5 = d["s"].view(1, -1, 1, 1, 1)
        fn = lambda: F.gelu(torch.clamp(F.leaky_relu(F.conv3d(d["x"], d["w"], d["b"]),  # noqa: E731
                                                     shape["slope"]) + s5, shape["lo"], shape["hi"]))
    else:
        fn = lambda: torch.tanh(torch.mean(F.hardtanh(F.max_pool2d(  # noqa: E731
            F.conv_transpose2d(d["x"], d["w"], d["b"], stride=1, padding=1), 2, 2),
            shape["lo"], shape["hi"]), dim=(2, 3), keepdim=True))
    for _ in range(3):  # first calls pick and compile the convolution kernels
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del d
    torch.cuda.empty_cache()
    return round(ms, 5)


class ErrorVsOracle:
    """Running comparison of GPU outputs with the oracle's, chunk by chunk:
    max abs error, max rel error where |ref| >= 1e-3, and how many outputs
    exceed the 1e-4 + 1e-4 |ref| tolerance."""

    def __init__(self):
        self.outputs, self.max_abs, self.max_rel, self.over, self.finite = 0, 0.0, 0.0, 0, True

    def add(self, gpu, ref):
        g = np.asarray(gpu, np.float64).reshape(-1)
        r = np.asarray(ref, np.float64).reshape(-1)
        err = np.abs(g - r)
        big = np.abs(r) >= 1e-3
        self.outputs += int(r.size)
        self.max_abs = max(self.max_abs, float(err.max()) if err.size else 0.0)
        if big.any():
            self.max_rel = max(self.max_rel, float((err[big] / np.abs(r[big])).max()))
        self.over += int(np.count_nonzero(~(err <= 1e-4 + 1e-4 * np.abs(r))))
        self.finite = self.finite and bool(np.all(np.isfinite(g)))

    def result(self):
        return {"outputs": self.outputs, "max_abs": self.max_abs, "max_rel_where_abs_ref_ge_1e-3": self.max_rel,
                "over_tolerance": self.over, "finite": self.finite}


def oracle_check(name, shape, p, gpu_y, budget_s=90.0, seed=0):
    """The CPU oracle (double precision, OpenMP over the host's cores) over
    the whole output of a workload, compared with the GPU's result `gpu_y`
    output by output.  Only the oracle's own compute is timed, and reported
    in the headline metric's unit (GFLOP/s of the convolution's
    multiply-adds; GB/s of the algorithmic bytes for the epilogue-only
    operators) as a CPU baseline.  Convolution and elementwise outputs are
    computed a few images at a time to bound host memory.  For the
    transposed convolution the first `cores` (image, channel) outputs
    estimate the whole run; if that exceeds `budget_s` seconds a random
    subset that fits the budget is computed instead (and named as such)."""
    import oracle as O
    op = shape["op"]
    cores = O.num_threads()
    acc = ErrorVsOracle()
    spent = 0.0

    def timed(fn, *a, **k):
        nonlocal spent
        t = time.perf_counter()
        r = fn(*a, **k)
        spent += time.perf_counter() - t
        return r

    N = shape["N"]
    sample = "every output"
    if op in (CONV2D, CONV3D, TAIL_GELU):
        step = 32 if op == CONV2D else 8
        for n0 in range(0, N, step):
            if op == CONV2D:
                ref = timed(O.conv2d_relu_hswish, np.ascontiguousarray(p["x"][n0:n0 + step]), p["w"], p["b"])
            elif op == CONV3D:
                ref = timed(O.conv3d_lrelu_add_clamp_gelu, np.ascontiguousarray(p["x"][n0:n0 + step]), p["w"],
                            p["b"], p["s"], shape["slope"], shape["lo"], shape["hi"])
            else:
                ref = timed(O.lrelu_add_clamp_gelu_array, np.ascontiguousarray(p["z"][n0:n0 + step]), p["s"],
                            shape["slope"], shape["lo"], shape["hi"])
            acc.add(gpu_y[n0:n0 + step], ref)
        work = work_counts(shape)
    elif op == TAIL_POOL:
        ref = timed(O.pool_htanh_mean_tanh, p["z"], shape["pool_k"], shape["pool_s"], shape["lo"], shape["hi"])
        acc.add(gpu_y[:, :, 0, 0], ref)
        work = work_counts(shape)
    else:
        total = N * shape["C_out"]
        gy = gpu_y.reshape(-1)
        first = np.arange(min(cores, total))
        acc.add(gy[first], timed(O.convT2d_pool_htanh_mean_tanh_at, p["x"], p["w"], p["b"], first))
        estimate = spent * total / max(1, first.size)
        if estimate <= budget_s:
            rest = np.arange(first.size, total)
        else:
            count = int(max(0, budget_s / spent * first.size - first.size))
            rest = np.sort(np.random.default_rng(seed).choice(np.arange(first.size, total), size=count,
                                                              replace=False))
            sample = f"{first.size + count} of {total} (image, channel) outputs"
        if rest.size:
            acc.add(gy[rest], timed(O.convT2d_pool_htanh_mean_tanh_at, p["x"], p["w"], p["b"], rest))
        per_output = work_counts(shape)["fma"] // total
        work = {"flop": 2 * per_output * (first.size + rest.size), "bytes": 0}
    if op in HBM_BOUND:
        value, unit = work["bytes"] / spent / 1e9, "GB/s"
    else:
        value, unit = work["flop"] / spent / 1e9, "GFLOP/s"
    base = {"value": round(value, 3), "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{sample} of {name}", "seconds": round(spent, 3)}
    return base, acc.result()


def main():
    ap = argparse.ArgumentParser(description="fused conv + epilogue benchmark (one MI355X)")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prewarm", type=float, default=1.0,
                    help="seconds of untimed calls before the warm-up steps (GPU clock ramp)")
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--ops", default="all", choices=["all", "none"],
                    help="also time every other fused workload (reported under 'ops')")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-probe", type=int, metavar="MIB",
                    help="only run a plain MIB-MiB device copy (counter calibration) and exit")
    ap.add_argument("--record-traffic", metavar="PMC_DIR",
                    help="only convert rocprofv3 FETCH_SIZE/WRITE_SIZE runs in PMC_DIR into "
                         "profiles/hbm_traffic.json and exit")
    ap.add_argument("--record-mfma", metavar="PMC_DIR",
                    help="only convert rocprofv3 MFMA/LDS counter runs in PMC_DIR into "
                         "profiles/mfma_counters.json and exit")
    ap.add_argument("--layer-shapes", action="store_true",
                    help="only time the fused operators at the other supported layer shapes and "
                         "print one JSON line")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size of the calibration copy")
    ap.add_argument("--unfused", action="store_true",
                    help="also time PyTorch-ROCm's unfused operator sequence per workload (context)")
    ap.add_argument("--cold-calls", type=int, default=20,
                    help="calls timed one by one after a 1 GiB cache-flushing write (0: skip)")
    args = ap.parse_args()

    if args.record_traffic:
        dest = ROOT / "profiles" / "hbm_traffic.json"
        prev = json.loads(dest.read_text()) if dest.exists() else None
        rec = record_traffic(Path(args.record_traffic), args.copy_mib, prev)
        dest.parent.mkdir(exist_ok=True)
        dest.write_text(json.dumps(rec, indent=1) + "\n")
        print(json.dumps(rec, indent=1))
        return

    if args.record_mfma:
        dest = ROOT / "profiles" / "mfma_counters.json"
        prev = json.loads(dest.read_text()) if dest.exists() else None
        rec = record_mfma(Path(args.record_mfma), prev)
        dest.parent.mkdir(exist_ok=True)
        dest.write_text(json.dumps(rec, indent=1) + "\n")
        print(json.dumps(rec, indent=1))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the fused kernels have no multi-GPU path. Images "
              "are independent, so a batch would shard by image across GPUs with no exchange.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args.copy_probe, max(1, args.steps))
        return
    import channel_convolution_epilogue_amd as cce
    cce.load()
    if args.layer_shapes:
        rows = time_layer_shapes(torch, cce, args.steps, args.warmup, args.seed, args.prewarm)
        print(json.dumps({"layer_shapes": rows, "steps": args.steps, "warmup": args.warmup}), flush=True)
        return

    check = not args.no_cpu_baseline

    def report(name, r):
        print(f"# {name}: {r['ms_per_call']:.4f} ms/call, {r['gflops']:.1f} GFLOP/s, {r['gbs']:.1f} GB/s, "
              f"{r['roofline']['frac']:.3f} of the {r['roofline']['bound']} roofline", file=sys.stderr, flush=True)

    def with_oracle(name, shape, r):
        """Every output of the workload against the CPU oracle (unless
        --no-cpu-baseline); frees the host copies afterwards."""
        gy, p = r.pop("y", None), r.pop("inputs", None)
        if gy is None:
            return
        base, err = oracle_check(name, shape, p, gy, seed=args.seed)
        r["oracle"], r["gpu_error_vs_oracle"] = base, err
        print(f"# {name}: oracle {base['seconds']:.1f} s on {base['cores']} threads ({base['sample']}); "
              f"GPU max abs error {err['max_abs']:.2e}, {err['over_tolerance']} of {err['outputs']} "
              f"outputs over tolerance", file=sys.stderr, flush=True)

    shape, head = time_workload(torch, cce, args.workload, args.steps, args.warmup, args.seed,
                                args.prewarm, args.cold_calls, keep_output=check)
    report(args.workload, head)
    ops = {}
    if args.ops == "all":
        for name in WORKLOADS:
            if name == args.workload:
                r = head
            else:
                shp, r = time_workload(torch, cce, name, max(3, min(args.steps, 50)), min(args.warmup, 10),
                                       args.seed, min(args.prewarm, 0.5), min(args.cold_calls, 10),
                                       keep_output=check)
                report(name, r)
                with_oracle(name, shp, r)
            ops[name] = {"ms_per_call": round(r["ms_per_call"], 5), "gflops": round(r["gflops"], 1),
                         "gbs": round(r["gbs"], 1), "roofline_bound": r["roofline"]["bound"],
                         "roofline_frac": r["roofline"]["frac"], "traffic": r["roofline"]["traffic"],
                         "hbm_frac": r["hbm_frac"], "hot": r["hot"]}
            if "cold" in r:
                ops[name]["cold"] = r["cold"]
            if "oracle" in r:
                ops[name]["oracle"], ops[name]["gpu_error_vs_oracle"] = r["oracle"], r["gpu_error_vs_oracle"]
            if name in PAGES_ESTIMATE:
                ops[name]["pages_estimate"] = PAGES_ESTIMATE[name]
    # The headline's oracle run last: the GPU is idle meanwhile, and the other
    # workloads' timings are not delayed by it.
    with_oracle(args.workload, shape, head)
    for name in ops:
        r = head if name == args.workload else None
        if r is not None and "oracle" in r:
            ops[name]["oracle"], ops[name]["gpu_error_vs_oracle"] = r["oracle"], r["gpu_error_vs_oracle"]

    line = {
        "metric": METRIC,
        "value": round(head["gflops"], 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_s": args.prewarm,
        "ms_per_step": round(head["ms_per_call"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, **{k: v for k, v in shape.items() if k != "op"},
                   "op": shape["op"], "global_batch": shape["N"], "parallelism": "none (1 GPU)"},
        "roofline": head["roofline"],
        "hbm": {"achieved": round(head["gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": head["hbm_frac"]},
        # per-call event timing: hot = back to back; cold = after a 1 GiB write
        # that flushes the L2s and the MALL (the event pair brackets the kernel only)
        "per_call": {k: head[k] for k in ("hot", "cold") if k in head},
    }
    counters = measured_mfma(shape["op"], args.workload)
    if counters:  # rocprofv3 cross-check of the dominant kernel (profiles/mfma_counters.json)
        line["mfma_counters"] = counters
    if args.workload in PAGES_ESTIMATE:
        line["pages_estimate"] = PAGES_ESTIMATE[args.workload]
    if args.unfused:
        names = list(WORKLOADS) if args.ops == "all" else [args.workload]
        ctx = {}
        for name in names:
            ms = unfused_torch(torch, name, max(3, min(args.steps, 20)), args.seed)
            if ms is None:
                continue
            fused = ops[name]["ms_per_call"] if name in ops else head["ms_per_call"]
            ctx[name] = {"ms_per_call": ms, "fused_speedup": round(ms / fused, 2)}
            print(f"# unfused torch {name}: {ms:.4f} ms/call ({ms / fused:.2f}x the fused kernel)",
                  file=sys.stderr, flush=True)
        line["unfused_torch"] = ctx
    if "oracle" in head:
        line["cpu_baseline"] = head["oracle"]
        line["gpu_error_vs_oracle"] = head["gpu_error_vs_oracle"]
    if ops:
        line["ops"] = ops
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
