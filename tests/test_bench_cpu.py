"""Host-side logic of bench.py (no GPU): algorithmic work counts, the HBM
counter conversion, and the refusal to run on more than one GPU."""
import csv
import json
import subprocess
import sys
from pathlib import Path

import pytest

import bench
from conv_inputs import WORKLOADS

ROOT = Path(__file__).resolve().parents[1]


def test_work_counts_match_page_counts():
    golden = json.load(open(ROOT / "tests" / "golden" / "page_values.json"))
    c2 = bench.work_counts(dict(WORKLOADS["conv2d_relu_hswish_n128"]))
    assert c2["fma"] == golden["conv2d_shapes"]["out_elements"] * 72
    assert c2["bytes"] == 4 * (128 * 8 * 128 * 128 + 64 * 72 + 64 + golden["conv2d_shapes"]["out_elements"])
    c3 = bench.work_counts(dict(WORKLOADS["conv3d_lrelu_add_clamp_gelu_n128"]))
    assert c3["fma"] == golden["conv3d_shapes"]["fmas"]
    ct = bench.work_counts(dict(WORKLOADS["convT2d_pool_htanh_mean_tanh_n128"]))
    assert ct["fma"] == golden["convT_shapes"]["macs"]
    assert ct["flop"] == 2 * ct["fma"]
    tp = bench.work_counts(dict(WORKLOADS["pool_htanh_mean_tanh_n128"]))
    assert tp["fma"] == 0 and tp["bytes"] == 4 * (128 * 64 * 256 * 256 + 128 * 64)
    tg = bench.work_counts(dict(WORKLOADS["lrelu_add_clamp_gelu_n128"]))
    assert tg["bytes"] == 4 * (2 * golden["conv3d_shapes"]["out_elements"] + 64)


def _write_counter_csv(path: Path, rows):
    path.mkdir(parents=True)
    with open(path / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_record_traffic_scales_by_copy_calibration(tmp_path):
    mib = 64
    # The copy reads as half its size on FETCH_SIZE and exactly on WRITE_SIZE.
    _write_counter_csv(tmp_path / "fetch_copy", [
        {"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE", "Counter_Value": mib * 512}])
    _write_counter_csv(tmp_path / "write_copy", [
        {"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE", "Counter_Value": mib * 1024}])
    k = "void cce::(anonymous namespace)::conv2d_relu_hswish_kernel<2, true, true, 4>(Args)"
    _write_counter_csv(tmp_path / "fetch_conv2d_relu_hswish_n8", [
        {"Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Counter_Value": 100.0},
        {"Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Counter_Value": 300.0},
        {"Kernel_Name": "other", "Counter_Name": "FETCH_SIZE", "Counter_Value": 1e9}])
    _write_counter_csv(tmp_path / "write_conv2d_relu_hswish_n8", [
        {"Kernel_Name": k, "Counter_Name": "WRITE_SIZE", "Counter_Value": 50.0}])
    rec = bench.record_traffic(tmp_path, mib)
    assert rec["copy_scale"] == {"fetch": 2.0, "write": 1.0}
    r = rec["conv2d_relu_hswish_n8"]
    assert r["fetch_bytes"] == 200 * 1024 * 2 and r["write_bytes"] == 50 * 1024
    assert r["bytes_per_launch"] == r["fetch_bytes"] + r["write_bytes"]
    assert r["source_sha256_16"] == bench.source_digest("conv2d_relu_hswish")
    assert "conv3d_lrelu_add_clamp_gelu_n128" not in rec

    # A record from an earlier run survives only while its kernel source is unchanged.
    prev = {"copy_scale": {"fetch": 2.0, "write": 1.0},
            "conv3d_lrelu_add_clamp_gelu_n128": {"source_sha256_16": bench.source_digest("conv3d_lrelu_add_clamp_gelu"),
                                                 "bytes_per_launch": 7},
            "convT2d_pool_htanh_mean_tanh_n16": {"source_sha256_16": "stale", "bytes_per_launch": 9},
            "conv2d_relu_hswish_n8": {"source_sha256_16": bench.source_digest("conv2d_relu_hswish"),
                                      "bytes_per_launch": 5}}
    rec = bench.record_traffic(tmp_path, mib, prev)
    assert rec["conv3d_lrelu_add_clamp_gelu_n128"]["bytes_per_launch"] == 7
    assert "convT2d_pool_htanh_mean_tanh_n16" not in rec
    assert rec["conv2d_relu_hswish_n8"]["bytes_per_launch"] == r["bytes_per_launch"]


def test_record_mfma_counters(tmp_path):
    k = "void cce::(anonymous namespace)::convT2d_pool_htanh_mean_tanh_kernel<OutCh<64>, true, 8>(Args)"
    vals = {"MfmaUtil": 87.5, "MfmaFlopsF32": 4.0e11, "SQ_INSTS_VALU_MFMA_F32": 2.0e8,
            "SQ_INSTS_LDS": 1.0e7, "SQ_LDS_BANK_CONFLICT": 3.0e5, "GRBM_GUI_ACTIVE": 1.0e7}
    rows = [{"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v} for c, v in vals.items()]
    rows += [{"Kernel_Name": k, "Counter_Name": "MfmaUtil", "Counter_Value": 85.5},  # second dispatch
             {"Kernel_Name": "convT_prepare_weight_kernel", "Counter_Name": "MfmaUtil", "Counter_Value": 0.0}]
    _write_counter_csv(tmp_path / "mfma_convT2d_pool_htanh_mean_tanh_n16", rows)
    _write_counter_csv(tmp_path / "mfma_pool_htanh_mean_tanh_n128", rows)  # no MFMA: ignored
    rec = bench.record_mfma(tmp_path)
    r = rec["convT2d_pool_htanh_mean_tanh_n16"]
    alg = bench.work_counts(dict(WORKLOADS["convT2d_pool_htanh_mean_tanh_n16"]))["flop"]
    assert r["mfma_util_pct"] == 86.5  # mean over the kernel's dispatches only
    assert r["mfma_flops_per_launch"] == 400_000_000_000 and r["algorithmic_flops"] == alg
    assert r["mfma_flops_over_algorithmic"] == round(4.0e11 / alg, 4)
    assert r["source_sha256_16"] == bench.source_digest("convT2d_pool_htanh_mean_tanh")
    assert "pool_htanh_mean_tanh_n128" not in rec
    prev = {"conv3d_lrelu_add_clamp_gelu_n128": {"source_sha256_16": "stale", "mfma_util_pct": 1.0}}
    assert "conv3d_lrelu_add_clamp_gelu_n128" not in bench.record_mfma(tmp_path, prev)


def test_committed_counter_records_match_the_kernel_sources():
    """bench.py reports `traffic` only from a record whose kernel source
    digest matches the tree: every workload's committed HBM-traffic record,
    and every convolution's MFMA-counter record, must have been taken on the
    kernels as they stand."""
    traffic = json.loads((ROOT / "profiles" / "hbm_traffic.json").read_text())
    mfma = json.loads((ROOT / "profiles" / "mfma_counters.json").read_text())
    for name, cfg in WORKLOADS.items():
        digest = bench.source_digest(cfg["op"])
        assert traffic[name]["source_sha256_16"] == digest, f"{name}: stale HBM traffic record"
        assert bench.measured_traffic(cfg["op"], name) == traffic[name]["bytes_per_launch"]
        if cfg["op"] in ("conv2d_relu_hswish", "conv3d_lrelu_add_clamp_gelu", "convT2d_pool_htanh_mean_tanh"):
            assert mfma[name]["source_sha256_16"] == digest, f"{name}: stale MFMA counter record"


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "8"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


@pytest.mark.parametrize("op,sizes", [
    ("conv2d_relu_hswish", dict(N=3, C_in=8, H=12, W=10, C_out=64, k=3)),
    ("conv3d_lrelu_add_clamp_gelu", dict(N=9, C_in=8, D=4, H=6, W=5, C_out=16, k=3, slope=0.2, lo=-1.0, hi=1.0)),
    ("convT2d_pool_htanh_mean_tanh", dict(N=2, C_in=8, H=6, W=8, C_out=16, k=3, stride=1, pad=1, pool_k=2,
                                          pool_s=2, lo=-1.0, hi=1.0)),
    ("pool_htanh_mean_tanh", dict(N=2, C=3, H=6, W=8, pool_k=2, pool_s=2, lo=-1.0, hi=1.0)),
    ("lrelu_add_clamp_gelu", dict(N=9, C=3, D=2, H=3, W=4, slope=0.2, lo=-1.0, hi=1.0)),
])
def test_oracle_check_counts_every_output_and_flags_errors(op, sizes):
    """The bench's oracle leg compares every output (in chunks of images) and
    counts those outside the tolerance: the oracle's own result passes, and
    one planted error is found."""
    import numpy as np
    import oracle as O
    from conv_inputs import make_inputs
    shape = dict(op=op, **sizes)
    keys = ("N", "C_in", "H", "W", "C_out", "k", "D", "C")
    p = make_inputs(op, 4, **{k: v for k, v in sizes.items() if k in keys})
    if op == "conv2d_relu_hswish":
        ref = O.conv2d_relu_hswish(p["x"], p["w"], p["b"])
    elif op == "conv3d_lrelu_add_clamp_gelu":
        ref = O.conv3d_lrelu_add_clamp_gelu(p["x"], p["w"], p["b"], p["s"])
    elif op == "convT2d_pool_htanh_mean_tanh":
        ref = O.convT2d_pool_htanh_mean_tanh(p["x"], p["w"], p["b"])[:, :, None, None]
    elif op == "pool_htanh_mean_tanh":
        ref = O.pool_htanh_mean_tanh(p["z"])[:, :, None, None]
    else:
        ref = O.lrelu_add_clamp_gelu_array(p["z"], p["s"])
    gpu = ref.astype(np.float32)
    base, err = bench.oracle_check("tiny", shape, p, gpu)
    assert err["outputs"] == ref.size and err["over_tolerance"] == 0 and err["finite"]
    assert base["kind"] == "oracle" and base["cores"] >= 1 and base["value"] > 0
    assert base["sample"].startswith("every output")
    bad = gpu.copy()
    bad.reshape(-1)[ref.size - 1] += 1e-2
    _, err = bench.oracle_check("tiny", shape, p, bad)
    assert err["over_tolerance"] == 1 and err["max_abs"] >= 9e-3


def test_oracle_check_samples_convT_within_budget():
    """Past its time budget the transposed-convolution check computes a
    random subset of (image, channel) outputs and says so."""
    import numpy as np
    import oracle as O
    from conv_inputs import make_inputs
    sizes = dict(N=4, C_in=16, H=16, W=16, C_out=64, k=3, stride=1, pad=1, pool_k=2, pool_s=2, lo=-1.0, hi=1.0)
    p = make_inputs("convT2d_pool_htanh_mean_tanh", 5, N=4, C_in=16, H=16, W=16, C_out=64, k=3)
    gpu = O.convT2d_pool_htanh_mean_tanh(p["x"], p["w"], p["b"]).astype(np.float32)[:, :, None, None]
    base, err = bench.oracle_check("tiny", dict(op="convT2d_pool_htanh_mean_tanh", **sizes), p, gpu, budget_s=1e-9)
    assert err["outputs"] < 256 and err["over_tolerance"] == 0
    assert "of 256 (image, channel) outputs" in base["sample"]
