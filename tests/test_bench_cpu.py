"""Host-side logic of bench.py and the workload registry (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from tiled_dense_gemm_scale_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_roofline_bound_follows_intensity():
    # 1024^3: 341 FLOP/B, just above the 315 FLOP/B ridge -> MFMA-bound, in TFLOP/s
    w = W.by_name("square_1024")
    r = bench.roofline_of(w, 0.006, None)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == bench.PEAK_FP16_TFLOPS
    assert r["achieved"] == pytest.approx(w.flops / 6e-6 / 1e12, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)
    # 256^3 (85 FLOP/B) and the skinny class (16 FLOP/B) -> HBM-bound, in GB/s
    for name, ms in (("square_256", 0.003), ("skinny_16x11008x4096", 0.0158)):
        w = W.by_name(name)
        r = bench.roofline_of(w, ms, 123)
        assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.PEAK_HBM_GBS
        assert r["achieved"] == pytest.approx(w.algorithmic_bytes / (ms * 1e-3) / 1e9, rel=1e-4)
        assert r["traffic"] == 123


def test_traffic_is_dropped_once_the_kernel_sources_change(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path))
    assert bench.load_traffic("square_1024", 1) is None  # no summary
    path = tmp_path / "traffic_square_1024.json"
    path.write_text(json.dumps({"kernel_source_digest": bench.kernel_source_digest(),
                                "hbm_bytes_per_launch": 14801353}))
    assert bench.load_traffic("square_1024", 1) == 14801353
    path.write_text(json.dumps({"kernel_source_digest": "0000000000000000", "hbm_bytes_per_launch": 1}))
    assert bench.load_traffic("square_1024", 1) is None


def test_committed_traffic_summaries_name_their_workloads():
    for name in list(W.WORKLOADS) + [W.SKINNY.name]:
        path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
        if not os.path.exists(path):
            continue
        t = json.load(open(path))
        assert len(t["kernel_source_digest"]) == 16
        assert t["hbm_bytes_per_launch"] > 0


def test_cpu_baseline_on_a_small_workload():
    w = W.Workload("tiny", 48, 40, 72, 0.5, 1.0, False, "test")
    a, b = W.workload_inputs(w)
    r = bench.cpu_baseline(w, a, b, target_s=0.2)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert "rows 0..47" in r["sample"]  # the whole of C, repeated to fill the time


def test_workload_registry():
    for name in list(W.WORKLOADS) + list(W.EXTRA):
        assert W.by_name(name).name == name
    with pytest.raises(KeyError):
        W.by_name("square_7")
    s = W.COLSHARD8
    assert (s.M, s.N, s.K) == (4097, 11008 // 8, 4096) and s.b_std == 4096 ** -0.5
    # every workload draws the same bits from its seed
    a1, b1 = W.workload_inputs(W.by_name("square_256"))
    a2, b2 = W.workload_inputs(W.by_name("square_256"))
    assert torch.equal(a1.view(torch.int16), a2.view(torch.int16))
    assert torch.equal(b1.view(torch.int16), b2.view(torch.int16))
