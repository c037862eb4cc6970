"""GPU side of the tuning machinery: explicit launch orders give bit-for-bit
the results of the compiled order, a loaded tuning table steers the plain
entry point, and the offline tuner runs end to end on a small shape."""
import os

import pytest
import torch

import parity as PT
from tiled_dense_gemm_scale_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def gsr(native):
    import tiled_dense_gemm_scale_amd as g

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    g.clear_tuning()
    yield g
    g.clear_tuning()


@pytest.mark.parametrize("cid,shape", [(28, (4097, 700, 264)), (16, (700, 1100, 264)), (17, (700, 1100, 264)),
                                       (18, (700, 1100, 264)), (21, (700, 1100, 264)), (22, (700, 1100, 264)),
                                       (25, (700, 1100, 264)), (29, (700, 1100, 264)),
                                       (25, (4096, 4096, 136)), (25, (8192, 4096, 72)), (28, (4096, 8192, 72)),
                                       (28, (700, 1100, 264)), (28, (4096, 4096, 136)), (31, (700, 1100, 264)),
                                       (31, (2048, 4096, 200)),
                                       (32, (700, 1100, 264)), (32, (2048, 2048, 200))],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_launch_order_does_not_change_results(gsr, orc, cid, shape):
    """Every launch order, including the chip rounds of 16 x 16 tiles (order 2,
    active on the 4096- and 8192-wide grids of 256 x 256 tiles), gives the
    compiled order's bits; the compiled order matches the oracle."""
    M, N, K = shape
    a, b = W.normal_inputs(M, N, K, seed=cid)
    ad, bd = a.to(DEV), b.to(DEV)
    ref = gsr.gemm_scale_relu_ex(ad, bd, 0.5, cid).clone()
    torch.cuda.synchronize()
    oref, _ = orc.gemm_scale_relu(W.fp16_bits(a), W.fp16_bits(b), 0.5)
    PT.assert_parity(f"cfg{cid} default order", W.fp16_bits(ref.cpu()), oref)
    for gm in (1, 2, 3, 8, 64):
        for xcd in (0, 1, 2):
            print(f"[gpu] launch order cfg {cid} group {gm} xcd {xcd}", flush=True)
            out = gsr.gemm_launch(ad, bd, 0.5, cid, gm, xcd)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (cid, gm, xcd)


def test_tuning_table_steers_the_plain_call(gsr, tmp_path):
    M, N, K = 300, 520, 200
    a, b = W.normal_inputs(M, N, K, seed=3)
    ad, bd = a.to(DEV), b.to(DEV)
    sel = gsr.select_config(M, N, K)["id"]
    forced = 21 if sel != 21 else 22
    want = gsr.gemm_scale_relu_ex(ad, bd, 0.5, forced).clone()
    p = tmp_path / "tuning.txt"
    p.write_text(f"{M} {N} {K} {forced} 2 0\n")
    gsr.load_tuning(str(p))
    try:
        assert gsr.select_config(M, N, K)["id"] == forced
        print(f"[gpu] tuned call {M}x{N}x{K} -> cfg {forced}", flush=True)
        got = gsr.gemm_scale_relu(ad, bd, 0.5)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    finally:
        gsr.clear_tuning()


def test_tuner_end_to_end(gsr, tmp_path):
    from tiled_dense_gemm_scale_amd import tune

    out = tmp_path / "t.txt"
    rep = tmp_path / "t.json"
    print("[gpu] tuner on 256x512x256", flush=True)
    assert tune.main(["--shapes", "256x512x256", "--out", str(out), "--report", str(rep), "--top", "1"]) == 0
    lines = [l for l in out.read_text().splitlines() if l and not l.startswith("#")]
    assert len(lines) == 1 and lines[0].split()[:3] == ["256", "512", "256"]
    import json
    r = json.loads(rep.read_text())["shapes"][0]
    assert r["best"]["us"] > 0 and r["pareto_time_vs_lds"]
    assert all(c["matches_selector_output"] for c in r["candidates"])
    assert gsr.tuning_entries() == 0
