"""The selector's fitted cost model (host-side, no GPU)."""
import os
import re

import numpy as np
import pytest

from tiled_dense_gemm_scale_amd import fit_selector as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSV = os.path.join(ROOT, "tiled_dense_gemm_scale_amd", "tuning", "mi355x_config_times.csv")
API = os.path.join(ROOT, "tiled_dense_gemm_scale_amd", "csrc", "gsr_api.hip")


def test_fit_recovers_a_known_model():
    """Times generated from known rates and fixed costs are fitted back."""
    tiles = {28: (256, 256), 31: (128, 256), 32: (128, 128),
             21: (64, 64), 22: (32, 64), 16: (64, 64), 18: (32, 64)}
    truth = {cid: (1.0 + 0.5 * i, 2.0 + 0.25 * i) for i, cid in enumerate(sorted(tiles))}
    a, pmin = 0.2, 0.6
    times = {}
    for M in (16, 200, 1000, 4100, 8200):
        for N in (512, 3000, 11008):
            for K in (128, 256, 1024, 4096):
                times[(M, N, K)] = {cid: F.waves(F.workgroups(tiles[cid], M, N), a, pmin)
                                    * (2.0 * tiles[cid][0] * tiles[cid][1] * K / (r * 1e6) + e)
                                    for cid, (r, e) in truth.items() if cid in F.candidates(M, N, K)}
    params = F.fit_params(times, tiles, a, pmin)
    for cid, (r, e) in truth.items():
        assert params[cid][0] == pytest.approx(r, rel=1e-6)
        assert params[cid][1] == pytest.approx(e, rel=1e-6, abs=1e-9)
    mean, worst = F.regret(times, tiles, params, a, pmin)
    assert mean == pytest.approx(1.0) and worst == pytest.approx(1.0)


def test_one_kernel_per_large_tile():
    """One 256x256 and one 128x256 kernel at every grid size (the copy-to-LDS
    16x16x32 kernels, the 128x256 one with copy waves; their twins and the
    32x32x16 128x256 kernel are never candidates), and the K-split kinds by K."""
    for M, N in ((16, 11008), (1024, 4096), (1280, 4096), (2048, 4096), (4096, 4096)):
        c = F.candidates(M, N, 4096)
        assert 28 in c and 31 in c and 32 in c
        assert not {5, 6, 7, 8, 10, 15, 23, 24, 25, 26, 29} & set(c)
    assert F.candidates(16, 11008, 256)[-2:] == F.FOUR_WAVE and F.candidates(16, 11008, 257)[-2:] == F.COPY_WAVE


def test_waves_price_a_partial_last_wave():
    assert F.waves(256, 0.0, 0.85) == 1.0
    assert F.waves(512, 0.0, 0.85) == 2.0
    assert F.waves(257, 0.0, 0.85) == pytest.approx(1.85)
    assert F.waves(256 + 240, 0.0, 0.85) == pytest.approx(1 + 240 / 256)
    assert F.workgroups((256, 256), 4097, 11008) == 17 * 43


def test_selector_table_is_the_fit_of_the_committed_measurements():
    """The constants in select() are what the fit of the committed times gives."""
    times, tiles = F.load(CSV)
    assert len(times) >= 50
    mean, worst, a, pmin, params = F.fit(times, tiles)
    src = open(API).read()
    table = src[src.index("const Candidate kCandidates[]"):]
    table = table[: table.index("};")]
    rows = {int(m.group(1)): (float(m.group(2)), float(m.group(3)))
            for m in re.finditer(r"\{(\d+),\s*([0-9.]+),\s*([0-9.]+)\}", table)}
    assert set(rows) == set(params)
    for cid, (rate, tile_us) in rows.items():
        assert rate == pytest.approx(params[cid][0], abs=0.006), cid
        assert tile_us == pytest.approx(params[cid][1], abs=0.006), cid
    consts = re.search(r"kPartMin = ([0-9.]+), kPartA = ([0-9.]+);", src)
    assert float(consts.group(1)) == pytest.approx(pmin) and float(consts.group(2)) == pytest.approx(a)
    assert re.search(r"kFullChipTiles", src) is None  # one kernel per large tile, no swap rule
    assert mean < 1.005 and worst < 1.05


def test_library_selector_matches_the_model(native):
    """select() in the library makes the model's choice on every measured shape."""
    times, tiles = F.load(CSV)
    src = open(API).read()
    consts = re.search(r"kPartMin = ([0-9.]+), kPartA = ([0-9.]+);", src)
    mean, worst, a, pmin, params = F.fit(times, tiles, a_grid=np.array([float(consts.group(2))]),
                                         p_grid=np.array([float(consts.group(1))]))
    disagree = []
    for (M, N, K), t in times.items():
        want = F.choose(params, tiles, M, N, K, a, pmin)
        got = native.select_config(M, N, K)["id"]
        if got != want:
            disagree.append(((M, N, K), got, want))
    assert not disagree, disagree
