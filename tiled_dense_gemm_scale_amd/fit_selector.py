"""Fit the tile selector's cost model to measured configuration times.

The selector in csrc/gsr_api.hip prices a candidate tile bm x bn as

    waves(wgs) * (2 * bm * bn * K / (rate * 1e6) + tile_us)        [us]

with wgs = ceil(M / bm) * ceil(N / bn) workgroups on 256 CUs and
waves(wgs) = full waves + (a part-filled last wave: max(pmin, a + (1 - a) * fill)).
The 256x256 tile has one kernel (config 28, 16x16x32 MFMAs with B copied to
LDS: measured faster than both other 256x256 kernels on every one of the 60
shapes).  The 128x256 tile has two: config 23 on 32x32x16 MFMAs (the higher
issue efficiency) and config 26 on 16x16x32 MFMAs (the higher engine clock
once enough CUs run for the power limit to bind); config 26 stands in for
config 23 when the 128x256 grid has at least full[0] workgroups.  This module
fits `rate` (TFLOP/s per CU) and `tile_us` per configuration by least squares
in relative error on the shapes where it is a candidate, and picks (a, pmin,
full) on grids whose choices come closest to the fastest measured
configuration (mean log ratio): first (a, pmin) with config 26 left out, then
full[0], then (a, pmin) again.  Input: the CSV written from a `tune.py --top 0`
report (tuning/mi355x_config_times.csv) or such a JSON report itself.

    python -m tiled_dense_gemm_scale_amd.fit_selector tuning/mi355x_config_times.csv
prints the candidate table for gsr_api.hip and the fit's distance from the
fastest configuration, in sample and on shapes held out of the fit.
"""
from __future__ import annotations

import argparse
import csv
import json
import math
import random
import sys
from typing import Dict, List, Tuple

import numpy as np

CUS = 256
Shape = Tuple[int, int, int]
# the selector's candidates; the copy-wave K-split tiles only for K > 256,
# their four-wave twins only for K <= 256
BASE = [28, 23, 24, 5, 6, 7, 10, 8]
COPY_WAVE = [21, 22]
FOUR_WAVE = [16, 18]
# (config, its 16x16x32 stand-in, the tile whose grid size decides)
FULL_CHIP = [(23, 26, (128, 256))]
ALL = BASE + [f for _, f, _ in FULL_CHIP] + COPY_WAVE + FOUR_WAVE
FULL_H_GRID = (128, 160, 176, 192, 208, 224, 256, 320)
NEVER = 1 << 30


def candidates(M: int, N: int, K: int, full) -> List[int]:
    base = list(BASE)
    for (cid, stand_in, tile), f in zip(FULL_CHIP, full):
        if workgroups(tile, M, N) >= f:
            base[base.index(cid)] = stand_in
    return base + (COPY_WAVE if K > 256 else FOUR_WAVE)


def load(path: str) -> Tuple[Dict[Shape, Dict[int, float]], Dict[int, Tuple[int, int]]]:
    """(times[(M, N, K)][config] in us, tiles[config] = (bm, bn))."""
    times: Dict[Shape, Dict[int, float]] = {}
    tiles: Dict[int, Tuple[int, int]] = {}
    if path.endswith(".json"):
        rep = json.load(open(path))
        for s in rep["shapes"]:
            for c in s["candidates"]:
                if not c.get("matches_selector_output", True):
                    continue
                bm, bn, _ = (int(v) for v in c["tile"].split("x"))
                tiles[c["config_id"]] = (bm, bn)
                times.setdefault((s["M"], s["N"], s["K"]), {})[c["config_id"]] = float(c["us"])
        return times, tiles
    with open(path) as f:
        for row in csv.DictReader(line for line in f if not line.startswith("#")):
            cid = int(row["config_id"])
            bm, bn, _ = (int(v) for v in row["tile"].split("x"))
            tiles[cid] = (bm, bn)
            times.setdefault((int(row["M"]), int(row["N"]), int(row["K"])), {})[cid] = float(row["us"])
    return times, tiles


def waves(wgs: int, a: float, pmin: float) -> float:
    full, rem = divmod(wgs, CUS)
    return full + (max(pmin, a + (1.0 - a) * rem / CUS) if rem else 0.0)


def workgroups(tile: Tuple[int, int], M: int, N: int) -> int:
    return -(-M // tile[0]) * -(-N // tile[1])


PAIRED = {c for c, _, _ in FULL_CHIP} | {f for _, f, _ in FULL_CHIP}


def fit_params(times, tiles, a: float, pmin: float, full) -> Dict[int, Tuple[float, float]]:
    """(rate, tile_us) per candidate: least squares of t ~ w * (flops/rate + e),
    rows scaled by 1/t (relative error); the paired configurations on the
    shapes where the full-chip rules make them candidates."""
    out = {}
    for cid in ALL:
        X, y = [], []
        for (M, N, K), t in times.items():
            if cid not in t:
                continue
            if cid in PAIRED and cid not in candidates(M, N, K, full):
                continue
            w = waves(workgroups(tiles[cid], M, N), a, pmin)
            X.append([w * 2.0 * tiles[cid][0] * tiles[cid][1] * K / 1e6, w])
            y.append(t[cid])
        if not X:
            continue
        X, y = np.asarray(X), np.asarray(y)
        coef, *_ = np.linalg.lstsq(X / y[:, None], np.ones_like(y), rcond=None)
        out[cid] = (1.0 / max(coef[0], 1e-12), max(coef[1], 0.0))
    return out


def choose(params, tiles, M: int, N: int, K: int, a: float, pmin: float, full, have=None) -> int:
    best, best_t = None, math.inf
    for cid in candidates(M, N, K, full):
        if cid not in params or (have is not None and cid not in have):
            continue
        rate, e = params[cid]
        t = waves(workgroups(tiles[cid], M, N), a, pmin) * (2.0 * tiles[cid][0] * tiles[cid][1] * K / (rate * 1e6) + e)
        if t < best_t:
            best, best_t = cid, t
    return best


def regret(times, tiles, params, a, pmin, full) -> Tuple[float, float]:
    """(mean, worst) of t[choice] / t[fastest] over the shapes."""
    logs, worst = [], 1.0
    for (M, N, K), t in times.items():
        c = choose(params, tiles, M, N, K, a, pmin, full, have=t)
        r = t[c] / min(t.values())
        logs.append(math.log(r))
        worst = max(worst, r)
    return math.exp(sum(logs) / len(logs)), worst


def _search(times, tiles, a_grid, p_grid, fulls):
    best = None
    for full in fulls:
        for a in a_grid:
            for p in p_grid:
                params = fit_params(times, tiles, float(a), float(p), full)
                mean, worst = regret(times, tiles, params, float(a), float(p), full)
                if best is None or mean < best[0] - 1e-12:
                    best = (mean, worst, float(a), float(p), full, params)
    return best


def fit(times, tiles, a_grid=None, p_grid=None, full_h_grid=None):
    """(mean, worst, a, pmin, (full[0],), params) of the best point, by
    coordinate search: (a, pmin) without config 26, then full[0], then
    (a, pmin) again."""
    a_grid = np.arange(0.0, 0.75, 0.05) if a_grid is None else a_grid
    p_grid = np.arange(0.30, 1.001, 0.05) if p_grid is None else p_grid
    full_h_grid = FULL_H_GRID if full_h_grid is None else full_h_grid
    best = _search(times, tiles, a_grid, p_grid, [(NEVER,)])
    a, p = best[2], best[3]
    best = _search(times, tiles, [a], [p], [(int(f),) for f in full_h_grid])
    return _search(times, tiles, a_grid, p_grid, [best[4]])


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("times", help="CSV of configuration times or a tune.py JSON report")
    ap.add_argument("--holdout-splits", type=int, default=6)
    args = ap.parse_args(argv)
    times, tiles = load(args.times)
    mean, worst, a, p, full, params = fit(times, tiles)
    print(f"# {len(times)} shapes; waves: part-filled last wave costs max({p:.2f}, {a:.2f} + {1 - a:.2f} * fill);"
          + "".join(f" config {f} for config {c} from {n} {t[0]}x{t[1]} tiles;" for (c, f, t), n in zip(FULL_CHIP, full)))
    for cid in ALL:
        if cid in params:
            bm, bn = tiles[cid]
            print(f"    {{{cid}, {params[cid][0]:.2f}, {params[cid][1]:.2f}}},  // {bm}x{bn}")
    print(f"# in sample: choice / fastest = x{mean:.4f} on average, x{worst:.3f} at worst")
    keys = sorted(times)
    for seed in range(args.holdout_splits):
        rnd = random.Random(seed)
        ks = keys[:]
        rnd.shuffle(ks)
        train = {k: times[k] for k in ks[: len(ks) // 2]}
        test = {k: times[k] for k in ks[len(ks) // 2:]}
        _, _, a_s, p_s, f_s, prm = fit(train, tiles)
        m, w = regret(test, tiles, prm, a_s, p_s, f_s)
        print(f"# held-out split {seed}: x{m:.4f} on average, x{w:.3f} at worst")
    return 0


if __name__ == "__main__":
    sys.exit(main())
