"""Fit the tile selector's cost model to measured configuration times.

The selector in csrc/gsr_api.hip prices a candidate tile bm x bn as

    waves(wgs) * (2 * bm * bn * K / (rate * 1e6) + tile_us)        [us]

with wgs = ceil(M / bm) * ceil(N / bn) workgroups on 256 CUs and
waves(wgs) = full waves + (a part-filled last wave: max(pmin, a + (1 - a) * fill)).
The 256x256, 128x256 and 128x128 tiles have one kernel each, the 16x16x32
kernels with B copied to LDS (configs 28, 31 and 32): each was measured faster
than every other kernel of its tile on every one of the 60 shapes.  This module fits `rate`
(TFLOP/s per CU) and `tile_us` per configuration by least squares in relative
error, and picks (a, pmin) on a grid whose choices come closest to the
fastest measured configuration (mean log ratio).  Input: the CSV written from
a `tune.py --top 0` report (tuning/mi355x_config_times.csv) or such a JSON
report itself.

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
BASE = [28, 31, 32]
COPY_WAVE = [21, 22]
FOUR_WAVE = [16, 18]
ALL = BASE + COPY_WAVE + FOUR_WAVE


def candidates(M: int, N: int, K: int) -> List[int]:
    return BASE + (COPY_WAVE if K > 256 else FOUR_WAVE)


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


def fit_params(times, tiles, a: float, pmin: float) -> Dict[int, Tuple[float, float]]:
    """(rate, tile_us) per candidate: least squares of t ~ w * (flops/rate + e),
    rows scaled by 1/t (relative error)."""
    out = {}
    for cid in ALL:
        X, y = [], []
        for (M, N, K), t in times.items():
            if cid not in t:
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


def choose(params, tiles, M: int, N: int, K: int, a: float, pmin: float, have=None) -> int:
    best, best_t = None, math.inf
    for cid in candidates(M, N, K):
        if cid not in params or (have is not None and cid not in have):
            continue
        rate, e = params[cid]
        t = waves(workgroups(tiles[cid], M, N), a, pmin) * (2.0 * tiles[cid][0] * tiles[cid][1] * K / (rate * 1e6) + e)
        if t < best_t:
            best, best_t = cid, t
    return best


def regret(times, tiles, params, a, pmin) -> Tuple[float, float]:
    """(mean, worst) of t[choice] / t[fastest] over the shapes."""
    logs, worst = [], 1.0
    for (M, N, K), t in times.items():
        c = choose(params, tiles, M, N, K, a, pmin, have=t)
        r = t[c] / min(t.values())
        logs.append(math.log(r))
        worst = max(worst, r)
    return math.exp(sum(logs) / len(logs)), worst


def fit(times, tiles, a_grid=None, p_grid=None):
    """(mean, worst, a, pmin, params) of the grid point whose choices come
    closest to the fastest configuration (first such point on ties)."""
    a_grid = np.arange(0.0, 0.75, 0.05) if a_grid is None else a_grid
    p_grid = np.arange(0.30, 1.001, 0.05) if p_grid is None else p_grid
    best = None
    for a in a_grid:
        for p in p_grid:
            params = fit_params(times, tiles, float(a), float(p))
            mean, worst = regret(times, tiles, params, float(a), float(p))
            if best is None or mean < best[0] - 1e-12:
                best = (mean, worst, float(a), float(p), params)
    return best


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("times", help="CSV of configuration times or a tune.py JSON report")
    ap.add_argument("--holdout-splits", type=int, default=6)
    args = ap.parse_args(argv)
    times, tiles = load(args.times)
    mean, worst, a, p, params = fit(times, tiles)
    print(f"# {len(times)} shapes; waves: part-filled last wave costs max({p:.2f}, {a:.2f} + {1 - a:.2f} * fill)")
    for cid in ALL:
        if cid in params:
            bm, bn = tiles[cid]
            print(f"    {{{cid}, {params[cid][0]:.3f}, {params[cid][1]:.3f}}},  // {bm}x{bn}")
    print(f"# in sample: choice / fastest = x{mean:.4f} on average, x{worst:.3f} at worst")
    keys = sorted(times)
    for seed in range(args.holdout_splits):
        rnd = random.Random(seed)
        ks = keys[:]
        rnd.shuffle(ks)
        train = {k: times[k] for k in ks[: len(ks) // 2]}
        test = {k: times[k] for k in ks[len(ks) // 2:]}
        _, _, a_s, p_s, prm = fit(train, tiles)
        m, w = regret(test, tiles, prm, a_s, p_s)
        print(f"# held-out split {seed}: x{m:.4f} on average, x{w:.3f} at worst")
    return 0


if __name__ == "__main__":
    sys.exit(main())
