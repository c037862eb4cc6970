"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle element by element.

Tolerance (the tutorial's own check, PKUHPC scow-tutorial "Tutorial14",
section 2 listing: assert_close with rtol = atol = 1e-2): every checked
output must satisfy |gpu - ref| <= 1e-2 + 1e-2 * |ref|, with both the GPU
output and the oracle's fp16 output decoded exactly; a NaN or Inf where the
oracle is finite fails; where the oracle itself is not finite (an fp16
overflow to +-inf) only the identical bit pattern passes, since no finite
bound can be formed there; +0 and -0 compare equal.
"""
from __future__ import annotations

import numpy as np
import torch

from tiled_dense_gemm_scale_amd import workloads as W

RTOL = 1e-2
ATOL = 1e-2


def f16(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def run_gpu(a: torch.Tensor, b: torch.Tensor, alpha: float, config_id: int = -1,
            c: torch.Tensor = None) -> np.ndarray:
    """a, b: CPU fp16 tensors.  Returns C's bit patterns (numpy uint16)."""
    import tiled_dense_gemm_scale_amd as gsr

    dev = torch.device("cuda:0")
    ad = a.to(dev)
    bd = b.to(dev)
    if config_id == -1:
        out = gsr.gemm_scale_relu(ad, bd, alpha, c=c)
    else:
        out = gsr.gemm_scale_relu_ex(ad, bd, alpha, config_id, c=c)
    torch.cuda.synchronize()
    return W.fp16_bits(out.cpu())


def run_gpu_variant(a: torch.Tensor, b: torch.Tensor, bias, alpha: float, act: str,
                    config_id: int = -1, c: torch.Tensor = None) -> np.ndarray:
    """act(alpha * a @ b + bias) through the epilogue-variant entry point.
    a, b, bias (or None): CPU fp16 tensors.  Returns C's bit patterns."""
    import tiled_dense_gemm_scale_amd as gsr

    dev = torch.device("cuda:0")
    bd = bias.to(dev) if bias is not None else None
    out = gsr.gemm_scale_bias_act(a.to(dev), b.to(dev), bd, alpha, act, c=c, config_id=config_id)
    torch.cuda.synchronize()
    return W.fp16_bits(out.cpu())


class Report:
    def __init__(self, name, n, max_abs, max_rel_excess, violations, worst, fro):
        self.name, self.n, self.max_abs = name, n, max_abs
        self.max_rel_excess, self.violations, self.worst, self.fro = max_rel_excess, violations, worst, fro

    def __str__(self):
        return (f"{self.name}: {self.n} checked, max|err|={self.max_abs:.3g}, "
                f"worst err/(atol+rtol|ref|)={self.max_rel_excess:.3g}, violations={self.violations}, "
                f"rel Frobenius={self.fro:.3g}, worst at {self.worst}")


def compare(name: str, gpu_bits: np.ndarray, ref_bits: np.ndarray, coords=None) -> Report:
    gb = np.asarray(gpu_bits, dtype=np.uint16).ravel()
    rb = np.asarray(ref_bits, dtype=np.uint16).ravel()
    g = f16(gb)
    r = f16(rb)
    if g.shape != r.shape:
        raise AssertionError(f"{name}: {g.shape} values vs {r.shape} expected")
    if g.size == 0:
        return Report(name, 0, 0.0, 0.0, 0, None, 0.0)
    fin = np.isfinite(r)
    err = np.zeros_like(r)
    bound = np.ones_like(r)
    err[fin] = np.abs(g[fin] - r[fin])          # NaN where the GPU gave NaN
    err[fin & ~np.isfinite(g)] = np.inf          # Inf or NaN where the oracle is finite
    bound[fin] = ATOL + RTOL * np.abs(r[fin])
    err[~fin] = np.where(gb[~fin] == rb[~fin], 0.0, np.inf)  # not finite: same bits or fail
    ratio = err / bound
    viol = int(np.count_nonzero(~(ratio <= 1.0)))  # NaN counts as a violation
    i = int(np.argmax(np.where(np.isnan(ratio), np.inf, ratio)))
    where = (tuple(np.unravel_index(i, np.asarray(ref_bits).shape)) if coords is None
             else (int(coords[0][i]), int(coords[1][i])))
    gf, rf = g[fin & np.isfinite(g)], r[fin & np.isfinite(g)]
    denom = float(np.sqrt(np.sum(rf * rf)))
    fro = float(np.sqrt(np.sum((gf - rf) ** 2)) / denom) if denom > 0 else float(np.sqrt(np.sum(gf * gf)))
    return Report(name, g.size, float(np.max(np.where(np.isnan(err), np.inf, err))),
                  float(np.max(np.where(np.isnan(ratio), np.inf, ratio))), viol, where, fro)


def assert_parity(name: str, gpu_bits, ref_bits, coords=None) -> Report:
    rep = compare(name, gpu_bits, ref_bits, coords)
    print(rep, flush=True)
    assert rep.violations == 0, str(rep)
    return rep


def assert_bitwise(name: str, gpu_bits, ref_bits) -> None:
    g = np.asarray(gpu_bits, dtype=np.uint16)
    r = np.asarray(ref_bits, dtype=np.uint16)
    # +0 and -0 are the same value
    gz = np.where((g & 0x7FFF) == 0, 0, g)
    rz = np.where((r & 0x7FFF) == 0, 0, r)
    bad = np.argwhere(gz != rz)
    assert bad.size == 0, (f"{name}: {len(bad)} bitwise mismatches, first at {tuple(bad[0])}: "
                           f"gpu 0x{int(g[tuple(bad[0])]):04x} oracle 0x{int(r[tuple(bad[0])]):04x}")
