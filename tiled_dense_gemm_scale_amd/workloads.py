"""Workload registry and seeded synthetic input generators.

This module only draws random numbers and names shapes.  It holds none of
the operation's arithmetic, so both the GPU path and the oracle may be fed
from it: each receives the same fp16 bit patterns and computes on its own.

Recipe (PKUHPC scow-tutorial "Tutorial14", section 2, the main() of the
listing): seed the CPU generator with 0, draw A = randn(M, K) and then
B = randn(K, N) in fp32 from the same generator, and narrow both to fp16 with
round-to-nearest-even.  The LLM-MLP workload scales B by 1/sqrt(K) before the
narrowing (weights ~ N(0, 1/K)); for K = 4096 that is an exact division by 64.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    alpha: float
    b_std: float  # standard deviation of B's entries before narrowing
    sampled: bool  # parity on sampled outputs instead of all of C
    note: str

    @property
    def flops(self) -> int:
        """2*M*N*K: one multiply and one add per term of every output."""
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """One fp16 read of A and B and one fp16 write of C."""
        return 2 * (self.M * self.K + self.K * self.N + self.M * self.N)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("square_256", 256, 256, 256, 0.5, 1.0, False,
                 "M=N=K=256, A,B ~ N(0,1) fp16, alpha=0.5"),
        Workload("square_1024", 1024, 1024, 1024, 0.5, 1.0, False,
                 "M=N=K=1024, A,B ~ N(0,1) fp16, alpha=0.5 (the tutorial's own shape)"),
        Workload("square_4096", 4096, 4096, 4096, 0.5, 1.0, False,
                 "M=N=K=4096, A,B ~ N(0,1) fp16, alpha=0.5"),
        Workload("llm_mlp_4097x11008x4096", 4097, 11008, 4096, 1.0, 4096 ** -0.5, False,
                 "LLM MLP up-projection, 4097 tokens (ragged M), N=11008, K=4096, "
                 "A ~ N(0,1), B ~ N(0,1/K), alpha=1.0"),
        Workload("square_16384", 16384, 16384, 16384, 0.5, 1.0, True,
                 "M=N=K=16384, A,B ~ N(0,1) fp16, alpha=0.5; parity on 4096 sampled outputs"),
    ]
}

WORKLOAD_ORDER = ["square_256", "square_1024", "square_4096",
                  "llm_mlp_4097x11008x4096", "square_16384"]

# A 16-token decode batch against the LLM-MLP weights: the skinny class.
SKINNY = Workload("skinny_16x11008x4096", 16, 11008, 4096, 1.0, 4096 ** -0.5, False,
                  "decode batch of 16 tokens against the 11008x4096 MLP weights")

# One GPU's share of the LLM-MLP up-projection when its columns are split over
# 8 GPUs (column parallelism: each GPU holds 11008/8 = 1376 columns of B and
# the whole A, and no partial sums are exchanged).
COLSHARD8 = Workload("llm_mlp_colshard8_4097x1376x4096", 4097, 1376, 4096, 1.0, 4096 ** -0.5, False,
                     "one GPU's column shard of the LLM-MLP up-projection split over 8 GPUs "
                     "(N = 11008/8), A ~ N(0,1), B ~ N(0,1/K), alpha=1.0")

# A 1024-row batch against 4096x4096 weights: a mid-size grid (256 tiles of
# 128x128, 64 of 256x256), the class the 128x128 tile serves.
MID = Workload("mid_1024x4096x4096", 1024, 4096, 4096, 1.0, 4096 ** -0.5, False,
               "a 1024-row batch against 4096x4096 weights, A ~ N(0,1), B ~ N(0,1/K), alpha=1.0")

# A 16-token decode batch against the MLP down-projection (11008 -> 4096): 64
# output tiles of 32x64 against 86 K-steps of 128, the class that splits K
# across workgroups when the call has a workspace.
DECODE_DOWN = Workload("decode_down_16x4096x11008", 16, 4096, 11008, 1.0, 11008 ** -0.5, False,
                       "decode batch of 16 tokens against the 4096x11008 MLP down-projection weights, "
                       "A ~ N(0,1), B ~ N(0,1/K), alpha=1.0")

# Shapes timed and tested besides the five workloads above.
EXTRA: Dict[str, Workload] = {w.name: w for w in [SKINNY, COLSHARD8, MID, DECODE_DOWN]}


def by_name(name: str) -> Workload:
    """A workload of either registry by name."""
    if name in WORKLOADS:
        return WORKLOADS[name]
    if name in EXTRA:
        return EXTRA[name]
    raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS) + sorted(EXTRA)}")


def normal_inputs(M: int, N: int, K: int, seed: int = 0, b_std: float = 1.0
                  ) -> Tuple[torch.Tensor, torch.Tensor]:
    """A (M,K) and B (K,N) fp16 CPU tensors: fp32 randn from one CPU
    generator seeded with `seed`, A drawn first, then narrowed to fp16."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    a = torch.randn(M, K, generator=g, dtype=torch.float32)
    b = torch.randn(K, N, generator=g, dtype=torch.float32)
    if b_std != 1.0:
        b.mul_(b_std)
    return a.half(), b.half()


def workload_inputs(w: Workload, seed: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    return normal_inputs(w.M, w.N, w.K, seed=seed, b_std=w.b_std)


def integer_inputs(M: int, N: int, K: int, seed: int = 0, lo: int = -4, hi: int = 4
                   ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Small-integer fp16 inputs (uniform in [lo, hi]).  With |partial sums|
    below 2^24 every fp32 accumulation order gives the exact integer sum, so
    results can be compared bit for bit."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    a = torch.randint(lo, hi + 1, (M, K), generator=g, dtype=torch.int32)
    b = torch.randint(lo, hi + 1, (K, N), generator=g, dtype=torch.int32)
    return a.half(), b.half()


def bias_input(N: int, seed: int = 0, std: float = 1.0, integer: bool = False) -> torch.Tensor:
    """A bias vector (N,) fp16 CPU tensor for the epilogue variants: fp32
    randn * std from its own CPU generator (seed + 1000003), narrowed to fp16;
    or, with integer=True, integers uniform in [-4, 4]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 1000003)
    if integer:
        return torch.randint(-4, 5, (N,), generator=g, dtype=torch.int32).half()
    return (torch.randn(N, generator=g, dtype=torch.float32) * std).half()


def pattern_inputs(M: int, N: int, K: int, device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """Integer-valued fp16 inputs with no random draw, built where they are
    used (so multi-GiB operands need no host copy to create):
    A[m,k] = ((7m + 13k) mod 9) - 4 and B[k,n] = ((5k + 11n) mod 7) - 3.
    Every fp32 partial sum stays an exact integer while |sums| < 2^24."""
    m = torch.arange(M, device=device, dtype=torch.int64)[:, None]
    k = torch.arange(K, device=device, dtype=torch.int64)
    a = ((7 * m + 13 * k[None, :]) % 9 - 4).to(torch.float16)
    n = torch.arange(N, device=device, dtype=torch.int64)[None, :]
    b = ((5 * k[:, None] + 11 * n) % 7 - 3).to(torch.float16)
    return a, b


def sample_points(M: int, N: int, count: int = 4096, seed: int = 1,
                  extra_rows: Optional[list] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Output coordinates to check on the largest shapes: the four corners,
    the centre and three edge midpoints, then distinct uniform points from a
    generator of its own (seed 1), `count` in all; plus every column of each
    row listed in `extra_rows` (e.g. a ragged last row)."""
    forced = [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1), (M // 2, N // 2),
              (M - 1, N // 2), (M // 2, N - 1), (0, N // 2)]
    seen = set()
    pts = []
    for p in forced:
        if p not in seen and 0 <= p[0] < M and 0 <= p[1] < N:
            seen.add(p)
            pts.append(p)
    rng = np.random.Generator(np.random.PCG64(seed))
    target = min(count, M * N)
    while len(pts) < target:
        m = int(rng.integers(0, M))
        n = int(rng.integers(0, N))
        if (m, n) not in seen:
            seen.add((m, n))
            pts.append((m, n))
    ms = [p[0] for p in pts]
    ns = [p[1] for p in pts]
    for r in extra_rows or []:
        ms.extend([r] * N)
        ns.extend(range(N))
    return np.asarray(ms, dtype=np.int64), np.asarray(ns, dtype=np.int64)


def fp16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw IEEE binary16 bit patterns of a CPU fp16 tensor."""
    if t.dtype != torch.float16:
        raise TypeError("expected an fp16 tensor")
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_tensor(bits: np.ndarray) -> torch.Tensor:
    """A CPU fp16 tensor holding the given bit patterns."""
    arr = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(arr.view(np.int16).copy()).view(torch.float16)
