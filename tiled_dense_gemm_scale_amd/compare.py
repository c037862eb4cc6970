"""The library against torch on many shapes (context, not the benchmark).

For each M x N x K: the library's gemm_scale_relu in the selector's
configuration, torch's unfused relu((a @ b) * alpha) (three kernels, the
comparison the PKUHPC tutorial makes for its fused kernel in section 2) and
torch's a @ b alone (hipBLASLt on ROCm, no epilogue).  Each is captured as a
HIP graph of `steps` calls and replayed three times; the fastest replay
counts.  Inputs: A ~ N(0, 1), B ~ N(0, 1/K) fp16 from a seeded CPU
generator, alpha = 1.

    python -m tiled_dense_gemm_scale_amd.compare [--shapes MxNxK,...] [--json out.json]

The default shapes: M in {1, 8, 32, ..., 8192} against 11008x4096, 4096x4096
and 4096x11008 weights, and squares from 512 to 8192.
"""
from __future__ import annotations

import argparse
import json
import sys
from typing import List, Tuple

import torch


def default_shapes() -> List[Tuple[int, int, int]]:
    shapes = []
    for (N, K) in [(11008, 4096), (4096, 4096), (4096, 11008)]:
        for M in [1, 8, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192]:
            shapes.append((M, N, K))
    for S in [512, 768, 1536, 2048, 3072, 6144, 8192]:
        shapes.append((S, S, S))
    return shapes


def time_graph(fn, stream, steps: int) -> float:
    """Microseconds per call: `steps` calls captured once, fastest of three replays."""
    with torch.cuda.stream(stream):
        for _ in range(3):
            fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(steps):
            fn()
    best = float("inf")
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        with torch.cuda.stream(stream):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / steps)
    del g
    return best


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--shapes", default=None, help="comma-separated MxNxK (default: the built-in list)")
    ap.add_argument("--json", default=None, help="write every timing to this file")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("compare: no GPU visible", file=sys.stderr)
        return 2
    import tiled_dense_gemm_scale_amd as gsr

    shapes = default_shapes() if args.shapes is None else \
        [tuple(int(v) for v in s.lower().split("x")) for s in args.shapes.split(",") if s.strip()]
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(0)
    out = []
    for (M, N, K) in shapes:
        a = torch.randn(M, K, generator=gen).half().to(dev)
        b = (torch.randn(K, N, generator=gen) * K ** -0.5).half().to(dev)
        c = torch.empty(M, N, dtype=torch.float16, device=dev)
        s = torch.cuda.Stream(dev)
        flops = 2.0 * M * N * K
        steps = max(10, min(200, int(3e13 / flops)))
        cfg = gsr.select_config(M, N, K)
        t_lib = time_graph(lambda: gsr.gemm_scale_relu(a, b, 1.0, c=c, stream=s), s, steps)
        t_unf = time_graph(lambda: torch.relu(torch.matmul(a, b) * 1.0), s, steps)
        t_mm = time_graph(lambda: torch.matmul(a, b), s, steps)
        r = {"M": M, "N": N, "K": K, "config_id": cfg["id"], "tile": f"{cfg['block_m']}x{cfg['block_n']}",
             "library_us": round(t_lib, 2), "torch_unfused_us": round(t_unf, 2), "torch_matmul_us": round(t_mm, 2),
             "library_tflops": round(flops / t_lib / 1e6, 1),
             "speedup_vs_unfused": round(t_unf / t_lib, 3), "speedup_vs_matmul": round(t_mm / t_lib, 3)}
        out.append(r)
        print(f"{M:5d}x{N:5d}x{K:5d} cfg {cfg['id']:2d} {r['tile']:>8s}  library {t_lib:9.2f} us "
              f"({r['library_tflops']:7.1f} TF/s)  torch unfused {t_unf:9.2f} ({r['speedup_vs_unfused']:5.2f}x)  "
              f"torch matmul {t_mm:9.2f} ({r['speedup_vs_matmul']:5.2f}x)", flush=True)
        del a, b, c
    if args.json:
        with open(args.json, "w") as f:
            json.dump({"device": torch.cuda.get_device_properties(0).name, "library_version": gsr.version(),
                       "shapes": out}, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
