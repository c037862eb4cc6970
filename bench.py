#!/usr/bin/env python3
"""Benchmark of the fused fp16 GEMM + scale + ReLU on one MI355X.

A step is one call of the whole operation, C = ReLU(alpha * A @ B), on one
batch of synthetic fp16 input already resident in HBM.  Timing follows the
tutorial's benchmark helper (PKUHPC scow-tutorial "Tutorial14", section 2:
warm-up calls, a synchronise, an event, the timed calls, an event, a
synchronise, mean time per call, TFLOP/s = 2*M*N*K / time), with the events
recorded on the stream the kernels are launched on.  By default the K timed
calls are captured once into a HIP graph and the graph is replayed, so host
launch overhead does not pace the GPU; --launch eager issues them one by one.

Prints one JSON line on stdout.  Diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2516.6   # MI355X dense fp16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
DEFAULT_WORKLOAD = "square_16384"
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    """Digest of the kernel and launch sources; a traffic measurement taken
    on other sources is stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_dense_gemm_scale_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, flops: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel sources changed since."""
    path = os.path.join(TRAFFIC_DIR, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_digest") != kernel_source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def roofline_of(w, ms: float, traffic):
    """The roofline object of one launch taking `ms` milliseconds.  The bound
    follows the workload's arithmetic intensity against the ridge point of the
    two published peaks (2516.6 TFLOP/s / 8 TB/s = 315 FLOP/B): above it the
    algorithmic FLOP per launch over the time against the MFMA peak, below it
    the algorithmic bytes 2(MK+KN+MN) over the time against the HBM peak."""
    ridge = PEAK_FP16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if w.flops / w.algorithmic_bytes >= ridge:
        achieved, peak, unit, bound = w.flops / (ms * 1e-3) / 1e12, PEAK_FP16_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = w.algorithmic_bytes / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    return {
        "bound": bound,
        "achieved": round(achieved, 3),
        "peak": peak,
        "unit": unit,
        "frac": round(achieved / peak, 4),
        "traffic": traffic,
    }


def device_info(index: int) -> dict:
    """CU count and maximum engine clock as the HIP runtime reports them."""
    import ctypes
    info = {}
    for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
        try:
            hip = ctypes.CDLL(name)
            break
        except OSError:
            hip = None
    if hip is None:
        return info
    for key, attr in (("clock_khz", 5), ("cus", 63)):  # hipDeviceAttributeClockRate, ...MultiprocessorCount
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, index) == 0:
            info[key] = v.value
    return info


class ClockSampler:
    """The engine (graphics) clock and the socket power the GPU reports while
    the benchmark's calls run, read from the driver's metrics table through
    amdsmi in a background thread.  The part is power-limited under dense fp16
    MFMA work, so this clock, not the maximum the runtime reports, is what the
    achieved rate follows.  The driver refreshes that table only about once a
    second, so a reading is trusted only from `settle_s` seconds after the
    sampling started (the caller keeps the GPU busy with the timed calls for
    longer than that).  Each reading is the mean over the XCDs of their
    current clocks.  Sampling only reads the driver's counters; any failure
    (no amdsmi, no permission, the device not found) leaves the result None."""

    def __init__(self, props, period_s: float = 0.05, settle_s: float = 1.5):
        import threading
        self.period_s, self.settle_s = period_s, settle_s
        self.samples = []  # (seconds since start, MHz, watts or None)
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        self._amdsmi = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            want = (int(props.pci_domain_id), int(props.pci_bus_id), int(props.pci_device_id))
            for h in amdsmi.amdsmi_get_processor_handles():
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self._handle = h
                    break
            if self._handle is None:
                self.error = f"no amdsmi device at {want}"
        except Exception as e:  # noqa: BLE001 - a missing clock reading is not an error of the benchmark
            self.error = f"{type(e).__name__}: {e}"

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        clks = [float(v) for v in (m.get("current_gfxclks") or []) if isinstance(v, (int, float)) and v > 0]
        if not clks and isinstance(m.get("current_gfxclk"), (int, float)):
            clks = [float(m["current_gfxclk"])]
        power = m.get("current_socket_power")
        return (sum(clks) / len(clks) if clks else None), (float(power) if isinstance(power, (int, float)) else None)

    def _run(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            try:
                mhz, watts = self._read()
            except Exception as e:  # noqa: BLE001
                self.error = f"{type(e).__name__}: {e}"
                return
            if mhz is not None:
                self.samples.append((time.perf_counter() - t0, mhz, watts))
            self._stop.wait(self.period_s)

    def start(self):
        import threading
        if self._handle is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def stop(self):
        """Median, min and max of the settled readings, or None."""
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        if self._amdsmi is not None:
            try:
                self._amdsmi.amdsmi_shut_down()
            except Exception:  # noqa: BLE001
                pass
        good = sorted(mhz for t, mhz, _ in self.samples if t >= self.settle_s)
        watts = sorted(w for t, _, w in self.samples if t >= self.settle_s and w is not None)
        if not good:
            if self.error is None:
                self.error = f"no reading after the first {self.settle_s} s"
            return None
        out = {"median_mhz": round(good[len(good) // 2], 1), "min_mhz": round(good[0], 1),
               "max_mhz": round(good[-1], 1), "samples": len(good)}
        if watts:
            out["socket_power_w"] = watts[len(watts) // 2]
        out["source"] = ("amdsmi metrics table (mean over XCDs of the current graphics clock), read every "
                         f"{self.period_s * 1e3:.0f} ms while the timed calls were replayed for the clock window; "
                         f"readings from the first {self.settle_s} s dropped (the table refreshes about once a second)")
        return out


def time_graph(graph, stream, steps: int, repeats: int):
    """Per-call milliseconds of `repeats` replays of a graph of `steps` calls,
    each bracketed by events on the launch stream."""
    import torch
    out = []
    for _ in range(repeats):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        with torch.cuda.stream(stream):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    return out


def capture(fn, stream, steps: int):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(steps):
            fn()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()  # one untimed replay
    torch.cuda.synchronize()
    return g


# --epilogue choices: (bias?, activation).  "relu" is the tutorial's operation
# through gemm_scale_relu; the others go through gemm_scale_bias_act.
EPILOGUES = {"relu": (False, "relu"), "bias-relu": (True, "relu"), "gelu": (False, "gelu"),
             "bias-gelu": (True, "gelu"), "bias-none": (True, "none")}


def cpu_baseline(w, a, b, target_s: float, epilogue: str = "relu", bias=None):
    """The oracle, as it is, on a bounded sample of the same workload: the
    first R rows of A against all of B, R sized for about `target_s` seconds."""
    from oracle import oracle
    from tiled_dense_gemm_scale_amd import workloads as W

    orc = oracle.load()
    threads = oracle.default_threads()
    a_bits = W.fp16_bits(a)
    b_bits = W.fp16_bits(b)
    act = {"relu": oracle.ACT_RELU, "gelu": oracle.ACT_GELU, "none": oracle.ACT_NONE}[EPILOGUES[epilogue][1]]
    bias_bits = W.fp16_bits(bias) if bias is not None else None

    def run(rows):
        if epilogue == "relu":
            orc.gemm_scale_relu(a_bits[:rows], b_bits, w.alpha, nthreads=threads)
        else:
            orc.gemm_bias_act(a_bits[:rows], b_bits, bias_bits, w.alpha, act, nthreads=threads)

    # size the sample from two timed runs (each run also decodes all of B: a
    # fixed cost beside the per-row cost); a workload the oracle finishes
    # whole in well under the target is repeated instead
    def timed(rows):
        t0 = time.perf_counter()
        run(rows)
        return time.perf_counter() - t0

    R1 = min(w.M, max(threads, 8))
    t1 = timed(R1)
    if R1 >= w.M:
        per_row, fixed = t1 / R1, 0.0
    else:
        R2 = min(w.M, R1 * 4)
        t2 = timed(R2)
        per_row = max((t2 - t1) / (R2 - R1), 1e-9)
        fixed = max(t1 - per_row * R1, 0.0)
    R = int(min(w.M, max(R1, (target_s - fixed) / per_row)))
    if R < w.M:
        R = max(threads, (R // threads) * threads)
        reps = 1
    else:
        R = w.M
        reps = int(max(1, min(1000, round(target_s / (fixed + per_row * w.M)))))
    t0 = time.perf_counter()
    for _ in range(reps):
        run(R)
    t = time.perf_counter() - t0
    flops = 2.0 * R * w.N * w.K * reps
    return {
        "value": round(flops / t / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"rows 0..{R - 1} of C ({R}x{w.N} outputs, K={w.K})" + (f", {reps} times" if reps > 1 else "")
                   + f", full fp64 oracle, {t:.2f} s"),
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--launch", choices=["graph", "eager"], default="graph")
    ap.add_argument("--config-id", type=int, default=-1, help="force a tile configuration")
    ap.add_argument("--workspace", action="store_true",
                    help="call the entry point with a workspace (K split across workgroups where the "
                         "library picks one), with the bytes gsr_workspace_bytes gives")
    ap.add_argument("--epilogue", choices=sorted(EPILOGUES), default="relu",
                    help="relu: the tutorial's C = ReLU(alpha A B); the others time the epilogue variants "
                         "C = act(alpha A B + bias) (bias: seeded N(0,1) fp16 per column)")
    ap.add_argument("--tuning", default=None,
                    help="load a tuning table (gsr_load_tuning format, e.g. written by "
                         "python -m tiled_dense_gemm_scale_amd.tune) before timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--repeats", type=int, default=5,
                    help="extra replays of the timed graph for median/min (graph launch only)")
    ap.add_argument("--no-context", action="store_true", help="skip the dispatch-floor measurement")
    ap.add_argument("--clock-window-s", type=float, default=3.0,
                    help="seconds of the same calls, after the timed region, during which the engine clock and "
                         "socket power are sampled (0: skip)")
    ap.add_argument("--no-torch-context", action="store_true",
                    help="skip timing torch's unfused matmul -> mul -> relu and its plain fp16 matmul")
    ap.add_argument("--cold", action="store_true",
                    help="also time single calls with L2 and the last-level cache flushed before each "
                         "(context only; eager launches, so each time holds one dispatch)")
    ap.add_argument("--zero-input", action="store_true",
                    help="also time the same kernel on all-zero inputs (runs the timed kernel again, "
                         "so leave it off when profiling per-kernel averages)")
    ap.add_argument("--inputs", choices=["normal", "zeros"], default="normal",
                    help="zeros: run everything, the timed region included, on all-zero A and B (a study of "
                         "the data-dependent engine clock under rocprofv3 counters; not the workload's number)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch
    import tiled_dense_gemm_scale_amd as gsr
    from tiled_dense_gemm_scale_amd import workloads as W

    w = W.by_name(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    dinfo = device_info(torch.cuda.current_device())
    log(f"[bench] device {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count} {dinfo}")
    log(f"[bench] workload {w.name}: {w.note}")

    a_cpu, b_cpu = W.workload_inputs(w)
    if args.inputs == "zeros":
        a_cpu, b_cpu = torch.zeros_like(a_cpu), torch.zeros_like(b_cpu)
        log("[bench] inputs: all zeros (clock study)")
    a = a_cpu.to(dev)
    b = b_cpu.to(dev)
    c = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    stream = torch.cuda.Stream(dev)
    torch.cuda.synchronize()
    if args.tuning:
        gsr.load_tuning(args.tuning)
        log(f"[bench] tuning table {args.tuning}: {gsr.tuning_entries()} entries")
    cfg = gsr.select_config(w.M, w.N, w.K) if args.config_id < 0 else gsr.get_config(args.config_id)
    log(f"[bench] tile config {cfg}")

    has_bias, act = EPILOGUES[args.epilogue]
    bias_cpu = W.bias_input(w.N) if has_bias else None
    bias = bias_cpu.to(dev) if has_bias else None

    ws, ws_bytes = None, None
    if args.workspace:
        ws_bytes = gsr.workspace_bytes(w.M, w.N, w.K)
        ws = gsr.new_workspace(ws_bytes, device=dev)
        log(f"[bench] workspace {ws_bytes} bytes ({'K split across workgroups' if ws_bytes else 'no split'})")

    def step():
        if ws is not None:
            gsr.gemm_scale_bias_act_ws(a, b, ws, bias, w.alpha, act, c=c, stream=stream, config_id=args.config_id)
        elif args.epilogue == "relu":
            gsr.gemm_scale_relu_ex(a, b, w.alpha, args.config_id, c=c, stream=stream)
        else:
            gsr.gemm_scale_bias_act(a, b, bias, w.alpha, act, c=c, stream=stream, config_id=args.config_id)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()

    graph = None
    if args.launch == "graph":
        graph = capture(step, stream, args.steps)

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()  # single rank: the barrier is this synchronise
    start.record(stream)
    if graph is not None:
        with torch.cuda.stream(stream):
            graph.replay()
    else:
        with torch.cuda.stream(stream):
            for _ in range(args.steps):
                step()
    end.record(stream)
    torch.cuda.synchronize()
    elapsed_ms = start.elapsed_time(end)
    ms = elapsed_ms / args.steps
    tflops = w.flops / (ms * 1e-3) / 1e12
    log(f"[bench] {args.steps} steps in {elapsed_ms:.3f} ms -> {ms * 1e3:.2f} us/step, {tflops:.1f} TFLOP/s "
        f"({100 * tflops / PEAK_FP16_TFLOPS:.1f}% of {PEAK_FP16_TFLOPS})")

    # Context, outside the timed region: the spread of further replays, the
    # dispatch floor (the same number of launches of the library's smallest
    # kernel: K = 0 on a 1x8 output) and, on request, the same kernel on
    # all-zero inputs (identical instruction stream; the engine clock is
    # power-limited and depends on the data, so this separates the schedule
    # from the clock).
    context = {}
    if graph is not None and args.repeats > 0:
        reps = sorted(time_graph(graph, stream, args.steps, args.repeats))
        context["repeat_ms_per_step"] = {"median": round(reps[len(reps) // 2], 6), "min": round(reps[0], 6),
                                         "max": round(reps[-1], 6), "n": len(reps)}
        log(f"[bench] repeats: {context['repeat_ms_per_step']}")
    if args.clock_window_s > 0:
        # The same calls again for a few seconds (the timed graph replayed, or
        # the eager calls), while the driver's clock and power readings are
        # sampled; outside the timed region.
        clock = ClockSampler(props)
        torch.cuda.synchronize()
        clock.start()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.clock_window_s:
            with torch.cuda.stream(stream):
                if graph is not None:
                    graph.replay()
                else:
                    for _ in range(args.steps):
                        step()
            torch.cuda.synchronize()
        observed = clock.stop()
        context["engine_clock_observed"] = observed
        if observed is None:
            log(f"[bench] engine clock not sampled ({clock.error})")
        else:
            log(f"[bench] engine clock under the timed calls: {observed}")
    if graph is not None and not args.no_context:
        a0 = torch.empty((1, 0), dtype=torch.float16, device=dev)
        b0 = torch.empty((0, 8), dtype=torch.float16, device=dev)
        c0 = torch.empty((1, 8), dtype=torch.float16, device=dev)
        g0 = capture(lambda: gsr.gemm_scale_relu(a0, b0, 1.0, c=c0, stream=stream), stream, args.steps)
        floor = min(time_graph(g0, stream, args.steps, 3))
        context["dispatch_floor_us"] = round(floor * 1e3, 3)
        del g0
        log(f"[bench] dispatch floor {context['dispatch_floor_us']} us/launch")
    if graph is not None and not args.no_torch_context and args.epilogue == "relu":
        # The tutorial's comparison: its fused kernel against torch's
        # relu((a @ b) * scale), three kernels with two fp16 round trips of C
        # through HBM; and torch's fp16 matmul alone (the vendor GEMM, no
        # epilogue).  Context only: another library, timed the same way.
        alpha = w.alpha
        with torch.cuda.stream(stream):  # the vendor GEMM sets itself up on first use, outside capture
            for _ in range(3):
                torch.relu(torch.matmul(a, b) * alpha)
        torch.cuda.synchronize()
        gu = capture(lambda: torch.relu(torch.matmul(a, b) * alpha), stream, args.steps)
        tu = min(time_graph(gu, stream, args.steps, 2))
        del gu
        gm = capture(lambda: torch.matmul(a, b), stream, args.steps)
        tm = min(time_graph(gm, stream, args.steps, 2))
        del gm
        torch.cuda.empty_cache()
        context["torch_unfused_tflops"] = round(w.flops / (tu * 1e-3) / 1e12, 3)
        context["torch_matmul_only_tflops"] = round(w.flops / (tm * 1e-3) / 1e12, 3)
        context["speedup_vs_torch_unfused"] = round(tu / ms, 3)
        log(f"[bench] torch unfused {tu * 1e3:.2f} us ({context['torch_unfused_tflops']} TFLOP/s), "
            f"torch matmul only {tm * 1e3:.2f} us ({context['torch_matmul_only_tflops']} TFLOP/s)")
    if args.cold:
        # Before every call: write 512 MiB (evicts A, B and C from L2, 4 MB
        # per XCD, and from the 256 MB last-level cache), then read another
        # 512 MiB one element per 64 bytes (every line is fetched, so the
        # dirty lines of the write are written back now, not during the
        # call).  The call alone is timed with events on the launch stream.
        flush = torch.empty(256 * 1024 * 1024, dtype=torch.float16, device=dev)
        clean = torch.ones(256 * 1024 * 1024, dtype=torch.float16, device=dev)
        sink = torch.empty(clean.numel() // 32, dtype=torch.float16, device=dev)
        cold = []
        with torch.cuda.stream(stream):
            for i in range(max(5, min(args.steps, 30))):
                flush.fill_(float(i))
                sink.copy_(clean.view(-1, 32)[:, 0])
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                step()
                e1.record(stream)
                cold.append((e0, e1))
        torch.cuda.synchronize()
        cold_ms = sorted(e0.elapsed_time(e1) for e0, e1 in cold)[len(cold) // 2]
        # the same single eager calls with the caches left warm (a small
        # kernel instead of the flush before each), so the cold penalty can be
        # told apart from the cost of timing one dispatch on its own
        warm = []
        with torch.cuda.stream(stream):
            for i in range(len(cold)):
                sink[:4096].fill_(float(i))  # a small kernel before the call, as in the cold loop
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                step()
                e1.record(stream)
                warm.append((e0, e1))
        torch.cuda.synchronize()
        warm_ms = sorted(e0.elapsed_time(e1) for e0, e1 in warm)[len(warm) // 2]
        # a reference from the same two states: a device-to-device copy of B
        # (its bytes read once and written once), timed the same way, so the
        # call's cold rate can be set beside what a plain stream of B reaches
        bcopy = torch.empty_like(b)
        ref = {"cold": [], "warm": []}
        with torch.cuda.stream(stream):
            for state in ("cold", "warm"):
                for i in range(len(cold)):
                    if state == "cold":
                        flush.fill_(float(i))
                        sink.copy_(clean.view(-1, 32)[:, 0])
                    else:
                        sink[:4096].fill_(float(i))
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    bcopy.copy_(b)
                    e1.record(stream)
                    ref[state].append((e0, e1))
        torch.cuda.synchronize()
        copy_ms = {k: sorted(e0.elapsed_time(e1) for e0, e1 in v)[len(v) // 2] for k, v in ref.items()}
        del flush, clean, sink, bcopy
        torch.cuda.empty_cache()
        context["cold_us_per_call"] = round(cold_ms * 1e3, 3)
        context["cold_tflops"] = round(w.flops / (cold_ms * 1e-3) / 1e12, 3)
        context["warm_single_call_us"] = round(warm_ms * 1e3, 3)
        if w.flops / w.algorithmic_bytes < PEAK_FP16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
            context["cold_hbm_gbs_algorithmic"] = round(w.algorithmic_bytes / (cold_ms * 1e-3) / 1e9, 1)
        b_bytes = b.numel() * b.element_size()
        context["cold_copy_of_b_us"] = round(copy_ms["cold"] * 1e3, 3)
        context["warm_copy_of_b_us"] = round(copy_ms["warm"] * 1e3, 3)
        context["cold_copy_of_b_gbs_read_plus_write"] = round(2 * b_bytes / (copy_ms["cold"] * 1e-3) / 1e9, 1)
        log(f"[bench] cold caches (median of {len(cold)}): {cold_ms * 1e3:.2f} us/call "
            f"({context['cold_tflops']} TFLOP/s); warm single calls {warm_ms * 1e3:.2f} us/call; "
            f"a copy of B ({b_bytes / 1e6:.1f} MB): {copy_ms['cold'] * 1e3:.2f} us cold, {copy_ms['warm'] * 1e3:.2f} us warm")
    if graph is not None and args.zero_input:
        za = torch.zeros_like(a)
        zb = torch.zeros_like(b)
        zc = torch.empty_like(c)
        gz = capture(lambda: gsr.gemm_scale_bias_act(za, zb, bias, w.alpha, act, c=zc, stream=stream,
                                                     config_id=args.config_id), stream, args.steps)
        zms = min(time_graph(gz, stream, args.steps, 1))
        context["zero_input_tflops"] = round(w.flops / (zms * 1e-3) / 1e12, 3)
        del gz, za, zb, zc
        torch.cuda.empty_cache()
        log(f"[bench] zero inputs {context['zero_input_tflops']} TFLOP/s")

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * 1024 * 1024 // 2
        src = torch.ones(n, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {n * 2} bytes read, {n * 2} bytes written")

    # a call that splits K across workgroups runs another kernel: its own record
    split = bool(ws_bytes)
    roofline = roofline_of(w, ms, load_traffic(w.name + ("_split" if split else ""), w.flops))
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host (cpu_baseline)")
        cpu = cpu_baseline(w, a_cpu, b_cpu, args.cpu_seconds, args.epilogue, bias_cpu)
        log(f"[bench] cpu_baseline {cpu}")

    out = {
        "metric": "TFLOP/s and % of dense fp16 MFMA peak for fused GEMM+scale+ReLU",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 (fp32 accumulate)",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha,
            "inputs": (f"seed 0 randn fp32 -> fp16, A then B, B std {w.b_std:g}" if args.inputs == "normal"
                       else "all zeros (clock study, not the workload's number)"),
            "launch": args.launch,
            "epilogue": args.epilogue,
            "tile": {k: cfg[k] for k in ("id", "block_m", "block_n", "block_k", "waves_m", "waves_n", "group_m",
                                         "xcd_remap")},
            "tuning": os.path.relpath(args.tuning, ROOT) if args.tuning else None,
            "workspace_bytes": ws_bytes,
            "pct_of_peak": round(100 * tflops / PEAK_FP16_TFLOPS, 2),
            "hbm_gbs_algorithmic": round(w.algorithmic_bytes / (ms * 1e-3) / 1e9, 1),
            "device": {"cus": dinfo.get("cus"), "max_clock_mhz": (dinfo["clock_khz"] / 1000.0) if "clock_khz" in dinfo else None,
                       # dense fp16: 4096 FLOP per clock per CU (256 per SIMD lane-op x 16) at the reported clock
                       "peak_tflops_from_device": (round(dinfo["cus"] * 4096 * dinfo["clock_khz"] * 1e3 / 1e12, 1)
                                                   if "cus" in dinfo and "clock_khz" in dinfo else None)},
            "caches": "warm: the timed calls reuse the same A and B, which stay in the 256 MB last-level cache "
                      "when they fit (all workloads but 16384^3)",
            "gpu_over_oracle": (round(tflops / cpu["value"], 1) if cpu else None),
            **context,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
