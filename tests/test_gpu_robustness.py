"""GPU robustness: the largest problems the 32-bit byte offsets allow (on the
128-bit and the element-wise path), concurrent calls from several host
threads on their own streams while the tuning table changes, graph
capture of the epilogue variants replayed against eager results, and a good
launch while an unrelated HIP error is pending on the thread."""
import threading

import numpy as np
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
    return g


@pytest.mark.parametrize("K", [32760, 32767], ids=["vec-path", "element-path"])
def test_largest_operand_under_2gib(gsr, orc, K):
    """A is M*K*2 bytes just under 2^31 (the documented limit): every offset
    near the top of the 32-bit range is exercised.  Integer inputs, so the
    sampled outputs, the last row and the last column match bit for bit."""
    M, N = 32768, 72
    assert M * K * 2 < 2 ** 31
    print(f"[gpu] largest A {M}x{K} ({M * K * 2} bytes), N={N}", flush=True)
    a, b = W.pattern_inputs(M, N, K, device=DEV)
    c = gsr.gemm_scale_relu(a, b, 0.5)
    torch.cuda.synchronize()
    ms, ns = W.sample_points(M, N, 2048, seed=1, extra_rows=[M - 1])
    ms = np.concatenate([ms, np.arange(M, dtype=np.int64)[::97], np.full(M // 97 + 1, 0, np.int64)])
    ns = np.concatenate([ns, np.full(len(range(0, M, 97)), N - 1, np.int64), np.arange(0, M, 97) % N])
    a_bits = W.fp16_bits(a.cpu())
    b_bits = W.fp16_bits(b.cpu())
    ref, _ = orc.gemm_scale_relu_points(a_bits, b_bits, 0.5, ms, ns)
    got = W.fp16_bits(c.cpu())
    PT.assert_bitwise(f"largest K={K}", got[ms, ns], ref)
    del a, b, c
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cid", [25, 28, 29, 31, 32])
def test_largest_operand_under_2gib_interleaved(gsr, orc, cid):
    """The same A just under 2^31 bytes through each interleaved 256x256 and
    128x256 kernel, forced: their per-lane copy offsets are formed from base
    registers plus strides of 32 and 64 rows, so the top of the 32-bit range
    is where a wrong stride or a wrap would show."""
    M, N, K = 32768, 72, 32760
    assert M * K * 2 < 2 ** 31
    print(f"[gpu] largest A {M}x{K}, N={N}, config {cid}", flush=True)
    a, b = W.pattern_inputs(M, N, K, device=DEV)
    c = gsr.gemm_scale_relu_ex(a, b, 0.5, cid)
    torch.cuda.synchronize()
    ms, ns = W.sample_points(M, N, 2048, seed=2, extra_rows=[M - 1])
    ms = np.concatenate([ms, np.arange(M, dtype=np.int64)[::61]])
    ns = np.concatenate([ns, np.arange(0, M, 61) % N])
    ref, _ = orc.gemm_scale_relu_points(W.fp16_bits(a.cpu()), W.fp16_bits(b.cpu()), 0.5, ms, ns)
    got = W.fp16_bits(c.cpu())
    PT.assert_bitwise(f"largest cfg{cid}", got[ms, ns], ref)
    del a, b, c
    torch.cuda.empty_cache()


def test_concurrent_host_threads(gsr, tmp_path):
    """Eight host threads, each on its own stream, call the library with
    different shapes, configurations and epilogues while a ninth thread keeps
    loading and clearing a tuning table; every result equals the
    single-threaded one bit for bit (launch order never changes a result)."""
    shapes = [(300, 520, 200), (257, 263, 129), (1024, 1024, 256), (64, 4096, 512),
              (513, 384, 1000), (17, 33, 65), (2048, 256, 64), (130, 136, 72)]
    inputs = []
    for i, (M, N, K) in enumerate(shapes):
        a, b = W.normal_inputs(M, N, K, seed=40 + i)
        bias = W.bias_input(N, seed=40 + i)
        inputs.append((a.to(DEV), b.to(DEV), bias.to(DEV)))
    acts = ["relu", "gelu", "none"]
    want = []
    for i, (a, b, bias) in enumerate(inputs):
        want.append(gsr.gemm_scale_bias_act(a, b, bias if i % 2 else None, 0.5, acts[i % 3]).clone())
    torch.cuda.synchronize()
    table = tmp_path / "t.txt"
    table.write_text("".join(f"{M} {N} {K} 21 2 0\n" for (M, N, K) in shapes[:2]))
    errors = []
    stop = threading.Event()

    def tuner():
        while not stop.is_set():
            try:
                gsr.load_tuning(str(table))
                gsr.clear_tuning()
            except Exception as e:  # pragma: no cover - reported below
                errors.append(repr(e))

    def worker(i):
        try:
            a, b, bias = inputs[i]
            s = torch.cuda.Stream(DEV)
            outs = []
            with torch.cuda.stream(s):
                for _ in range(20):
                    outs.append(gsr.gemm_scale_bias_act(a, b, bias if i % 2 else None, 0.5, acts[i % 3],
                                                        stream=s))
            s.synchronize()
            for o in outs:
                # the tuning table may or may not be in force for shapes 0 and
                # 1: a different tile sums in a different order, so compare by
                # value there and bit for bit elsewhere
                if i < 2:
                    PT.assert_parity(f"thread {i}", W.fp16_bits(o.cpu()), W.fp16_bits(want[i].cpu()))
                elif not torch.equal(o.view(torch.int16), want[i].view(torch.int16)):
                    errors.append(f"thread {i}: result differs")
        except Exception as e:
            errors.append(f"thread {i}: {e!r}")

    print("[gpu] 8 threads x 20 calls with a tuning thread", flush=True)
    tt = threading.Thread(target=tuner)
    tt.start()
    ths = [threading.Thread(target=worker, args=(i,)) for i in range(len(shapes))]
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    stop.set()
    tt.join()
    gsr.clear_tuning()
    assert not errors, errors[:5]


@pytest.mark.parametrize("act,with_bias", [("gelu", True), ("none", True), ("relu", False)])
def test_graph_capture_of_variants(gsr, act, with_bias):
    """Capture several calls of a variant, replay the graph repeatedly with
    eager work and synchronisations in between, check every replay."""
    M, N, K = 520, 1100, 264
    a, b = W.normal_inputs(M, N, K, seed=77)
    bias = W.bias_input(N, seed=77).to(DEV) if with_bias else None
    ad, bd = a.to(DEV), b.to(DEV)
    want = gsr.gemm_scale_bias_act(ad, bd, bias, 1.0, act).clone()
    outs = [torch.empty((M, N), dtype=torch.float16, device=DEV) for _ in range(3)]
    s = torch.cuda.Stream(DEV)
    with torch.cuda.stream(s):
        gsr.gemm_scale_bias_act(ad, bd, bias, 1.0, act, c=outs[0], stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for o in outs:
            gsr.gemm_scale_bias_act(ad, bd, bias, 1.0, act, c=o, stream=s)
    print(f"[gpu] graph replays of {act} bias={with_bias}", flush=True)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o in outs:
            assert torch.equal(o.view(torch.int16), want.view(torch.int16)), f"replay {rep}"
        gsr.gemm_scale_relu(ad, bd, 0.5)  # eager work between replays
        torch.cuda.synchronize()


def test_pending_unrelated_hip_error_is_not_taken_for_a_launch_error(gsr, orc):
    """A HIP error that an earlier call left pending on the thread (here a
    failed hipSetDevice, a host-side check that touches no device) must not
    turn a good launch into GSR_ERROR_LAUNCH, on the tile path nor on the
    K = 0 fill; the caller's pending error is left for the caller."""
    import ctypes
    import os

    from tiled_dense_gemm_scale_amd import _native as nat

    # the HIP runtime torch and the library already share: reopen that very
    # file (dlopen returns the loaded copy), never load a second runtime
    nat.lib()
    loaded = sorted({ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln.split()[-1]})
    assert len(loaded) == 1, loaded
    hip = ctypes.CDLL(loaded[0], mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    M, N, K = 200, 136, 72
    a, b = W.integer_inputs(M, N, K, seed=3)
    ref, _ = orc.gemm_scale_relu(W.fp16_bits(a), W.fp16_bits(b), 0.5)
    ad, bd = a.to(DEV), b.to(DEV)
    c = torch.full((M, N), 7.0, dtype=torch.float16, device=DEV)
    c0 = torch.full((M, N), 7.0, dtype=torch.float16, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    print("[gpu] launch with an unrelated HIP error pending", flush=True)
    bad = hip.hipSetDevice(1 << 20)
    try:
        assert bad != 0 and hip.hipPeekAtLastError() == bad
        st = nat.gemm_scale_relu(M, N, K, ad.data_ptr(), bd.data_ptr(), c.data_ptr(), 0.5, stream)
        st0 = nat.gemm_scale_relu(M, N, 0, ad.data_ptr(), bd.data_ptr(), c0.data_ptr(), 0.5, stream)
    finally:
        hip.hipGetLastError()  # clear it before torch launches anything
    assert (st, st0) == (0, 0), (st, st0)
    torch.cuda.synchronize()
    PT.assert_bitwise("pending-error launch", W.fp16_bits(c.cpu()), ref)
    assert not torch.any(c0.view(torch.int16) != 0)
