"""The allocation-free entry point (gemm_scale_bias_act_noalloc) through the
C ABI: its K split runs in the library's per-device scratch array, and its
outputs match those of the entry point with a caller-owned workspace
(gemm_scale_bias_act_ws) bit for bit, and the oracle within the tolerance,
on two calls in a row, the second with a smaller input; a forced split
larger than the array is rejected before anything is enqueued."""
import pytest
import torch

import parity as PT
from tiled_dense_gemm_scale_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def bits(t):
    return W.fp16_bits(t)


def call_ws(native, a, b, c, alpha, ws, stream):
    M, K = a.shape
    N = b.shape[1]
    return native.gemm_scale_bias_act_ws(M, N, K, a.data_ptr(), b.data_ptr(), 0, c.data_ptr(), alpha, 0,
                                         ws.data_ptr(), ws.numel(), stream, -1, 0)


def call_noalloc(native, a, b, c, alpha, stream, config_id=-1, splits=0):
    M, K = a.shape
    N = b.shape[1]
    return native.gemm_scale_bias_act_noalloc(M, N, K, a.data_ptr(), b.data_ptr(), 0, c.data_ptr(), alpha, 0,
                                              stream, config_id, splits)


def test_noalloc_matches_the_workspace_entry_point(native, orc):
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    stream = torch.cuda.current_stream().cuda_stream
    # the first call splits 64 tiles four ways (2 MiB of partial sums), the
    # second, smaller one 32 tiles four ways
    for (M, N, K, alpha) in [(16, 4096, 11008, 1.0), (3, 2048, 4096, 0.5)]:
        need = native.workspace_bytes(M, N, K)
        assert 0 < need <= (4 << 20) + 512
        a, b = W.normal_inputs(M, N, K, seed=M + N, b_std=K ** -0.5 if alpha == 1.0 else 1.0)
        ad, bd = a.to(DEV), b.to(DEV)
        ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
        c_ws = torch.empty((M, N), dtype=torch.float16, device=DEV)
        c_na = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        print(f"[gpu] noalloc {M}x{N}x{K}", flush=True)
        torch.cuda.synchronize()
        assert call_ws(native, ad, bd, c_ws, alpha, ws, stream) == 0
        assert call_noalloc(native, ad, bd, c_na, alpha, stream) == 0
        torch.cuda.synchronize()
        assert torch.equal(c_na.view(torch.int16), c_ws.view(torch.int16)), (M, N, K)
        ref, _ = orc.gemm_scale_relu(bits(a), bits(b), alpha)
        PT.assert_parity(f"noalloc {M}x{N}x{K}", bits(c_na.cpu()), ref)


def test_noalloc_rejects_a_split_beyond_its_scratch(native, orc):
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    stream = torch.cuda.current_stream().cuda_stream
    M, N, K = 1024, 1024, 4096  # 256 tiles of 64 x 64: two parts already need 8 MiB
    a, b = W.normal_inputs(M, N, K, seed=5)
    ad, bd = a.to(DEV), b.to(DEV)
    c = torch.full((M, N), 7.0, dtype=torch.float16, device=DEV)
    torch.cuda.synchronize()
    for parts in (2, 16):
        assert call_noalloc(native, ad, bd, c, 0.5, stream, config_id=21, splits=parts) == 2
    torch.cuda.synchronize()
    assert bool((c == 7.0).all().item())
    # a split that fills the scratch exactly still runs: 64 tiles of 64 x 64
    # in four parts are 4 MiB of partial sums and 256 bytes of counters
    M, N, K = 512, 512, 4096
    a, b = W.normal_inputs(M, N, K, seed=6)
    ad, bd = a.to(DEV), b.to(DEV)
    c = torch.empty((M, N), dtype=torch.float16, device=DEV)
    assert call_noalloc(native, ad, bd, c, 0.5, stream, config_id=21, splits=4) == 0
    torch.cuda.synchronize()
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 0.5)
    PT.assert_parity("noalloc 512^2x4096 four parts", bits(c.cpu()), ref)


def test_noalloc_under_graph_capture(native, orc):
    """The callers it is for include code under HIP graph capture: after one
    call outside capture (which looks the scratch array's address up), a
    captured split call replays with the eager call's bits, eager work in
    between, and a bias + GELU variant too."""
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    M, N, K = 8, 4096, 4096
    a, b = W.normal_inputs(M, N, K, seed=9, b_std=K ** -0.5)
    g = torch.Generator().manual_seed(10)
    bias = torch.randn(N, generator=g).half()
    ad, bd, biasd = a.to(DEV), b.to(DEV), bias.to(DEV)
    assert native.workspace_bytes(M, N, K) > 0
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = {}
    for act in (0, 1):  # ReLU without a bias, GELU with one
        bp = biasd.data_ptr() if act else 0
        eager = torch.empty((M, N), dtype=torch.float16, device=DEV)
        c = torch.empty_like(eager)
        with torch.cuda.stream(s):
            assert native.gemm_scale_bias_act_noalloc(M, N, K, ad.data_ptr(), bd.data_ptr(), bp, eager.data_ptr(),
                                                      1.0, act, s.cuda_stream, -1, 0) == 0
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            assert native.gemm_scale_bias_act_noalloc(M, N, K, ad.data_ptr(), bd.data_ptr(), bp, c.data_ptr(),
                                                      1.0, act, s.cuda_stream, -1, 0) == 0
        print(f"[gpu] noalloc graph replays, activation {act}", flush=True)
        for i in range(4):
            c.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(c.view(torch.int16), eager.view(torch.int16)), (act, i)
            _ = (ad.float() * 2).sum()
            torch.cuda.synchronize()
        outs[act] = eager
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 1.0)
    PT.assert_parity("noalloc relu", bits(outs[0].cpu()), ref)
    ref, _ = orc.gemm_bias_act(bits(a), bits(b), bits(bias), 1.0, 1)
    PT.assert_parity("noalloc bias+gelu", bits(outs[1].cpu()), ref)
