"""GPU parity of the entry points with a workspace, which split K across
workgroups (configurations 21 and 22): the split sums against the oracle,
integer inputs bit for bit for every part count, the epilogue variants,
the workspace's arrival counters back at zero after every call, a workspace
too small for the split, graph replays and concurrent streams."""
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


def bits(t):
    return W.fp16_bits(t)


def say(msg):
    print(msg, flush=True)


def counters_zero(ws, tiles):
    torch.cuda.synchronize()
    return bool((ws[:4 * tiles] == 0).all().item())


def tiles_of(gsr, M, N, cid):
    c = gsr.get_config(cid)
    return -(-M // c["block_m"]) * -(-N // c["block_n"])


# Shapes the library splits (gsr_workspace_bytes > 0): decode rows against
# 4096-wide weights, K = 4096 and 11008, one and two tile rows, a ragged N
# against the 64-wide tile and a K that ends inside the last part's step.
SPLIT_SHAPES = [(1, 4096, 4096), (16, 4096, 11008), (40, 2048, 4096), (5, 1000, 4104), (64, 4096, 4096),
                (3, 512, 8192)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_library_split_every_output(gsr, orc, shape):
    M, N, K = shape
    need = gsr.workspace_bytes(M, N, K)
    assert need > 0, f"{shape}: the library no longer splits this shape"
    alpha = 1.0 if K == 11008 else 0.5
    a, b = W.normal_inputs(M, N, K, seed=M + N + K, b_std=K ** -0.5 if alpha == 1.0 else 1.0)
    ws = gsr.new_workspace(need)
    say(f"[gpu] split {shape}: library choice, workspace {need} bytes")
    c = gsr.gemm_scale_relu_ws(a.to(DEV), b.to(DEV), alpha, ws)
    torch.cuda.synchronize()
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), alpha)
    PT.assert_parity(f"split {shape}", bits(c.cpu()), ref)
    cid = gsr.select_config(M, N, K)["id"]
    assert counters_zero(ws, tiles_of(gsr, M, N, cid))


# Every part count on integer inputs, whose fp32 sums are exact: bit for bit
# with the oracle, for both K-split tiles.  K of 2000 is 16 steps of 128
# (parts of 1-16 steps, uneven ones included), 4100 ends inside the 33rd step,
# 128 is a single step (any part count collapses to one part).
@pytest.mark.parametrize("shape", [(33, 520, 2000), (1, 4096, 4100), (7, 64, 128), (96, 192, 1536)],
                         ids=lambda s: "x".join(map(str, s)))
def test_forced_parts_integer_bitwise(gsr, orc, shape):
    M, N, K = shape
    a, b = W.integer_inputs(M, N, K, seed=21)
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 0.5)
    ad, bd = a.to(DEV), b.to(DEV)
    ws = gsr.new_workspace(16 << 20)
    for cid in (22, 21):
        for parts in (1, 2, 3, 4, 5, 7, 8, 16):
            say(f"[gpu] split {shape} config {cid} parts {parts} integer")
            c = gsr.gemm_scale_bias_act_ws(ad, bd, ws, alpha=0.5, config_id=cid, splits=parts)
            torch.cuda.synchronize()
            PT.assert_bitwise(f"split {shape} cfg{cid} parts{parts}", bits(c.cpu()), ref)
            assert counters_zero(ws, tiles_of(gsr, M, N, cid)), (cid, parts)


@pytest.mark.parametrize("act", ["relu", "gelu", "none"])
def test_split_epilogue_variants(gsr, orc, act):
    M, N, K = 9, 1024, 4096
    a, b = W.normal_inputs(M, N, K, seed=31, b_std=K ** -0.5)
    g = torch.Generator().manual_seed(32)
    bias = torch.randn(N, generator=g).half()
    ws = gsr.new_workspace(8 << 20)
    say(f"[gpu] split epilogue {act}")
    for parts in (0, 3, 4):
        c = gsr.gemm_scale_bias_act_ws(a.to(DEV), b.to(DEV), ws, bias=bias.to(DEV), alpha=1.0, activation=act,
                                       splits=parts)
        torch.cuda.synchronize()
        ref, _ = orc.gemm_bias_act(bits(a), bits(b), bits(bias), 1.0, gsr.ACTIVATIONS[act])
        PT.assert_parity(f"split {act} parts {parts}", bits(c.cpu()), ref)


def test_split_repeats_and_workspace_reuse(gsr):
    """The kernels leave the counters at zero, so one workspace serves
    consecutive calls of different shapes in stream order; repeated calls
    give the same bits."""
    ws = gsr.new_workspace(8 << 20)
    runs = []
    for (M, N, K) in [(1, 4096, 4096), (16, 2048, 11008), (1, 4096, 4096)]:
        assert gsr.workspace_bytes(M, N, K) > 0
        a, b = W.normal_inputs(M, N, K, seed=41)
        ad, bd = a.to(DEV), b.to(DEV)
        say(f"[gpu] split reuse {M}x{N}x{K}")
        first = gsr.gemm_scale_relu_ws(ad, bd, 0.5, ws).clone()
        for _ in range(5):
            again = gsr.gemm_scale_relu_ws(ad, bd, 0.5, ws)
            assert torch.equal(first.view(torch.int16), again.view(torch.int16))
        assert counters_zero(ws, tiles_of(gsr, M, N, gsr.select_config(M, N, K)["id"]))
        runs.append(first)
    assert torch.equal(runs[0].view(torch.int16), runs[2].view(torch.int16))


def test_small_workspace(gsr, orc):
    """The library's choice takes fewer parts (or none) when the workspace is
    smaller than its split needs; a forced split that does not fit is an
    error, and nothing is launched."""
    M, N, K = 4, 4096, 4096
    need = gsr.workspace_bytes(M, N, K)
    assert need > 0
    a, b = W.normal_inputs(M, N, K, seed=51)
    ad, bd = a.to(DEV), b.to(DEV)
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 0.5)
    for nbytes in (need - 1, need // 2, 300, 16):
        ws = gsr.new_workspace(nbytes)
        say(f"[gpu] split with a {nbytes}-byte workspace")
        c = gsr.gemm_scale_relu_ws(ad, bd, 0.5, ws)
        torch.cuda.synchronize()
        PT.assert_parity(f"workspace {nbytes}", bits(c.cpu()), ref)
    ws = gsr.new_workspace(need // 2)
    c = torch.full((M, N), 7.0, dtype=torch.float16, device=DEV)
    with pytest.raises(gsr.GsrError) as e:
        gsr.gemm_scale_bias_act_ws(ad, bd, ws, alpha=0.5, c=c, config_id=22, splits=4)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert bool((c == 7.0).all().item())
    with pytest.raises(gsr.GsrError) as e:  # a tile configuration that cannot split
        gsr.gemm_scale_bias_act_ws(ad, bd, ws, alpha=0.5, config_id=28, splits=2)
    assert e.value.status == 6


def test_element_path_ignores_the_workspace(gsr, orc):
    """N not a multiple of 8 takes the element-wise kernel, which does not
    split: the result is right and the workspace untouched."""
    M, N, K = 3, 1001, 4096
    a, b = W.normal_inputs(M, N, K, seed=61)
    ws = gsr.new_workspace(8 << 20)
    say("[gpu] split request on the element path")
    c = gsr.gemm_scale_bias_act_ws(a.to(DEV), b.to(DEV), ws, alpha=0.5, config_id=22, splits=4)
    torch.cuda.synchronize()
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 0.5)
    PT.assert_parity("element path with workspace", bits(c.cpu()), ref)
    assert bool((ws == 0).all().item())


def test_split_graph_replays(gsr):
    """A split call captured in a HIP graph: every replay, with eager work in
    between, matches the eager result, and the counters stay at zero."""
    M, N, K = 8, 4096, 4096
    a, b = W.normal_inputs(M, N, K, seed=71)
    ad, bd = a.to(DEV), b.to(DEV)
    ws = gsr.new_workspace(gsr.workspace_bytes(M, N, K))
    say("[gpu] split graph capture")
    eager = gsr.gemm_scale_relu_ws(ad, bd, 0.5, ws).clone()
    torch.cuda.synchronize()
    c = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gsr.gemm_scale_relu_ws(ad, bd, 0.5, ws, c=c)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        gsr.gemm_scale_relu_ws(ad, bd, 0.5, ws, c=c)
    for i in range(4):
        c.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        assert counters_zero(ws, 64)
        _ = (ad.float() * 2).sum()
        torch.cuda.synchronize()


def test_split_on_two_streams(gsr, orc):
    """Calls that may overlap use workspaces of their own."""
    shapes = [(1, 4096, 4096), (12, 2048, 8192)]
    ins = [W.normal_inputs(M, N, K, seed=81 + i) for i, (M, N, K) in enumerate(shapes)]
    refs = [orc.gemm_scale_relu(bits(a), bits(b), 0.5)[0] for a, b in ins]
    dev_in = [(a.to(DEV), b.to(DEV)) for a, b in ins]
    wss = [gsr.new_workspace(gsr.workspace_bytes(*s)) for s in shapes]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    say("[gpu] split on two streams")
    outs = [None, None]
    for rep in range(10):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                outs[i] = gsr.gemm_scale_relu_ws(*dev_in[i], 0.5, wss[i])
        torch.cuda.synchronize()
        for i in range(2):
            PT.assert_parity(f"stream {i} rep {rep}", bits(outs[i].cpu()), refs[i])


def _random_split_cases(n=12, seed=2024):
    """Seeded ragged shapes on the 128-bit path (N and K multiples of 8) with a
    random part count and K-split tile."""
    import random
    rng = random.Random(seed)
    cases = []
    for _ in range(n):
        M = rng.randint(1, 100)
        N = 8 * rng.randint(1, 150)
        K = 8 * rng.randint(1, 400)
        cases.append((M, N, K, rng.choice((21, 22)), rng.randint(2, 16)))
    return cases


@pytest.mark.parametrize("case", _random_split_cases(), ids=lambda c: "x".join(map(str, c[:3])) + f"-c{c[3]}-p{c[4]}")
def test_random_shapes_forced_parts_bitwise(gsr, orc, case):
    """Integer inputs (exact fp32 sums): the split call gives the oracle's bits
    on seeded ragged shapes, whatever the part count (1 part when K has fewer
    K-steps than parts asked for collapses them)."""
    M, N, K, cid, parts = case
    a, b = W.integer_inputs(M, N, K, seed=M + N + K)
    alpha = -0.5 if parts % 3 == 0 else 0.5
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), alpha)
    ws = gsr.new_workspace(16 << 20)
    say(f"[gpu] split random {case}")
    c = gsr.gemm_scale_bias_act_ws(a.to(DEV), b.to(DEV), ws, alpha=alpha, config_id=cid, splits=parts)
    torch.cuda.synchronize()
    PT.assert_bitwise(f"split random {case}", bits(c.cpu()), ref)
    assert counters_zero(ws, tiles_of(gsr, M, N, cid))


@pytest.mark.parametrize("c_off", [1, 2, 4], ids=lambda o: f"c+{2 * o}B")
def test_split_with_a_less_aligned_c(gsr, orc, c_off):
    """C at a 2-, 4- or 8-byte offset keeps the split on the 128-bit path and
    is written in stores of the size its alignment allows."""
    M, N, K = 5, 2048, 4096
    assert gsr.workspace_bytes(M, N, K) > 0
    a, b = W.integer_inputs(M, N, K, seed=91)
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 0.5)
    buf = torch.full((M * N + 16,), 3.0, dtype=torch.float16, device=DEV)
    c = buf[c_off:c_off + M * N].view(M, N)
    ws = gsr.new_workspace(gsr.workspace_bytes(M, N, K))
    say(f"[gpu] split with C at +{2 * c_off} bytes")
    gsr.gemm_scale_relu_ws(a.to(DEV), b.to(DEV), 0.5, ws, c=c)
    torch.cuda.synchronize()
    PT.assert_bitwise(f"split C+{2 * c_off}B", bits(c.cpu()), ref)
    host = buf.cpu()
    assert bool((host[:c_off] == 3.0).all()) and bool((host[c_off + M * N:] == 3.0).all()), "guard values written"
