"""GPU parity of the epilogue variants C = act(alpha * A @ B + bias[n]) (the
aikraft.ru TileLang guide, section 4, GEMM + Bias + GELU) against the oracle:
every tile configuration on ragged shapes, the LLM-MLP shape with bias and
GELU at full size (sampled), bit-exact integer cases for ReLU and the
identity, K = 0, an unaligned bias, and the plain entry point as the special
case bias = None, act = ReLU."""
import numpy as np
import pytest
import torch

import parity as PT
from tiled_dense_gemm_scale_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ACT = {"relu": 0, "gelu": 1, "none": 2}


@pytest.fixture(scope="module")
def gsr(native):
    import tiled_dense_gemm_scale_amd as g

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return g


def bits(t):
    return W.fp16_bits(t)


def say(msg):
    print(msg, flush=True)


def oracle_full(orc, a, b, bias, alpha, act):
    ref, _ = orc.gemm_bias_act(bits(a), bits(b), bits(bias) if bias is not None else None, alpha, ACT[act])
    return ref


SHAPES = [(17, 33, 65), (300, 520, 200), (257, 263, 129), (129, 1031, 72), (1000, 1500, 704)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("act", ["relu", "gelu", "none"])
def test_variant_selector(gsr, orc, shape, act):
    M, N, K = shape
    a, b = W.normal_inputs(M, N, K, seed=M + 2 * N + 3 * K)
    bias = W.bias_input(N, seed=M)
    for alpha, bb in ((1.0, bias), (0.5, bias), (0.5, None)):
        say(f"[gpu] variant {shape} act={act} alpha={alpha} bias={'yes' if bb is not None else 'no'} selector")
        got = PT.run_gpu_variant(a, b, bb, alpha, act)
        PT.assert_parity(f"{shape} {act} alpha={alpha} bias={bb is not None}", got,
                         oracle_full(orc, a, b, bb, alpha, act))


@pytest.mark.parametrize("shape", [(300, 520, 200), (257, 263, 129)], ids=lambda s: "x".join(map(str, s)))
def test_variant_every_config(gsr, orc, shape):
    M, N, K = shape
    a, b = W.normal_inputs(M, N, K, seed=7 * M + N)
    bias = W.bias_input(N, seed=N)
    refs = {act: oracle_full(orc, a, b, bias, 1.0, act) for act in ("gelu", "none")}
    for cid in gsr.config_ids():
        for act in ("gelu", "none"):
            say(f"[gpu] variant {shape} act={act} config {cid}")
            got = PT.run_gpu_variant(a, b, bias, 1.0, act, config_id=cid)
            PT.assert_parity(f"{shape} {act} cfg{cid}", got, refs[act])


@pytest.mark.parametrize("shape", [(256, 256, 256), (300, 520, 200), (257, 263, 129), (4097, 384, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_variant_integer_bitwise(gsr, orc, shape):
    """Integer inputs and bias: the fp32 value alpha*s + b is exact, so ReLU
    and the identity match the oracle bit for bit on every configuration."""
    M, N, K = shape
    a, b = W.integer_inputs(M, N, K, seed=9)
    bias = W.bias_input(N, seed=9, integer=True)
    for act in ("relu", "none"):
        for alpha in (0.5, -1.0):
            ref = oracle_full(orc, a, b, bias, alpha, act)
            for cid in [-1] + gsr.config_ids():
                say(f"[gpu] variant integer {shape} act={act} alpha={alpha} config {cid}")
                got = PT.run_gpu_variant(a, b, bias, alpha, act, config_id=cid)
                PT.assert_bitwise(f"integer {shape} {act} alpha={alpha} cfg{cid}", got, ref)


def test_variant_llm_bias_gelu(gsr, orc):
    """The guide's GEMM + Bias + GELU at the LLM-MLP shape (alpha = 1), in
    the selector's configuration: every output, and whole-output properties."""
    w = W.WORKLOADS["llm_mlp_4097x11008x4096"]
    a, b = W.workload_inputs(w)
    bias = W.bias_input(w.N)
    say("[gpu] variant llm bias+gelu, every output")
    got = PT.run_gpu_variant(a, b, bias, 1.0, "gelu")
    PT.assert_parity("llm bias+gelu", got, oracle_full(orc, a, b, bias, 1.0, "gelu"))
    v = PT.f16(got)
    assert np.all(np.isfinite(v))
    # GELU's minimum is about -0.17: nothing below it, and a good share negative
    assert v.min() >= -0.1701
    assert 0.2 < float(np.mean(v < 0)) < 0.6


def test_variant_skinny_bias_gelu(gsr, orc):
    w = W.SKINNY
    a, b = W.workload_inputs(w)
    bias = W.bias_input(w.N)
    say("[gpu] variant skinny bias+gelu, full")
    got = PT.run_gpu_variant(a, b, bias, 1.0, "gelu")
    PT.assert_parity("skinny bias+gelu", got, oracle_full(orc, a, b, bias, 1.0, "gelu"))


def test_variant_square_4096_identity_sampled(gsr, orc):
    w = W.WORKLOADS["square_4096"]
    a, b = W.workload_inputs(w)
    bias = W.bias_input(w.N, std=8.0)
    say("[gpu] variant 4096^3 bias+identity, sampled")
    got = PT.run_gpu_variant(a, b, bias, w.alpha, "none")
    ms, ns = W.sample_points(w.M, w.N, 4096, seed=1)
    ref, _ = orc.gemm_bias_act_points(bits(a), bits(b), bits(bias), w.alpha, ACT["none"], ms, ns)
    PT.assert_parity("4096 bias+identity (sampled)", got[ms, ns], ref, coords=(ms, ns))


@pytest.mark.parametrize("act", ["relu", "gelu", "none"])
def test_variant_k_zero(gsr, orc, act):
    M, N = 37, 45
    bias = W.bias_input(N, seed=3)
    a = torch.empty((M, 0), dtype=torch.float16)
    b = torch.empty((0, N), dtype=torch.float16)
    say(f"[gpu] variant K=0 act={act}")
    for bb in (bias, None):
        c = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        got = PT.run_gpu_variant(a, b, bb, 0.5, act, c=c)
        PT.assert_parity(f"K=0 {act} bias={bb is not None}", got, oracle_full(orc, a, b, bb, 0.5, act))
        if bb is None:
            assert np.all(got == 0), "K=0 without a bias must give +0"


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_variant_unaligned_bias(gsr, orc, offset):
    """A bias at a 2-byte but not 8-byte aligned address takes the
    element-wise path and gives the same results."""
    M, N, K = 130, 136, 72
    a, b = W.normal_inputs(M, N, K, seed=offset)
    bias = W.bias_input(N, seed=offset)
    buf = torch.zeros(N + 8, dtype=torch.float16, device=DEV)
    bd = buf[offset:offset + N]
    bd.copy_(bias.to(DEV))
    say(f"[gpu] variant unaligned bias +{offset}")
    out = gsr.gemm_scale_bias_act(a.to(DEV), b.to(DEV), bd, 1.0, "gelu")
    torch.cuda.synchronize()
    PT.assert_parity(f"unaligned bias +{offset}", bits(out.cpu()), oracle_full(orc, a, b, bias, 1.0, "gelu"))


@pytest.mark.parametrize("cid", [-1, 28, 31, 32, 16, 22, 21])
def test_variant_plain_case_is_the_operation(gsr, cid):
    """bias = None with ReLU is gemm_scale_relu itself (same kernel, same bits)."""
    M, N, K = 520, 300, 264
    a, b = W.normal_inputs(M, N, K, seed=21)
    ad, bd = a.to(DEV), b.to(DEV)
    say(f"[gpu] variant plain == scale_relu config {cid}")
    c1 = gsr.gemm_scale_bias_act(ad, bd, None, 0.5, "relu", config_id=cid)
    c2 = gsr.gemm_scale_relu_ex(ad, bd, 0.5, cid)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_variant_zero_bias_matches_no_bias(gsr):
    M, N, K = 256, 264, 128
    a, b = W.normal_inputs(M, N, K, seed=4)
    ad, bd = a.to(DEV), b.to(DEV)
    z = torch.zeros(N, dtype=torch.float16, device=DEV)
    say("[gpu] variant zero bias")
    for act in ("relu", "gelu", "none"):
        c1 = gsr.gemm_scale_bias_act(ad, bd, z, 0.5, act)
        c2 = gsr.gemm_scale_bias_act(ad, bd, None, 0.5, act)
        torch.cuda.synchronize()
        v1, v2 = c1.float(), c2.float()
        assert torch.equal(v1, v2), act
