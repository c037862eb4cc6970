"""GPU parity: the HIP path (through the C ABI) against the oracle.

Every workload up to the LLM-MLP shape (4097 x 11008 x 4096) is checked on
every output, in the launch configuration the benchmark times (the
selector's choice), with seeded N(0,1) inputs against the tolerance and with
integer inputs bit for bit; 16384^3, whose full oracle pass would take
minutes, on 4096 sampled outputs and on properties that hold at any size.
Small and ragged shapes are checked on every output for every tile
configuration.  Integer-valued inputs make the fp32 sums exact, so there
the comparison is bit for bit.
"""
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


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["square_256", "square_1024", "square_4096", "llm_mlp_4097x11008x4096"])
def test_workload_full(gsr, orc, name):
    w = W.WORKLOADS[name]
    a, b = W.workload_inputs(w)
    say(f"[gpu] {name} {w.M}x{w.N}x{w.K} alpha={w.alpha} selector")
    got = PT.run_gpu(a, b, w.alpha)
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), w.alpha)
    PT.assert_parity(name, got, ref)


def test_skinny_full(gsr, orc):
    """The HBM-bound skinny class (16 x 11008 x 4096, B ~ N(0, 1/K)), every
    output, in the selector's launch."""
    w = W.SKINNY
    a, b = W.workload_inputs(w)
    say(f"[gpu] {w.name} {w.M}x{w.N}x{w.K} alpha={w.alpha} selector")
    got = PT.run_gpu(a, b, w.alpha)
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), w.alpha)
    PT.assert_parity(w.name, got, ref)


def test_column_shard_full(gsr, orc):
    """One GPU's column shard of the LLM-MLP layer under 8-way column
    parallelism (4097 x 1376 x 4096, ragged M and N against 256-wide tiles),
    every output, in the selector's launch."""
    w = W.COLSHARD8
    a, b = W.workload_inputs(w)
    say(f"[gpu] {w.name} {w.M}x{w.N}x{w.K} alpha={w.alpha} selector")
    got = PT.run_gpu(a, b, w.alpha)
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), w.alpha)
    PT.assert_parity(w.name, got, ref)


def test_mid_size_full(gsr, orc):
    """A 1024-row batch against 4096 x 4096 weights (the 128 x 128 tile's
    class), every output, in the selector's launch."""
    w = W.MID
    a, b = W.workload_inputs(w)
    say(f"[gpu] {w.name} {w.M}x{w.N}x{w.K} alpha={w.alpha} selector")
    got = PT.run_gpu(a, b, w.alpha)
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), w.alpha)
    PT.assert_parity(w.name, got, ref)


@pytest.mark.parametrize("name", ["square_16384"])
def test_workload_sampled(gsr, orc, name):
    w = W.WORKLOADS[name]
    a, b = W.workload_inputs(w)
    say(f"[gpu] {name} {w.M}x{w.N}x{w.K} alpha={w.alpha} selector, sampled")
    got = PT.run_gpu(a, b, w.alpha)
    extra = [w.M - 1] if w.M % 256 else []
    ms, ns = W.sample_points(w.M, w.N, 4096, seed=1, extra_rows=extra)
    ref, _ = orc.gemm_scale_relu_points(bits(a), bits(b), w.alpha, ms, ns)
    PT.assert_parity(name + " (sampled)", got[ms, ns], ref, coords=(ms, ns))
    # properties of the whole output: finite, non-negative, about half zeros
    v = PT.f16(got)
    assert np.all(np.isfinite(v))
    assert not np.any(got & 0x8000), "negative or -0 output"
    assert np.all(v >= 0)
    zf = float(np.mean(got == 0))
    assert 0.45 < zf < 0.55, zf


def test_square_16384_every_output_periodic_inputs(gsr, orc):
    """16384^3 in the selector's launch (the benchmark's), every output bit
    for bit.  With the periodic integer inputs A[m,k] = ((7m + 13k) mod 9) - 4
    and B[k,n] = ((5k + 11n) mod 7) - 3, row m of A depends only on m mod 9
    and column n of B only on n mod 7, so C[m,n] is one of 63 values, chosen
    by (m mod 9, n mod 7); the oracle computes those 63 (every fp32 partial
    sum is an exact integer), and each of the 2^28 outputs must equal its
    class's value.  alpha = 0.5 and -0.5, so the classes with negative sums
    are seen too."""
    w = W.WORKLOADS["square_16384"]
    M, N, K = w.M, w.N, w.K
    a, b = W.pattern_inputs(M, N, K, device=DEV)
    a9 = bits(a[:9].cpu())
    b7 = bits(b[:, :7].contiguous().cpu())
    ms = np.repeat(np.arange(9, dtype=np.int64), 7)
    ns = np.tile(np.arange(7, dtype=np.int64), 9)
    ncls = torch.arange(N, device=DEV) % 7
    for alpha in (0.5, -0.5):
        say(f"[gpu] square_16384 periodic integer inputs, alpha={alpha}, selector, every output")
        c = gsr.gemm_scale_relu(a, b, alpha)
        torch.cuda.synchronize()
        ref, _ = orc.gemm_scale_relu_points(a9, b7, alpha, ms, ns)
        assert len(set(int(v) for v in ref)) >= 5, "the classes should differ"
        table = torch.from_numpy(np.asarray(ref, dtype=np.uint16).reshape(9, 7).view(np.int16).copy()).to(DEV)
        got = c.view(torch.int16)
        for r0 in range(0, M, 1024):
            rows = torch.arange(r0, min(M, r0 + 1024), device=DEV) % 9
            bad = got[r0:r0 + rows.numel()] != table[rows][:, ncls]
            if bool(bad.any()):
                i, j = (int(x) for x in torch.nonzero(bad)[0])
                i += r0
                raise AssertionError(f"16384^3 periodic, alpha={alpha}: output ({i},{j}) is "
                                     f"0x{int(got[i, j]) & 0xffff:04x}, its class ({i % 9},{j % 7}) gives "
                                     f"0x{int(table[i % 9, j % 7]) & 0xffff:04x}")
        del c, got
    del a, b
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# every tile configuration, several tiles and ragged tails
# --------------------------------------------------------------------------

RAGGED = [
    (1, 1, 1),
    (17, 33, 65),
    (64, 64, 64),
    (300, 520, 200),      # K multiple of 8, not of 64; 128-bit path
    (257, 263, 129),      # N, K odd: element path
    (513, 384, 1000),
    (129, 1031, 72),      # N % 8 != 0: element path
    (1000, 1500, 704),
    (200, 262, 130),      # rows of 2N, 2K = 4 mod 8 bytes: element path, 4-byte loads
    (96, 300, 100),       # rows of 2N, 2K = 8 mod 16 bytes: element path, 8-byte loads
]


def _configs(gsr):
    return gsr.config_ids()


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_ragged_every_config(gsr, orc, shape):
    M, N, K = shape
    a, b = W.normal_inputs(M, N, K, seed=M * 7 + N * 3 + K)
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 0.5)
    for cid in [-1] + _configs(gsr):
        say(f"[gpu] ragged {shape} config {cid}")
        got = PT.run_gpu(a, b, 0.5, config_id=cid)
        PT.assert_parity(f"{shape} cfg{cid}", got, ref)


# K-split tiles with separate copy waves against the four-wave K-split kernel
# of the same tile: same K split, same summation order, so the same bits.
# K covers 1, 2, 3, 4, 8, 9 and 32 steps of 128; M and N ragged against the
# tile (M of 1, 5, 16, 33 and 40 against 32- and 64-row tiles).
COPY_WAVE_TWINS = [(21, 16), (22, 18)]


@pytest.mark.parametrize("shape", [(64, 64, 8), (100, 72, 136), (1024, 1024, 264), (33, 200, 392),
                                   (520, 1000, 1032), (16, 11008, 4096), (1, 4096, 1000), (5, 300, 777),
                                   (40, 520, 2000)], ids=lambda s: "x".join(map(str, s)))
def test_copy_wave_ksplit_matches_its_twin(gsr, orc, shape):
    M, N, K = shape
    a, b = W.normal_inputs(M, N, K, seed=M + 3 * N + 5 * K)
    ad, bd = a.to(DEV), b.to(DEV)
    for new, old in COPY_WAVE_TWINS:
        say(f"[gpu] copy-wave K split {shape}: config {new} vs {old}")
        c_new = gsr.gemm_scale_relu_ex(ad, bd, 0.5, new).clone()
        c_old = gsr.gemm_scale_relu_ex(ad, bd, 0.5, old).clone()
        torch.cuda.synchronize()
        assert torch.equal(c_new.view(torch.int16), c_old.view(torch.int16)), (shape, new, old)
    if M * N * K <= 2e8:  # and the 64x64 copy-wave tile against the oracle
        ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 0.5)
        PT.assert_parity(f"{shape} cfg21", PT.run_gpu(a, b, 0.5, config_id=21), ref)


# The 16x16x32 kernels pair the same k in every MFMA and sum in the same
# order, so they give the same bits: the 256x256 kernel with B copied to LDS
# (config 28) and its register-transpose twin (config 25); the 128x256
# kernel with its copies on separate waves (config 31) and the same plan with
# the copies among the MFMAs (config 29); the 128x128 copy-wave kernel with a
# four-stage ring (config 32) and config 31, whose tiles differ but whose
# MFMA chains per output do not.  K covers 1 to 65 steps of 64, M and N
# ragged against the tile, the element path included (N or K odd); the last
# three shapes run the 128-bit path with 3, 17 and 66 K-steps, so the ring
# of four ends on a tail of 3, 1 and 2 steps.
@pytest.mark.parametrize("pair", [(28, 25), (31, 29), (32, 31)], ids=lambda p: f"{p[0]}vs{p[1]}")
@pytest.mark.parametrize("shape", [(256, 256, 8), (300, 520, 200), (257, 1031, 72), (1000, 1500, 704),
                                   (513, 777, 4160), (4097, 2048, 1000), (2048, 4096, 1031),
                                   (384, 1024, 192), (640, 768, 1088), (1024, 2048, 4224)],
                         ids=lambda s: "x".join(map(str, s)))
def test_copy_transpose_twin_matches_register_transpose(gsr, orc, shape, pair):
    M, N, K = shape
    new, old = pair
    a, b = W.normal_inputs(M, N, K, seed=M + 7 * N + 3 * K)
    ad, bd = a.to(DEV), b.to(DEV)
    say(f"[gpu] config {new} vs {old} {shape}")
    c_new = gsr.gemm_scale_relu_ex(ad, bd, 0.5, new).clone()
    c_old = gsr.gemm_scale_relu_ex(ad, bd, 0.5, old).clone()
    torch.cuda.synchronize()
    assert torch.equal(c_new.view(torch.int16), c_old.view(torch.int16)), shape
    if M * N * K <= 3e9:
        ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 0.5)
        PT.assert_parity(f"{shape} cfg{new}", bits(c_new.cpu()), ref)


@pytest.mark.parametrize("shape", [(256, 256, 256), (300, 520, 200), (257, 263, 129), (1024, 1024, 512),
                                   (4097, 384, 256)], ids=lambda s: "x".join(map(str, s)))
def test_integer_inputs_bitwise(gsr, orc, shape):
    M, N, K = shape
    a, b = W.integer_inputs(M, N, K, seed=5)
    for alpha in (0.5, 1.0, -0.5):
        ref, _ = orc.gemm_scale_relu(bits(a), bits(b), alpha)
        for cid in [-1] + _configs(gsr):
            say(f"[gpu] integer {shape} alpha={alpha} config {cid}")
            got = PT.run_gpu(a, b, alpha, config_id=cid)
            PT.assert_bitwise(f"integer {shape} alpha={alpha} cfg{cid}", got, ref)


@pytest.mark.parametrize("name", ["square_4096", "llm_mlp_4097x11008x4096"])
def test_integer_full_size_every_output(gsr, orc, name):
    """The 4096^3 and LLM-MLP shapes with integer inputs in [-2, 2], in the
    selector's launch: every output bit for bit (|partial sums| <= 4K < 2^24,
    so the fp32 sum is exact)."""
    w = W.WORKLOADS[name]
    a, b = W.integer_inputs(w.M, w.N, w.K, seed=11, lo=-2, hi=2)
    say(f"[gpu] integer {name} {w.M}x{w.N}x{w.K} alpha=0.5 selector, every output")
    got = PT.run_gpu(a, b, 0.5)
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 0.5)
    PT.assert_bitwise(f"integer {name}", got, ref)


# --------------------------------------------------------------------------
# edges, layout, guard bands
# --------------------------------------------------------------------------

def test_k_zero_fills_zero(gsr):
    say("[gpu] K=0")
    c = torch.full((37, 45), float("nan"), dtype=torch.float16, device=DEV)
    a = torch.empty((37, 0), dtype=torch.float16, device=DEV)
    b = torch.empty((0, 45), dtype=torch.float16, device=DEV)
    gsr.gemm_scale_relu(a, b, 0.5, c=c)
    torch.cuda.synchronize()
    assert torch.all(c == 0) and not torch.any(torch.signbit(c))


def test_empty_outputs(gsr):
    say("[gpu] M=0 / N=0")
    a = torch.empty((0, 8), dtype=torch.float16, device=DEV)
    b = torch.ones((8, 16), dtype=torch.float16, device=DEV)
    assert gsr.gemm_scale_relu(a, b, 0.5).shape == (0, 16)
    b2 = torch.ones((8, 0), dtype=torch.float16, device=DEV)
    a2 = torch.ones((4, 8), dtype=torch.float16, device=DEV)
    assert gsr.gemm_scale_relu(a2, b2, 0.5).shape == (4, 0)


@pytest.mark.parametrize("cid", [-1, 16, 17, 18, 21, 22, 25, 28, 29, 31, 32])
@pytest.mark.parametrize("c_off", [4, 2, 1], ids=lambda o: f"C+{2 * o}B")
def test_c_less_aligned_than_16_bytes(gsr, orc, cid, c_off):
    """A and B 16-byte aligned with K and N multiples of 8, C only 8-, 4- or
    2-byte aligned (1, 2 or 4 elements into a 16-byte aligned buffer): the
    vector kernels run and write C in 8-, 4- or 2-byte stores.  The bands
    around C stay untouched and every output matches the oracle."""
    M, N, K = 300, 264, 200
    a, b = W.normal_inputs(M, N, K, seed=31)
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 0.5)
    say(f"[gpu] C at a {2 * c_off}-byte offset, config {cid}")
    buf = torch.full((M * N + 64,), 0x7E5A, dtype=torch.int16, device=DEV).view(torch.float16)
    assert buf.data_ptr() % 16 == 0
    c = buf[c_off:c_off + M * N].view(M, N)
    PT.run_gpu(a, b, 0.5, config_id=cid, c=c)
    hb = bits(buf.cpu())
    assert np.all(hb[:c_off] == 0x7E5A) and np.all(hb[c_off + M * N:] == 0x7E5A)
    PT.assert_parity(f"C+{2 * c_off} bytes cfg{cid}", hb[c_off:c_off + M * N].reshape(M, N), ref)


@pytest.mark.parametrize("offset", [1, 2, 3, 4, 8])
def test_unaligned_pointers(gsr, orc, offset):
    """Operands at 2-, 4- or 8-byte (but not 16-byte) aligned addresses take
    the element-wise path, whose loads narrow to the alignment (2-, 4- or
    8-byte units), and give the same results."""
    M, N, K = 130, 136, 72
    a, b = W.normal_inputs(M, N, K, seed=offset)
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 0.5)
    say(f"[gpu] unaligned offset {offset}")
    abuf = torch.zeros(M * K + 64, dtype=torch.float16, device=DEV)
    bbuf = torch.zeros(K * N + 64, dtype=torch.float16, device=DEV)
    cbuf = torch.zeros(M * N + 64, dtype=torch.float16, device=DEV)
    ad = abuf[offset:offset + M * K].view(M, K)
    bd = bbuf[offset:offset + K * N].view(K, N)
    cd = cbuf[offset:offset + M * N].view(M, N)
    ad.copy_(a.to(DEV))
    bd.copy_(b.to(DEV))
    gsr.gemm_scale_relu(ad, bd, 0.5, c=cd)
    torch.cuda.synchronize()
    PT.assert_parity(f"unaligned+{offset}", bits(cd.cpu()), ref)


@pytest.mark.parametrize("cid", [-1, 21, 22, 25, 28, 29, 31, 32])
def test_guard_bands_and_full_coverage(gsr, orc, cid):
    """C sits inside a larger buffer filled with a sentinel: the bands before
    and after stay untouched and every element of C is written."""
    M, N, K = 333, 264, 136
    a, b = W.normal_inputs(M, N, K, seed=21)
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 1.0)
    say(f"[gpu] guard bands config {cid}")
    guard = 4096
    # a NaN payload no kernel would produce; filled as int16 so the exact bits survive
    buf = torch.full((guard + M * N + guard,), 0x7E5A, dtype=torch.int16, device=DEV).view(torch.float16)
    c = buf[guard:guard + M * N].view(M, N)
    PT.run_gpu(a, b, 1.0, config_id=cid, c=c)
    hb = bits(buf.cpu())
    assert np.all(hb[:guard] == 0x7E5A) and np.all(hb[guard + M * N:] == 0x7E5A)
    PT.assert_parity(f"guard cfg{cid}", hb[guard:guard + M * N].reshape(M, N), ref)


def test_zero_padding_equivalence(gsr):
    """A ragged problem and its zero-padded, tile-multiple version agree bit
    for bit on the shared block (adding exact zeros leaves fp32 sums alone)."""
    # K and N multiples of 8 so both problems take the same (128-bit) path
    M, N, K = 261, 296, 152
    a, b = W.normal_inputs(M, N, K, seed=4)
    ap = torch.zeros(512, 512, dtype=torch.float16)
    bp = torch.zeros(192, 512, dtype=torch.float16)
    ap[:M, :K] = a
    bp[:K, :N] = b
    ap = ap[:, :192].contiguous()
    for cid in gsr.config_ids():
        say(f"[gpu] zero padding config {cid}")
        got = PT.run_gpu(a, b, 0.5, config_id=cid)
        gotp = PT.run_gpu(ap, bp, 0.5, config_id=cid)
        PT.assert_bitwise(f"padding cfg{cid}", got, gotp[:M, :N])
        assert np.all(gotp[M:, :] == 0) and np.all(gotp[:, N:] == 0)


def test_nonpositive_results_are_plus_zero(gsr):
    """An exactly-zero sum times a negative alpha is -0 in fp32; ReLU must
    still store +0."""
    say("[gpu] -0 handling")
    a = torch.zeros((64, 64), dtype=torch.float16, device=DEV)
    b = torch.ones((64, 64), dtype=torch.float16, device=DEV)
    c = gsr.gemm_scale_relu(a, b, -0.5)
    torch.cuda.synchronize()
    assert not torch.any(torch.signbit(c))


def test_alpha_sign_flip(gsr):
    M, N, K = 512, 640, 384
    a, b = W.normal_inputs(M, N, K, seed=8)
    say("[gpu] alpha sign flip")
    p = PT.run_gpu(a, b, 0.75)
    n = PT.run_gpu(a, b, -0.75)
    assert not np.any((p != 0) & (n != 0))
    assert not np.any(p & 0x8000) and not np.any(n & 0x8000)


def test_transpose_invariant(gsr):
    """(A B)^T = B^T A^T, bit for bit with integer inputs."""
    M, N, K = 320, 200, 264
    a, b = W.integer_inputs(M, N, K, seed=9)
    say("[gpu] transpose")
    c = PT.run_gpu(a, b, 0.5)
    ct = PT.run_gpu(b.t().contiguous(), a.t().contiguous(), 0.5)
    PT.assert_bitwise("transpose", ct, c.T)


def test_deterministic(gsr):
    w = W.WORKLOADS["square_1024"]
    a, b = W.workload_inputs(w)
    ad, bd = a.to(DEV), b.to(DEV)
    say("[gpu] determinism")
    first = gsr.gemm_scale_relu(ad, bd, w.alpha)
    for _ in range(20):
        again = gsr.gemm_scale_relu(ad, bd, w.alpha)
        assert torch.equal(first.view(torch.int16), again.view(torch.int16))


def test_side_stream(gsr, orc):
    M, N, K = 256, 512, 320
    a, b = W.normal_inputs(M, N, K, seed=13)
    ref, _ = orc.gemm_scale_relu(bits(a), bits(b), 0.5)
    say("[gpu] side stream")
    s = torch.cuda.Stream()
    ad, bd = a.to(DEV), b.to(DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        c = gsr.gemm_scale_relu(ad, bd, 0.5)
    s.synchronize()
    PT.assert_parity("side stream", bits(c.cpu()), ref)


def test_graph_capture_replays(gsr, orc):
    """The launch can be captured into a HIP graph; each replay, with eager
    work in between, matches the eager result."""
    M, N, K = 1024, 1024, 1024
    a, b = W.normal_inputs(M, N, K, seed=17)
    ad, bd = a.to(DEV), b.to(DEV)
    say("[gpu] graph capture")
    eager = gsr.gemm_scale_relu(ad, bd, 0.5)
    torch.cuda.synchronize()
    c = torch.empty_like(eager)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gsr.gemm_scale_relu(ad, bd, 0.5, c=c)  # warm-up outside capture
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        gsr.gemm_scale_relu(ad, bd, 0.5, c=c)
    for i in range(4):
        c.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        _ = (ad.float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
