"""GPU pins of the fp16 narrowing of C at its edges, bit for bit.

The hand-worked cases of tests/golden/worked_examples.txt fix the single
round-to-nearest-even store of the tutorial's kernel (PKUHPC scow-tutorial
"Tutorial14", section 2 listing: the accumulator fragment is scaled, clamped
at zero and copied to the fp16 C in one store): ties to even at 2048,
subnormal outputs and a subnormal tie that rounds to zero, overflow to +inf,
the same sum halved back into range, and a negative alpha.

Each case is a few outputs of a tiny problem.  So that every tile
configuration runs its real path (several tiles, several K-steps, ragged
edges), R copies of the case are placed block-diagonally in one larger
problem: copy i owns rows r_i.., columns c_i.. and k-indices k_i.., A is the
case's A on (rows of i) x (k of i) and zero elsewhere, B the case's B on
(k of i) x (columns of i) and zero elsewhere.  Every other product is an
exact zero, so C holds the case's hand-worked outputs in each diagonal block
and +0 everywhere else.  The gaps between copies vary, so the copies meet
tile and K-step boundaries at every offset.

The case whose point is that an fp32 running sum loses a term against the
fp64 oracle (cancellation_needs_wide_sum) is left out: the kernel accumulates
in fp32 by design (the listing's float accumulator), so there the oracle and
the GPU are meant to differ.
"""
import numpy as np
import pytest
import torch

import parity as PT
from oracle_pins import load_golden
from tiled_dense_gemm_scale_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SKIP = {"cancellation_needs_wide_sum"}
CASES = [c for c in load_golden() if c["name"] not in SKIP]


def embed(case, copies: int, pad8: bool):
    """The block-diagonal problem for one golden case: (A, B, expected C bits,
    alpha).  pad8 rounds N and K up to multiples of 8 (the 128-bit path);
    otherwise they end one element past such a multiple (the element path)."""
    Mc, Nc, Kc = case["M"], case["N"], case["K"]
    a_c = np.array(case["A"], dtype=np.float64)
    b_c = np.array(case["B"], dtype=np.float64)
    c_c = np.array(case["C"], dtype=np.uint16)
    rows, cols, ks = [], [], []
    r = c = k = 0
    for i in range(copies):
        r += i % 3          # gaps of 0, 1, 2 between copies
        c += (i * 5) % 7
        k += (i * 3) % 11
        rows.append(r)
        cols.append(c)
        ks.append(k)
        r += Mc
        c += Nc
        k += Kc
    M, N, K = r + 3, c + 5, k + 9
    if pad8:
        N, K = -(-N // 8) * 8, -(-K // 8) * 8
    else:
        N, K = N // 8 * 8 + 1, K // 8 * 8 + 1
    a = np.zeros((M, K), dtype=np.float64)
    b = np.zeros((K, N), dtype=np.float64)
    want = np.zeros((M, N), dtype=np.uint16)
    for r0, c0, k0 in zip(rows, cols, ks):
        a[r0:r0 + Mc, k0:k0 + Kc] = a_c
        b[k0:k0 + Kc, c0:c0 + Nc] = b_c
        want[r0:r0 + Mc, c0:c0 + Nc] = c_c
    a16 = torch.from_numpy(a.astype(np.float16))
    b16 = torch.from_numpy(b.astype(np.float16))
    assert np.array_equal(a16.double().numpy(), a) and np.array_equal(b16.double().numpy(), b)
    return a16, b16, want, case["alpha"]


@pytest.fixture(scope="module")
def gsr(native):
    import tiled_dense_gemm_scale_amd as g

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return g


def test_golden_fixture_covers_the_edges():
    names = {c["name"] for c in CASES}
    for n in ("ties_to_even_at_2048", "subnormal_outputs", "subnormal_tie_to_zero", "overflow_to_inf",
              "overflow_halved", "negative_alpha_flips"):
        assert n in names


@pytest.mark.parametrize("pad8", [True, False], ids=["vec", "elem"])
@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_case_every_config_bitwise(gsr, orc, case, pad8):
    a, b, want, alpha = embed(case, copies=150, pad8=pad8)
    M, K = a.shape
    N = b.shape[1]
    # the embedding itself: the oracle gives the hand-worked blocks and zeros
    ref, _ = orc.gemm_scale_relu(W.fp16_bits(a), W.fp16_bits(b), alpha)
    np.testing.assert_array_equal(ref, want)
    for cid in [-1] + gsr.config_ids():
        print(f"[gpu] golden {case['name']} {M}x{N}x{K} alpha={alpha} config {cid}", flush=True)
        got = PT.run_gpu(a, b, alpha, config_id=cid)
        # bit for bit, the sign of zero included: every non-positive result is +0
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"{case['name']} cfg{cid}: {len(bad)} mismatches, first at {tuple(bad[0])}: "
                               f"gpu 0x{int(got[tuple(bad[0])]):04x} expected 0x{int(want[tuple(bad[0])]):04x}")
