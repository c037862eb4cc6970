"""The tolerance gate of the GPU parity tests, checked on the CPU with
planted GPU outputs (no device): every output that the tutorial's
assert_close(rtol = atol = 1e-2) rejects must count as a violation, and an
oracle output that overflowed to +-inf must be matched bit for bit."""
import numpy as np
import pytest

import parity as PT

INF, NINF, NAN, MAX = 0x7C00, 0xFC00, 0x7E00, 0x7BFF  # +inf, -inf, a NaN, 65504


def h(*vals):
    return np.array(vals, dtype=np.float16).view(np.uint16)


def viol(gpu_bits, ref_bits):
    return PT.compare("t", np.asarray(gpu_bits, np.uint16), np.asarray(ref_bits, np.uint16)).violations


@pytest.mark.parametrize("gpu", [h(1.0)[0], NINF, MAX, NAN, 0])
def test_oracle_inf_needs_the_same_bits(gpu):
    assert viol([gpu], [INF]) == 1


def test_oracle_inf_matched():
    assert viol([INF, 0x3C00], [INF, 0x3C00]) == 0
    assert viol([NINF], [NINF]) == 0


@pytest.mark.parametrize("gpu", [INF, NINF, NAN])
def test_nonfinite_gpu_where_oracle_finite(gpu):
    assert viol([gpu], h(2.0)) == 1


def test_tolerance_edges():
    ref = h(1.0, 100.0, 0.0)
    # 1 + 0.02 is the largest allowed error at 1.0; fp16 steps there are 2^-10
    ok = h(1.0 + 19 * 2.0 ** -10, 100.0 + 1.0, 0.0078125)
    bad = h(1.0 + 21 * 2.0 ** -10, 100.0 + 1.25, 0.0117)
    assert viol(ok, ref) == 0
    assert viol(bad, ref) == 3


def test_signed_zero_is_equal():
    assert viol([0x8000], [0x0000]) == 0
