"""Pins for the CPU oracle: checks that tie it to things other than itself.

Each pin takes an oracle object (oracle.oracle.Oracle) and returns a list of
failure messages (empty = pass).  The same pins run against the real oracle
(tests/test_oracle_pins.py, must all pass) and against builds with a planted
mistake (tests/test_oracle_mutants.py, at least one pin must fail for each).

What pins what:
  * fp16 decode / encode -- numpy's float16 conversions and struct's 'e'
    format, exhaustively over all 65536 patterns, every tie midpoint and the
    overflow / subnormal boundaries (IEEE 754 binary16 definition);
  * the dot product, scale, ReLU and rounding -- exact rational arithmetic
    (fractions.Fraction) with a rational -> fp16 round-to-nearest-even
    written here from the IEEE definition, no float intermediate;
  * closed forms -- all-ones inputs give alpha*K, an identity B returns
    ReLU(alpha*A), a one-hot row of A returns ReLU(alpha*B[k,:]), a diagonal
    B scales columns, small-integer inputs give exact integer sums;
  * invariants -- outputs are never negative, flipping alpha's sign zeroes
    every output that was positive, doubling alpha doubles outputs,
    transposition, permutation of k, zero padding;
  * hand-worked examples in tests/golden/worked_examples.txt;
  * the epilogue variants (bias per output column; ReLU, GELU or nothing):
    GELU against the tanh form as usually written with the library tanh,
    against the exact GELU x*Phi(x) from the library erf (the tanh form is an
    approximation of it to 5e-4), and its odd-part identity
    gelu(y) - gelu(-y) = y; bias and activation against exact rationals; K=0
    and zero-bias closed forms; the identity that a bias equals one more k
    term (a column of ones in A, the bias as a row of B).
The operation itself: PKUHPC scow-tutorial "Tutorial14", section 3, display
formula; the listing in section 2 fixes scale-then-max and the fp16 output.
The epilogue variants: the aikraft.ru TileLang guide, section 4 (GEMM + Bias
+ GELU, with an exponent-based GELU approximation).
"""
from __future__ import annotations

import math
import os
import struct
from fractions import Fraction
from typing import List

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.txt")


# ---------------------------------------------------------------------------
# Independent helpers (exact arithmetic; nothing shared with the oracle)
# ---------------------------------------------------------------------------

def fraction_to_fp16_bits(r: Fraction) -> int:
    """Round an exact rational to IEEE binary16, ties to even, from the
    definition: pick the binade, scale to an integer significand, round."""
    if r == 0:
        return 0
    sign = 0x8000 if r < 0 else 0
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -14)                     # below 2^-14 the quantum stays 2^-24
    n = a / (Fraction(2) ** (e - 10))   # significand in units of the quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    if fl == 2048:
        fl = 1024
        e += 1
    if e > 15:
        return sign | 0x7C00
    if fl < 1024:                       # subnormal (only reachable with e == -14)
        return sign | fl
    return sign | ((e + 15) << 10) | (fl - 1024)


def fp16_value(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", int(bits)))[0]


def exact_reference(a_bits: np.ndarray, b_bits: np.ndarray, alpha: float) -> np.ndarray:
    """Brute force in exact rationals: C bits for tiny shapes."""
    M, K = a_bits.shape
    N = b_bits.shape[1]
    A = [[Fraction(fp16_value(a_bits[m, k])) for k in range(K)] for m in range(M)]
    B = [[Fraction(fp16_value(b_bits[k, n])) for n in range(N)] for k in range(K)]
    al = Fraction(float(np.float32(alpha)))
    out = np.zeros((M, N), dtype=np.uint16)
    for m in range(M):
        for n in range(N):
            s = sum((A[m][k] * B[k][n] for k in range(K)), Fraction(0))
            y = al * s
            out[m, n] = fraction_to_fp16_bits(y if y > 0 else Fraction(0))
    return out


def random_fp16_bits(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    return (rng.standard_normal(shape) * scale).astype(np.float16).view(np.uint16)


def to_bits(x) -> np.ndarray:
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def _cmp(name: str, got: np.ndarray, want: np.ndarray, fails: List[str]) -> None:
    got = np.asarray(got)
    want = np.asarray(want)
    if got.shape != want.shape:
        fails.append(f"{name}: shape {got.shape} != {want.shape}")
        return
    bad = np.argwhere(got != want)
    if bad.size:
        idx = tuple(bad[0])
        fails.append(f"{name}: {len(bad)} mismatches, first at {idx}: "
                     f"got 0x{int(got[idx]):04x} want 0x{int(want[idx]):04x}")


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

def pin_decode(orc) -> List[str]:
    fails: List[str] = []
    bits = np.arange(65536, dtype=np.uint16)
    got = orc.decode(bits)
    want = bits.view(np.float16).astype(np.float64)
    nan_w = np.isnan(want)
    if not np.array_equal(np.isnan(got), nan_w):
        fails.append("decode: NaN classification differs from numpy")
    ok = got[~nan_w] == want[~nan_w]
    if not ok.all():
        i = int(np.flatnonzero(~ok)[0])
        fails.append(f"decode: 0x{i:04x} -> {got[~nan_w][i]!r}, numpy says {want[~nan_w][i]!r}")
    # sign of zero and a spot check against struct's own binary16 codec
    if math.copysign(1.0, got[0x8000]) != -1.0:
        fails.append("decode: 0x8000 is not -0.0")
    for b in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0xFBFF, 0x8001, 0x3555):
        if got[b] != fp16_value(b):
            fails.append(f"decode: 0x{b:04x} differs from struct")
    return fails


def pin_encode(orc) -> List[str]:
    fails: List[str] = []
    bits = np.arange(65536, dtype=np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    fin = ~np.isnan(vals)
    _cmp("encode round trip", orc.encode(vals[fin]), bits[fin], fails)
    # every midpoint between consecutive positive finite fp16 values
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2.0   # exact in binary64
    _cmp("encode midpoints", orc.encode(mids), to_bits(mids), fails)
    _cmp("encode -midpoints", orc.encode(-mids), to_bits(-mids), fails)
    # boundaries: overflow threshold, subnormal ties, tiny values
    edge = np.array([65504.0, 65519.99, 65519.999999, 65520.0, 65536.0, 1e10, 2.0 ** -24,
                     2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -25, 2.0 ** -26, 1e-30,
                     2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 0.0, -0.0, np.inf, -np.inf])
    _cmp("encode edges", orc.encode(edge), to_bits(edge), fails)
    for x in edge[:-2]:
        want = struct.unpack("<H", struct.pack("<e", x))[0] if abs(x) < 65520 else (0x7C00 if x > 0 else 0xFC00)
        got = int(orc.encode(np.array([x]))[0])
        if got != want:
            fails.append(f"encode {x!r}: 0x{got:04x}, struct says 0x{want:04x}")
    rng = np.random.Generator(np.random.PCG64(12345))
    r = np.concatenate([
        rng.standard_normal(300000),
        rng.standard_normal(300000) * 1000.0,
        np.exp(rng.uniform(-25 * math.log(2), 17 * math.log(2), 400000)) * rng.choice([-1.0, 1.0], 400000),
    ])
    _cmp("encode random", orc.encode(r), to_bits(r), fails)
    if int(orc.encode(np.array([np.nan]))[0]) & 0x7C00 != 0x7C00 or int(orc.encode(np.array([np.nan]))[0]) & 0x3FF == 0:
        fails.append("encode: NaN does not map to a NaN pattern")
    return fails


def pin_bruteforce(orc, shapes=(1, 2, 3, 5, 8, 13, 17), alphas=(0.5, 1.0, -0.75, 3.0), seed=7) -> List[str]:
    """Bit-exact against exact rationals.  A mismatch is allowed only where
    the exact value is so close to an fp16 rounding midpoint that the fp64
    summation error bound (K * 2^-53 * sum|alpha a b|) straddles it."""
    fails: List[str] = []
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i, M in enumerate(shapes):
        N = shapes[(i + 2) % len(shapes)]
        K = shapes[(i + 4) % len(shapes)]
        cases.append((M, N, K))
    cases += [(3, 4, 17), (17, 13, 8), (2, 2, 1), (1, 17, 13)]
    for ci, (M, N, K) in enumerate(cases):
        a = random_fp16_bits(rng, (M, K))
        b = random_fp16_bits(rng, (K, N))
        for alpha in alphas:
            want = exact_reference(a, b, alpha)
            got, _ = orc.gemm_scale_relu(a, b, alpha, nthreads=1)
            gp, _ = orc.gemm_scale_relu_points(a, b, alpha, *np.divmod(np.arange(M * N), N), nthreads=2)
            for name, g in (("full", got), ("points", gp.reshape(M, N))):
                bad = np.argwhere(g != want)
                for (m, n) in bad:
                    av = np.abs(a[m].view(np.float16).astype(np.float64))
                    bv = np.abs(b[:, n].view(np.float16).astype(np.float64))
                    bound = K * 2.0 ** -53 * abs(alpha) * float(np.dot(av, bv))
                    exact = sum(Fraction(fp16_value(a[m, k])) * Fraction(fp16_value(b[k, n])) for k in range(K))
                    y = Fraction(float(np.float32(alpha))) * exact
                    lo = fraction_to_fp16_bits(max(y - Fraction(bound), Fraction(0)))
                    hi = fraction_to_fp16_bits(max(y + Fraction(bound), Fraction(0)))
                    if lo == hi:
                        fails.append(f"bruteforce {name} case {ci} {(M, N, K)} alpha={alpha} at {(m, n)}: "
                                     f"0x{int(g[m, n]):04x} != exact 0x{int(want[m, n]):04x}")
                        break
    return fails


def pin_closed_forms(orc) -> List[str]:
    fails: List[str] = []
    one = np.uint16(0x3C00)
    # all-ones: every output is alpha*K, exact in fp16 at these sizes
    for K, alpha, want in ((256, 0.5, 128.0), (1024, 0.5, 512.0), (4096, 0.5, 2048.0),
                           (16384, 0.5, 8192.0), (4096, 1.0, 4096.0), (7, 1.0, 7.0), (1, 0.5, 0.5)):
        a = np.full((2, K), one, dtype=np.uint16)
        b = np.full((K, 3), one, dtype=np.uint16)
        c, r = orc.gemm_scale_relu(a, b, alpha, want_fp64=True)
        _cmp(f"all-ones K={K}", c, np.full((2, 3), to_bits(want), dtype=np.uint16), fails)
        if not np.all(r == want):
            fails.append(f"all-ones K={K}: fp64 value {r.flat[0]!r} != {want}")
        c, _ = orc.gemm_scale_relu(a, b, -alpha)
        _cmp(f"all-ones K={K} negated alpha", c, np.zeros((2, 3), np.uint16), fails)
    rng = np.random.Generator(np.random.PCG64(99))
    # identity B: ReLU(alpha*A) rounded once
    for alpha in (0.5, 1.0, -1.0, 0.3):
        a = random_fp16_bits(rng, (9, 12), 3.0)
        eye = np.where(np.eye(12, dtype=bool), np.uint16(0x3C00), np.uint16(0)).astype(np.uint16)
        c, _ = orc.gemm_scale_relu(a, eye, alpha)
        y = a.view(np.float16).astype(np.float64) * float(np.float32(alpha))
        _cmp(f"identity B alpha={alpha}", c, to_bits(np.where(y > 0, y, 0.0)), fails)
    # one-hot rows of A pick rows of B
    b = random_fp16_bits(rng, (6, 10), 2.0)
    a = np.zeros((6, 6), dtype=np.uint16)
    perm = [3, 0, 5, 1, 4, 2]
    for m, k in enumerate(perm):
        a[m, k] = 0x3C00
    c, _ = orc.gemm_scale_relu(a, b, 0.5)
    y = b.view(np.float16).astype(np.float64)[perm] * 0.5
    _cmp("one-hot A", c, to_bits(np.where(y > 0, y, 0.0)), fails)
    # diagonal B scales each column of A
    a = random_fp16_bits(rng, (5, 7))
    d = np.array([1.0, -2.0, 0.5, 4.0, -0.25, 8.0, 1.0])
    bd = np.diag(d).astype(np.float16).view(np.uint16)
    c, _ = orc.gemm_scale_relu(a, bd, 1.0)
    y = a.view(np.float16).astype(np.float64) * d[None, :]
    _cmp("diagonal B", c, to_bits(np.where(y > 0, y, 0.0)), fails)
    # small integers: exact integer arithmetic
    ai = rng.integers(-4, 5, (11, 40))
    bi = rng.integers(-4, 5, (40, 13))
    s = ai.astype(np.int64) @ bi.astype(np.int64)
    for alpha in (0.5, 1.0, -0.5):
        c, _ = orc.gemm_scale_relu(to_bits(ai), to_bits(bi), alpha)
        y = s.astype(np.float64) * alpha
        _cmp(f"integer inputs alpha={alpha}", c, to_bits(np.where(y > 0, y, 0.0)), fails)
    # K = 0: the empty sum, so every output is +0
    c, _ = orc.gemm_scale_relu(np.zeros((3, 0), np.uint16), np.zeros((0, 4), np.uint16), 0.5)
    _cmp("K=0", c, np.zeros((3, 4), np.uint16), fails)
    c, _ = orc.gemm_scale_relu(np.zeros((0, 5), np.uint16), np.zeros((5, 4), np.uint16), 0.5)
    if c.shape != (0, 4):
        fails.append("M=0: wrong shape")
    return fails


def pin_invariants(orc, seed=3) -> List[str]:
    fails: List[str] = []
    rng = np.random.Generator(np.random.PCG64(seed))
    M, N, K = 23, 19, 37
    a = random_fp16_bits(rng, (M, K))
    b = random_fp16_bits(rng, (K, N))
    c, _ = orc.gemm_scale_relu(a, b, 0.5)
    if np.any(c & 0x8000) or np.any((c & 0x7C00) == 0x7C00):
        fails.append("invariant: an output is negative, -0, inf or NaN")
    frac_zero = float(np.mean(c == 0))
    if not 0.3 < frac_zero < 0.7:
        fails.append(f"invariant: fraction of zeros {frac_zero:.2f} far from 1/2 for symmetric inputs")
    # flipping alpha's sign zeroes every output that was positive
    cn, _ = orc.gemm_scale_relu(a, b, -0.5)
    if np.any((c != 0) & (cn != 0)):
        fails.append("invariant: C(alpha) and C(-alpha) both nonzero somewhere")
    # ... and the two together carry |alpha*s|
    both = np.where(c != 0, c, cn)
    s_abs = np.abs(a.view(np.float16).astype(np.float64) @ b.view(np.float16).astype(np.float64))
    _cmp("invariant: C(a) | C(-a) == fp16(|a s|)", both, to_bits(0.5 * s_abs), fails)
    # doubling alpha doubles the outputs (powers of two, no overflow here)
    c2, _ = orc.gemm_scale_relu(a, b, 1.0)
    _cmp("invariant: C(2a) == 2 C(a)", c2, to_bits(2.0 * c.view(np.float16).astype(np.float64)), fails)
    # transposition: (A B)^T = B^T A^T
    ct, _ = orc.gemm_scale_relu(np.ascontiguousarray(b.T), np.ascontiguousarray(a.T), 0.5)
    _cmp("invariant: transpose", ct, c.T, fails)
    # permuting k in A's columns and B's rows together (integer inputs keep
    # every fp64 partial sum exact, so the result is order independent)
    ai = to_bits(rng.integers(-8, 9, (M, K)))
    bi = to_bits(rng.integers(-8, 9, (K, N)))
    ci, _ = orc.gemm_scale_relu(ai, bi, 0.5)
    p = rng.permutation(K)
    cp, _ = orc.gemm_scale_relu(ai[:, p], bi[p, :], 0.5)
    _cmp("invariant: k permutation", cp, ci, fails)
    # zero padding: extra zero k-terms change nothing; extra rows/columns of
    # C only add ReLU(0) = +0 ... for zero rows/cols of A/B
    ap = np.concatenate([a, np.zeros((M, 5), np.uint16)], axis=1)
    bp = np.concatenate([b, np.zeros((5, N), np.uint16)], axis=0)
    cz, _ = orc.gemm_scale_relu(ap, bp, 0.5)
    _cmp("invariant: zero k padding", cz, c, fails)
    ar = np.concatenate([a, np.zeros((4, K), np.uint16)], axis=0)
    bc = np.concatenate([b, np.zeros((K, 3), np.uint16)], axis=1)
    cr, _ = orc.gemm_scale_relu(ar, bc, 0.5)
    _cmp("invariant: zero row/col padding (core)", cr[:M, :N], c, fails)
    if np.any(cr[M:, :] != 0) or np.any(cr[:, N:] != 0):
        fails.append("invariant: zero row/col padding produced nonzero outputs")
    # point mode agrees with full mode
    ms = rng.integers(0, M, 50)
    ns = rng.integers(0, N, 50)
    cpnt, _ = orc.gemm_scale_relu_points(a, b, 0.5, ms, ns)
    _cmp("invariant: points == full", cpnt, c[ms, ns], fails)
    # thread count does not change results
    c7, _ = orc.gemm_scale_relu(a, b, 0.5, nthreads=7)
    _cmp("invariant: threads", c7, c, fails)
    return fails


def load_golden(path: str = GOLDEN):
    cases = []
    cur = None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            key, *rest = line.split()
            if key == "case":
                cur = {"name": rest[0], "A": [], "B": [], "C": []}
            elif key in ("M", "N", "K"):
                cur[key] = int(rest[0])
            elif key == "alpha":
                cur["alpha"] = float(rest[0])
            elif key in ("A", "B"):
                cur[key].append([float.fromhex(v) if "0x" in v else float(v) for v in rest])
            elif key == "C":
                cur["C"].append([int(v, 16) for v in rest])
            elif key == "end":
                cases.append(cur)
                cur = None
    return cases


def pin_golden(orc) -> List[str]:
    fails: List[str] = []
    cases = load_golden()
    if len(cases) < 8:
        fails.append("golden: fixture incomplete")
    for cs in cases:
        a = np.array(cs["A"], dtype=np.float64)
        b = np.array(cs["B"], dtype=np.float64)
        if a.shape != (cs["M"], cs["K"]) or b.shape != (cs["K"], cs["N"]):
            fails.append(f"golden {cs['name']}: malformed")
            continue
        if not np.array_equal(a.astype(np.float16).astype(np.float64), a):
            fails.append(f"golden {cs['name']}: inputs not exact in fp16")
        want = np.array(cs["C"], dtype=np.uint16)
        got, _ = orc.gemm_scale_relu(to_bits(a), to_bits(b), cs["alpha"])
        _cmp(f"golden {cs['name']}", got, want, fails)
        ms, ns = np.divmod(np.arange(cs["M"] * cs["N"]), cs["N"])
        gp, _ = orc.gemm_scale_relu_points(to_bits(a), to_bits(b), cs["alpha"], ms, ns)
        _cmp(f"golden {cs['name']} (points)", gp.reshape(want.shape), want, fails)
        # the exact-rational brute force agrees with the hand working too
        _cmp(f"golden {cs['name']} (exact)", exact_reference(to_bits(a), to_bits(b), cs["alpha"]), want, fails)
    return fails


# ---------------------------------------------------------------------------
# Epilogue variants: C = act(alpha * A B + bias[n])
# ---------------------------------------------------------------------------

ACT_RELU, ACT_GELU, ACT_NONE = 0, 1, 2
ACTS = (ACT_RELU, ACT_GELU, ACT_NONE)
_GELU_C = math.sqrt(2.0 / math.pi)


def gelu_textbook(y: float) -> float:
    """The tanh form of GELU as it is usually written, with the library tanh."""
    return 0.5 * y * (1.0 + math.tanh(_GELU_C * (y + 0.044715 * y ** 3)))


def gelu_exact(y: float) -> float:
    """GELU itself: y * Phi(y), Phi the standard normal CDF via erf."""
    return 0.5 * y * (1.0 + math.erf(y / math.sqrt(2.0)))


def _fp16_ulps_apart(x: int, y: int) -> int:
    """Distance in representable steps between two fp16 bit patterns."""
    def key(b):
        b = int(b)
        return -(b & 0x7FFF) if b & 0x8000 else b
    return abs(key(x) - key(y))


def exact_reference_bias_act(a_bits, b_bits, bias_bits, alpha, act):
    """C bits of act(alpha * A B + bias) for tiny shapes: the sum, scale and
    bias in exact rationals; ReLU and the identity exact too; GELU of the
    exact value rounded once to binary64, by the textbook formula."""
    M, K = a_bits.shape
    N = b_bits.shape[1]
    A = [[Fraction(fp16_value(a_bits[m, k])) for k in range(K)] for m in range(M)]
    B = [[Fraction(fp16_value(b_bits[k, n])) for n in range(N)] for k in range(K)]
    bias = [Fraction(fp16_value(bias_bits[n])) if bias_bits is not None else Fraction(0) for n in range(N)]
    al = Fraction(float(np.float32(alpha)))
    out = np.zeros((M, N), dtype=np.uint16)
    exact = {}
    for m in range(M):
        for n in range(N):
            y = al * sum((A[m][k] * B[k][n] for k in range(K)), Fraction(0)) + bias[n]
            exact[m, n] = y
            if act == ACT_RELU:
                out[m, n] = fraction_to_fp16_bits(y if y > 0 else Fraction(0))
            elif act == ACT_NONE:
                out[m, n] = fraction_to_fp16_bits(y)
            else:
                out[m, n] = fraction_to_fp16_bits(Fraction(gelu_textbook(float(y))))
    return out, exact


def pin_gelu(orc) -> List[str]:
    fails: List[str] = []
    rng = np.random.Generator(np.random.PCG64(2024))
    ys = np.concatenate([np.linspace(-12.0, 12.0, 8001), rng.standard_normal(20000) * 4.0,
                         [0.0, -0.0, 1e-300, -1e-300, 1e-8, -1e-8, 30.0, -30.0]])
    worst_t = worst_e = worst_s = 0.0
    for y in ys:
        g = orc.gelu(float(y))
        worst_t = max(worst_t, abs(g - gelu_textbook(float(y))) / max(1.0, abs(y)))
        worst_e = max(worst_e, abs(g - gelu_exact(float(y))))
        worst_s = max(worst_s, abs(g - orc.gelu(-float(y)) - y) / max(1.0, abs(y)))
    if worst_t > 4e-15:
        fails.append(f"gelu: differs from the textbook tanh form by {worst_t:.3g} (relative)")
    if worst_e > 5e-4:
        fails.append(f"gelu: differs from y*Phi(y) by {worst_e:.3g} (the tanh form is within 4.8e-4)")
    if worst_s > 4e-15:
        fails.append(f"gelu: gelu(y) - gelu(-y) differs from y by {worst_s:.3g}")
    if orc.gelu(0.0) != 0.0 or orc.gelu(60.0) != 60.0 or abs(orc.gelu(-60.0)) > 1e-300:
        fails.append("gelu: wrong at 0 or in the tails")
    return fails


def pin_bias_act_bruteforce(orc, seed=11) -> List[str]:
    """Bias and activation against exact rationals (M <= N everywhere, so a
    bias indexed by row would still stay inside the bias array).  ReLU and
    the identity must be bit-exact unless the fp64 error bound straddles a
    rounding midpoint; GELU (a transcendental of the exact sum) may differ by
    one fp16 step."""
    fails: List[str] = []
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = [(1, 3, 2), (2, 5, 3), (3, 7, 5), (4, 4, 17), (5, 13, 8), (2, 17, 1), (3, 3, 0), (6, 9, 13)]
    for ci, (M, N, K) in enumerate(cases):
        a = random_fp16_bits(rng, (M, K))
        b = random_fp16_bits(rng, (K, N))
        bias = random_fp16_bits(rng, (N,), 2.0)
        for alpha in (1.0, 0.5, -0.75):
            for act in ACTS:
                want, exact = exact_reference_bias_act(a, b, bias, alpha, act)
                got, _ = orc.gemm_bias_act(a, b, bias, alpha, act, nthreads=1)
                gp, _ = orc.gemm_bias_act_points(a, b, bias, alpha, act, *np.divmod(np.arange(M * N), N), nthreads=2)
                for name, g in (("full", got), ("points", gp.reshape(M, N))):
                    for (m, n) in np.argwhere(g != want):
                        if act == ACT_GELU:
                            if _fp16_ulps_apart(g[m, n], want[m, n]) <= 1:
                                continue
                        else:
                            av = np.abs(a[m].view(np.float16).astype(np.float64))
                            bv = np.abs(b[:, n].view(np.float16).astype(np.float64))
                            bound = Fraction((K + 2) * 2.0 ** -53 * (abs(alpha) * float(np.dot(av, bv))
                                                                    + abs(fp16_value(bias[n]))))
                            y = exact[m, n]
                            lo, hi = y - bound, y + bound
                            if act == ACT_RELU:
                                lo, hi = max(lo, Fraction(0)), max(hi, Fraction(0))
                            if fraction_to_fp16_bits(lo) != fraction_to_fp16_bits(hi):
                                continue
                        fails.append(f"bias/act {name} case {ci} {(M, N, K)} alpha={alpha} act={act} at "
                                     f"{(int(m), int(n))}: 0x{int(g[m, n]):04x} != 0x{int(want[m, n]):04x}")
                        break
    return fails


def pin_bias_act_forms(orc, seed=13) -> List[str]:
    fails: List[str] = []
    rng = np.random.Generator(np.random.PCG64(seed))
    M, N, K = 7, 11, 29
    a = random_fp16_bits(rng, (M, K))
    b = random_fp16_bits(rng, (K, N))
    bias = random_fp16_bits(rng, (N,), 3.0)
    bv = bias.view(np.float16).astype(np.float64)
    # K = 0: every output is act(bias[n]), the empty sum plus the bias
    for act in ACTS:
        c, _ = orc.gemm_bias_act(np.zeros((M, 0), np.uint16), np.zeros((0, N), np.uint16), bias, 0.5, act)
        if act == ACT_RELU:
            _cmp("bias K=0 relu", c, np.tile(to_bits(np.where(bv > 0, bv, 0.0)), (M, 1)), fails)
        elif act == ACT_NONE:
            _cmp("bias K=0 identity", c, np.tile(bias, (M, 1)), fails)
        else:
            want = to_bits([gelu_textbook(float(v)) for v in bv])
            if any(_fp16_ulps_apart(x, y) > 1 for x, y in zip(c[0], want)) or np.any(c != c[0]):
                fails.append("bias K=0 gelu: not gelu(bias) in every row")
    # no bias, ReLU: the tutorial's operation; a zero bias changes nothing
    c0, _ = orc.gemm_scale_relu(a, b, 0.5)
    c1, _ = orc.gemm_bias_act(a, b, None, 0.5, ACT_RELU)
    c2, _ = orc.gemm_bias_act(a, b, np.zeros(N, np.uint16), 0.5, ACT_RELU)
    _cmp("bias None == scale_relu", c1, c0, fails)
    _cmp("zero bias == no bias", c2, c0, fails)
    # a bias is one more k term: A gets a column of ones, B the row bias/alpha
    # (alpha a power of two, so bias/alpha is exact in fp16)
    for alpha in (1.0, 0.5):
        aa = np.concatenate([a, np.full((M, 1), 0x3C00, np.uint16)], axis=1)
        ba = np.concatenate([b, to_bits(bv / alpha)[None, :]], axis=0)
        for act in ACTS:
            cb, _ = orc.gemm_bias_act(a, b, bias, alpha, act)
            ck, _ = orc.gemm_bias_act(aa, ba, None, alpha, act)
            _cmp(f"bias == extra k term alpha={alpha} act={act}", cb, ck, fails)
    # the identity activation is signed; ReLU of it is the ReLU variant
    cn, rn = orc.gemm_bias_act(a, b, bias, 0.5, ACT_NONE, want_fp64=True)
    cr, _ = orc.gemm_bias_act(a, b, bias, 0.5, ACT_RELU)
    _cmp("relu == max(identity, 0)", cr, to_bits(np.where(rn > 0, rn, 0.0)), fails)
    if not np.any(cn & 0x8000):
        fails.append("identity activation produced no negative output")
    # points agree with full mode
    ms = rng.integers(0, M, 40)
    ns = rng.integers(0, N, 40)
    for act in ACTS:
        cf, _ = orc.gemm_bias_act(a, b, bias, 0.5, act)
        cp, _ = orc.gemm_bias_act_points(a, b, bias, 0.5, act, ms, ns)
        _cmp(f"bias points == full act={act}", cp, cf[ms, ns], fails)
    return fails


ALL_PINS = [pin_decode, pin_encode, pin_bruteforce, pin_closed_forms, pin_invariants, pin_golden,
            pin_gelu, pin_bias_act_bruteforce, pin_bias_act_forms]
