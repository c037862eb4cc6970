"""ctypes front end of the CPU oracle (gsr_oracle.c).

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg may import this module.  The product library in
tiled_dense_gemm_scale_amd/ never imports it, and it imports nothing from
the product.

The oracle evaluates C[m,n] = ReLU(alpha * sum_k A[m,k] B[k,n]) in binary64
from the fp16 bit patterns and rounds once to fp16 (PKUHPC scow-tutorial
"Tutorial14", section 3, display formula; kernel listing in section 2 for the
scale-then-max epilogue and the fp16 output).  The epilogue variants add an
optional fp16 bias per output column after the scale and apply ReLU, the
tanh-form GELU or nothing (the aikraft.ru TileLang guide, section 4, GEMM +
Bias + GELU): C = act(alpha * A B + bias).  Arrays cross the boundary as
numpy uint16 bit patterns so that no library fp16 conversion touches them.

Parity status: every function here is pinned by tests/test_oracle_*.py
(exhaustive codec checks against numpy and struct, exact rational brute
force, closed forms, invariants, a hand-worked golden example, and planted
mutants that the pins must reject).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "gsr_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")


def build(output: str = LIBRARY, mutant: int = 0) -> str:
    """Compile gsr_oracle.c with gcc.  mutant != 0 plants a deliberate
    mistake (pin tests only)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-pthread", f"-DORACLE_MUTANT={int(mutant)}",
           SOURCE, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


ACT_RELU, ACT_GELU, ACT_NONE = 0, 1, 2

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


class Oracle:
    """One loaded copy of the oracle library."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library not built: {path}")
        lib = ctypes.CDLL(path)
        lib.oracle_fp16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_fp16_to_f64.restype = ctypes.c_double
        lib.oracle_f64_to_fp16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_fp16.restype = ctypes.c_uint16
        lib.oracle_decode_array.argtypes = [ctypes.c_int64, _u16p, _f64p]
        lib.oracle_decode_array.restype = None
        lib.oracle_encode_array.argtypes = [ctypes.c_int64, _f64p, _u16p]
        lib.oracle_encode_array.restype = None
        lib.oracle_gemm_scale_relu.argtypes = [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _u16p, _u16p,
            ctypes.c_float, _u16p, _f64p, ctypes.c_int]
        lib.oracle_gemm_scale_relu.restype = ctypes.c_int
        lib.oracle_gemm_scale_relu_points.argtypes = [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _u16p, _u16p,
            ctypes.c_float, ctypes.c_int64, _i64p, _i64p, _u16p, _f64p, ctypes.c_int]
        lib.oracle_gemm_scale_relu_points.restype = ctypes.c_int
        lib.oracle_gemm_bias_act.argtypes = [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _u16p, _u16p, _u16p,
            ctypes.c_float, ctypes.c_int, _u16p, _f64p, ctypes.c_int]
        lib.oracle_gemm_bias_act.restype = ctypes.c_int
        lib.oracle_gemm_bias_act_points.argtypes = [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _u16p, _u16p, _u16p,
            ctypes.c_float, ctypes.c_int, ctypes.c_int64, _i64p, _i64p, _u16p, _f64p, ctypes.c_int]
        lib.oracle_gemm_bias_act_points.restype = ctypes.c_int
        lib.oracle_gelu.argtypes = [ctypes.c_double]
        lib.oracle_gelu.restype = ctypes.c_double
        lib.oracle_mutant_id.argtypes = []
        lib.oracle_mutant_id.restype = ctypes.c_int
        self._lib = lib
        self.path = path
        self.mutant = lib.oracle_mutant_id()

    # -- codec -------------------------------------------------------------
    def decode(self, bits: np.ndarray) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float64)
        self._lib.oracle_decode_array(bits.size, bits.ctypes.data_as(_u16p), out.ctypes.data_as(_f64p))
        return out

    def encode(self, values: np.ndarray) -> np.ndarray:
        values = np.ascontiguousarray(values, dtype=np.float64)
        out = np.empty(values.shape, dtype=np.uint16)
        self._lib.oracle_encode_array(values.size, values.ctypes.data_as(_f64p), out.ctypes.data_as(_u16p))
        return out

    # -- the operation -----------------------------------------------------
    def gemm_scale_relu(self, a_bits: np.ndarray, b_bits: np.ndarray, alpha: float,
                        nthreads: Optional[int] = None, want_fp64: bool = False
                        ) -> Tuple[np.ndarray, Optional[np.ndarray]]:
        """All outputs.  a_bits: (M,K) uint16, b_bits: (K,N) uint16.
        Returns (C bits (M,N) uint16, fp64 values before narrowing or None)."""
        a = np.ascontiguousarray(a_bits, dtype=np.uint16)
        b = np.ascontiguousarray(b_bits, dtype=np.uint16)
        if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
            raise ValueError(f"shape mismatch {a.shape} x {b.shape}")
        M, K = a.shape
        N = b.shape[1]
        c = np.zeros((M, N), dtype=np.uint16)
        r = np.zeros((M, N), dtype=np.float64) if want_fp64 else None
        rc = self._lib.oracle_gemm_scale_relu(
            M, N, K, a.ctypes.data_as(_u16p), b.ctypes.data_as(_u16p), ctypes.c_float(alpha),
            c.ctypes.data_as(_u16p), r.ctypes.data_as(_f64p) if r is not None else None,
            int(nthreads or default_threads()))
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_scale_relu failed with code {rc}")
        return c, r

    def gemm_scale_relu_points(self, a_bits: np.ndarray, b_bits: np.ndarray, alpha: float,
                               ms: np.ndarray, ns: np.ndarray, nthreads: Optional[int] = None
                               ) -> Tuple[np.ndarray, np.ndarray]:
        """Outputs at (ms[i], ns[i]) only.  Returns (fp16 bits, fp64 values)."""
        a = np.ascontiguousarray(a_bits, dtype=np.uint16)
        b = np.ascontiguousarray(b_bits, dtype=np.uint16)
        if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
            raise ValueError(f"shape mismatch {a.shape} x {b.shape}")
        M, K = a.shape
        N = b.shape[1]
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        if ms.shape != ns.shape or ms.ndim != 1:
            raise ValueError("ms and ns must be 1-D and of equal length")
        out = np.zeros(ms.shape, dtype=np.uint16)
        r = np.zeros(ms.shape, dtype=np.float64)
        rc = self._lib.oracle_gemm_scale_relu_points(
            M, N, K, a.ctypes.data_as(_u16p), b.ctypes.data_as(_u16p), ctypes.c_float(alpha),
            ms.size, ms.ctypes.data_as(_i64p), ns.ctypes.data_as(_i64p),
            out.ctypes.data_as(_u16p), r.ctypes.data_as(_f64p), int(nthreads or default_threads()))
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_scale_relu_points failed with code {rc}")
        return out, r

    # -- the epilogue variants ---------------------------------------------
    def gelu(self, y: float) -> float:
        """The tanh-form GELU in binary64."""
        return float(self._lib.oracle_gelu(float(y)))

    def gemm_bias_act(self, a_bits: np.ndarray, b_bits: np.ndarray, bias_bits: Optional[np.ndarray],
                      alpha: float, act: int, nthreads: Optional[int] = None, want_fp64: bool = False
                      ) -> Tuple[np.ndarray, Optional[np.ndarray]]:
        """All outputs of act(alpha * A B + bias).  bias_bits: (N,) uint16 or
        None; act: ACT_RELU, ACT_GELU or ACT_NONE."""
        a = np.ascontiguousarray(a_bits, dtype=np.uint16)
        b = np.ascontiguousarray(b_bits, dtype=np.uint16)
        if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
            raise ValueError(f"shape mismatch {a.shape} x {b.shape}")
        M, K = a.shape
        N = b.shape[1]
        bias = None
        if bias_bits is not None:
            bias = np.ascontiguousarray(bias_bits, dtype=np.uint16)
            if bias.shape != (N,):
                raise ValueError(f"bias must have shape ({N},), got {bias.shape}")
        c = np.zeros((M, N), dtype=np.uint16)
        r = np.zeros((M, N), dtype=np.float64) if want_fp64 else None
        rc = self._lib.oracle_gemm_bias_act(
            M, N, K, a.ctypes.data_as(_u16p), b.ctypes.data_as(_u16p),
            bias.ctypes.data_as(_u16p) if bias is not None else None, ctypes.c_float(alpha), int(act),
            c.ctypes.data_as(_u16p), r.ctypes.data_as(_f64p) if r is not None else None,
            int(nthreads or default_threads()))
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_bias_act failed with code {rc}")
        return c, r

    def gemm_bias_act_points(self, a_bits: np.ndarray, b_bits: np.ndarray, bias_bits: Optional[np.ndarray],
                             alpha: float, act: int, ms: np.ndarray, ns: np.ndarray,
                             nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
        """act(alpha * A B + bias) at (ms[i], ns[i]) only."""
        a = np.ascontiguousarray(a_bits, dtype=np.uint16)
        b = np.ascontiguousarray(b_bits, dtype=np.uint16)
        if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
            raise ValueError(f"shape mismatch {a.shape} x {b.shape}")
        M, K = a.shape
        N = b.shape[1]
        bias = None
        if bias_bits is not None:
            bias = np.ascontiguousarray(bias_bits, dtype=np.uint16)
            if bias.shape != (N,):
                raise ValueError(f"bias must have shape ({N},), got {bias.shape}")
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        if ms.shape != ns.shape or ms.ndim != 1:
            raise ValueError("ms and ns must be 1-D and of equal length")
        out = np.zeros(ms.shape, dtype=np.uint16)
        r = np.zeros(ms.shape, dtype=np.float64)
        rc = self._lib.oracle_gemm_bias_act_points(
            M, N, K, a.ctypes.data_as(_u16p), b.ctypes.data_as(_u16p),
            bias.ctypes.data_as(_u16p) if bias is not None else None, ctypes.c_float(alpha), int(act),
            ms.size, ms.ctypes.data_as(_i64p), ns.ctypes.data_as(_i64p),
            out.ctypes.data_as(_u16p), r.ctypes.data_as(_f64p), int(nthreads or default_threads()))
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_bias_act_points failed with code {rc}")
        return out, r


def default_threads() -> int:
    """Host threads for the oracle: the CPUs this process may use, capped at
    16 (the host share of one GPU on a shared node)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


_DEFAULT: Optional[Oracle] = None


def load(build_if_missing: bool = True) -> Oracle:
    """The default oracle library, compiled with gcc on first use if absent."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(LIBRARY) and build_if_missing:
            build()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT
