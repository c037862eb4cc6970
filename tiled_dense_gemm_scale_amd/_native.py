"""ctypes binding of libgsr.so (include/gsr.h).  Argument marshalling only:
every step of the operation runs in the library's HIP kernels.

The library is loaded on first use.  If it has not been built the call raises
at once -- there is no fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgsr.so")

GSR_SUCCESS = 0
GSR_ERROR_INVALID_VALUE = 1
GSR_ERROR_TOO_LARGE = 2
GSR_ERROR_NO_DEVICE = 3
GSR_ERROR_UNSUPPORTED_DEVICE = 4
GSR_ERROR_LAUNCH = 5
GSR_ERROR_INVALID_CONFIG = 6

GSR_ACT_RELU = 0
GSR_ACT_GELU = 1
GSR_ACT_NONE = 2


class GsrConfig(ctypes.Structure):
    """Mirror of struct gsr_config."""
    _fields_ = [
        ("id", ctypes.c_int32),
        ("block_m", ctypes.c_int32),
        ("block_n", ctypes.c_int32),
        ("block_k", ctypes.c_int32),
        ("waves_m", ctypes.c_int32),
        ("waves_n", ctypes.c_int32),
        ("stages", ctypes.c_int32),
        ("group_m", ctypes.c_int32),
        ("xcd_remap", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


class GsrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libgsr.so; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY):
                raise RuntimeError(
                    f"{LIBRARY} is not built: run `python -m tiled_dense_gemm_scale_amd.build` "
                    "(there is no non-HIP fallback)")
            L = ctypes.CDLL(LIBRARY)
            i64, vp, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int32
            L.gemm_scale_relu.argtypes = [i64, i64, i64, vp, vp, vp, f32, vp]
            L.gemm_scale_relu.restype = ctypes.c_int
            L.gemm_scale_relu_ex.argtypes = [i64, i64, i64, vp, vp, vp, f32, vp, i32]
            L.gemm_scale_relu_ex.restype = ctypes.c_int
            L.gemm_scale_bias_act.argtypes = [i64, i64, i64, vp, vp, vp, vp, f32, i32, vp]
            L.gemm_scale_bias_act.restype = ctypes.c_int
            L.gemm_scale_bias_act_ex.argtypes = [i64, i64, i64, vp, vp, vp, vp, f32, i32, vp, i32]
            L.gemm_scale_bias_act_ex.restype = ctypes.c_int
            L.gemm_scale_bias_act_cfg.argtypes = [i64, i64, i64, vp, vp, vp, vp, f32, i32, vp,
                                                   ctypes.POINTER(GsrConfig)]
            L.gemm_scale_bias_act_cfg.restype = ctypes.c_int
            L.gemm_scale_bias_act_ws.argtypes = [i64, i64, i64, vp, vp, vp, vp, f32, i32, vp, i64, vp, i32, i32]
            L.gemm_scale_bias_act_ws.restype = ctypes.c_int
            L.gemm_scale_relu_ws.argtypes = [i64, i64, i64, vp, vp, vp, f32, vp, i64, vp]
            L.gemm_scale_relu_ws.restype = ctypes.c_int
            L.gemm_scale_bias_act_noalloc.argtypes = [i64, i64, i64, vp, vp, vp, vp, f32, i32, vp, i32, i32]
            L.gemm_scale_bias_act_noalloc.restype = ctypes.c_int
            L.gsr_workspace_bytes.argtypes = [i64, i64, i64]
            L.gsr_workspace_bytes.restype = i64
            L.gsr_load_tuning.argtypes = [ctypes.c_char_p]
            L.gsr_load_tuning.restype = ctypes.c_int
            L.gsr_clear_tuning.argtypes = []
            L.gsr_clear_tuning.restype = ctypes.c_int
            L.gsr_tuning_entries.argtypes = []
            L.gsr_tuning_entries.restype = ctypes.c_int
            L.gsr_select_config.argtypes = [i64, i64, i64, ctypes.POINTER(GsrConfig)]
            L.gsr_select_config.restype = ctypes.c_int
            L.gsr_num_configs.argtypes = []
            L.gsr_num_configs.restype = ctypes.c_int
            L.gsr_config_ids.argtypes = [ctypes.POINTER(i32), i32]
            L.gsr_config_ids.restype = ctypes.c_int
            L.gsr_get_config.argtypes = [i32, ctypes.POINTER(GsrConfig)]
            L.gsr_get_config.restype = ctypes.c_int
            L.gsr_status_string.argtypes = [ctypes.c_int]
            L.gsr_status_string.restype = ctypes.c_char_p
            L.gsr_version.argtypes = []
            L.gsr_version.restype = ctypes.c_int
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().gsr_status_string(int(status)).decode()


def check(status: int) -> None:
    if status != GSR_SUCCESS:
        raise GsrError(status, status_string(status))


def gemm_scale_relu(M: int, N: int, K: int, A: int, B: int, C: int, alpha: float, stream: int) -> int:
    """Raw entry point: device addresses and a hipStream_t as integers.
    Returns the gsr_status."""
    return lib().gemm_scale_relu(M, N, K, A or None, B or None, C or None, float(alpha), stream or None)


def gemm_scale_relu_ex(M: int, N: int, K: int, A: int, B: int, C: int, alpha: float, stream: int,
                       config_id: int) -> int:
    return lib().gemm_scale_relu_ex(M, N, K, A or None, B or None, C or None, float(alpha),
                                    stream or None, int(config_id))


def gemm_scale_bias_act(M: int, N: int, K: int, A: int, B: int, bias: int, C: int, alpha: float,
                        activation: int, stream: int, config_id: int = -1) -> int:
    """Raw entry point of the epilogue variants (bias 0 = none).  Returns the
    gsr_status."""
    return lib().gemm_scale_bias_act_ex(M, N, K, A or None, B or None, bias or None, C or None, float(alpha),
                                        int(activation), stream or None, int(config_id))


def gemm_scale_bias_act_cfg(M: int, N: int, K: int, A: int, B: int, bias: int, C: int, alpha: float,
                            activation: int, stream: int, config_id: int, group_m: int, xcd_remap: int) -> int:
    """Raw entry point with an explicit launch (tile config id, group_m,
    xcd_remap).  Returns the gsr_status."""
    cfg = GsrConfig()
    cfg.id, cfg.group_m, cfg.xcd_remap = int(config_id), int(group_m), int(xcd_remap)
    return lib().gemm_scale_bias_act_cfg(M, N, K, A or None, B or None, bias or None, C or None, float(alpha),
                                         int(activation), stream or None, ctypes.byref(cfg))


def gemm_scale_bias_act_ws(M: int, N: int, K: int, A: int, B: int, bias: int, C: int, alpha: float,
                           activation: int, workspace: int, workspace_bytes: int, stream: int,
                           config_id: int = -1, splits: int = 0) -> int:
    """Raw entry point with a workspace (K split across workgroups).
    Returns the gsr_status."""
    return lib().gemm_scale_bias_act_ws(M, N, K, A or None, B or None, bias or None, C or None, float(alpha),
                                        int(activation), workspace or None, int(workspace_bytes), stream or None,
                                        int(config_id), int(splits))


def gemm_scale_relu_ws(M: int, N: int, K: int, A: int, B: int, C: int, alpha: float, workspace: int,
                       workspace_bytes: int, stream: int) -> int:
    return lib().gemm_scale_relu_ws(M, N, K, A or None, B or None, C or None, float(alpha), workspace or None,
                                    int(workspace_bytes), stream or None)


def gemm_scale_bias_act_noalloc(M: int, N: int, K: int, A: int, B: int, bias: int, C: int, alpha: float,
                                activation: int, stream: int, config_id: int = -1, splits: int = 0) -> int:
    """Raw entry point that allocates nothing: the K split's workspace is
    the library's per-device scratch array.  Returns the gsr_status."""
    return lib().gemm_scale_bias_act_noalloc(M, N, K, A or None, B or None, bias or None, C or None, float(alpha),
                                             int(activation), stream or None, int(config_id), int(splits))


def workspace_bytes(M: int, N: int, K: int) -> int:
    """Workspace bytes the library's K split needs for this shape (0: none)."""
    got = int(lib().gsr_workspace_bytes(int(M), int(N), int(K)))
    if got < 0:
        raise GsrError(GSR_ERROR_INVALID_VALUE, status_string(GSR_ERROR_INVALID_VALUE))
    return got


def load_tuning(path: str) -> None:
    """Load a tuning table (text: "M N K config_id group_m xcd_remap" per line)."""
    check(lib().gsr_load_tuning(os.fsencode(path)))


def clear_tuning() -> None:
    check(lib().gsr_clear_tuning())


def tuning_entries() -> int:
    return int(lib().gsr_tuning_entries())


def select_config(M: int, N: int, K: int) -> dict:
    out = GsrConfig()
    check(lib().gsr_select_config(M, N, K, ctypes.byref(out)))
    return out.as_dict()


def num_configs() -> int:
    return int(lib().gsr_num_configs())


def config_ids() -> list:
    """The ids of the compiled tile configurations, ascending (ids are stable
    across library versions and not contiguous)."""
    n = int(lib().gsr_num_configs())
    buf = (ctypes.c_int32 * max(n, 1))()
    got = int(lib().gsr_config_ids(buf, n))
    if got != n:
        raise GsrError(GSR_ERROR_INVALID_VALUE, f"gsr_config_ids returned {got}, expected {n}")
    return [int(buf[i]) for i in range(n)]


def get_config(config_id: int) -> dict:
    out = GsrConfig()
    check(lib().gsr_get_config(int(config_id), ctypes.byref(out)))
    return out.as_dict()


def version() -> int:
    return int(lib().gsr_version())
