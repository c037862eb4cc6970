"""Fused fp16 GEMM + scale + ReLU for AMD Instinct MI355X (gfx950).

    C = ReLU(alpha * A @ B)    A: (M,K) fp16, B: (K,N) fp16, C: (M,N) fp16

fp32 accumulation, scale and ReLU applied to the fp32 sum in registers, one
fp16 store (PKUHPC scow-tutorial "Tutorial14", section 3 display formula;
section 2 listing for the types and the epilogue order).

    C = act(alpha * A @ B + bias)    gemm_scale_bias_act: bias (N,) fp16 or
                                     None; act "relu", "gelu" (tanh form) or
                                     "none"

is the epilogue-variant family (the aikraft.ru TileLang guide, section 4,
GEMM + Bias + GELU) on the same kernels.

The compute runs in libgsr.so's hand-written HIP kernels; this package only
marshals torch tensors (device memory and the current stream) into the C ABI
of include/gsr.h.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _native
from ._native import (GsrError, clear_tuning, config_ids, get_config, load_tuning, num_configs, select_config,
                      status_string, tuning_entries, version, workspace_bytes)

__all__ = ["gemm_scale_relu", "gemm_scale_relu_ex", "gemm_scale_bias_act", "gemm_launch", "GsrError",
           "gemm_scale_relu_ws", "gemm_scale_bias_act_ws", "workspace_bytes", "new_workspace",
           "select_config", "get_config", "num_configs", "config_ids", "status_string", "version", "configs",
           "ACTIVATIONS",
           "load_tuning", "clear_tuning", "tuning_entries"]

ACTIVATIONS = {"relu": _native.GSR_ACT_RELU, "gelu": _native.GSR_ACT_GELU, "none": _native.GSR_ACT_NONE}


def _check_operands(a: torch.Tensor, b: torch.Tensor, c: Optional[torch.Tensor]):
    if a.dtype != torch.float16 or b.dtype != torch.float16:
        raise TypeError("A and B must be float16")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"shape mismatch: A {tuple(a.shape)} @ B {tuple(b.shape)}")
    if not (a.is_cuda and b.is_cuda):
        raise ValueError("A and B must be device tensors")
    if b.device != a.device:
        raise ValueError(f"A and B must be on one device, got {a.device} and {b.device}")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("A and B must be row-major contiguous")
    M, K = a.shape
    N = b.shape[1]
    if c is None:
        c = torch.empty((M, N), dtype=torch.float16, device=a.device)
    elif c.dtype != torch.float16 or tuple(c.shape) != (M, N) or not c.is_contiguous() or not c.is_cuda:
        raise ValueError("C must be a contiguous (M,N) float16 device tensor")
    elif c.device != a.device:
        raise ValueError(f"C must be on A's device {a.device}, got {c.device}")
    return int(M), int(N), int(K), c


def _stream_handle(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def gemm_scale_relu(a: torch.Tensor, b: torch.Tensor, alpha: float,
                    c: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """C = ReLU(alpha * a @ b), enqueued on `stream` (default: the current
    stream of a's device).  Allocates C when `c` is not given, as the
    tutorial's kernel wrapper does; returns C."""
    M, N, K, c = _check_operands(a, b, c)
    with torch.cuda.device(a.device):
        s = _stream_handle(a.device, stream)
        st = _native.gemm_scale_relu(M, N, K, a.data_ptr(), b.data_ptr(), c.data_ptr(), alpha, s)
    _native.check(st)
    return c


def gemm_scale_relu_ex(a: torch.Tensor, b: torch.Tensor, alpha: float, config_id: int,
                       c: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """As gemm_scale_relu with a forced tile configuration (-1 = selector)."""
    M, N, K, c = _check_operands(a, b, c)
    with torch.cuda.device(a.device):
        s = _stream_handle(a.device, stream)
        st = _native.gemm_scale_relu_ex(M, N, K, a.data_ptr(), b.data_ptr(), c.data_ptr(), alpha, s,
                                        config_id)
    _native.check(st)
    return c


def gemm_scale_bias_act(a: torch.Tensor, b: torch.Tensor, bias: Optional[torch.Tensor] = None,
                        alpha: float = 1.0, activation: str = "relu", c: Optional[torch.Tensor] = None,
                        stream=None, config_id: int = -1) -> torch.Tensor:
    """C = act(alpha * a @ b + bias), bias one fp16 value per output column
    (or None), act "relu", "gelu" or "none"; enqueued on `stream`.  With
    bias=None and "relu" it is gemm_scale_relu.  Returns C."""
    M, N, K, c = _check_operands(a, b, c)
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}, got {activation!r}")
    bptr = 0
    if bias is not None:
        if (bias.dtype != torch.float16 or tuple(bias.shape) != (N,) or not bias.is_cuda or not bias.is_contiguous()
                or bias.device != a.device):
            raise ValueError(f"bias must be a contiguous ({N},) float16 tensor on A's device")
        bptr = bias.data_ptr()
    with torch.cuda.device(a.device):
        s = _stream_handle(a.device, stream)
        st = _native.gemm_scale_bias_act(M, N, K, a.data_ptr(), b.data_ptr(), bptr, c.data_ptr(), alpha,
                                         ACTIVATIONS[activation], s, config_id)
    _native.check(st)
    return c


def new_workspace(nbytes: int, device=None) -> torch.Tensor:
    """A zero-filled workspace of `nbytes` bytes (uint8) for the entry points
    that split K across workgroups.  The kernels leave its counters at zero,
    so one workspace serves any number of calls in stream order; calls that
    may overlap need one each."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device if device is not None else "cuda")


def _check_workspace(workspace: torch.Tensor, device: torch.device):
    if (workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_cuda
            or not workspace.is_contiguous() or workspace.device != device):
        raise ValueError(f"workspace must be a contiguous 1-D uint8 tensor on {device}")
    return workspace.data_ptr(), workspace.numel()


def gemm_scale_bias_act_ws(a: torch.Tensor, b: torch.Tensor, workspace: torch.Tensor,
                           bias: Optional[torch.Tensor] = None, alpha: float = 1.0, activation: str = "relu",
                           c: Optional[torch.Tensor] = None, stream=None, config_id: int = -1,
                           splits: int = 0) -> torch.Tensor:
    """gemm_scale_bias_act with a workspace (see new_workspace), so that K
    can be split across workgroups: splits 0 is the library's choice, n >= 1
    at most n parts.  Returns C."""
    M, N, K, c = _check_operands(a, b, c)
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}, got {activation!r}")
    bptr = 0
    if bias is not None:
        if (bias.dtype != torch.float16 or tuple(bias.shape) != (N,) or not bias.is_cuda or not bias.is_contiguous()
                or bias.device != a.device):
            raise ValueError(f"bias must be a contiguous ({N},) float16 tensor on A's device")
        bptr = bias.data_ptr()
    wptr, wbytes = _check_workspace(workspace, a.device)
    with torch.cuda.device(a.device):
        s = _stream_handle(a.device, stream)
        st = _native.gemm_scale_bias_act_ws(M, N, K, a.data_ptr(), b.data_ptr(), bptr, c.data_ptr(), alpha,
                                            ACTIVATIONS[activation], wptr, wbytes, s, config_id, splits)
    _native.check(st)
    return c


def gemm_scale_relu_ws(a: torch.Tensor, b: torch.Tensor, alpha: float, workspace: torch.Tensor,
                       c: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """gemm_scale_relu with a workspace (see new_workspace and
    workspace_bytes): the library may split K across workgroups.  Returns C."""
    M, N, K, c = _check_operands(a, b, c)
    wptr, wbytes = _check_workspace(workspace, a.device)
    with torch.cuda.device(a.device):
        s = _stream_handle(a.device, stream)
        st = _native.gemm_scale_relu_ws(M, N, K, a.data_ptr(), b.data_ptr(), c.data_ptr(), alpha, wptr, wbytes, s)
    _native.check(st)
    return c


def gemm_launch(a: torch.Tensor, b: torch.Tensor, alpha: float, config_id: int, group_m: int, xcd_remap: int,
                bias: Optional[torch.Tensor] = None, activation: str = "relu", c: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """act(alpha * a @ b + bias) with an explicit launch: tile configuration,
    tile rows per launch group and XCD regrouping (tuning sweeps)."""
    M, N, K, c = _check_operands(a, b, c)
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}, got {activation!r}")
    bptr = 0
    if bias is not None:
        if (bias.dtype != torch.float16 or tuple(bias.shape) != (N,) or not bias.is_cuda or not bias.is_contiguous()
                or bias.device != a.device):
            raise ValueError(f"bias must be a contiguous ({N},) float16 tensor on A's device")
        bptr = bias.data_ptr()
    with torch.cuda.device(a.device):
        s = _stream_handle(a.device, stream)
        st = _native.gemm_scale_bias_act_cfg(M, N, K, a.data_ptr(), b.data_ptr(), bptr, c.data_ptr(), alpha,
                                             ACTIVATIONS[activation], s, config_id, group_m, xcd_remap)
    _native.check(st)
    return c


def configs() -> list:
    """Every compiled tile configuration, by ascending id."""
    return [get_config(i) for i in config_ids()]
