"""MI355X (gfx950) weight-only 4-bit GEMM: Python binding of the C-ABI library.

Argument marshalling only: tensors supply device memory and
``torch.cuda.current_stream()`` supplies the stream; every step of the
computation runs in the library's HIP kernels (``csrc/``).  There is no CPU
fallback.

    y = gemm(x, qweight, scales, qzeros, group_size)        # W4A16
    y = gemm_grouped(x, m_offsets, qweight, scales, qzeros, group_size)
    y = mxfp4_moe_gemm(x, topk_ids, w_fp4, w_scale)         # MoE stage 1

Layouts are those of ``include/weight_only_bit.h``.
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import (ACT_NONE, ACT_SILU_MUL, BF16, DTYPE, F16, F32, INVALID_ARG, OK, PATH_AUTO,
                   PATH_SKINNY, PATH_TILED, U4X8_I32, UNSUPPORTED, WobArgError, WobDtypeError,
                   WobError)

__all__ = [
    "gemm", "gemm_grouped", "mxfp4_moe_gemm", "moe_workspace_size", "w4a16_dequant",
    "mxfp4_dequant", "stream_read", "device_check", "WobError", "WobDtypeError", "WobArgError",
    "PATH_AUTO", "PATH_SKINNY", "PATH_TILED", "ACT_NONE", "ACT_SILU_MUL",
]


def _torch():
    import torch
    return torch


def _tag(t):
    torch = _torch()
    return {torch.float16: F16, torch.bfloat16: BF16, torch.int32: U4X8_I32,
            torch.float32: F32}.get(t.dtype, -1)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_device(*tensors):
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all operands must be device tensors")
        if not t.is_contiguous():
            raise ValueError("all operands must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("operands live on different devices")
    return dev


def device_check() -> None:
    """Raise unless the current device is gfx950."""
    _lib.check(_lib.lib().wob_device_check(), "device_check")


def gemm(x, qweight, scales, qzeros, group_size: int, out=None, path: int = PATH_AUTO):
    """W4A16 GEMM: y[M,N] = x[M,K] . ((q - z) * s)^T.

    x [M,K] fp16/bf16; qweight [N,K/8] int32; scales [N,K/g] x.dtype;
    qzeros [N/8,K/g] int32 (packed) or None (symmetric, z = 8).
    """
    torch = _torch()
    M, K = x.shape
    N = qweight.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    dev = _check_device(x, qweight, scales, qzeros, out)
    with torch.cuda.device(dev):
        st = _lib.lib().w4a16_gemm_ex(
            _ptr(x), _tag(x), _ptr(qweight), _ptr(scales), _tag(scales), _ptr(qzeros),
            _tag(qzeros) if qzeros is not None else U4X8_I32, _ptr(out), M, N, K, group_size,
            path, _stream(dev))
    _lib.check(st, "w4a16_gemm")
    return out


def gemm_grouped(x, m_offsets, qweight, scales, qzeros, group_size: int, out=None):
    """Ragged grouped W4A16 GEMM; m_offsets is a device int64 tensor [E+1]."""
    torch = _torch()
    total_m, K = x.shape
    E, N = qweight.shape[0], qweight.shape[1]
    if m_offsets.dtype != torch.int64 or m_offsets.numel() != E + 1:
        raise ValueError("m_offsets must be int64 with num_groups + 1 entries")
    if out is None:
        out = torch.empty((total_m, N), dtype=x.dtype, device=x.device)
    dev = _check_device(x, m_offsets, qweight, scales, qzeros, out)
    with torch.cuda.device(dev):
        st = _lib.lib().w4a16_gemm_grouped(
            _ptr(x), _tag(x), _ptr(m_offsets), E, total_m, _ptr(qweight), _ptr(scales),
            _tag(scales), _ptr(qzeros), _tag(qzeros) if qzeros is not None else U4X8_I32,
            _ptr(out), N, K, group_size, _stream(dev))
    _lib.check(st, "w4a16_gemm_grouped")
    return out


def moe_workspace_size(T: int, topk: int, E: int) -> int:
    return int(_lib.lib().mxfp4_moe_gemm_workspace_size(T, topk, E))


def mxfp4_moe_gemm(x, topk_ids, w_fp4, w_scale, out=None, workspace=None, act: int = ACT_NONE):
    """MoE stage 1: x [T,K] bf16, topk_ids [T,topk] int32, w_fp4 [E,N,K/2] uint8 and
    w_scale [E,N,K/32] uint8 (E8M0) -> y [T,topk,N] bf16 (act=ACT_NONE) or
    y [T,topk,N/2] = silu(gate) * up (act=ACT_SILU_MUL)."""
    torch = _torch()
    T, K = x.shape
    topk = topk_ids.shape[1]
    E, N = w_fp4.shape[0], w_fp4.shape[1]
    if x.dtype != torch.bfloat16 or topk_ids.dtype != torch.int32:
        raise TypeError("x must be bfloat16 and topk_ids int32")
    if w_fp4.dtype != torch.uint8 or w_scale.dtype != torch.uint8:
        raise TypeError("w_fp4 and w_scale must be uint8")
    if out is None:
        nout = N // 2 if act == ACT_SILU_MUL else N
        out = torch.empty((T, topk, nout), dtype=torch.bfloat16, device=x.device)
    need = moe_workspace_size(T, topk, E)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    dev = _check_device(x, topk_ids, w_fp4, w_scale, out, workspace)
    with torch.cuda.device(dev):
        st = _lib.lib().mxfp4_moe_gemm_act(
            _ptr(x), _ptr(topk_ids), _ptr(w_fp4), _ptr(w_scale), _ptr(out), T, topk, E, N, K, act,
            _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check(st, "mxfp4_moe_gemm")
    return out


def w4a16_dequant(qweight, scales, qzeros, group_size: int, out_dtype=None):
    """Probe: the kernels' dequantized weights [N,K] (float32 skinny form, or
    the scales' dtype for the MFMA operand form)."""
    torch = _torch()
    N = qweight.shape[0]
    K = qweight.shape[1] * 8
    out_dtype = out_dtype or torch.float32
    out = torch.empty((N, K), dtype=out_dtype, device=qweight.device)
    dev = _check_device(qweight, scales, qzeros, out)
    with torch.cuda.device(dev):
        st = _lib.lib().w4a16_dequant(
            _ptr(qweight), _ptr(scales), _tag(scales), _ptr(qzeros),
            _tag(qzeros) if qzeros is not None else U4X8_I32, _ptr(out), _tag(out), N, K,
            group_size, _stream(dev))
    _lib.check(st, "w4a16_dequant")
    return out


def mxfp4_dequant(w_fp4, w_scale):
    """Probe: the MoE kernel's bf16 B-operand values [N,K] for one expert."""
    torch = _torch()
    N = w_fp4.shape[0]
    K = w_fp4.shape[1] * 2
    out = torch.empty((N, K), dtype=torch.bfloat16, device=w_fp4.device)
    dev = _check_device(w_fp4, w_scale, out)
    with torch.cuda.device(dev):
        st = _lib.lib().mxfp4_dequant(_ptr(w_fp4), _ptr(w_scale), _ptr(out), N, K, _stream(dev))
    _lib.check(st, "mxfp4_dequant")
    return out


def stream_read(buf, nbytes: int, sink) -> None:
    """Measurement aid: read nbytes of the device tensor buf once (the device's
    streaming-read reference for a byte count); sink: >= 1024 bytes of scratch."""
    torch = _torch()
    dev = _check_device(buf, sink)
    if nbytes > buf.numel() * buf.element_size() or sink.numel() * sink.element_size() < 1024:
        raise ValueError("buffer smaller than nbytes or sink under 1024 bytes")
    with torch.cuda.device(dev):
        st = _lib.lib().wob_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(dev))
    _lib.check(st, "wob_stream_read")
