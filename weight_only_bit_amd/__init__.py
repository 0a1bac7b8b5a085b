"""MI355X (gfx950) weight-only 4-bit GEMM: Python binding of the C-ABI library.

Argument marshalling only: tensors supply device memory and
``torch.cuda.current_stream()`` supplies the stream; every step of the
computation runs in the library's HIP kernels (``csrc/``).  There is no CPU
fallback.

    y = gemm(x, qweight, scales, qzeros, group_size)        # W4A16
    y = gemm_grouped(x, m_offsets, qweight, scales, qzeros, group_size)
    y = mxfp4_moe_gemm(x, topk_ids, w_fp4, w_scale)         # MoE stage 1
    y = mxfp4_moe_stage2(a, topk_ids, topk_weights, w2_fp4, w2_scale)  # MoE stage 2

Layouts are those of ``include/weight_only_bit.h``.
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import (ACT_NONE, ACT_SILU_MUL, BF16, DTYPE, F16, F32, INVALID_ARG, OK, PATH_AUTO,
                   PATH_SKINNY, PATH_TILED, U4X8_I32, UNSUPPORTED, WobArgError, WobDtypeError,
                   WobError)

__all__ = [
    "gemm", "gemm_grouped", "mxfp4_moe_gemm", "moe_workspace_size", "mxfp4_moe_stage2",
    "moe_stage2_workspace_size", "w4a16_dequant",
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


# Shape and dtype checks.  They read only .shape and .dtype, so they run
# before any device access (and work on CPU or meta tensors): the C ABI sees
# raw pointers and could not detect an operand smaller than its shape says.

def _want(t, name, shape, dtypes):
    """t must exist, have exactly `shape`, and one of `dtypes`."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected one of {[str(d) for d in dtypes]}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")


def _act_dtypes():
    torch = _torch()
    return (torch.float16, torch.bfloat16)


def _w4_group_count(K: int, group_size: int) -> int:
    if group_size <= 0 or K % group_size != 0:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")
    return K // group_size


def _check_w4_weights(qweight, scales, qzeros, N, K, group_size, act, lead=()):
    """qweight [*lead, N, K/8] int32; scales [*lead, N, K/g] act; qzeros
    [*lead, N/8, K/g] int32 or None (activation-dtype zero-points are refused)."""
    torch = _torch()
    if K % 8 != 0 or N % 8 != 0:
        raise ValueError(f"K={K} and N={N} must be multiples of 8")
    G = _w4_group_count(K, group_size)
    _want(qweight, "qweight", (*lead, N, K // 8), (torch.int32,))
    _want(scales, "scales", (*lead, N, G), (act,))
    if qzeros is not None:
        if qzeros.dtype != torch.int32:
            raise TypeError(f"qzeros must be packed 4-bit zero-points (int32); dtype {qzeros.dtype} "
                            "is refused, not reinterpreted")
        _want(qzeros, "qzeros", (*lead, N // 8, G), (torch.int32,))


def device_check() -> None:
    """Raise unless the current device is gfx950."""
    _lib.check(_lib.lib().wob_device_check(), "device_check")


def gemm(x, qweight, scales, qzeros, group_size: int, out=None, path: int = PATH_AUTO):
    """W4A16 GEMM: y[M,N] = x[M,K] . ((q - z) * s)^T.

    x [M,K] fp16/bf16; qweight [N,K/8] int32; scales [N,K/g] x.dtype;
    qzeros [N/8,K/g] int32 (packed) or None (symmetric, z = 8); out [M,N] x.dtype.
    """
    torch = _torch()
    if x.dim() != 2 or qweight.dim() != 2:
        raise ValueError("x must be [M, K] and qweight [N, K/8]")
    _want(x, "x", tuple(x.shape), _act_dtypes())
    M, K = x.shape
    N = qweight.shape[0]
    _check_w4_weights(qweight, scales, qzeros, N, K, group_size, x.dtype)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _want(out, "out", (M, N), (x.dtype,))
    dev = _check_device(x, qweight, scales, qzeros, out)
    with torch.cuda.device(dev):
        st = _lib.lib().w4a16_gemm_ex(
            _ptr(x), _tag(x), _ptr(qweight), _ptr(scales), _tag(scales), _ptr(qzeros),
            _tag(qzeros) if qzeros is not None else U4X8_I32, _ptr(out), M, N, K, group_size,
            path, _stream(dev))
    _lib.check(st, "w4a16_gemm")
    return out


def gemm_grouped(x, m_offsets, qweight, scales, qzeros, group_size: int, out=None):
    """Ragged grouped W4A16 GEMM: x [total_M,K]; m_offsets device int64 [E+1];
    qweight [E,N,K/8] int32; scales [E,N,K/g]; qzeros [E,N/8,K/g] int32 or None;
    out [total_M,N] x.dtype."""
    torch = _torch()
    if x.dim() != 2 or qweight.dim() != 3:
        raise ValueError("x must be [total_M, K] and qweight [E, N, K/8]")
    _want(x, "x", tuple(x.shape), _act_dtypes())
    total_m, K = x.shape
    E, N = qweight.shape[0], qweight.shape[1]
    _check_w4_weights(qweight, scales, qzeros, N, K, group_size, x.dtype, lead=(E,))
    _want(m_offsets, "m_offsets", (E + 1,), (torch.int64,))
    if out is None:
        out = torch.empty((total_m, N), dtype=x.dtype, device=x.device)
    _want(out, "out", (total_m, N), (x.dtype,))
    dev = _check_device(x, m_offsets, qweight, scales, qzeros, out)
    with torch.cuda.device(dev):
        st = _lib.lib().w4a16_gemm_grouped(
            _ptr(x), _tag(x), _ptr(m_offsets), E, total_m, _ptr(qweight), _ptr(scales),
            _tag(scales), _ptr(qzeros), _tag(qzeros) if qzeros is not None else U4X8_I32,
            _ptr(out), N, K, group_size, _stream(dev))
    _lib.check(st, "w4a16_gemm_grouped")
    return out


def moe_workspace_size(T: int, topk: int, E: int, N: int = 0, K: int = 0) -> int:
    """Bytes of workspace mxfp4_moe_gemm needs (0 for arguments it refuses)."""
    return int(_lib.lib().mxfp4_moe_gemm_workspace_size(T, topk, E, N, K))


def mxfp4_moe_gemm(x, topk_ids, w_fp4, w_scale, out=None, workspace=None, act: int = ACT_NONE,
                   tile_m: int = 32):
    """MoE stage 1: x [T,K] bf16, topk_ids [T,topk] int32, w_fp4 [E,N,K/2] uint8 and
    w_scale [E,N,K/32] uint8 (E8M0) -> y [T,topk,N] bf16 (act=ACT_NONE) or
    y [T,topk,N/2] = silu(gate) * up (act=ACT_SILU_MUL).  workspace: device memory of
    at least moe_workspace_size(T, topk, E, N, K) bytes (allocated when None).
    tile_m: 32 (the default, mxfp4_moe_gemm) or 16 (mxfp4_moe_gemm_tile_m), the
    row padding of each expert's tile."""
    torch = _torch()
    if x.dim() != 2 or topk_ids.dim() != 2 or w_fp4.dim() != 3:
        raise ValueError("x must be [T, K], topk_ids [T, topk] and w_fp4 [E, N, K/2]")
    _want(x, "x", tuple(x.shape), (torch.bfloat16,))
    T, K = x.shape
    topk = topk_ids.shape[1]
    E, N = w_fp4.shape[0], w_fp4.shape[1]
    if K % 32 != 0:
        raise ValueError(f"K={K} must be a multiple of 32 (one E8M0 scale per 32)")
    _want(topk_ids, "topk_ids", (T, topk), (torch.int32,))
    _want(w_fp4, "w_fp4", (E, N, K // 2), (torch.uint8,))
    _want(w_scale, "w_scale", (E, N, K // 32), (torch.uint8,))
    if act not in (ACT_NONE, ACT_SILU_MUL):
        raise ValueError(f"unknown activation {act}")
    if tile_m not in (16, 32):
        raise ValueError(f"tile_m={tile_m} must be 16 or 32")
    nout = N // 2 if act == ACT_SILU_MUL else N
    if out is None:
        out = torch.empty((T, topk, nout), dtype=torch.bfloat16, device=x.device)
    _want(out, "out", (T, topk, nout), (torch.bfloat16,))
    need = moe_workspace_size(T, topk, E, N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    if ws_bytes < need:
        raise ValueError(f"workspace holds {ws_bytes} bytes; {need} are needed")
    dev = _check_device(x, topk_ids, w_fp4, w_scale, out, workspace)
    with torch.cuda.device(dev):
        if tile_m == 32:
            st = _lib.lib().mxfp4_moe_gemm(
                _ptr(x), _ptr(topk_ids), _ptr(w_fp4), _ptr(w_scale), _ptr(out), T, topk, E, N, K,
                act, _ptr(workspace), ws_bytes, _stream(dev))
        else:
            st = _lib.lib().mxfp4_moe_gemm_tile_m(
                _ptr(x), _ptr(topk_ids), _ptr(w_fp4), _ptr(w_scale), _ptr(out), T, topk, E, N, K,
                act, tile_m, _ptr(workspace), ws_bytes, _stream(dev))
    _lib.check(st, "mxfp4_moe_gemm")
    return out


def moe_stage2_workspace_size(T: int, topk: int, E: int, H: int, I: int) -> int:
    """Bytes of workspace mxfp4_moe_stage2 needs (0 for arguments it refuses)."""
    return int(_lib.lib().mxfp4_moe_stage2_workspace_size(T, topk, E, H, I))


def mxfp4_moe_stage2(a, topk_ids, topk_weights, w2_fp4, w2_scale, out=None, workspace=None):
    """MoE stage 2: a [T,topk,I] bf16 (the stage-1 activation rows), topk_ids
    [T,topk] int32, topk_weights [T,topk] float32, w2_fp4 [E,H,I/2] uint8,
    w2_scale [E,H,I/32] uint8 (E8M0) -> y [T,H] bf16 = sum over slots of
    weight * (a row . expert's W2)."""
    torch = _torch()
    if a.dim() != 3 or topk_ids.dim() != 2 or w2_fp4.dim() != 3:
        raise ValueError("a must be [T, topk, I], topk_ids [T, topk] and w2_fp4 [E, H, I/2]")
    _want(a, "a", tuple(a.shape), (torch.bfloat16,))
    T, topk, I = a.shape
    E, H = w2_fp4.shape[0], w2_fp4.shape[1]
    if I % 32 != 0:
        raise ValueError(f"I={I} must be a multiple of 32 (one E8M0 scale per 32)")
    _want(topk_ids, "topk_ids", (T, topk), (torch.int32,))
    _want(topk_weights, "topk_weights", (T, topk), (torch.float32,))
    _want(w2_fp4, "w2_fp4", (E, H, I // 2), (torch.uint8,))
    _want(w2_scale, "w2_scale", (E, H, I // 32), (torch.uint8,))
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=a.device)
    _want(out, "out", (T, H), (torch.bfloat16,))
    need = moe_stage2_workspace_size(T, topk, E, H, I)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    if ws_bytes < need:
        raise ValueError(f"workspace holds {ws_bytes} bytes; {need} are needed")
    dev = _check_device(a, topk_ids, topk_weights, w2_fp4, w2_scale, out, workspace)
    with torch.cuda.device(dev):
        st = _lib.lib().mxfp4_moe_stage2(
            _ptr(a), _ptr(topk_ids), _ptr(topk_weights), _ptr(w2_fp4), _ptr(w2_scale), _ptr(out),
            T, topk, E, H, I, _ptr(workspace), ws_bytes, _stream(dev))
    _lib.check(st, "mxfp4_moe_stage2")
    return out


def w4a16_dequant(qweight, scales, qzeros, group_size: int, out_dtype=None):
    """Probe: the kernels' dequantized weights [N,K] (float32 skinny form, or
    the scales' dtype for the MFMA operand form)."""
    torch = _torch()
    if qweight.dim() != 2:
        raise ValueError("qweight must be [N, K/8]")
    N, K = qweight.shape[0], qweight.shape[1] * 8
    if scales.dtype not in _act_dtypes():
        raise TypeError(f"scales must be float16 or bfloat16, not {scales.dtype}")
    _check_w4_weights(qweight, scales, qzeros, N, K, group_size, scales.dtype)
    out_dtype = out_dtype or torch.float32
    if out_dtype not in (torch.float32, scales.dtype):
        raise TypeError("out_dtype must be float32 or the scales' dtype")
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
    """Probe: the MoE kernels' bf16 weight-operand values [N,K] for one expert."""
    torch = _torch()
    if w_fp4.dim() != 2:
        raise ValueError("w_fp4 must be [N, K/2]")
    N, K = w_fp4.shape[0], w_fp4.shape[1] * 2
    if K % 32 != 0:
        raise ValueError(f"K={K} must be a multiple of 32")
    _want(w_fp4, "w_fp4", (N, K // 2), (torch.uint8,))
    _want(w_scale, "w_scale", (N, K // 32), (torch.uint8,))
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
    if nbytes > buf.numel() * buf.element_size() or sink.numel() * sink.element_size() < 1024:
        raise ValueError("buffer smaller than nbytes or sink under 1024 bytes")
    dev = _check_device(buf, sink)
    with torch.cuda.device(dev):
        st = _lib.lib().wob_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(dev))
    _lib.check(st, "wob_stream_read")
