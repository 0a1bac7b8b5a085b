"""ctypes wrapper around the C reference oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module; the ``weight_only_bit_amd`` library never
imports it and has no CPU fallback.  The oracle is single-threaded C that
dequantizes each weight exactly in binary32 and accumulates in binary64
(definitions and readings in the header of ``oracle.c``).

Functions whose parity is not pinned by a test independent of the oracle:
none (every entry point is covered by ``tests/test_oracle_*.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F16 = 0
BF16 = 1

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc -O2 (no fast-math, no threads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
             "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = ctypes.CDLL(_LIB)
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --- codecs -----------------------------------------------------------------

def f16_decode(bits):
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_f16_decode(_p(bits), _p(out), ctypes.c_int64(bits.size))
    return out


def bf16_decode(bits):
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_bf16_decode(_p(bits), _p(out), ctypes.c_int64(bits.size))
    return out


def act_decode(bits, dtype):
    return f16_decode(bits) if dtype == F16 else bf16_decode(bits)


def f16_encode(values):
    v = _c(values, np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_f16_encode(_p(v), _p(out), ctypes.c_int64(v.size))
    return out


def bf16_encode(values):
    v = _c(values, np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_bf16_encode(_p(v), _p(out), ctypes.c_int64(v.size))
    return out


def e2m1_decode(codes):
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e2m1_decode(_p(c), _p(out), ctypes.c_int64(c.size))
    return out


def e8m0_decode(b):
    b = _c(b, np.uint8)
    out = np.empty(b.shape, np.float64)
    _load().oracle_e8m0_decode(_p(b), _p(out), ctypes.c_int64(b.size))
    return out


# --- W4A16 ------------------------------------------------------------------

def w4a16_unpack_codes(qweight, N, K):
    qw = _c(qweight, np.int32)
    out = np.empty((N, K), np.uint8)
    _load().oracle_w4a16_unpack_codes(_p(qw), ctypes.c_int64(N), ctypes.c_int64(K), _p(out))
    return out


def w4a16_unpack_zeros(qzeros, N, G):
    qz = _c(qzeros, np.int32)
    out = np.empty((N, G), np.uint8)
    _load().oracle_w4a16_unpack_zeros(_p(qz), ctypes.c_int64(N), ctypes.c_int64(G), _p(out))
    return out


def w4a16_dequant(qweight, scales, sdtype, qzeros, N, K, g):
    """Exact binary32 dequantized weights [N][K]."""
    qw = _c(qweight, np.int32)
    sc = _c(scales, np.uint16)
    qz = None if qzeros is None else _c(qzeros, np.int32)
    out = np.empty((N, K), np.float32)
    _load().oracle_w4a16_dequant(_p(qw), _p(sc), ctypes.c_int(sdtype), _p(qz), ctypes.c_int64(N),
                                 ctypes.c_int64(K), ctypes.c_int64(g), _p(out))
    return out


def w4a16_dequant_act(qweight, scales, sdtype, qzeros, N, K, g):
    """Dequantized weights rounded (RNE) to the activation dtype, as uint16 bits [N][K]."""
    qw = _c(qweight, np.int32)
    sc = _c(scales, np.uint16)
    qz = None if qzeros is None else _c(qzeros, np.int32)
    scratch = np.empty(K, np.float32)
    out = np.empty((N, K), np.uint16)
    _load().oracle_w4a16_dequant_act(_p(qw), _p(sc), ctypes.c_int(sdtype), _p(qz),
                                     ctypes.c_int64(N), ctypes.c_int64(K), ctypes.c_int64(g),
                                     _p(scratch), _p(out))
    return out


def w4a16_gemm(x, xdtype, qweight, scales, qzeros, M, N, K, g):
    """fp64 y[M][N]."""
    xx = _c(x, np.uint16)
    qw = _c(qweight, np.int32)
    sc = _c(scales, np.uint16)
    qz = None if qzeros is None else _c(qzeros, np.int32)
    scratch = np.empty(K, np.float32)
    y = np.empty((M, N), np.float64)
    _load().oracle_w4a16_gemm(_p(xx), ctypes.c_int(xdtype), _p(qw), _p(sc), _p(qz),
                              ctypes.c_int64(M), ctypes.c_int64(N), ctypes.c_int64(K),
                              ctypes.c_int64(g), _p(scratch), _p(y))
    return y


def w4a16_gemm_sampled(x, xdtype, qweight, scales, qzeros, K, g, ms, ns):
    """fp64 y at positions (ms[i], ns[i]); pass ns sorted for speed."""
    xx = _c(x, np.uint16)
    qw = _c(qweight, np.int32)
    sc = _c(scales, np.uint16)
    qz = None if qzeros is None else _c(qzeros, np.int32)
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    scratch = np.empty(K, np.float32)
    out = np.empty(ms.shape, np.float64)
    _load().oracle_w4a16_gemm_sampled(_p(xx), ctypes.c_int(xdtype), _p(qw), _p(sc), _p(qz),
                                      ctypes.c_int64(K), ctypes.c_int64(g), _p(ms), _p(ns),
                                      ctypes.c_int64(ms.size), _p(scratch), _p(out))
    return out


def w4a16_gemm_grouped(x, xdtype, m_offsets, qweight, scales, qzeros, N, K, g):
    xx = _c(x, np.uint16)
    off = _c(m_offsets, np.int64)
    qw = _c(qweight, np.int32)
    sc = _c(scales, np.uint16)
    qz = None if qzeros is None else _c(qzeros, np.int32)
    total_m = int(off[-1])
    scratch = np.empty(K, np.float32)
    y = np.zeros((total_m, N), np.float64)
    _load().oracle_w4a16_gemm_grouped(_p(xx), ctypes.c_int(xdtype), _p(off),
                                      ctypes.c_int64(off.size - 1), _p(qw), _p(sc), _p(qz),
                                      ctypes.c_int64(N), ctypes.c_int64(K), ctypes.c_int64(g),
                                      _p(scratch), _p(y))
    return y


# --- MXFP4 MoE ----------------------------------------------------------------

def mxfp4_dequant(w_fp4, w_scale, N, K):
    w = _c(w_fp4, np.uint8)
    s = _c(w_scale, np.uint8)
    out = np.empty((N, K), np.float32)
    _load().oracle_mxfp4_dequant(_p(w), _p(s), ctypes.c_int64(N), ctypes.c_int64(K), _p(out))
    return out


def mxfp4_moe_gemm(x, ids, w_fp4, w_scale, T, topk, E, N, K):
    """fp64 y[T][topk][N]."""
    xx = _c(x, np.uint16)
    ii = _c(ids, np.int32)
    w = _c(w_fp4, np.uint8)
    s = _c(w_scale, np.uint8)
    scratch = np.empty(K, np.float32)
    y = np.empty((T, topk, N), np.float64)
    _load().oracle_mxfp4_moe_gemm(_p(xx), _p(ii), _p(w), _p(s), ctypes.c_int64(T),
                                  ctypes.c_int64(topk), ctypes.c_int64(E), ctypes.c_int64(N),
                                  ctypes.c_int64(K), _p(scratch), _p(y))
    return y


def silu_mul(ypre):
    """Stage-1 activation of pre-activation rows [..., N]: silu(gate) * up -> [..., N/2]."""
    y = _c(ypre, np.float64)
    N = y.shape[-1]
    rows = y.size // N
    out = np.empty(y.shape[:-1] + (N // 2,), np.float64)
    _load().oracle_silu_mul(_p(y), ctypes.c_int64(rows), ctypes.c_int64(N), _p(out))
    return out


def mxfp4_moe_gemm_sampled(x, ids, w_fp4, w_scale, topk, E, N, K, ts, slots, ns):
    xx = _c(x, np.uint16)
    ii = _c(ids, np.int32)
    w = _c(w_fp4, np.uint8)
    s = _c(w_scale, np.uint8)
    ts = _c(ts, np.int64)
    slots = _c(slots, np.int64)
    ns = _c(ns, np.int64)
    scratch = np.empty(K, np.float32)
    out = np.empty(ts.shape, np.float64)
    _load().oracle_mxfp4_moe_gemm_sampled(_p(xx), _p(ii), _p(w), _p(s), ctypes.c_int64(topk),
                                          ctypes.c_int64(E), ctypes.c_int64(N), ctypes.c_int64(K),
                                          _p(ts), _p(slots), _p(ns), ctypes.c_int64(ts.size),
                                          _p(scratch), _p(out))
    return out


def mxfp4_moe_stage2(a, ids, w, w2_fp4, w2_scale, T, topk, E, H, I):
    """fp64 y[T][H] of MoE stage 2 (a [T][topk][I] bf16 bits, w [T][topk] fp32)."""
    aa = _c(a, np.uint16)
    ii = _c(ids, np.int32)
    ww = _c(w, np.float32)
    w2 = _c(w2_fp4, np.uint8)
    s2 = _c(w2_scale, np.uint8)
    scratch = np.empty(I, np.float32)
    pre = np.empty(T * topk * H, np.float64)
    y = np.empty((T, H), np.float64)
    _load().oracle_mxfp4_moe_stage2(_p(aa), _p(ii), _p(ww), _p(w2), _p(s2), ctypes.c_int64(T),
                                    ctypes.c_int64(topk), ctypes.c_int64(E), ctypes.c_int64(H),
                                    ctypes.c_int64(I), _p(scratch), _p(pre), _p(y))
    return y


def mxfp4_moe_stage2_sampled(a, ids, w, w2_fp4, w2_scale, topk, E, H, I, ts, hs):
    aa = _c(a, np.uint16)
    ii = _c(ids, np.int32)
    ww = _c(w, np.float32)
    w2 = _c(w2_fp4, np.uint8)
    s2 = _c(w2_scale, np.uint8)
    ts = _c(ts, np.int64)
    hs = _c(hs, np.int64)
    scratch = np.empty(I, np.float32)
    out = np.empty(ts.shape, np.float64)
    _load().oracle_mxfp4_moe_stage2_sampled(_p(aa), _p(ii), _p(ww), _p(w2), _p(s2),
                                            ctypes.c_int64(topk), ctypes.c_int64(E),
                                            ctypes.c_int64(H), ctypes.c_int64(I), _p(ts), _p(hs),
                                            ctypes.c_int64(ts.size), _p(scratch), _p(out))
    return out


def tolerance_ok(y_test, y_ref):
    """The parity rule: |y - y_ref| <= 1e-3 + 1e-2 * max|y_ref| elementwise, no NaN/Inf.

    Returns (ok, max_abs_err, bound).
    """
    y_test = np.asarray(y_test, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    if y_ref.size == 0:
        return True, 0.0, 0.0
    bound = 1e-3 + 1e-2 * float(np.max(np.abs(y_ref)))
    if not np.all(np.isfinite(y_test)):
        return False, float("inf"), bound
    err = float(np.max(np.abs(y_test - y_ref)))
    return err <= bound, err, bound
