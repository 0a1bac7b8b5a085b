"""Parity-check harness: the oracle's own routines run on disjoint slices of
one problem in host threads, so full-size outputs can be checked element by
element in seconds.  The oracle is unchanged; each slice is an independent
call of the same single-threaded C function (ctypes releases the GIL while it
runs), and the slices are stitched back together without any arithmetic."""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np


def host_threads() -> int:
    """Worker threads for the harness: the host's CPUs, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _slices(n, parts, align):
    """[(lo, hi)] covering range(n) in at most `parts` pieces, cut at multiples of align."""
    step = max(align, -(-n // parts) // align * align)
    return [(lo, min(n, lo + step)) for lo in range(0, n, step)]


def w4a16_gemm(oracle, d, threads=None):
    """The oracle's fp64 y[M][N] of a W4A16 problem, computed on N-slices cut at
    multiples of 8 (one packed zero-point word holds 8 rows)."""
    M, N, K, g = d["M"], d["N"], d["K"], d["g"]
    y = np.empty((M, N), np.float64)
    qz = d["qzeros"]

    def run(lo_hi):
        lo, hi = lo_hi
        y[:, lo:hi] = oracle.w4a16_gemm(
            d["x"], d["dtype"], d["qweight"][lo:hi], d["scales"][lo:hi],
            None if qz is None else qz[lo // 8:hi // 8], M, hi - lo, K, g)

    with cf.ThreadPoolExecutor(threads or host_threads()) as ex:
        list(ex.map(run, _slices(N, 4 * (threads or host_threads()), 8)))
    return y


def w4a16_gemm_sampled(oracle, d, ms, ns, threads=None):
    """The oracle's fp64 y at (ms[i], ns[i]), the sample list cut into pieces."""
    ms = np.asarray(ms, np.int64)
    ns = np.asarray(ns, np.int64)
    out = np.empty(ms.shape, np.float64)

    def run(lo_hi):
        lo, hi = lo_hi
        out[lo:hi] = oracle.w4a16_gemm_sampled(d["x"], d["dtype"], d["qweight"], d["scales"],
                                               d["qzeros"], d["K"], d["g"], ms[lo:hi], ns[lo:hi])

    with cf.ThreadPoolExecutor(threads or host_threads()) as ex:
        list(ex.map(run, _slices(ms.size, 4 * (threads or host_threads()), 1)))
    return out


def mxfp4_moe_gemm_sampled(oracle, d, ts, ss, ns, ids=None, threads=None):
    """The oracle's fp64 MoE stage-1 output at (ts[i], ss[i], ns[i])."""
    ids = d["ids"] if ids is None else ids
    ts, ss, ns = (np.asarray(a, np.int64) for a in (ts, ss, ns))
    out = np.empty(ts.shape, np.float64)

    def run(lo_hi):
        lo, hi = lo_hi
        out[lo:hi] = oracle.mxfp4_moe_gemm_sampled(d["x"], ids, d["w_fp4"], d["w_scale"],
                                                   d["topk"], d["E"], d["N"], d["K"],
                                                   ts[lo:hi], ss[lo:hi], ns[lo:hi])

    with cf.ThreadPoolExecutor(threads or host_threads()) as ex:
        list(ex.map(run, _slices(ts.size, 4 * (threads or host_threads()), 1)))
    return out


def mxfp4_moe_stage2_sampled(oracle, d, ts, hs, threads=None):
    """The oracle's fp64 MoE stage-2 output at (ts[i], hs[i])."""
    ts, hs = (np.asarray(v, np.int64) for v in (ts, hs))
    out = np.empty(ts.shape, np.float64)

    def run(lo_hi):
        lo, hi = lo_hi
        out[lo:hi] = oracle.mxfp4_moe_stage2_sampled(d["a"], d["ids"], d["w"], d["w2_fp4"],
                                                     d["w2_scale"], d["topk"], d["E"], d["H"],
                                                     d["I"], ts[lo:hi], hs[lo:hi])

    with cf.ThreadPoolExecutor(threads or host_threads()) as ex:
        list(ex.map(run, _slices(ts.size, 4 * (threads or host_threads()), 1)))
    return out
