"""Seeded synthetic inputs for the weight-only 4-bit GEMM, shared by the tests,
the smoke check and the benchmark.

This module only draws random numbers and lays them out in the packed formats;
it holds none of the method's arithmetic (no unpacking, no dequantization, no
products), so the oracle and the HIP path can both consume its output without
sharing code.

Packed formats (weight-only 4-bit GEMM pages; see the library header):
  * ``qweight[N][K/8]`` int32: eight 4-bit codes along K, code k%8 in bits 4*(k%8);
  * ``scales[N][K/g]`` in the activation dtype (float16 or bfloat16 bit patterns);
  * ``qzeros[N/8][K/g]`` int32: eight 4-bit zero-points along N, row n%8 in bits 4*(n%8);
  * MXFP4: ``w_fp4[E][N][K/2]`` uint8 with the even-k code in the low nibble,
    ``w_scale[E][N][K/32]`` uint8 E8M0 exponents.

Activation-dtype arrays are returned as uint16 bit patterns (numpy has no
bfloat16); float16 values are rounded with numpy's RNE cast, bfloat16 values
with torch's RNE cast on the CPU.

Recipe, drawn in this order from ``numpy.random.default_rng(seed)``:
  W4A16: X ~ N(0,1) [M,K] float32 -> act dtype; packed weight words uniform over
  all 2^32 values (so each of the eight codes is an independent uniform 0..15);
  scales ~ U[1e-3, 2e-2] [N,G] -> act dtype; packed zero-point words uniform over
  2^32 values (each zero-point uniform 0..15).
  MoE: X ~ N(0,1) [T,K] -> bfloat16; per token a uniformly random ordered set of
  ``topk`` distinct experts (argsort of uniform keys); FP4 bytes uniform over 256
  values (both codes uniform over the 16 E2M1 codes); E8M0 bytes uniform in
  [118, 126].
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F16 = 0
BF16 = 1
DTYPE_NAMES = {F16: "fp16", BF16: "bf16"}


def to_act_bits(values: np.ndarray, dtype: int) -> np.ndarray:
    """Round float32/float64 values to the activation dtype; return uint16 bits."""
    values = np.ascontiguousarray(values, np.float32)
    if dtype == F16:
        return values.astype(np.float16).view(np.uint16)
    import torch  # CPU-only use: torch's float32 -> bfloat16 cast rounds to nearest even

    t = torch.from_numpy(values).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def pack_u4_along_k(codes: np.ndarray) -> np.ndarray:
    """codes[N][K] in 0..15 -> int32 words [N][K/8], code k%8 at bits 4*(k%8)."""
    codes = np.asarray(codes, np.uint32)
    n, k = codes.shape
    assert k % 8 == 0
    c = codes.reshape(n, k // 8, 8)
    words = np.zeros((n, k // 8), np.uint32)
    for i in range(8):
        words |= (c[:, :, i] & 0xF) << np.uint32(4 * i)
    return words.view(np.int32)


def pack_u4_along_n(zeros: np.ndarray) -> np.ndarray:
    """zeros[N][G] in 0..15 -> int32 words [N/8][G], row n%8 at bits 4*(n%8)."""
    zeros = np.asarray(zeros, np.uint32)
    n, g = zeros.shape
    assert n % 8 == 0
    z = zeros.reshape(n // 8, 8, g)
    words = np.zeros((n // 8, g), np.uint32)
    for i in range(8):
        words |= (z[:, i, :] & 0xF) << np.uint32(4 * i)
    return words.view(np.int32)


def pack_fp4_pairs(codes: np.ndarray) -> np.ndarray:
    """codes[..., K] in 0..15 -> bytes [..., K/2], even k in the low nibble."""
    codes = np.asarray(codes, np.uint8)
    assert codes.shape[-1] % 2 == 0
    lo = codes[..., 0::2] & 0xF
    hi = codes[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def _uniform_words(rng, shape):
    return rng.integers(0, 1 << 32, size=shape, dtype=np.uint32).view(np.int32)


def w4a16_inputs(M, N, K, g, dtype, seed=0, symmetric=False, signed_scales=False):
    """Seeded W4A16 operands.  ``signed_scales`` draws |s| log-uniform over two
    decades [1e-3, 1e-1] with a random sign (robustness case, not a config)."""
    assert K % g == 0 and N % 8 == 0 and K % 8 == 0
    G = K // g
    rng = np.random.default_rng(seed)
    x = to_act_bits(rng.standard_normal((M, K), dtype=np.float32), dtype)
    qweight = _uniform_words(rng, (N, K // 8))
    scales = _scales(rng, (N, G), dtype, signed_scales)
    qzeros = None if symmetric else _uniform_words(rng, (N // 8, G))
    return dict(x=x, qweight=qweight, scales=scales, qzeros=qzeros,
                M=M, N=N, K=K, g=g, dtype=dtype)


def _scales(rng, shape, dtype, signed):
    if signed:
        mag = 10.0 ** rng.uniform(-3.0, -1.0, size=shape)
        sign = np.where(rng.integers(0, 2, size=shape) == 1, -1.0, 1.0)
        return to_act_bits((mag * sign).astype(np.float32), dtype)
    return to_act_bits(rng.uniform(1e-3, 2e-2, size=shape).astype(np.float32), dtype)


def w4a16_degenerate_inputs(M, N, K, g, dtype, seed=0, live_groups=0.1, outlier_cols=0.02,
                            symmetric=False):
    """Weights that mostly dequantize to zero under activations with outliers.

    Every (row, group) draws a zero-point z uniform 0..15 (8 when symmetric);
    the group's codes all equal z, except in a fraction ``live_groups`` of the
    (row, group) pairs whose codes are uniform 0..15.  X ~ N(0,1), with a
    fraction ``outlier_cols`` of the K columns scaled by +-U[100, 1000].
    ``live_groups=0`` gives a matrix that dequantizes to all zeros.  Scales as
    in w4a16_inputs.  Draw order: zero-points, live mask, live codes, X,
    outlier columns, outlier factors, scales."""
    assert K % g == 0 and N % 8 == 0
    G = K // g
    rng = np.random.default_rng(seed)
    zeros = np.full((N, G), 8, np.int64) if symmetric else rng.integers(0, 16, (N, G))
    live = rng.random((N, G)) < live_groups
    codes = np.repeat(zeros, g, axis=1)
    rand = rng.integers(0, 16, (N, K))
    codes = np.where(np.repeat(live, g, axis=1), rand, codes)
    x = rng.standard_normal((M, K)).astype(np.float32)
    cols = rng.choice(K, max(1, int(K * outlier_cols)), replace=False)
    fac = rng.uniform(100.0, 1000.0, cols.size) * np.where(rng.integers(0, 2, cols.size) == 1, -1, 1)
    x[:, cols] *= fac.astype(np.float32)
    scales = to_act_bits(rng.uniform(1e-3, 2e-2, size=(N, G)).astype(np.float32), dtype)
    return dict(x=to_act_bits(x, dtype), qweight=pack_u4_along_k(codes), scales=scales,
                qzeros=None if symmetric else pack_u4_along_n(zeros), M=M, N=N, K=K, g=g,
                dtype=dtype)


def w4a16_grouped_inputs(group_rows, N, K, g, dtype, seed=0, symmetric=False,
                         signed_scales=False):
    """Ragged grouped operands: group e has group_rows[e] rows and its own weights."""
    E = len(group_rows)
    G = K // g
    rng = np.random.default_rng(seed)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(group_rows)
    total = int(offsets[-1])
    x = to_act_bits(rng.standard_normal((total, K), dtype=np.float32), dtype)
    qweight = _uniform_words(rng, (E, N, K // 8))
    scales = _scales(rng, (E, N, G), dtype, signed_scales)
    qzeros = None if symmetric else _uniform_words(rng, (E, N // 8, G))
    return dict(x=x, m_offsets=offsets, qweight=qweight, scales=scales, qzeros=qzeros,
                N=N, K=K, g=g, dtype=dtype)


def moe_inputs(T, E, topk, N, K, seed=0, exp_lo=118, exp_hi=126):
    assert K % 32 == 0 and topk <= E
    rng = np.random.default_rng(seed)
    x = to_act_bits(rng.standard_normal((T, K), dtype=np.float32), BF16)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :topk].astype(np.int32)
    w_fp4 = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    w_scale = rng.integers(exp_lo, exp_hi + 1, size=(E, N, K // 32), dtype=np.uint8)
    return dict(x=np.ascontiguousarray(x), ids=np.ascontiguousarray(ids), w_fp4=w_fp4,
                w_scale=w_scale, T=T, E=E, topk=topk, N=N, K=K)


def moe_stage2_inputs(T, E, topk, H, I, seed=0, exp_lo=118, exp_hi=126):
    """MoE stage-2 operands: the stage-1 activation rows a [T][topk][I] ~ N(0,1)
    in bfloat16, ids as in moe_inputs, routing weights [T][topk] fp32 (uniform
    keys normalised to sum 1 per token), W2 codes [E][H][I/2] uniform bytes,
    E8M0 scales [E][H][I/32] uniform in [exp_lo, exp_hi].  Draw order: a, ids,
    weights, codes, scales."""
    assert I % 32 == 0 and topk <= E
    rng = np.random.default_rng(seed)
    a = to_act_bits(rng.standard_normal((T, topk, I), dtype=np.float32), BF16)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :topk].astype(np.int32)
    r = rng.random((T, topk)).astype(np.float32) + np.float32(0.05)
    w = (r / r.sum(axis=1, keepdims=True)).astype(np.float32)
    w2_fp4 = rng.integers(0, 256, size=(E, H, I // 2), dtype=np.uint8)
    w2_scale = rng.integers(exp_lo, exp_hi + 1, size=(E, H, I // 32), dtype=np.uint8)
    return dict(a=np.ascontiguousarray(a), ids=np.ascontiguousarray(ids), w=np.ascontiguousarray(w),
                w2_fp4=w2_fp4, w2_scale=w2_scale, T=T, E=E, topk=topk, H=H, I=I)


def routed_group_rows(T, E, topk, seed=0):
    """Rows per expert of a uniform top-k routing (the recipe of moe_inputs)."""
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :topk]
    return np.bincount(ids.ravel(), minlength=E).astype(np.int64)


def moe_decode_bytes(ids, E, N, K):
    """Algorithmic bytes of one MoE stage-1 call with few tokens: FP4 codes and
    E8M0 scales of the experts the ids name (each streamed once), X, ids and Y."""
    T, topk = ids.shape
    used = len(np.unique(ids[(ids >= 0) & (ids < E)]))
    return used * (N * K // 2 + N * K // 32) + 2 * T * K + 4 * T * topk + 2 * T * topk * N


def grouped_bytes(total_m, E, N, K, g, act_bytes=2):
    """Algorithmic bytes of one grouped W4A16 call: every group's packed codes,
    scales and packed zero-points, X and Y."""
    G = K // g
    return E * (N * K // 2 + act_bytes * N * G + N * G // 2) + act_bytes * total_m * (K + N)


@dataclass(frozen=True)
class Workload:
    key: str
    kind: str  # "w4a16", "grouped", "moe" or "moe2"
    desc: str
    params: dict

    def make(self, seed=0):
        p = dict(self.params)
        if self.kind == "w4a16":
            return w4a16_inputs(p["M"], p["N"], p["K"], p["g"], p["dtype"], seed=seed)
        if self.kind == "moe2":
            return moe_stage2_inputs(p["T"], p["E"], p["topk"], p["H"], p["I"], seed=seed)
        if self.kind == "grouped":
            rows = routed_group_rows(p["T"], p["E"], p["topk"], seed=seed)
            return w4a16_grouped_inputs(rows, p["N"], p["K"], p["g"], p["dtype"], seed=seed)
        return moe_inputs(p["T"], p["E"], p["topk"], p["N"], p["K"], seed=seed)


# The five measured shapes of the weight-only 4-bit GEMM pages' workloads.
WORKLOADS = [
    Workload("tiny_gemv", "w4a16", "tiny W4A16 asymmetric GEMV 1x256x512 g=32 fp16",
             dict(M=1, N=256, K=512, g=32, dtype=F16)),
    Workload("decode_gemv", "w4a16", "decode skinny GEMV 1x43008x5376 g=32 fp16 (gate_up shape)",
             dict(M=1, N=43008, K=5376, g=32, dtype=F16)),
    Workload("small_batch", "w4a16", "small-batch skinny 4x2048x2048 g=128 bf16",
             dict(M=4, N=2048, K=2048, g=128, dtype=BF16)),
    Workload("prefill", "w4a16", "prefill tiled GEMM 2048x16384x5376 g=128 fp16",
             dict(M=2048, N=16384, K=5376, g=128, dtype=F16)),
    Workload("moe_stage1", "moe", "MoE stage-1 BF16xMXFP4 1024 tokens, 32 experts, top-4, K=2880, N=5760",
             dict(T=1024, E=32, topk=4, N=5760, K=2880)),
]
# The zero-point page's other measured shapes (its per-shape timing table and
# its batch-4, g = 128 regression table), read as M x N x K with the shapes
# of the batch-4 table given as N x K; fp16 like that table's "-zp" rows.
EXTRA_WORKLOADS = [
    Workload("decode_qkv", "w4a16", "decode skinny GEMV 1x16384x5376 g=32 fp16 (qkv shape)",
             dict(M=1, N=16384, K=5376, g=32, dtype=F16)),
    Workload("decode_down", "w4a16", "decode skinny GEMV 1x5376x21504 g=32 fp16 (down shape)",
             dict(M=1, N=5376, K=21504, g=32, dtype=F16)),
    Workload("bs4_2048x2560", "w4a16", "batch-4 skinny 4x2048x2560 g=128 fp16",
             dict(M=4, N=2048, K=2560, g=128, dtype=F16)),
    Workload("bs4_6144x2048", "w4a16", "batch-4 skinny 4x6144x2048 g=128 fp16",
             dict(M=4, N=6144, K=2048, g=128, dtype=F16)),
    Workload("bs4_4096x2048", "w4a16", "batch-4 skinny 4x4096x2048 g=128 fp16",
             dict(M=4, N=4096, K=2048, g=128, dtype=F16)),
    # MoE stage 1 with a decode batch: the memory-bound path.
    Workload("moe_decode", "moe",
             "MoE stage-1 BF16xMXFP4 decode: 4 tokens, 32 experts, top-4, K=2880, N=5760",
             dict(T=4, E=32, topk=4, N=5760, K=2880)),
    # MoE stage 2 after the stage-1 shape: the down projection of the
    # 2880-wide activation rows back to the 2880-wide model dimension, with
    # the routing-weight combine (a reading: the pages define stage 1 only).
    Workload("moe_stage2", "moe2",
             "MoE stage-2 BF16xMXFP4 1024 tokens, 32 experts, top-4, I=2880, H=2880, "
             "routing-weight combine",
             dict(T=1024, E=32, topk=4, H=2880, I=2880)),
    # The grouped GEMM on an MoE-like uint4 configuration: the MoE stage-1
    # shape with W4A16 experts, rows per expert from a uniform top-4 routing.
    Workload("grouped_moe_like", "grouped",
             "grouped W4A16 32 experts x rows of 1024 tokens top-4 (4096 rows), N=5760, K=2880, "
             "g=32 bf16",
             dict(T=1024, E=32, topk=4, N=5760, K=2880, g=32, dtype=BF16)),
]

BY_KEY = {w.key: w for w in WORKLOADS + EXTRA_WORKLOADS}


def w4a16_bytes(M, N, K, g, act_bytes=2, symmetric=False):
    """Algorithmic bytes of one W4A16 call: packed codes, scales, packed
    zero-points, X and Y."""
    G = K // g
    b = N * K // 2 + act_bytes * N * G + (0 if symmetric else N * G // 2)
    return b + act_bytes * M * K + act_bytes * M * N


def moe_stage2_bytes(T, E, topk, H, I):
    """Algorithmic bytes of one MoE stage-2 call: W2 codes and E8M0 scales, the
    activation rows, ids, routing weights and y."""
    return E * H * I // 2 + E * H * I // 32 + 2 * T * topk * I + 8 * T * topk + 2 * T * H


def moe_bytes(T, E, topk, N, K):
    """Algorithmic bytes of one MoE stage-1 call: FP4 codes, E8M0 scales, X,
    routing ids and Y."""
    return E * N * K // 2 + E * N * K // 32 + 2 * T * K + 4 * T * topk + 2 * T * topk * N
