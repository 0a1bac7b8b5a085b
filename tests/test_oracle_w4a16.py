"""Pins of the W4A16 oracle against things other than itself.

* brute-force integer matmul when every scale is 1 and every zero-point 0, and
  with random zero-points and power-of-two scales (all sums exact);
* the packed-nibble layout: hand words from the zero-point layout statement of
  the zero-point page ("Keep W4A16 zero-points packed at 4 bits...", section
  Change), a pack/unpack round trip with an independent packer, and one-hot
  codes;
* dequantization against numpy on unpacked codes, bit for bit;
* the GEMM against numpy fp64 and fp32 matmuls of the oracle's own
  dequantized matrix, within rounding-error bounds;
* the grouped form against per-group dense calls of numpy.
"""
import json
import os

import numpy as np
import pytest

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _act_bits(values, dtype):
    return wl.to_act_bits(np.asarray(values, np.float32), dtype)


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("M,N,K,g", [(1, 8, 32, 32), (3, 16, 64, 32), (8, 24, 256, 128),
                                     (17, 8, 256, 32), (2, 16, 128, 64)])
def test_bruteforce_integer_matmul_unit_scale_zero_zp(oracle, dtype, M, N, K, g):
    rng = np.random.default_rng(M * 1000 + N * 10 + K + g + dtype)
    codes = rng.integers(0, 16, (N, K))
    xi = rng.integers(-8, 9, (M, K))
    G = K // g
    qweight = wl.pack_u4_along_k(codes)
    qzeros = wl.pack_u4_along_n(np.zeros((N, G), np.int64))  # packed zeros, not "symmetric"
    scales = _act_bits(np.ones((N, G)), dtype)
    x = _act_bits(xi, dtype)
    y = oracle.w4a16_gemm(x, dtype, qweight, scales, qzeros, M, N, K, g)
    ref = xi.astype(np.int64) @ codes.astype(np.int64).T
    assert np.array_equal(y, ref.astype(np.float64))


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
def test_bruteforce_random_zero_points_pow2_scales(oracle, dtype):
    M, N, K, g = 5, 32, 256, 32
    G = K // g
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, (N, K))
    zeros = rng.integers(0, 16, (N, G))
    exps = rng.integers(-12, -1, (N, G))
    xi = rng.integers(-8, 9, (M, K))
    y = oracle.w4a16_gemm(_act_bits(xi, dtype), dtype, wl.pack_u4_along_k(codes),
                          _act_bits(np.ldexp(1.0, exps), dtype), wl.pack_u4_along_n(zeros),
                          M, N, K, g)
    # integer sum per group, then the power-of-two scale: every step is exact
    ref = np.zeros((M, N), np.float64)
    d = codes - np.repeat(zeros, g, axis=1)  # (N, K) integers
    for j in range(G):
        part = xi[:, j * g:(j + 1) * g].astype(np.int64) @ d[:, j * g:(j + 1) * g].T.astype(np.int64)
        ref += part * np.ldexp(1.0, exps[:, j])[None, :]
    assert np.array_equal(y, ref)


def test_zero_point_hand_words_from_layout_statement(oracle):
    with open(os.path.join(GOLDEN, "p1_zero_point_words.json")) as f:
        fx = json.load(f)
    words = np.array([[int(w, 16) for w in row] for row in fx["words_hex"]], np.uint32).view(np.int32)
    z = oracle.w4a16_unpack_zeros(words, fx["N"], fx["G"])
    assert np.array_equal(z, np.array(fx["expected_zeros"], np.uint8))


def test_weight_hand_words_and_sign_extension(oracle):
    words = np.array([[0x76543210, 0xFEDCBA98]], np.uint32).view(np.int32)
    codes = oracle.w4a16_unpack_codes(words, 1, 16)
    assert codes.tolist() == [list(range(16))]


def test_symmetric_codes_are_offset_by_eight(oracle):
    """No zero-point tensor means z = 8: a code c dequantizes to (c - 8) * s,
    the offset-8 codes of the q4_0 page ("qsa_prompt_attn: Q4_0 KV on tensor
    cores (mode 4)", What: each block's codes become (code - 8) with one fp16
    scale per 32, which may be negative).  Expected values written from that
    statement for the hand words 0x76543210, 0xFEDCBA98 (codes 0..15)."""
    words = np.array([[0x76543210, 0xFEDCBA98, 0x76543210, 0xFEDCBA98]], np.uint32).view(np.int32)
    scales = np.array([[0x3C00]], np.uint16)   # fp16 1.0 for the single group of 32
    w = oracle.w4a16_dequant(words, scales, 0, None, 1, 32, 32)
    assert w.tolist() == [[float(c - 8) for c in list(range(16)) * 2]]
    scales = np.array([[0xB800]], np.uint16)   # fp16 -0.5 (a negative q4_0 scale)
    w = oracle.w4a16_dequant(words, scales, 0, None, 1, 32, 32)
    expect = [(c - 8) * -0.5 for c in list(range(16)) * 2]
    assert w[0].tolist() == expect
    # code 8 gives (8 - 8) * -0.5 = -0.0: the sign of a zero product is kept
    assert np.signbit(w[0, 8]) and np.signbit(w[0, 24])


def test_pack_unpack_round_trip(oracle):
    rng = np.random.default_rng(3)
    N, K, G = 48, 512, 16
    codes = rng.integers(0, 16, (N, K))
    zeros = rng.integers(0, 16, (N, G))
    assert np.array_equal(oracle.w4a16_unpack_codes(wl.pack_u4_along_k(codes), N, K), codes)
    assert np.array_equal(oracle.w4a16_unpack_zeros(wl.pack_u4_along_n(zeros), N, G), zeros)


def test_one_hot_code_moves_exactly_one_weight(oracle):
    N, K, g = 8, 64, 32  # N = 8: exactly one zero-point word per group
    G = K // g
    scales = _act_bits(np.full((N, G), 0.5), wl.F16)
    qzeros = wl.pack_u4_along_n(np.zeros((N, G), np.int64))
    base = oracle.w4a16_dequant(wl.pack_u4_along_k(np.zeros((N, K), np.int64)), scales, wl.F16,
                                qzeros, N, K, g)
    assert not base.any()
    for n, k in [(0, 0), (3, 9), (7, 63), (5, 31), (2, 32)]:
        codes = np.zeros((N, K), np.int64)
        codes[n, k] = 15
        w = oracle.w4a16_dequant(wl.pack_u4_along_k(codes), scales, wl.F16, qzeros, N, K, g)
        nz = np.argwhere(w != 0)
        assert nz.tolist() == [[n, k]] and w[n, k] == 7.5
    # one-hot zero-point: row n, group j shifts exactly that row-group
    for n, j in [(0, 0), (6, 1), (7, 0)]:
        zeros = np.zeros((N, G), np.int64)
        zeros[n, j] = 15
        w = oracle.w4a16_dequant(wl.pack_u4_along_k(np.zeros((N, K), np.int64)), scales, wl.F16,
                                 wl.pack_u4_along_n(zeros), N, K, g)
        expect = np.zeros((N, K), np.float32)
        expect[n, j * g:(j + 1) * g] = -7.5
        assert np.array_equal(w, expect)


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("symmetric", [False, True])
def test_dequant_matches_unpacked_numpy(oracle, dtype, g, symmetric):
    N, K = 24, 256
    G = K // g
    rng = np.random.default_rng(g + 3 * dtype + symmetric)
    codes = rng.integers(0, 16, (N, K))
    zeros = rng.integers(0, 16, (N, G))
    sc_bits = _act_bits(rng.uniform(-2e-2, 2e-2, (N, G)), dtype)
    sc = oracle.act_decode(sc_bits, dtype)  # decoders pinned exhaustively elsewhere
    w = oracle.w4a16_dequant(wl.pack_u4_along_k(codes), sc_bits, dtype,
                             None if symmetric else wl.pack_u4_along_n(zeros), N, K, g)
    zz = np.full((N, G), 8) if symmetric else zeros
    ref = (codes - np.repeat(zz, g, axis=1)).astype(np.float64) * np.repeat(sc, g, axis=1)
    assert np.array_equal(w.astype(np.float64), ref)
    # activation-dtype form is the RNE rounding of the exact weight
    wa = oracle.w4a16_dequant_act(wl.pack_u4_along_k(codes), sc_bits, dtype,
                                  None if symmetric else wl.pack_u4_along_n(zeros), N, K, g)
    assert np.array_equal(wa, _act_bits(ref, dtype))


def _gamma(n, u):
    return n * u / (1 - n * u)


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
def test_gemm_vs_dense_matmul_of_dequantized_weights(oracle, dtype):
    M, N, K, g = 7, 40, 512, 32
    d = wl.w4a16_inputs(M, N, K, g, dtype, seed=11)
    y = oracle.w4a16_gemm(d["x"], dtype, d["qweight"], d["scales"], d["qzeros"], M, N, K, g)
    w = oracle.w4a16_dequant(d["qweight"], d["scales"], dtype, d["qzeros"], N, K, g).astype(np.float64)
    x = oracle.act_decode(d["x"], dtype)
    absprod = np.abs(x) @ np.abs(w).T
    ref64 = x @ w.T
    assert np.all(np.abs(y - ref64) <= _gamma(K, 2.0 ** -53) * absprod * 2 + 1e-300)
    ref32 = x.astype(np.float32) @ w.astype(np.float32).T
    assert np.all(np.abs(y - ref32) <= _gamma(K, 2.0 ** -24) * absprod + 1e-30)


def test_gemm_sampled_equals_full(oracle):
    M, N, K, g = 3, 32, 256, 128
    d = wl.w4a16_inputs(M, N, K, g, wl.F16, seed=5)
    y = oracle.w4a16_gemm(d["x"], wl.F16, d["qweight"], d["scales"], d["qzeros"], M, N, K, g)
    rng = np.random.default_rng(0)
    ns = np.sort(rng.integers(0, N, 50))
    ms = rng.integers(0, M, 50)
    ys = oracle.w4a16_gemm_sampled(d["x"], wl.F16, d["qweight"], d["scales"], d["qzeros"], K, g, ms, ns)
    assert np.array_equal(ys, y[ms, ns])


def test_grouped_equals_per_group_dense(oracle):
    rows = [3, 0, 17, 1]
    N, K, g = 16, 128, 32
    d = wl.w4a16_grouped_inputs(rows, N, K, g, wl.BF16, seed=9)
    y = oracle.w4a16_gemm_grouped(d["x"], wl.BF16, d["m_offsets"], d["qweight"], d["scales"],
                                  d["qzeros"], N, K, g)
    x = oracle.act_decode(d["x"], wl.BF16)
    off = d["m_offsets"]
    for e in range(len(rows)):
        w = oracle.w4a16_dequant(d["qweight"][e], d["scales"][e], wl.BF16, d["qzeros"][e], N, K, g)
        ref = x[off[e]:off[e + 1]] @ w.astype(np.float64).T
        absprod = np.abs(x[off[e]:off[e + 1]]) @ np.abs(w.astype(np.float64)).T
        assert np.all(np.abs(y[off[e]:off[e + 1]] - ref) <= _gamma(K, 2.0 ** -53) * 2 * absprod)


def test_parity_rule_catches_a_wrong_nibble_index(oracle):
    """A plausible indexing slip (zero-point nibble taken from row n+1) must
    break the parity rule at a config-like scale: planted on the CPU only."""
    M, N, K, g = 1, 256, 512, 32
    d = wl.w4a16_inputs(M, N, K, g, wl.F16, seed=0)
    y = oracle.w4a16_gemm(d["x"], wl.F16, d["qweight"], d["scales"], d["qzeros"], M, N, K, g)
    G = K // g
    zeros = oracle.w4a16_unpack_zeros(d["qzeros"], N, G)
    wrong = np.roll(zeros, -1, axis=0)
    y_bad = oracle.w4a16_gemm(d["x"], wl.F16, d["qweight"], d["scales"], wl.pack_u4_along_n(wrong),
                              M, N, K, g)
    ok, err, bound = oracle.tolerance_ok(y_bad, y)
    assert not ok, (err, bound)
