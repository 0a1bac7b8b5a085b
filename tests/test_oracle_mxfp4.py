"""Pins of the MXFP4 / MoE stage-1 oracle.

* dequantization against numpy on unpacked E2M1 codes and E8M0 exponents
  (the OCP MX definition, fixture ocp_mx_fp4_e2m1.json), bit for bit;
* nibble order of the packed FP4 bytes: hand bytes;
* top-1 routing of every token to expert 0 reduces to a dense GEMM with that
  expert's weights (numpy fp64 matmul, within the reordering bound);
* random top-k routing against per-(token, slot) numpy dot products;
* out-of-range expert ids give zero rows.
"""
import json
import os

import numpy as np
import pytest

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _table():
    with open(os.path.join(GOLDEN, "ocp_mx_fp4_e2m1.json")) as f:
        return np.array(json.load(f)["e2m1_values"], np.float64)


def _unpacked(w_fp4, K):
    lo = w_fp4 & 0xF
    hi = w_fp4 >> 4
    codes = np.empty(w_fp4.shape[:-1] + (K,), np.uint8)
    codes[..., 0::2] = lo
    codes[..., 1::2] = hi
    return codes


def test_fp4_byte_nibble_order(oracle):
    # byte 0x71: even k -> code 1 (0.5), odd k -> code 7 (6.0); scale byte 127 -> 1.0
    w = np.array([[0x71, 0xF8] + [0] * 14], np.uint8)
    s = np.array([[127]], np.uint8)
    out = oracle.mxfp4_dequant(w, s, 1, 32)
    assert out[0, :4].tolist() == [0.5, 6.0, -0.0, -6.0]
    assert np.signbit(out[0, 2])


def test_mxfp4_dequant_matches_definition(oracle):
    rng = np.random.default_rng(4)
    N, K = 16, 256
    codes = rng.integers(0, 16, (N, K))
    exps = rng.integers(110, 135, (N, K // 32)).astype(np.uint8)
    w = oracle.mxfp4_dequant(wl.pack_fp4_pairs(codes), exps, N, K)
    ref = _table()[codes] * np.ldexp(1.0, np.repeat(exps.astype(np.int64) - 127, 32, axis=1))
    assert np.array_equal(w.astype(np.float64), ref)


def _decode_bf16(oracle, bits):
    return oracle.bf16_decode(bits)


def test_moe_top1_expert0_is_dense_gemm(oracle):
    T, E, N, K = 9, 3, 32, 128
    d = wl.moe_inputs(T, E, 1, N, K, seed=2)
    ids = np.zeros((T, 1), np.int32)
    y = oracle.mxfp4_moe_gemm(d["x"], ids, d["w_fp4"], d["w_scale"], T, 1, E, N, K)
    x = _decode_bf16(oracle, d["x"])
    w0 = _table()[_unpacked(d["w_fp4"][0], K)] * np.ldexp(
        1.0, np.repeat(d["w_scale"][0].astype(np.int64) - 127, 32, axis=1))
    ref = x @ w0.T
    bound = 2 * K * 2.0 ** -53 / (1 - K * 2.0 ** -53) * (np.abs(x) @ np.abs(w0).T)
    assert np.all(np.abs(y[:, 0, :] - ref) <= bound)


def test_moe_random_routing_per_slot(oracle):
    T, E, topk, N, K = 12, 5, 3, 16, 96
    d = wl.moe_inputs(T, E, topk, N, K, seed=3)
    ids = d["ids"].copy()
    ids[2, 1] = E      # out of range -> zero row
    ids[5, 0] = -1     # out of range -> zero row
    y = oracle.mxfp4_moe_gemm(d["x"], ids, d["w_fp4"], d["w_scale"], T, topk, E, N, K)
    x = _decode_bf16(oracle, d["x"])
    tab = _table()
    for t in range(T):
        for s in range(topk):
            e = ids[t, s]
            if e < 0 or e >= E:
                assert not y[t, s].any()
                continue
            w = tab[_unpacked(d["w_fp4"][e], K)] * np.ldexp(
                1.0, np.repeat(d["w_scale"][e].astype(np.int64) - 127, 32, axis=1))
            ref = w @ x[t]
            bound = 2 * K * 2.0 ** -53 / (1 - K * 2.0 ** -53) * (np.abs(w) @ np.abs(x[t]))
            assert np.all(np.abs(y[t, s] - ref) <= bound)
    # sampled form agrees exactly with the full form
    rng = np.random.default_rng(1)
    ts = rng.integers(0, T, 40)
    ss = rng.integers(0, topk, 40)
    ns = rng.integers(0, N, 40)
    ys = oracle.mxfp4_moe_gemm_sampled(d["x"], ids, d["w_fp4"], d["w_scale"], topk, E, N, K, ts, ss, ns)
    assert np.array_equal(ys, y[ts, ss, ns])


def test_parity_rule_catches_swapped_fp4_nibbles(oracle):
    """Reading the odd-k code from the low nibble (a plausible slip) breaks
    the parity rule; planted on the CPU only."""
    T, E, topk, N, K = 8, 4, 2, 32, 256
    d = wl.moe_inputs(T, E, topk, N, K, seed=0)
    y = oracle.mxfp4_moe_gemm(d["x"], d["ids"], d["w_fp4"], d["w_scale"], T, topk, E, N, K)
    swapped = ((d["w_fp4"] >> 4) | (d["w_fp4"] << 4)).astype(np.uint8)
    y_bad = oracle.mxfp4_moe_gemm(d["x"], d["ids"], swapped, d["w_scale"], T, topk, E, N, K)
    ok, err, bound = oracle.tolerance_ok(y_bad, y)
    assert not ok


# --- stage-1 activation: silu(gate) * up ----------------------------------------

def test_silu_mul_matches_library_sigmoid(oracle):
    """silu(v) = v * sigmoid(v), with scipy's logistic sigmoid as the library
    routine; gate is the first half of each row, up the second."""
    from scipy.special import expit
    rng = np.random.default_rng(9)
    y = rng.normal(0.0, 30.0, (7, 64))
    y[0, :4] = [0.0, -0.0, 750.0, -750.0]  # exact zero, saturated sigmoid both ways
    out = oracle.silu_mul(y)
    g, u = y[:, :32], y[:, 32:]
    ref = g * expit(g) * u
    assert np.allclose(out, ref, rtol=1e-14, atol=1e-300)
    assert out[0, 0] == 0.0 and out[0, 2] == 750.0 * u[0, 2] and out[0, 3] == 0.0


def test_silu_mul_odd_part_pins_the_gate_up_pairing(oracle):
    """silu(g) - silu(-g) = g, so negating the gate half of W1 (flipping the
    E2M1 sign bit of its codes) changes the activated output by exactly
    gate_pre * up_pre; a swapped gate/up pairing fails this."""
    T, E, topk, N, K = 10, 3, 2, 32, 128
    d = wl.moe_inputs(T, E, topk, N, K, seed=12)
    pre = oracle.mxfp4_moe_gemm(d["x"], d["ids"], d["w_fp4"], d["w_scale"], T, topk, E, N, K)
    neg = d["w_fp4"].copy()
    neg[:, : N // 2, :] ^= 0x88  # sign bit of both codes of every gate byte
    pre_neg = oracle.mxfp4_moe_gemm(d["x"], d["ids"], neg, d["w_scale"], T, topk, E, N, K)
    assert np.array_equal(pre_neg[..., : N // 2], -pre[..., : N // 2])
    diff = oracle.silu_mul(pre) - oracle.silu_mul(pre_neg)
    ref = pre[..., : N // 2] * pre[..., N // 2:]
    assert np.allclose(diff, ref, rtol=1e-12, atol=1e-9)
    # the same difference with the halves' roles swapped is 2 silu(up) gate
    g, u = pre[..., : N // 2], pre[..., N // 2:]
    swapped = u / (1.0 + np.exp(-u)) * g - u / (1.0 + np.exp(-u)) * (-g)
    assert not np.allclose(swapped, ref, rtol=1e-3, atol=1e-3)
