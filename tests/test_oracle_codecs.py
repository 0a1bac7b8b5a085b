"""Pins of the oracle's number codecs against independent definitions.

binary16 is checked exhaustively against numpy's float16, bfloat16 against
torch's CPU bfloat16, and E2M1/E8M0 against the OCP MX definition (fixture
tests/golden/ocp_mx_fp4_e2m1.json).
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_f16_decode_all_patterns(oracle):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_decode(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_all_patterns(oracle):
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _edge_values():
    v = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e30, -1e30,
         2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26, 1.5 * 2.0 ** -24,
         2.5 * 2.0 ** -24, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8,
         3.0e38, 3.4e38, 1e-40, 1e-45, np.inf, -np.inf]
    return np.array(v, np.float64)


def test_f16_encode_rne_vs_numpy(oracle):
    rng = np.random.default_rng(1)
    v = np.concatenate([
        _edge_values(),
        rng.standard_normal(200000) * 10.0 ** rng.uniform(-9, 5, 200000),
        # exact ties of binary16 neighbours in the normal and subnormal ranges
        (np.arange(1, 20000, dtype=np.float64) + 0.5) * 2.0 ** -24,
        (2048 + np.arange(0, 2048) + 0.5) * 2.0 ** -10,
    ]).astype(np.float32).astype(np.float64)  # encoder input is binary32 in use
    got = oracle.f16_encode(v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    nanbits = oracle.f16_encode(np.array([np.nan]))
    assert (nanbits[0] & 0x7C00) == 0x7C00 and (nanbits[0] & 0x3FF) != 0


def test_bf16_encode_rne_vs_torch(oracle):
    import torch
    rng = np.random.default_rng(2)
    v = np.concatenate([
        _edge_values(),
        rng.standard_normal(200000) * 10.0 ** rng.uniform(-38, 38, 200000),
        (256 + np.arange(0, 256) + 0.5) * 2.0 ** -7,
    ]).astype(np.float32)
    got = oracle.bf16_encode(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_e2m1_table_matches_ocp_definition(oracle):
    with open(os.path.join(GOLDEN, "ocp_mx_fp4_e2m1.json")) as f:
        fx = json.load(f)
    got = oracle.e2m1_decode(np.arange(16, dtype=np.uint8))
    ref = np.array(fx["e2m1_values"], np.float64)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))  # code 8 is -0.0


def test_e8m0_closed_form(oracle):
    # the MXFP4 page builds the scale by placing the byte in the binary32
    # exponent field (shift left by 23); for b in 1..254 that is exactly 2^(b-127)
    b = np.arange(1, 255, dtype=np.uint8)
    got = oracle.e8m0_decode(b)
    via_shift = (b.astype(np.uint32) << np.uint32(23)).view(np.float32).astype(np.float64)
    assert np.array_equal(got, via_shift)
    assert np.array_equal(got, np.ldexp(1.0, b.astype(np.int64) - 127))
    with open(os.path.join(GOLDEN, "ocp_mx_fp4_e2m1.json")) as f:
        fx = json.load(f)
    for byte, val in fx["e8m0_examples"]:
        assert oracle.e8m0_decode(np.array([byte], np.uint8))[0] == pytest.approx(val, rel=0, abs=0)
    assert np.isnan(oracle.e8m0_decode(np.array([255], np.uint8))[0])
