"""The generated operands have the sizes and byte accounting the zero-point
page prints (fixture tests/golden/p1_byte_accounting.json)."""
import json
import os

import numpy as np

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fx():
    with open(os.path.join(GOLDEN, "p1_byte_accounting.json")) as f:
        return json.load(f)["cases"]


def test_gate_up_sizes_match_problem_section():
    c = _fx()[0]
    M, N, K, g = c["M"], c["N"], c["K"], c["g"]
    d = wl.w4a16_inputs(1, 64, K, g, wl.F16)  # same per-row layout, few rows
    rows = N / 64
    weights = d["qweight"].nbytes * rows
    zp = d["qzeros"].nbytes * rows
    zp_expanded = 2 * N * (K // g)  # one activation-dtype value per (row, group)
    assert round(weights / 1e6, 1) == c["weights_MB"]
    assert round(zp / 1e6, 1) == c["zp_packed_MB"]
    assert round(zp_expanded / 1e6, 1) == c["zp_expanded_MB"]
    assert weights == 115_605_504 and zp == 3_612_672 and zp_expanded == 14_450_688


def _weight_side(N, K, g, zp_bytes_per_value):
    G = K // g
    return N * K / 2 + 2 * N * G + zp_bytes_per_value * N * G


def test_decode_byte_reduction_is_7_5_percent():
    c = _fx()[1]
    for (M, N, K) in c["shapes"]:
        before = _weight_side(N, K, c["g"], 2.0)
        after = _weight_side(N, K, c["g"], 0.5)
        assert round(100 * (1 - after / before), 1) == c["reduction_pct"]
        # the library's own byte accounting counts the packed form
        assert wl.w4a16_bytes(M, N, K, c["g"]) == after + 2 * M * K + 2 * M * N


def test_g128_saving_is_about_2_2_percent():
    c = _fx()[2]
    M, N, K = c["shape"]
    before = _weight_side(N, K, c["g"], 2.0)
    after = _weight_side(N, K, c["g"], 0.5)
    assert round(100 * (1 - after / before), 1) == c["reduction_pct"]


def test_generator_is_deterministic_and_in_range():
    a = wl.w4a16_inputs(2, 16, 64, 32, wl.BF16, seed=0)
    b = wl.w4a16_inputs(2, 16, 64, 32, wl.BF16, seed=0)
    for k in ("x", "qweight", "scales", "qzeros"):
        assert np.array_equal(a[k], b[k])
    m = wl.moe_inputs(16, 8, 4, 32, 64, seed=0)
    assert all(len(set(r)) == 4 for r in m["ids"].tolist())
    assert m["w_scale"].min() >= 118 and m["w_scale"].max() <= 126
