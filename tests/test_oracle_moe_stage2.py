"""Pins of the oracle's MoE stage 2 (down projection with the routing-weight
combine), each against something other than the oracle's own formula:

* top-1 routing, weight 1, every id 0: a dense numpy fp64 GEMM of the
  activation rows with expert 0's dequantized W2 (the dequantization is
  pinned separately against the OCP E2M1 table and the E8M0 closed form);
* a one-hot routing weight (one token, one slot): exactly that slot's dense
  product with its own expert, zeros for every other token (pins the (t, s)
  indexing of the weights and the expert chosen per slot);
* linearity in the routing weights: doubling them doubles y exactly;
* the slot sum: y equals the sum of the single-slot problems;
* an id outside [0, E) contributes what a zero routing weight does.
"""
import numpy as np
import pytest

import workloads as wl


def _dense(oracle, d, e, rows):
    """fp64 rows @ W2_e^T with the oracle's dequantized (exact) weights."""
    H, I = d["H"], d["I"]
    w2 = oracle.mxfp4_dequant(d["w2_fp4"][e], d["w2_scale"][e], H, I).astype(np.float64)
    return oracle.bf16_decode(rows) @ w2.T


def _run(oracle, d, ids=None, w=None):
    return oracle.mxfp4_moe_stage2(d["a"], d["ids"] if ids is None else ids,
                                   d["w"] if w is None else w, d["w2_fp4"], d["w2_scale"],
                                   d["T"], d["topk"], d["E"], d["H"], d["I"])


def test_top1_single_expert_is_a_dense_gemm(oracle):
    d = wl.moe_stage2_inputs(9, 3, 1, 48, 96, seed=1)
    ids = np.zeros((9, 1), np.int32)
    w = np.ones((9, 1), np.float32)
    y = _run(oracle, d, ids, w)
    ref = _dense(oracle, d, 0, d["a"][:, 0, :])
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_one_hot_routing_weight_selects_one_slot(oracle):
    d = wl.moe_stage2_inputs(7, 5, 3, 32, 64, seed=2)
    t0, s0 = 4, 2
    w = np.zeros((7, 3), np.float32)
    w[t0, s0] = 0.75
    y = _run(oracle, d, w=w)
    e = int(d["ids"][t0, s0])
    ref = 0.75 * _dense(oracle, d, e, d["a"][t0, s0][None, :])[0]
    assert np.allclose(y[t0], ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    others = np.delete(y, t0, axis=0)
    assert np.all(others == 0.0)


def test_linear_in_the_routing_weights(oracle):
    d = wl.moe_stage2_inputs(6, 4, 2, 32, 64, seed=3)
    y1 = _run(oracle, d)
    y2 = _run(oracle, d, w=(2 * d["w"]).astype(np.float32))
    assert np.array_equal(y2, 2 * y1)


def test_slots_add_up(oracle):
    d = wl.moe_stage2_inputs(5, 6, 3, 32, 128, seed=4)
    y = _run(oracle, d)
    parts = []
    for s in range(3):
        w = np.zeros_like(d["w"])
        w[:, s] = d["w"][:, s]
        parts.append(_run(oracle, d, w=w))
    assert np.allclose(y, sum(parts), rtol=0, atol=1e-12 * np.abs(y).max())


def test_out_of_range_id_is_a_zero_weight(oracle):
    d = wl.moe_stage2_inputs(5, 4, 2, 32, 64, seed=5)
    ids = d["ids"].copy()
    ids[1, 0] = -1
    ids[3, 1] = 4
    w = d["w"].copy()
    w[1, 0] = 0
    w[3, 1] = 0
    assert np.array_equal(_run(oracle, d, ids=ids), _run(oracle, d, w=w))


def test_sampled_form_equals_the_full_form(oracle):
    d = wl.moe_stage2_inputs(6, 4, 2, 48, 64, seed=6)
    d["ids"][2, 1] = 7  # out of range
    y = _run(oracle, d)
    ts = np.array([0, 2, 5, 5, 3])
    hs = np.array([0, 47, 1, 20, 33])
    got = oracle.mxfp4_moe_stage2_sampled(d["a"], d["ids"], d["w"], d["w2_fp4"], d["w2_scale"],
                                          2, 4, 48, 64, ts, hs)
    assert np.allclose(got, y[ts, hs], rtol=1e-15, atol=0)
