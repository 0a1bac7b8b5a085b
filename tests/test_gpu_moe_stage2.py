"""GPU parity of MoE stage 2 (BF16 x MXFP4 down projection with the
routing-weight combine) against the oracle, through the C ABI.

Bar: |y - y_ref| <= 1e-3 + 1e-2 * max|y_ref| per element, no NaN/Inf, no
write outside y.  Cases: random top-k routing at several shapes (H not a
multiple of the 384-row weight tile, I with a K tail), experts with 16 to 161
rows (one and two expert tiles), out-of-range ids (their slots add nothing),
top-1 with unit weights (a plain grouped GEMM), determinism, the empty batch,
and the full 1024-token, 32-expert, top-4, H = I = 2880 shape on sampled
outputs covering every 128-column block.
"""
import numpy as np
import pytest

import workloads as wl
from tests import oracle_threads
from tests.gpu_util import dev, host_bits, is_nan_bits, require_gpu, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wob():
    require_gpu()
    import weight_only_bit_amd as w
    w.device_check()
    return w


def _run(wob, d, ids=None, w=None):
    torch = torch_mod()
    T, H = d["T"], d["H"]
    ids = d["ids"] if ids is None else ids
    w = d["w"] if w is None else w
    out = torch.empty((T + 2, H), dtype=torch.bfloat16, device="cuda")
    out.fill_(float("nan"))
    a = dev(d["a"].view(np.int16)).view(torch.bfloat16)
    wob.mxfp4_moe_stage2(a, dev(ids), dev(w), dev(d["w2_fp4"]), dev(d["w2_scale"]),
                         out=out[1:T + 1])
    torch.cuda.synchronize()
    bits = host_bits(out)
    assert np.all(is_nan_bits(bits[0], wl.BF16)), "write before y"
    assert np.all(is_nan_bits(bits[-1], wl.BF16)), "write after y"
    return bits[1:-1]


def _check(oracle, d, ybits, ids=None, w=None):
    ids = d["ids"] if ids is None else ids
    w = d["w"] if w is None else w
    yref = oracle.mxfp4_moe_stage2(d["a"], ids, w, d["w2_fp4"], d["w2_scale"], d["T"], d["topk"],
                                   d["E"], d["H"], d["I"])
    ok, err, bound = oracle.tolerance_ok(oracle.bf16_decode(ybits), yref)
    assert ok, f"max err {err} > bound {bound}"


@pytest.mark.parametrize("T,E,topk,H,I", [(64, 8, 2, 512, 256), (37, 4, 3, 400, 192),
                                          (200, 16, 4, 2880, 640), (5, 32, 4, 48, 64),
                                          (3, 4, 1, 16, 128)])
def test_stage2_random_routing(wob, oracle, T, E, topk, H, I):
    d = wl.moe_stage2_inputs(T, E, topk, H, I, seed=T + H)
    _check(oracle, d, _run(wob, d))


@pytest.mark.parametrize("rows_per_expert", [16, 100, 160, 161])
def test_stage2_tile_heights(wob, oracle, rows_per_expert):
    """Every expert gets exactly `rows_per_expert` routed rows (one or two
    expert tiles of at most 160 rows)."""
    E, topk = 3, 1
    T = E * rows_per_expert
    d = wl.moe_stage2_inputs(T, E, topk, 400, 320, seed=rows_per_expert)
    ids = (np.arange(T) % E).astype(np.int32).reshape(T, 1)
    _check(oracle, d, _run(wob, d, ids=ids), ids=ids)


def test_stage2_out_of_range_ids_add_nothing(wob, oracle):
    d = wl.moe_stage2_inputs(40, 6, 3, 272, 128, seed=7)
    ids = d["ids"].copy()
    ids[0, 0] = -1
    ids[5, 2] = 6
    ids[9, :] = 1000  # every slot invalid: a zero row
    ybits = _run(wob, d, ids=ids)
    _check(oracle, d, ybits, ids=ids)
    assert np.all(oracle.bf16_decode(ybits[9]) == 0.0)


def test_stage2_top1_unit_weights_is_a_grouped_gemm(wob, oracle):
    """topk = 1 with weight 1: each token's row times its expert's W2 (a dense
    product per expert), checked against numpy on the oracle's dequantized W2."""
    d = wl.moe_stage2_inputs(48, 3, 1, 96, 128, seed=8)
    w = np.ones((48, 1), np.float32)
    y = oracle.bf16_decode(_run(wob, d, w=w))
    x = oracle.bf16_decode(d["a"][:, 0, :])
    ref = np.empty_like(y)
    for e in range(3):
        rows = np.flatnonzero(d["ids"][:, 0] == e)
        w2 = oracle.mxfp4_dequant(d["w2_fp4"][e], d["w2_scale"][e], 96, 128).astype(np.float64)
        ref[rows] = x[rows] @ w2.T
    assert np.max(np.abs(y - ref)) <= 1e-3 + 1e-2 * np.max(np.abs(ref))


def test_stage2_deterministic(wob):
    d = wl.moe_stage2_inputs(300, 8, 4, 528, 384, seed=9)
    assert np.array_equal(_run(wob, d), _run(wob, d))


def test_stage2_empty_batch_is_a_noop(wob):
    torch = torch_mod()
    d = wl.moe_stage2_inputs(1, 2, 1, 64, 64, seed=0)
    a = torch.empty((0, 1, 64), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, 1), dtype=torch.int32, device="cuda")
    w = torch.empty((0, 1), dtype=torch.float32, device="cuda")
    y = wob.mxfp4_moe_stage2(a, ids, w, dev(d["w2_fp4"]), dev(d["w2_scale"]))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 64)


def test_config_moe_stage2_full_size(wob, oracle):
    """1024 tokens, 32 experts, top-4, H = I = 2880 in the benchmark's launch
    configuration: every output finite; for every 128-column block, 16
    sampled tokens (the first, the last and random ones) at both block edges
    and two random columns, against the oracle."""
    d = wl.BY_KEY["moe_stage2"].make()
    y = oracle.bf16_decode(_run(wob, d))
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(0)
    T, H = d["T"], d["H"]
    ts, hs = [], []
    for c0 in range(0, H, 128):
        width = min(128, H - c0)  # 2880 = 22.5 blocks: the last one is half wide
        toks = np.concatenate([[0, T - 1], rng.integers(0, T, 14)])
        cols = c0 + np.concatenate([[0, width - 1], rng.integers(0, width, 2)])
        for t in toks:
            ts.append(np.full(cols.size, t))
            hs.append(cols)
    ts, hs = np.concatenate(ts), np.concatenate(hs)
    yref = oracle_threads.mxfp4_moe_stage2_sampled(oracle, d, ts, hs)
    ok, err, bound = oracle.tolerance_ok(y[ts, hs], yref)
    assert ok, (err, bound)
