"""GPU parity of MoE stage 1 (BF16 x MXFP4, routed) against the oracle, through
the C ABI.

Bar: |y - y_ref| <= 1e-3 + 1e-2 * max|y_ref| per element, no NaN/Inf, and every
(token, slot) row written exactly where it belongs.  The matrix follows the
MXFP4 MoE page (section Test: the kernel per tile height x activation;
experts holding 16, 32 and 64 rows; the store-guard fix for a tile that
overhangs the weight rows) widened to skewed and empty experts, top-1
routing, out-of-range ids, ragged N and K, and the full 1024-token,
32-expert, top-4, K=2880, N=5760 shape on sampled outputs.  The tile-kernel
tests run at both tile heights the library builds (tile_m 16 and 32).
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


TILE_M = [32, 16]


def _run(wob, d, ids=None, tile_m=32):
    """Run with NaN-filled guard rows around y; return y's bf16 bits [T, topk, N]."""
    torch = torch_mod()
    T, topk, N = d["T"], d["topk"], d["N"]
    ids = d["ids"] if ids is None else ids
    out = torch.empty((T * topk + 2, N), dtype=torch.bfloat16, device="cuda")
    out.fill_(float("nan"))
    y = out[1:T * topk + 1].view(T, topk, N)
    x = dev(d["x"].view(np.int16)).view(torch.bfloat16)
    wob.mxfp4_moe_gemm(x, dev(ids), dev(d["w_fp4"]), dev(d["w_scale"]), out=y, tile_m=tile_m)
    torch.cuda.synchronize()
    bits = host_bits(out)
    assert np.all(is_nan_bits(bits[0], wl.BF16)), "write before y"
    assert np.all(is_nan_bits(bits[-1], wl.BF16)), "write after y"
    return bits[1:-1].reshape(T, topk, N)


def _check(oracle, d, ybits, ids=None):
    ids = d["ids"] if ids is None else ids
    yref = oracle.mxfp4_moe_gemm(d["x"], ids, d["w_fp4"], d["w_scale"], d["T"], d["topk"],
                                 d["E"], d["N"], d["K"])
    y = oracle.bf16_decode(ybits)
    ok, err, bound = oracle.tolerance_ok(y, yref)
    assert ok, f"max err {err} > bound {bound}"
    return y, yref


@pytest.mark.parametrize("tile_m", TILE_M)
@pytest.mark.parametrize("T,E,topk,N,K", [(64, 8, 2, 512, 256), (37, 4, 3, 400, 192),
                                          (200, 16, 4, 256, 2880), (5, 32, 4, 48, 64)])
def test_moe_random_routing(wob, oracle, T, E, topk, N, K, tile_m):
    d = wl.moe_inputs(T, E, topk, N, K, seed=T + N)
    _check(oracle, d, _run(wob, d, tile_m=tile_m))


@pytest.mark.parametrize("tile_m", TILE_M)
@pytest.mark.parametrize("rows_per_expert", [16, 17, 32, 64, 100, 160, 161, 256, 257])
def test_moe_tile_heights(wob, oracle, rows_per_expert, tile_m):
    """Every expert gets exactly `rows_per_expert` rows (16/32/64 as on the page,
    one row past a 16-row block, a ragged 100, a full 160-row expert tile and
    one row past it, 256 and 257)."""
    E, topk = 4, 1
    T = E * rows_per_expert
    d = wl.moe_inputs(T, E, topk, 528, 320, seed=rows_per_expert)
    ids = (np.arange(T) % E).astype(np.int32).reshape(T, 1)
    _check(oracle, d, _run(wob, d, ids, tile_m), ids)


@pytest.mark.parametrize("tile_m", TILE_M)
def test_moe_skewed_and_empty_experts(wob, oracle, tile_m):
    """All tokens on one expert (several expert tiles plus a tail) while the
    other experts stay empty."""
    d = wl.moe_inputs(600, 8, 1, 256, 128, seed=11)
    ids = np.full((600, 1), 5, np.int32)
    _check(oracle, d, _run(wob, d, ids, tile_m), ids)


def test_moe_top1_single_expert_is_dense(wob, oracle):
    d = wl.moe_inputs(96, 1, 1, 272, 256, seed=3)
    ids = np.zeros((96, 1), np.int32)
    y, _ = _check(oracle, d, _run(wob, d, ids), ids)
    dense = d["x"].astype(np.uint32) << 16
    xf = dense.view(np.float32).astype(np.float64)
    w = oracle.mxfp4_dequant(d["w_fp4"][0], d["w_scale"][0], 272, 256).astype(np.float64)
    ref = xf @ w.T
    assert np.max(np.abs(y[:, 0, :] - ref)) <= 1e-3 + 1e-2 * np.max(np.abs(ref))


@pytest.mark.parametrize("tile_m", TILE_M)
def test_moe_out_of_range_ids_write_zero_rows(wob, oracle, tile_m):
    d = wl.moe_inputs(40, 6, 2, 304, 128, seed=7)
    ids = d["ids"].copy()
    ids[0, 0] = -1
    ids[3, 1] = 6
    ids[17, 0] = 1000
    ids[39, 1] = -2147483648
    ybits = _run(wob, d, ids, tile_m)
    y, _ = _check(oracle, d, ybits, ids)
    for t, s in [(0, 0), (3, 1), (17, 0), (39, 1)]:
        assert np.all(ybits[t, s] == 0), (t, s)


def test_moe_zero_tokens_is_noop(wob):
    torch = torch_mod()
    d = wl.moe_inputs(1, 2, 1, 64, 64, seed=0)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, 1), dtype=torch.int32, device="cuda")
    y = wob.mxfp4_moe_gemm(x, ids, dev(d["w_fp4"]), dev(d["w_scale"]))
    assert y.shape == (0, 1, 64)


def test_moe_deterministic(wob):
    d = wl.moe_inputs(300, 8, 4, 528, 384, seed=5)
    assert np.array_equal(_run(wob, d), _run(wob, d))


def _moe_tile_samples(d, rng, width=128, per=4):
    """(token, slot, n) samples covering every (expert, column block) pair:
    for each expert its first and last routed pair and `per` - 2 random ones,
    each at both edges and two random columns of every `width`-wide block."""
    T, topk, N, E = d["T"], d["topk"], d["N"], d["E"]
    pairs = d["ids"].reshape(-1)
    ts, ss, ns = [], [], []
    for e in range(E):
        ps = np.flatnonzero(pairs == e)
        if ps.size == 0:
            continue
        pick = np.concatenate([[ps[0], ps[-1]], rng.choice(ps, per - 2)])
        for c0 in range(0, N, width):
            cols = c0 + np.concatenate([[0, min(width, N - c0) - 1],
                                        rng.integers(0, min(width, N - c0), 2)])
            for p in pick:
                ts.append(np.full(cols.size, p // topk))
                ss.append(np.full(cols.size, p % topk))
                ns.append(cols)
    return np.concatenate(ts), np.concatenate(ss), np.concatenate(ns)


@pytest.mark.parametrize("tile_m", TILE_M)
def test_config_moe_stage1_full_size(wob, oracle, tile_m):
    """1024 tokens, 32 experts, top-4, K=2880, N=5760 in the benchmark's launch
    configuration (tile_m 32; 16 as well): every output finite, and for every
    expert and every 128-column block, four of its routed rows at four columns
    each (both block edges) against the oracle."""
    d = wl.BY_KEY["moe_stage1"].make()
    ybits = _run(wob, d, tile_m=tile_m)
    y = oracle.bf16_decode(ybits)
    assert np.all(np.isfinite(y))
    ts, ss, ns = _moe_tile_samples(d, np.random.default_rng(0))
    yref = oracle_threads.mxfp4_moe_gemm_sampled(oracle, d, ts, ss, ns)
    # the bound takes the sampled outputs' max|y_ref|: no looser than the global one
    ok, err, bound = oracle.tolerance_ok(y[ts, ss, ns], yref)
    assert ok, (err, bound)


# --- fused stage-1 activation: silu(gate) * up -------------------------------------

def _run_act(wob, d, ids=None, tile_m=32):
    torch = torch_mod()
    T, topk, N = d["T"], d["topk"], d["N"]
    ids = d["ids"] if ids is None else ids
    out = torch.empty((T * topk + 2, N // 2), dtype=torch.bfloat16, device="cuda")
    out.fill_(float("nan"))
    y = out[1:T * topk + 1].view(T, topk, N // 2)
    x = dev(d["x"].view(np.int16)).view(torch.bfloat16)
    wob.mxfp4_moe_gemm(x, dev(ids), dev(d["w_fp4"]), dev(d["w_scale"]), out=y,
                       act=wob.ACT_SILU_MUL, tile_m=tile_m)
    torch.cuda.synchronize()
    bits = host_bits(out)
    assert np.all(is_nan_bits(bits[0], wl.BF16)) and np.all(is_nan_bits(bits[-1], wl.BF16))
    return bits[1:-1].reshape(T, topk, N // 2)


@pytest.mark.parametrize("tile_m", TILE_M)
@pytest.mark.parametrize("T,E,topk,N,K", [(64, 8, 2, 512, 256), (37, 4, 3, 416, 192),
                                          (200, 16, 4, 5760, 640), (5, 32, 4, 32, 64)])
def test_moe_silu_mul_parity(wob, oracle, T, E, topk, N, K, tile_m):
    d = wl.moe_inputs(T, E, topk, N, K, seed=T + N + 1)
    ids = d["ids"].copy()
    ids[0, 0] = -1  # out-of-range id: zero row
    pre = oracle.mxfp4_moe_gemm(d["x"], ids, d["w_fp4"], d["w_scale"], T, topk, E, N, K)
    ref = oracle.silu_mul(pre)
    ybits = _run_act(wob, d, ids, tile_m)
    ok, err, bound = oracle.tolerance_ok(oracle.bf16_decode(ybits), ref)
    assert ok, f"max err {err} > bound {bound}"
    assert np.all(ybits[0, 0] == 0)


@pytest.mark.parametrize("tile_m", TILE_M)
@pytest.mark.parametrize("rows_per_expert", [16, 17, 100, 161, 225, 257])
def test_moe_silu_mul_tile_heights(wob, oracle, rows_per_expert, tile_m):
    E = 3
    T = E * rows_per_expert
    d = wl.moe_inputs(T, E, 1, 288, 320, seed=rows_per_expert + 5)
    ids = (np.arange(T) % E).astype(np.int32).reshape(T, 1)
    pre = oracle.mxfp4_moe_gemm(d["x"], ids, d["w_fp4"], d["w_scale"], T, 1, E, 288, 320)
    ok, err, bound = oracle.tolerance_ok(oracle.bf16_decode(_run_act(wob, d, ids, tile_m)),
                                         oracle.silu_mul(pre))
    assert ok, f"max err {err} > bound {bound}"


@pytest.mark.parametrize("tile_m", TILE_M)
def test_config_moe_stage1_silu_mul_full_size(wob, oracle, tile_m):
    """The full MoE shape with the fused activation: all outputs finite, 2000
    sampled outputs against the oracle's silu(gate) * up of sampled gate and
    up pre-activations."""
    d = wl.BY_KEY["moe_stage1"].make()
    ybits = _run_act(wob, d, tile_m=tile_m)
    y = oracle.bf16_decode(ybits)
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(1)
    T, topk, N = d["T"], d["topk"], d["N"]
    I = N // 2
    ts = rng.integers(0, T, 2000)
    ss = rng.integers(0, topk, 2000)
    ns = rng.integers(0, I, 2000)
    ns[:2] = [0, I - 1]
    args = (d["x"], d["ids"], d["w_fp4"], d["w_scale"], topk, d["E"], N, d["K"])
    gate = oracle.mxfp4_moe_gemm_sampled(*args, ts, ss, ns)
    up = oracle.mxfp4_moe_gemm_sampled(*args, ts, ss, ns + I)
    ref = oracle.silu_mul(np.stack([gate, up], axis=-1))[..., 0]
    ok, err, bound = oracle.tolerance_ok(y[ts, ss, ns], ref)
    assert ok, (err, bound)


# --- decode path: at most 8 tokens (split weight rows, no MFMA tiles) -------------

@pytest.mark.parametrize("T,E,topk,N,K", [
    (1, 32, 4, 5760, 2880), (8, 32, 4, 5760, 2880),  # the MoE shape with decode batches
    (2, 8, 2, 528, 192), (3, 4, 4, 48, 64), (5, 16, 3, 272, 640),
    (8, 64, 8, 96, 4160),    # K past 4096: four staged rows per pass, several passes per tile
    (3, 4, 2, 64, 32768),    # one staged row per pass
    (2, 4, 2, 32, 32832)])   # K too long to stage: the tile kernel runs instead
def test_moe_decode_parity(wob, oracle, T, E, topk, N, K):
    d = wl.moe_inputs(T, E, topk, N, K, seed=T * 7 + N + K)
    _check(oracle, d, _run(wob, d))


def test_moe_decode_invalid_and_repeated_ids(wob, oracle):
    """Out-of-range ids write zero rows; an expert named twice by one token gets
    two rows of the same activation."""
    d = wl.moe_inputs(6, 8, 4, 304, 256, seed=9)
    ids = d["ids"].copy()
    ids[0, 0] = -1
    ids[2, 3] = 8
    ids[4, :] = 3  # all four slots of token 4 on expert 3
    ids[5, 1] = ids[5, 0]
    ybits = _run(wob, d, ids)
    _check(oracle, d, ybits, ids)
    assert np.all(ybits[0, 0] == 0) and np.all(ybits[2, 3] == 0)
    assert np.array_equal(ybits[4, 0], ybits[4, 3]) and np.array_equal(ybits[5, 0], ybits[5, 1])


@pytest.mark.parametrize("T,E,topk,N,K", [(1, 32, 4, 5760, 2880), (4, 8, 2, 32, 64),
                                          (8, 16, 4, 576, 4160)])
def test_moe_decode_silu_mul(wob, oracle, T, E, topk, N, K):
    d = wl.moe_inputs(T, E, topk, N, K, seed=T + K)
    ids = d["ids"].copy()
    ids[0, topk - 1] = E  # out-of-range id: zero row
    pre = oracle.mxfp4_moe_gemm(d["x"], ids, d["w_fp4"], d["w_scale"], T, topk, E, N, K)
    ybits = _run_act(wob, d, ids)
    ok, err, bound = oracle.tolerance_ok(oracle.bf16_decode(ybits), oracle.silu_mul(pre))
    assert ok, f"max err {err} > bound {bound}"
    assert np.all(ybits[0, topk - 1] == 0)


@pytest.mark.parametrize("T,N,K", [(16, 16384, 262144), (4, 131072, 32768)])
def test_moe_expert_past_4gib(wob, oracle, T, N, K):
    """Expert 2 of three 2 GiB experts starts 4 GiB into w_fp4, so its base
    offset needs 64 bits (tile path at T = 16, decode path at T = 4).  Only that
    expert is filled and named by the ids; sampled outputs are checked against
    the one-expert problem."""
    torch = torch_mod()
    E = 3
    d = wl.moe_inputs(T, 1, 1, N, K, seed=21)
    w = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty((E, N, K // 32), dtype=torch.uint8, device="cuda")
    assert w[2].data_ptr() - w.data_ptr() == 1 << 32
    w[2].copy_(torch.from_numpy(d["w_fp4"][0]))
    s[2].copy_(torch.from_numpy(d["w_scale"][0]))
    ids = torch.full((T, 1), 2, dtype=torch.int32, device="cuda")
    x = dev(d["x"].view(np.int16)).view(torch.bfloat16)
    out = torch.empty((T + 2, N), dtype=torch.bfloat16, device="cuda")
    out.fill_(float("nan"))
    wob.mxfp4_moe_gemm(x, ids, w, s, out=out[1:T + 1].view(T, 1, N))
    torch.cuda.synchronize()
    bits = host_bits(out)
    assert np.all(is_nan_bits(bits[0], wl.BF16)) and np.all(is_nan_bits(bits[-1], wl.BF16))
    y = oracle.bf16_decode(bits[1:-1])
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(4)
    ts = rng.integers(0, T, 64)
    ns = rng.integers(0, N, 64)
    ts[:2], ns[:2] = [0, T - 1], [0, N - 1]
    ss = np.zeros_like(ts)
    yref = oracle.mxfp4_moe_gemm_sampled(d["x"], np.zeros((T, 1), np.int32), d["w_fp4"],
                                         d["w_scale"], 1, 1, N, K, ts, ss, ns)
    ok, err, bound = oracle.tolerance_ok(y[ts, ns], yref)
    assert ok, (err, bound)
