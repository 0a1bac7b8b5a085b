"""GPU parity of the ragged grouped W4A16 GEMM against the oracle, through the
C ABI.

Group e owns rows [m_offsets[e], m_offsets[e+1]) and its own packed weights.
Cases: empty groups, groups shorter than one 32-row block, groups spanning
several 256-row tiles, more than 64 groups (the device-side tile lookup walks
the offsets 64 at a time), symmetric codes, both activation dtypes, and NaN
guard rows around y to catch stray writes.
"""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import dev, dev_act, host_bits, is_nan_bits, require_gpu, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wob():
    require_gpu()
    import weight_only_bit_amd as w
    w.device_check()
    return w


def _run(wob, d, symmetric=False):
    torch = torch_mod()
    total = int(d["m_offsets"][-1])
    N = d["N"]
    out = torch.empty((total + 2, N), dtype=torch.float16 if d["dtype"] == wl.F16 else torch.bfloat16,
                      device="cuda")
    out.fill_(float("nan"))
    y = out[1:total + 1]
    wob.gemm_grouped(dev_act(d["x"], d["dtype"]), dev(d["m_offsets"]), dev(d["qweight"]),
                     dev_act(d["scales"], d["dtype"]), None if symmetric else dev(d["qzeros"]),
                     d["g"], out=y)
    torch.cuda.synchronize()
    bits = host_bits(out)
    assert np.all(is_nan_bits(bits[0], d["dtype"])) and np.all(is_nan_bits(bits[-1], d["dtype"]))
    return bits[1:-1]


def _check(oracle, d, ybits, symmetric=False):
    yref = oracle.w4a16_gemm_grouped(d["x"], d["dtype"], d["m_offsets"], d["qweight"], d["scales"],
                                     None if symmetric else d["qzeros"], d["N"], d["K"], d["g"])
    ok, err, bound = oracle.tolerance_ok(oracle.act_decode(ybits, d["dtype"]), yref)
    assert ok, f"max err {err} > bound {bound}"


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("rows", [[0, 5, 300, 17, 0, 64], [1], [256, 256], [513, 0, 31]])
def test_grouped_ragged(wob, oracle, dtype, rows):
    d = wl.w4a16_grouped_inputs(rows, 264, 544, 32, dtype, seed=sum(rows))
    _check(oracle, d, _run(wob, d))


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
def test_grouped_g128_scale_batches(wob, oracle, dtype):
    # g = 128, G = 6: each group's tiles take the scales of four spans per load
    d = wl.w4a16_grouped_inputs([70, 0, 300, 9], 264, 768, 128, dtype, seed=5)
    _check(oracle, d, _run(wob, d))


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
def test_grouped_many_groups_symmetric(wob, oracle, dtype):
    rng = np.random.default_rng(1)
    rows = list(rng.integers(0, 40, 100))
    d = wl.w4a16_grouped_inputs(rows, 64, 256, 128, dtype, seed=2)
    _check(oracle, d, _run(wob, d, symmetric=True), symmetric=True)


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
def test_grouped_q4_0_arithmetic(wob, oracle, dtype):
    """Symmetric codes (z = 8) with signed two-decade scales at g = 32 on the
    grouped path (the Q4_0 KV page's sections What and Signed scales)."""
    d = wl.w4a16_grouped_inputs([37, 0, 300, 5], 264, 544, 32, dtype, seed=8, symmetric=True,
                                signed_scales=True)
    _check(oracle, d, _run(wob, d, symmetric=True), symmetric=True)


def test_grouped_single_group_matches_dense(wob):
    """One group covering every row gives the dense GEMM's bits."""
    torch = torch_mod()
    d = wl.w4a16_grouped_inputs([300], 512, 1024, 64, wl.F16, seed=4)
    a = _run(wob, d)
    y = wob.gemm(dev_act(d["x"], wl.F16), dev(d["qweight"][0]), dev_act(d["scales"][0], wl.F16),
                 dev(d["qzeros"][0]), 64)
    torch.cuda.synchronize()
    assert np.array_equal(a, host_bits(y))


def test_grouped_moe_like_full_size(wob, oracle):
    """The MoE-like grouped configuration at full size (32 experts, 4096 routed
    rows, N 5760, K 2880, g 32, bf16): every output finite, sampled outputs of
    every group (its first and last row and random ones, at random columns)
    against the oracle run on that group's rows and weights."""
    d = wl.BY_KEY["grouped_moe_like"].make()
    bits = _run(wob, d)
    y = oracle.act_decode(bits, d["dtype"])
    assert np.all(np.isfinite(y))
    off = d["m_offsets"]
    rng = np.random.default_rng(2)
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 4)]))
        ms = np.repeat(rows - lo, 16)
        ns = rng.integers(0, d["N"], ms.size)
        order = np.argsort(ns, kind="stable")
        ms, ns = ms[order], ns[order]
        yref = oracle.w4a16_gemm_sampled(d["x"][lo:hi], d["dtype"], d["qweight"][e],
                                         d["scales"][e], d["qzeros"][e], d["K"], d["g"], ms, ns)
        ok, err, bound = oracle.tolerance_ok(y[lo + ms, ns], yref)
        assert ok, (e, err, bound)


def test_grouped_all_groups_empty_is_a_noop(wob):
    """Every group empty (total_M = 0): nothing is written, no error."""
    torch = torch_mod()
    d = wl.w4a16_grouped_inputs([0, 0, 0], 64, 256, 32, wl.F16, seed=3)
    out = torch.full((2, 64), float("nan"), dtype=torch.float16, device="cuda")
    x = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    wob.gemm_grouped(x, dev(d["m_offsets"]), dev(d["qweight"]), dev_act(d["scales"], d["dtype"]),
                     dev(d["qzeros"]), 32, out=out[1:1])
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
