"""GPU parity of the cooperative-tile MFMA W4A16 GEMM against the oracle.

Covers every tile height (M up to 32, 64, 128, above), ragged M, N and K
tails (N not a multiple of the 256-row tile, K not a multiple of the 128 span),
g in {32, 64, 128}, fp16/bf16, symmetric codes and signed two-decade scales,
the q4_0 combination of both at g = 32, weights that dequantize to zeros under
activations with outliers, plus the full prefill shape 2048x16384x5376 (g=128)
on sampled outputs from every output tile.
"""
import numpy as np
import pytest

import workloads as wl
from tests import oracle_threads
from tests.gpu_util import host_bits, is_nan_bits, require_gpu, torch_mod, w4a16_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wob():
    require_gpu()
    import weight_only_bit_amd as w
    w.device_check()
    return w


def _run(wob, d, path):
    torch = torch_mod()
    t = w4a16_to_device(d)
    M, N = d["M"], d["N"]
    out = torch.empty((M + 2, N), dtype=t["x"].dtype, device="cuda")
    out.fill_(float("nan"))
    wob.gemm(t["x"], t["qweight"], t["scales"], t["qzeros"], d["g"], out=out[1:M + 1], path=path)
    torch.cuda.synchronize()
    bits = host_bits(out)
    assert np.all(is_nan_bits(bits[0], d["dtype"])) and np.all(is_nan_bits(bits[M + 1], d["dtype"]))
    return bits[1:M + 1]


def _check(oracle, d, ybits):
    yref = oracle.w4a16_gemm(d["x"], d["dtype"], d["qweight"], d["scales"], d["qzeros"],
                             d["M"], d["N"], d["K"], d["g"])
    ok, err, bound = oracle.tolerance_ok(oracle.act_decode(ybits, d["dtype"]), yref)
    assert ok, f"max err {err} > bound {bound}"


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("M", [1, 9, 16, 17, 33, 64, 100, 129, 256, 300])
def test_tiled_m_sweep(wob, oracle, dtype, M):
    d = wl.w4a16_inputs(M, 264, 544, 32, dtype, seed=M)
    _check(oracle, d, _run(wob, d, wob.PATH_TILED))


# every (N, K) with each group size that divides K
TILED_SHAPES = [(N, K, g) for N, K in [(8, 128), (24, 32), (256, 256), (520, 1088), (1024, 384)]
                for g in (32, 64, 128) if K % g == 0]


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("N,K,g", TILED_SHAPES)
def test_tiled_shapes(wob, oracle, dtype, g, N, K):
    d = wl.w4a16_inputs(40, N, K, g, dtype, seed=N + K + g)
    _check(oracle, d, _run(wob, d, wob.PATH_TILED))


# g = 128 with an even number of groups G >= 4: the scales of four spans come
# from one load; G = 6 and 10 end on a batch that overlaps the one before it,
# G = 8 does not.  Ragged M and N, asymmetric and symmetric codes.
G128_BATCHED = [(300, 520, 768), (40, 264, 1280), (129, 1024, 1024), (17, 24, 1280)]


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("M,N,K", G128_BATCHED)
def test_tiled_g128_scale_batches(wob, oracle, dtype, M, N, K):
    d = wl.w4a16_inputs(M, N, K, 128, dtype, seed=M + N + K, symmetric=(N == 24))
    _check(oracle, d, _run(wob, d, wob.PATH_TILED))


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
def test_tiled_symmetric_and_signed(wob, oracle, dtype):
    d = wl.w4a16_inputs(70, 512, 512, 64, dtype, seed=5, symmetric=True)
    _check(oracle, d, _run(wob, d, wob.PATH_TILED))
    d = wl.w4a16_inputs(70, 512, 512, 128, dtype, seed=6, signed_scales=True)
    _check(oracle, d, _run(wob, d, wob.PATH_TILED))


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("M", [40, 300])
def test_tiled_q4_0_arithmetic(wob, oracle, dtype, M):
    """Codes offset by 8 with signed two-decade scales, one per 32 (the Q4_0 KV
    page's sections What and Signed scales), on the MFMA path, with N and K
    tails (520 rows, K = 1088)."""
    d = wl.w4a16_inputs(M, 520, 1088, 32, dtype, seed=M + 9, symmetric=True, signed_scales=True)
    _check(oracle, d, _run(wob, d, wob.PATH_TILED))


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("live", [0.0, 0.01])
def test_tiled_degenerate_weights_outlier_activations(wob, oracle, dtype, live):
    """Weights that dequantize to zero in most (or all) groups under activations
    with +-1e2..1e3 outlier columns; all-zero weights give all-zero outputs."""
    d = wl.w4a16_degenerate_inputs(70, 264, 2080, 32, dtype, seed=int(live * 100) + dtype,
                                   live_groups=live)
    ybits = _run(wob, d, wob.PATH_TILED)
    _check(oracle, d, ybits)
    if live == 0.0:
        assert np.all(oracle.act_decode(ybits, dtype) == 0.0)


def test_tiled_matches_skinny_on_small_m(wob):
    """Both paths on the same M <= 8 input agree to the parity bound of each other."""
    d = wl.w4a16_inputs(4, 512, 1024, 128, wl.F16, seed=3)
    a = _run(wob, d, wob.PATH_TILED).view(np.float16).astype(np.float64)
    b = _run(wob, d, wob.PATH_SKINNY).view(np.float16).astype(np.float64)
    assert np.max(np.abs(a - b)) <= 1e-2 * np.max(np.abs(b)) + 1e-3


def test_config_prefill_full_size(wob, oracle):
    """2048x16384x5376 g=128 fp16 in the benchmark's launch configuration: all
    outputs finite; 16 sampled outputs in each of the 8 x 64 output tiles
    (256 x 256), including each tile's four corners, against the oracle."""
    d = wl.BY_KEY["prefill"].make()
    ybits = _run(wob, d, wob.PATH_AUTO)
    y = oracle.act_decode(ybits, d["dtype"])
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(0)
    ms, ns = [], []
    for mt in range(d["M"] // 256):
        for nt in range(d["N"] // 256):
            m = mt * 256 + np.concatenate([[0, 0, 255, 255], rng.integers(0, 256, 12)])
            n = nt * 256 + np.concatenate([[0, 255, 0, 255], rng.integers(0, 256, 12)])
            ms.append(m)
            ns.append(n)
    ms, ns = np.concatenate(ms), np.concatenate(ns)
    order = np.argsort(ns, kind="stable")
    ms, ns = ms[order], ns[order]
    yref = oracle_threads.w4a16_gemm_sampled(oracle, d, ms, ns)
    ok, err, bound = oracle.tolerance_ok(y[ms, ns], yref)
    assert ok, (err, bound)


def test_tiled_deterministic(wob):
    d = wl.w4a16_inputs(300, 520, 1088, 32, wl.BF16, seed=2)
    assert np.array_equal(_run(wob, d, wob.PATH_TILED), _run(wob, d, wob.PATH_TILED))


def test_tiled_codes_past_2gib(wob, oracle):
    """2 GiB of packed codes (N = 16384, K = 262144, g = 128): byte offsets into
    the code matrix pass 2^31 (the ABI allows up to 2^32), so an offset kept in
    a signed 32-bit integer would fail here.  Sampled outputs, including the
    last weight rows and both activation rows of the tile's ends."""
    d = wl.w4a16_inputs(16, 16384, 262144, 128, wl.F16, seed=11)
    assert d["qweight"].nbytes == 1 << 31
    ybits = _run(wob, d, wob.PATH_TILED)
    y = oracle.act_decode(ybits, d["dtype"])
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(3)
    ns = np.sort(np.concatenate([[0, 8191, 8192, 16383, 16376], rng.integers(0, 16384, 59)]))
    ms = rng.integers(0, 16, ns.size)
    ms[-1] = 15
    yref = oracle.w4a16_gemm_sampled(d["x"], d["dtype"], d["qweight"], d["scales"], d["qzeros"],
                                     d["K"], d["g"], ms, ns)
    ok, err, bound = oracle.tolerance_ok(y[ms, ns], yref)
    assert ok, (err, bound)
