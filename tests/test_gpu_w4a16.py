"""GPU parity of the W4A16 kernels against the oracle (through the C ABI).

Bar (weight-only 4-bit GEMM contract): every output element satisfies
|y - y_ref| <= 1e-3 + 1e-2 * max|y_ref|, no NaN/Inf; the dequantization
probes are bit-exact.  The matrix follows the zero-point page's value-level
tests (section Testing: fp16/bf16 x g32/g128 x three shapes including N = 8,
one packed word, plus the refusal of activation-dtype zero-points) widened to
g = 64, symmetric codes, signed two-decade scales and ragged K, the q4_0
arithmetic of the Q4_0 KV page ((code - 8) * d per 32 with signed d), weights
that dequantize to zeros under activations with outliers, scales at the ends
of the fp16 / bf16 ranges, and the full decode shapes element by element.
"""
import numpy as np
import pytest

import workloads as wl
from tests import oracle_threads
from tests.gpu_util import dev, host_bits, is_nan_bits, require_gpu, torch_mod, w4a16_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wob():
    require_gpu()
    import weight_only_bit_amd as w
    w.device_check()
    return w


def _run(wob, d, path, sentinel=True):
    torch = torch_mod()
    t = w4a16_to_device(d)
    M, N = d["M"], d["N"]
    out = torch.empty((M + 2, N), dtype=t["x"].dtype, device="cuda")
    out.fill_(float("nan"))
    y = out[1:M + 1]
    wob.gemm(t["x"], t["qweight"], t["scales"], t["qzeros"], d["g"], out=y, path=path)
    torch.cuda.synchronize()
    bits = host_bits(out)
    if sentinel:
        # rows outside y must still hold the NaN sentinel (no stray writes)
        assert np.all(is_nan_bits(bits[0], d["dtype"]))
        assert np.all(is_nan_bits(bits[M + 1], d["dtype"]))
    return bits[1:M + 1]


def _check(oracle, d, ybits):
    yref = oracle.w4a16_gemm(d["x"], d["dtype"], d["qweight"], d["scales"], d["qzeros"],
                             d["M"], d["N"], d["K"], d["g"])
    y = oracle.act_decode(ybits, d["dtype"])
    ok, err, bound = oracle.tolerance_ok(y, yref)
    assert ok, f"max err {err} > bound {bound}"
    return err, bound


SHAPES = [(8, 256), (256, 512), (2048, 2048)]


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
def test_skinny_parity_matrix(wob, oracle, dtype, g, N, K, M):
    d = wl.w4a16_inputs(M, N, K, g, dtype, seed=M * 7 + g + N)
    _check(oracle, d, _run(wob, d, wob.PATH_SKINNY))


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("M,N,K,g", [(1, 8, 32, 32), (3, 16, 96, 32), (4, 24, 160, 32),
                                     (2, 40, 384, 128), (8, 64, 1088, 64), (1, 4104, 4096, 128),
                                     # 2049 octets, K split 2 ways over 8-wave workgroups of
                                     # 4 octets: the last workgroup holds one octet
                                     (1, 16392, 2048, 32), (3, 16392, 1024, 128)])
def test_skinny_ragged_shapes(wob, oracle, dtype, M, N, K, g):
    d = wl.w4a16_inputs(M, N, K, g, dtype, seed=N + K)
    _check(oracle, d, _run(wob, d, wob.PATH_SKINNY))


SPLIT_K = [(1, 1056, 32), (1, 2176, 128), (1, 4224, 64), (1, 5408, 32), (1, 6944, 32),
           (1, 16416, 32), (1, 16512, 128), (4, 1056, 32), (4, 4224, 64), (4, 5408, 32),
           (4, 7040, 128), (8, 1056, 32), (8, 2176, 128), (8, 3200, 128)]


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("M,K,g", SPLIT_K)
def test_skinny_split_k_ring(wob, oracle, dtype, M, K, g):
    # N = 2048 splits K 2, 4 or 8 ways over the waves of a workgroup: 1 to 9
    # chunks per lane, lanes of one wave one chunk apart in the last K slice,
    # so the load ring's steady state, its drain and the clamped refills all
    # run.
    d = wl.w4a16_inputs(M, 2048, K, g, dtype, seed=K + M, symmetric=(K % 3 == 0))
    _check(oracle, d, _run(wob, d, wob.PATH_SKINNY))


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("M", [1, 4])
def test_skinny_symmetric_and_signed_scales(wob, oracle, dtype, M):
    d = wl.w4a16_inputs(M, 256, 1024, 32, dtype, seed=3, symmetric=True)
    _check(oracle, d, _run(wob, d, wob.PATH_SKINNY))
    d = wl.w4a16_inputs(M, 256, 1024, 128, dtype, seed=4, signed_scales=True)
    _check(oracle, d, _run(wob, d, wob.PATH_SKINNY))


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("M,N,K", [(1, 256, 1024), (4, 256, 1024), (1, 2048, 4224),
                                   (4, 2048, 5408)])
def test_skinny_q4_0_arithmetic(wob, oracle, dtype, M, N, K):
    """The Q4_0 KV page's arithmetic (section What: codes offset by 8, one
    scale per 32; section Signed scales): symmetric codes (z = 8) together with
    signed two-decade scales at g = 32, on the row-octet layout (N = 256) and
    on the split-K layout with scales through the load ring (N = 2048)."""
    d = wl.w4a16_inputs(M, N, K, 32, dtype, seed=M + K, symmetric=True, signed_scales=True)
    _check(oracle, d, _run(wob, d, wob.PATH_SKINNY))


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("M,K", [(1, 5376), (4, 5376), (8, 2048)])
@pytest.mark.parametrize("live", [0.0, 0.01, 0.1])
@pytest.mark.parametrize("symmetric", [False, True])
def test_skinny_degenerate_weights_outlier_activations(wob, oracle, dtype, M, K, live, symmetric):
    """Most (or all) groups have q = z, so y_ref is small (or exactly zero, and
    the parity bound its 1e-3 floor) while 2 % of the activation columns reach
    +-1e2..1e3 (g = 32, a split-K layout at N = 2048 and the row-octet layout
    at N = 256).  This is the case that separates exact (q - z) operands from
    a zero-point folded out of the sums (sum (B + q) x - (B + z) sum x), whose
    rounding grows with B: with B = 1024 it misses the bound here 15-fold.
    With all weights zero every output must be zero."""
    for N in (256, 2048):
        d = wl.w4a16_degenerate_inputs(M, N, K, 32, dtype, seed=M * 3 + N, live_groups=live,
                                       symmetric=symmetric)
        ybits = _run(wob, d, wob.PATH_SKINNY)
        _check(oracle, d, ybits)
        if live == 0.0:
            assert np.all(oracle.act_decode(ybits, dtype) == 0.0)


def test_config_tiny_gemv(wob, oracle):
    d = wl.BY_KEY["tiny_gemv"].make()
    _check(oracle, d, _run(wob, d, wob.PATH_AUTO))


def test_config_small_batch(wob, oracle):
    d = wl.BY_KEY["small_batch"].make()
    _check(oracle, d, _run(wob, d, wob.PATH_AUTO))


def _check_full(oracle, d, ybits):
    """Every output against the oracle, which runs on N-slices in host threads."""
    yref = oracle_threads.w4a16_gemm(oracle, d)
    ok, err, bound = oracle.tolerance_ok(oracle.act_decode(ybits, d["dtype"]), yref)
    assert ok, f"max err {err} > bound {bound}"


def test_config_decode_gemv_full_size(wob, oracle):
    """1x43008x5376 g=32 at full size, in the launch configuration the
    benchmark times: all 43008 outputs against the oracle."""
    d = wl.BY_KEY["decode_gemv"].make()
    _check_full(oracle, d, _run(wob, d, wob.PATH_AUTO, sentinel=True))


@pytest.mark.parametrize("key", ["bs4_2048x2560", "bs4_6144x2048", "bs4_4096x2048"])
def test_page_batch4_shapes(wob, oracle, key):
    """The zero-point page's batch-4, g = 128 asymmetric shapes, every output."""
    d = wl.BY_KEY[key].make()
    _check(oracle, d, _run(wob, d, wob.PATH_AUTO))


@pytest.mark.parametrize("key", ["decode_qkv", "decode_down"])
def test_page_decode_shapes_full_size(wob, oracle, key):
    """The page's qkv and down decode shapes at full size: every output against
    the oracle."""
    d = wl.BY_KEY[key].make()
    _check_full(oracle, d, _run(wob, d, wob.PATH_AUTO, sentinel=True))


def test_refuses_act_dtype_zero_points(wob):
    torch = torch_mod()
    d = wl.w4a16_inputs(1, 16, 64, 32, wl.F16)
    t = w4a16_to_device(d)
    zp_act = torch.zeros((16, 2), dtype=torch.float16, device="cuda")
    with pytest.raises(TypeError):
        wob.gemm(t["x"], t["qweight"], t["scales"], zp_act, 32)


def test_deterministic_repeat(wob):
    d = wl.w4a16_inputs(4, 2048, 2048, 128, wl.BF16, seed=1)
    a = _run(wob, d, wob.PATH_AUTO)
    b = _run(wob, d, wob.PATH_AUTO)
    assert np.array_equal(a, b)


# --- dequantization probes: bit-exact ---------------------------------------

@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("variant", ["asym", "sym", "signed", "q4_0"])
def test_dequant_probe_bit_exact(wob, oracle, dtype, g, variant):
    N, K = 64, 512
    d = wl.w4a16_inputs(1, N, K, g, dtype, seed=g + dtype,
                        symmetric=variant in ("sym", "q4_0"),
                        signed_scales=variant in ("signed", "q4_0"))
    _probe_bit_exact(wob, oracle, d)


def _probe_bit_exact(wob, oracle, d):
    """Both probe forms against the oracle's exact (q - z) * s, bit for bit."""
    dtype, N, K, g = d["dtype"], d["N"], d["K"], d["g"]
    t = w4a16_to_device(d)
    w32_ref = oracle.w4a16_dequant(d["qweight"], d["scales"], dtype, d["qzeros"], N, K, g)
    w32 = wob.w4a16_dequant(t["qweight"], t["scales"], t["qzeros"], g).cpu().numpy()
    assert np.array_equal(w32.view(np.uint32), w32_ref.view(np.uint32))
    wa_ref = oracle.w4a16_dequant_act(d["qweight"], d["scales"], dtype, d["qzeros"], N, K, g)
    wa = host_bits(wob.w4a16_dequant(t["qweight"], t["scales"], t["qzeros"], g,
                                     out_dtype=t["scales"].dtype))
    assert np.array_equal(wa, wa_ref)


# fp16 and bf16 bit patterns of scales at the ends of each format's range:
# subnormals, the smallest normals, and magnitudes whose products with
# |q - z| = 15 overflow to infinity.
_SCALE_BANDS = {wl.F16: [(0x0001, 0x03FF), (0x0400, 0x0800), (0x7800, 0x7BFF)],
                wl.BF16: [(0x0001, 0x007F), (0x0080, 0x0100), (0x7E80, 0x7F7F)]}


@pytest.mark.parametrize("dtype", [wl.F16, wl.BF16])
@pytest.mark.parametrize("symmetric", [False, True])
def test_dequant_probe_scale_extremes(wob, oracle, dtype, symmetric):
    """Scales drawn from the subnormal, smallest-normal and near-overflow bands
    of the scale dtype, both signs: the fp32 form and the MFMA operand form
    (whose rounding produces subnormals and infinities here) stay bit-exact."""
    N, K, g = 64, 512, 32
    d = wl.w4a16_inputs(1, N, K, g, dtype, seed=7 + dtype, symmetric=symmetric)
    rng = np.random.default_rng(17 + dtype)
    bands = _SCALE_BANDS[dtype]
    pick = rng.integers(0, len(bands), d["scales"].shape)
    lo = np.array([b[0] for b in bands])[pick]
    hi = np.array([b[1] for b in bands])[pick]
    bits = lo + (rng.random(d["scales"].shape) * (hi - lo + 1)).astype(np.int64)
    sign = rng.integers(0, 2, d["scales"].shape) << 15
    d["scales"] = (bits | sign).astype(np.uint16)
    _probe_bit_exact(wob, oracle, d)


def test_mxfp4_dequant_probe_bit_exact(wob, oracle):
    """Every E2M1 code under every E8M0 byte 0..255: subnormal and overflowing
    bfloat16 results, the OCP ends 2^-127 (byte 0) and NaN (byte 255)."""
    rng = np.random.default_rng(0)
    N, K = 256, 512  # 16 scale blocks per row: 4096 blocks, each byte 16 times
    codes = rng.integers(0, 16, (N, K))
    codes[:, :16] = np.arange(16)  # every code once in the first block of each row
    w_fp4 = wl.pack_fp4_pairs(codes)
    w_scale = (np.arange(N * (K // 32)) % 256).astype(np.uint8).reshape(N, K // 32)
    rng.shuffle(w_scale.reshape(-1))
    w_scale[:, 0] = np.arange(N)  # the first block of row n has byte n
    ref = oracle.mxfp4_dequant(w_fp4, w_scale, N, K).astype(np.float64)
    out = wob.mxfp4_dequant(dev(w_fp4), dev(w_scale))
    got = oracle.bf16_decode(host_bits(out))
    assert np.array_equal(got, ref, equal_nan=True), (got[0, :16], ref[0, :16])
    # the sign of zero (code 8 is -0) must match too; a NaN's sign carries no
    # meaning (IEEE 754) and is not compared
    num = ~np.isnan(ref)
    assert np.array_equal(np.signbit(got[num]), np.signbit(ref[num]))
    assert np.all(np.isnan(got[:, 0][w_scale[:, 0] == 255]))


def test_stream_read_reference_runs(wob):
    """The streaming-read measurement aid reads a buffer and returns OK; its
    sink is scratch (it holds no result to check)."""
    torch = torch_mod()
    buf = torch.ones(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    wob.stream_read(buf, buf.numel(), sink)
    wob.stream_read(buf, 4096 + 16, sink)  # a tail shorter than one grid step
    torch.cuda.synchronize()
    assert torch.all(buf == 1)


@pytest.mark.parametrize("path_name", ["PATH_AUTO", "PATH_SKINNY", "PATH_TILED"])
def test_empty_batch_is_a_noop(wob, path_name):
    """M = 0 (an empty batch) returns an empty result on every path and
    enqueues nothing."""
    torch = torch_mod()
    d = wl.w4a16_inputs(1, 64, 256, 32, wl.F16, seed=5)
    t = w4a16_to_device(d)
    x0 = t["x"][:0]
    y = wob.gemm(x0, t["qweight"], t["scales"], t["qzeros"], 32, path=getattr(wob, path_name))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 64)
