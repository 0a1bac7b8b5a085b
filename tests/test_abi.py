"""The C-ABI library loads, exports every entry point its header declares, and
rejects bad arguments before touching a device (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from weight_only_bit_amd import _lib, build
    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    return _lib


def _declared_functions():
    names = []
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            text = open(os.path.join(ROOT, "include", f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                                text, flags=re.M)
    return sorted(set(names))


def test_header_declarations_are_exported(L):
    declared = _declared_functions()
    assert "w4a16_gemm" in declared and "mxfp4_moe_gemm" in declared
    lib = L.lib()
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(L.EXPORTS)


def test_status_strings(L):
    assert L.status_str(0) == "ok"
    assert "dtype" in L.status_str(2)


class _Fake:
    """16-byte aligned host buffer standing in for device pointers: the
    library must refuse every case below before dereferencing anything."""

    def __init__(self):
        self.buf = np.zeros(64, np.uint8)
        addr = self.buf.ctypes.data
        self.p = ctypes.c_void_p(addr + (-addr) % 16)


def _gemm(L, x=True, xdt=0, sdt=0, zdt=2, zeros=True, M=1, N=8, K=64, g=32, path=0):
    f = _Fake()
    p = f.p
    return L.lib().w4a16_gemm_ex(p if x else None, xdt, p, p, sdt, p if zeros else None, zdt, p,
                                 M, N, K, g, path, None)


def test_act_dtype_zero_points_are_refused(L):
    assert _gemm(L, zdt=0) == L.DTYPE  # fp16 zero-points
    assert _gemm(L, zdt=1) == L.DTYPE
    assert _gemm(L, zdt=3) == L.DTYPE
    assert "packed" in L.last_error()


def test_dtype_checks(L):
    assert _gemm(L, xdt=3, sdt=3) == L.DTYPE
    assert _gemm(L, xdt=0, sdt=1) == L.DTYPE


def test_shape_checks(L):
    assert _gemm(L, N=12) == L.INVALID_ARG     # N % 8
    assert _gemm(L, K=48, g=32) == L.INVALID_ARG  # K % g
    assert _gemm(L, K=16) == L.INVALID_ARG
    assert _gemm(L, M=-1) == L.INVALID_ARG
    assert _gemm(L, g=16) == L.UNSUPPORTED
    assert _gemm(L, g=256, K=256) == L.UNSUPPORTED
    assert _gemm(L, x=False) == L.INVALID_ARG
    assert _gemm(L, path=7) == L.INVALID_ARG
    assert _gemm(L, M=9, path=L.PATH_SKINNY) == L.INVALID_ARG
    # empty problems are no-ops
    assert _gemm(L, M=0) == L.OK
    assert _gemm(L, N=0) == L.OK


def test_tiled_activation_offsets_bound(L):
    """The tile kernels keep a tile's activation row offsets in 32 bits: a long
    K with a full 256-row tile is refused (2*K*min(M, 256) must stay below
    2^32), on the dense and the grouped form.  (Every call here must be refused
    before any device access: the pointers are host stand-ins.)"""
    K = 1 << 23  # 2*K*256 = 2^32
    assert _gemm(L, M=256, N=8, K=K, g=128) == L.INVALID_ARG
    assert "tiled path" in L.last_error()
    f = _Fake()
    p = f.p
    grouped = L.lib().w4a16_gemm_grouped(p, 0, p, 2, 512, p, p, 0, p, 2, p, 8, K, 128, None)
    assert grouped == L.INVALID_ARG


def test_misaligned_pointer_refused(L):
    f = _Fake()
    bad = ctypes.c_void_p(f.p.value + 2)
    st = L.lib().w4a16_gemm(bad, 0, f.p, f.p, 0, f.p, 2, f.p, 1, 8, 64, 32, None)
    assert st == L.INVALID_ARG


def test_moe_checks(L):
    f = _Fake()
    p = f.p
    need = L.lib().mxfp4_moe_gemm_workspace_size(1024, 4, 32, 5760, 2880)
    assert need > 0
    assert L.lib().mxfp4_moe_gemm_workspace_size(-1, 4, 32, 64, 64) == 0
    assert L.lib().mxfp4_moe_gemm_workspace_size(4, 65, 32, 64, 64) == 0
    call = lambda K=64, N=32, ws=need, T=4: L.lib().mxfp4_moe_gemm(p, p, p, p, p, T, 4, 32, N, K,
                                                                   0, p, ws, None)
    assert call(K=48) == L.INVALID_ARG
    assert call(K=96) == L.INVALID_ARG  # the K tile is 64 wide
    assert call(N=24) == L.INVALID_ARG
    assert call(T=1 << 21, K=1 << 11) == L.INVALID_ARG  # x past 32-bit byte offsets
    act = lambda a, N=32: L.lib().mxfp4_moe_gemm(p, p, p, p, p, 4, 4, 32, N, 64, a, p, need, None)
    assert act(2) == L.INVALID_ARG          # unknown activation
    assert act(1, N=48) == L.INVALID_ARG    # silu(gate) * up needs N % 32 == 0
    assert call(ws=0) == L.INVALID_ARG
    assert call(T=0) == L.OK
    tm = lambda t, T=4, K=64: L.lib().mxfp4_moe_gemm_tile_m(p, p, p, p, p, T, 4, 32, 32, K, 0, t,
                                                             p, need, None)
    for bad_tm in (0, 8, 24, 64, -16):
        assert tm(bad_tm) == L.INVALID_ARG, bad_tm
    assert tm(16, K=48) == L.INVALID_ARG    # the other checks still apply
    assert tm(16, T=0) == L.OK and tm(32, T=0) == L.OK


def test_grouped_checks(L):
    f = _Fake()
    p = f.p
    g = lambda E=2, zdt=2: L.lib().w4a16_gemm_grouped(p, 0, p, E, 8, p, p, 0, p, zdt, p, 16, 64, 32, None)
    assert g(zdt=0) == L.DTYPE
    assert g(E=-1) == L.INVALID_ARG
    assert g(E=0) == L.OK


def test_probe_checks(L):
    f = _Fake()
    p = f.p
    assert L.lib().w4a16_dequant(p, p, 0, p, 2, p, 1, 8, 64, 32, None) == L.DTYPE  # bf16 out, fp16 scales
    assert L.lib().mxfp4_dequant(p, p, p, 8, 48, None) == L.INVALID_ARG


def test_stream_read_checks(L):
    f = _Fake()
    p = f.p
    assert L.lib().wob_stream_read(p, 24, p, None) == L.INVALID_ARG   # not a multiple of 16
    assert L.lib().wob_stream_read(None, 32, p, None) == L.INVALID_ARG
    assert L.lib().wob_stream_read(p, 32, None, None) == L.INVALID_ARG
    assert L.lib().wob_stream_read(p, 0, None, None) == L.OK           # nothing to read


def test_no_gpu_means_an_error_not_a_fallback(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _gemm(L) in (L.HIP, L.UNSUPPORTED)


# --- Python binding: operand shapes and dtypes are checked before any device access ---

@pytest.fixture(scope="module")
def wobpkg(L):
    import weight_only_bit_amd as w
    return w


def _w4_cpu(M=4, N=16, K=64, g=32, dtype=None):
    import torch
    dt = dtype or torch.float16
    G = K // g
    return dict(x=torch.zeros((M, K), dtype=dt), q=torch.zeros((N, K // 8), dtype=torch.int32),
                s=torch.zeros((N, G), dtype=dt), z=torch.zeros((N // 8, G), dtype=torch.int32))


def test_binding_gemm_shape_checks(wobpkg):
    import torch
    t = _w4_cpu()
    with pytest.raises(ValueError, match="scales"):   # scales for another group size
        wobpkg.gemm(t["x"], t["q"], torch.zeros((16, 4), dtype=torch.float16), t["z"], 32)
    with pytest.raises(ValueError, match="qweight"):  # qweight for another K
        wobpkg.gemm(t["x"], torch.zeros((16, 4), dtype=torch.int32), t["s"], t["z"], 32)
    with pytest.raises(ValueError, match="qzeros"):
        wobpkg.gemm(t["x"], t["q"], t["s"], torch.zeros((1, 1), dtype=torch.int32), 32)
    with pytest.raises(ValueError, match="out"):      # too small an output
        wobpkg.gemm(t["x"], t["q"], t["s"], t["z"], 32, out=torch.empty((4, 8), dtype=torch.float16))
    with pytest.raises(TypeError, match="out"):
        wobpkg.gemm(t["x"], t["q"], t["s"], t["z"], 32, out=torch.empty((4, 16), dtype=torch.float32))
    with pytest.raises(TypeError, match="scales"):
        wobpkg.gemm(t["x"], t["q"], t["s"].to(torch.bfloat16), t["z"], 32)
    with pytest.raises(TypeError, match="qzeros"):    # activation-dtype zero-points
        wobpkg.gemm(t["x"], t["q"], t["s"], torch.zeros((16, 2), dtype=torch.float16), 32)
    with pytest.raises(ValueError, match="group_size"):
        wobpkg.gemm(t["x"], t["q"], t["s"], t["z"], 48)
    with pytest.raises(ValueError, match="device"):   # shapes right: then the device check
        wobpkg.gemm(t["x"], t["q"], t["s"], t["z"], 32)


def test_binding_grouped_and_moe_shape_checks(wobpkg):
    import torch
    x = torch.zeros((10, 64), dtype=torch.float16)
    q = torch.zeros((3, 16, 8), dtype=torch.int32)
    s = torch.zeros((3, 16, 2), dtype=torch.float16)
    z = torch.zeros((3, 2, 2), dtype=torch.int32)
    off = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError, match="m_offsets"):
        wobpkg.gemm_grouped(x, torch.zeros(3, dtype=torch.int64), q, s, z, 32)
    with pytest.raises(ValueError, match="scales"):
        wobpkg.gemm_grouped(x, off, q, s[:2], z, 32)
    with pytest.raises(ValueError, match="device"):
        wobpkg.gemm_grouped(x, off, q, s, z, 32)
    xb = torch.zeros((4, 128), dtype=torch.bfloat16)
    ids = torch.zeros((4, 2), dtype=torch.int32)
    w = torch.zeros((3, 32, 64), dtype=torch.uint8)
    ws = torch.zeros((3, 32, 4), dtype=torch.uint8)
    with pytest.raises(ValueError, match="w_scale"):
        wobpkg.mxfp4_moe_gemm(xb, ids, w, ws[:, :, :3])
    with pytest.raises(ValueError, match="out"):
        wobpkg.mxfp4_moe_gemm(xb, ids, w, ws, out=torch.empty((4, 2, 32), dtype=torch.bfloat16),
                              act=wobpkg.ACT_SILU_MUL)
    with pytest.raises(TypeError, match="topk_ids"):
        wobpkg.mxfp4_moe_gemm(xb, ids.to(torch.int64), w, ws)
    with pytest.raises(ValueError, match="workspace"):
        wobpkg.mxfp4_moe_gemm(xb, ids, w, ws, workspace=torch.zeros(4, dtype=torch.uint8))
    with pytest.raises(ValueError, match="activation"):
        wobpkg.mxfp4_moe_gemm(xb, ids, w, ws, act=5)
    with pytest.raises(ValueError, match="tile_m"):
        wobpkg.mxfp4_moe_gemm(xb, ids, w, ws, tile_m=64)
    with pytest.raises(ValueError, match="device"):
        wobpkg.mxfp4_moe_gemm(xb, ids, w, ws)
    with pytest.raises(ValueError, match="w_scale"):
        wobpkg.mxfp4_dequant(w[0], ws[0, :, :2])


def test_moe_stage2_checks(L):
    """MoE stage 2 refuses bad shapes, pointers and workspaces before any
    device access."""
    f = _Fake()
    p = f.p
    need = L.lib().mxfp4_moe_stage2_workspace_size(1024, 4, 32, 2880, 2880)
    assert need >= 1024 * 4 * 2880 * 4  # the fp32 per-pair rows
    assert L.lib().mxfp4_moe_stage2_workspace_size(4, 0, 32, 64, 64) == 0
    call = lambda I=64, H=32, ws=need, T=4, wp=p: L.lib().mxfp4_moe_stage2(
        p, p, wp, p, p, p, T, 4, 32, H, I, p, ws, None)
    assert call(I=96) == L.INVALID_ARG    # the K tile is 64 wide
    assert call(I=32) == L.INVALID_ARG
    assert call(H=24) == L.INVALID_ARG
    assert call(T=1 << 20, I=1 << 10) == L.INVALID_ARG  # gathered rows past 32-bit offsets
    assert call(ws=16) == L.INVALID_ARG
    assert call(wp=None) == L.INVALID_ARG
    assert call(T=0) == L.OK
    assert call(H=0) == L.OK
