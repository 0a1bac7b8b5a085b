"""The allocation-free MoE stage-1 entry point (routing scratch in a static
device array) against the entry point with a caller workspace, through the C
ABI: identical bits on two calls in a row, the second one smaller (the
static array keeps the first call's contents, which must not leak into the
second), on the tile path and on the decode path."""
import ctypes

import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import dev, host_bits, require_gpu, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wob():
    require_gpu()
    import weight_only_bit_amd as w
    w.device_check()
    return w


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _both(wob, d, act):
    """(bits of the workspace entry point, bits of the allocation-free one)."""
    from weight_only_bit_amd import _lib
    torch = torch_mod()
    T, topk, E, N, K = d["T"], d["topk"], d["E"], d["N"], d["K"]
    nout = N // 2 if act else N
    x = dev(d["x"].view(np.int16)).view(torch.bfloat16)
    ids, w, s = dev(d["ids"]), dev(d["w_fp4"]), dev(d["w_scale"])
    ref = wob.mxfp4_moe_gemm(x, ids, w, s, act=act)
    out = torch.full((T, topk, nout), float("nan"), dtype=torch.bfloat16, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = _lib.lib().mxfp4_moe_gemm_noalloc(_p(x), _p(ids), _p(w), _p(s), _p(out), T, topk, E, N,
                                           K, act, stream)
    _lib.check(st, "mxfp4_moe_gemm_noalloc")
    torch.cuda.synchronize()
    return host_bits(ref), host_bits(out)


@pytest.mark.parametrize("act", [0, 1])
def test_noalloc_matches_workspace_entry_point(wob, act):
    # tile path: a large call, then a smaller one with other experts and ids
    big = wl.moe_inputs(600, 16, 4, 544, 256, seed=31)
    small = wl.moe_inputs(40, 8, 2, 288, 192, seed=32)
    small["ids"][3, 1] = -1  # an out-of-range id: a zero row
    for d in (big, small):
        a, b = _both(wob, d, act)
        assert np.array_equal(a, b)
    # decode path (at most 8 tokens), after the tile path used the array
    d = wl.moe_inputs(5, 16, 4, 544, 256, seed=33)
    a, b = _both(wob, d, act)
    assert np.array_equal(a, b)


def test_noalloc_refuses_a_problem_beyond_its_scratch(wob):
    from weight_only_bit_amd import _lib
    torch = torch_mod()
    T, topk, E, N, K = 65536, 8, 32, 32, 64  # 524288 pairs: over 2 MiB of routing scratch
    assert wob.moe_workspace_size(T, topk, E, N, K) > 1 << 20
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")  # never read: refused first
    st = _lib.lib().mxfp4_moe_gemm_noalloc(_p(buf), _p(buf), _p(buf), _p(buf), _p(buf), T, topk,
                                           E, N, K, 0, None)
    assert st == _lib.INVALID_ARG
    assert "static scratch" in _lib.last_error()
