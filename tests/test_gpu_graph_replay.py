"""HIP-graph replays of every hot path equal its eager result, bit for bit.

The timed measurements capture each call in a HIP graph, over several copies
of the operands, and replay it back to back.  This checks that mode at full
size: the calls of one graph cycle over three copies of the same operands
(each call writing its own output), the graph is replayed three times with
eager work and synchronizations between the replays, the outputs are
refilled with NaN before each replay, and every output of every replay must
equal the eager call's output bit for bit (the kernels are deterministic).
The K spans of the 2880-wide shapes are odd in number (23), so the tile
kernels' tail span runs in every call.
"""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import dev, dev_act, require_gpu, torch_mod

pytestmark = pytest.mark.gpu

COPIES = 3
CALLS = 6
REPLAYS = 3


@pytest.fixture(scope="module")
def wob():
    require_gpu()
    import weight_only_bit_amd as w
    w.device_check()
    return w


def _operands(wob, key):
    """(list of per-copy argument dicts, call(copy, out), output shape, dtype)."""
    torch = torch_mod()
    w = wl.BY_KEY[key]
    d = w.make()
    if w.kind == "w4a16":
        M, N, g = d["M"], d["N"], d["g"]
        ops = [dict(x=dev_act(d["x"], d["dtype"]), q=dev(d["qweight"]),
                    s=dev_act(d["scales"], d["dtype"]), z=dev(d["qzeros"])) for _ in range(COPIES)]
        dt = torch.float16 if d["dtype"] == wl.F16 else torch.bfloat16

        def call(o, out):
            wob.gemm(o["x"], o["q"], o["s"], o["z"], g, out=out)
        return ops, call, (M, N), dt
    if w.kind == "grouped":
        N, g = d["N"], d["g"]
        total = int(d["m_offsets"][-1])
        ops = [dict(x=dev_act(d["x"], d["dtype"]), off=dev(d["m_offsets"]), q=dev(d["qweight"]),
                    s=dev_act(d["scales"], d["dtype"]), z=dev(d["qzeros"])) for _ in range(COPIES)]

        def call(o, out):
            wob.gemm_grouped(o["x"], o["off"], o["q"], o["s"], o["z"], g, out=out)
        return ops, call, (total, N), torch.bfloat16
    if w.kind == "moe2":
        T, E, topk, H, I = d["T"], d["E"], d["topk"], d["H"], d["I"]
        need = max(wob.moe_stage2_workspace_size(T, topk, E, H, I), 16)
        ops = [dict(a=dev(d["a"].view(np.int16)).view(torch.bfloat16), ids=dev(d["ids"]),
                    w=dev(d["w"]), w2=dev(d["w2_fp4"]), s2=dev(d["w2_scale"]),
                    ws=torch.empty(need, dtype=torch.uint8, device="cuda")) for _ in range(COPIES)]

        def call(o, out):
            wob.mxfp4_moe_stage2(o["a"], o["ids"], o["w"], o["w2"], o["s2"], out=out,
                                 workspace=o["ws"])
        return ops, call, (T, H), torch.bfloat16
    T, E, topk, N, K = d["T"], d["E"], d["topk"], d["N"], d["K"]
    need = max(wob.moe_workspace_size(T, topk, E, N, K), 16)
    ops = [dict(x=dev(d["x"].view(np.int16)).view(torch.bfloat16), ids=dev(d["ids"]),
                wf=dev(d["w_fp4"]), ws_=dev(d["w_scale"]),
                ws=torch.empty(need, dtype=torch.uint8, device="cuda")) for _ in range(COPIES)]
    return ops, (lambda o, out, act=0: wob.mxfp4_moe_gemm(o["x"], o["ids"], o["wf"], o["ws_"],
                                                           out=out, workspace=o["ws"], act=act)), \
        (T, topk, N), torch.bfloat16


@pytest.mark.parametrize("key,act", [("decode_gemv", 0), ("decode_down", 0), ("small_batch", 0),
                                     ("prefill", 0), ("grouped_moe_like", 0), ("moe_stage1", 0),
                                     ("moe_stage1", 1), ("moe_decode", 0), ("moe_stage2", 0)])
def test_graph_replays_match_eager(wob, key, act):
    torch = torch_mod()
    ops, call, shape, dt = _operands(wob, key)
    if act:
        shape = shape[:-1] + (shape[-1] // 2,)
        base = call
        call = lambda o, out: base(o, out, act=wob.ACT_SILU_MUL)  # noqa: E731
    ref = torch.empty(shape, dtype=dt, device="cuda")
    call(ops[0], ref)
    torch.cuda.synchronize()
    outs = [torch.empty(shape, dtype=dt, device="cuda") for _ in range(CALLS)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(CALLS):
            call(ops[i % COPIES], outs[i])
    ref_bits = ref.view(torch.int16)
    for r in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))
        scratch = torch.empty(shape, dtype=dt, device="cuda")
        call(ops[r % COPIES], scratch)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(scratch.view(torch.int16), ref_bits), f"eager call before replay {r}"
        for i, o in enumerate(outs):
            assert torch.equal(o.view(torch.int16), ref_bits), f"replay {r}, call {i} (copy {i % COPIES})"
