#!/usr/bin/env python3
"""Benchmark of the weight-only 4-bit GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R] [--workload decode_gemv]

Prints ONE JSON line.  A step is one call of the library on one batch of
synthetic operands of the named workload (default: the decode GEMV
1x43008x5376, g=32, fp16 -- the gate_up decode shape of the zero-point page,
section Results).

Operand rotation.  Every call reads its own copy of the operands; n copies
rotate so that the bytes touched between two uses of one copy, (n - 1) times
the bytes of a call, are at least twice the 256 MB Infinity Cache: the timing
sees HBM, not cache.  The rotation continues across replays (below), so this
distance holds for every step, the first of a replay included.

Timed region.  W untimed eager warm-up steps; then the K steps of a replay
are captured in HIP graphs (graph j holds the K steps that start at copy
j*K mod n; n / gcd(n, K) graphs close the cycle) and every graph is replayed
once untimed (the first replay uploads it), then in whole cycles for 0.3 s
(untimed: the clocks ramp after an idle period, and the first replays ran up
to a quarter slower).  Then R replays (default 5) of K
steps each are timed one by one, each bracketed by torch.cuda.synchronize(),
with HIP events recorded on the stream the kernels run on.  The step time is
the median over the R replays of elapsed / K (the minimum is reported
beside it); `value` = algorithmic bytes (or FLOPs) per step / that time.  In
a graph the kernels run back to back, so for a one-kernel step the step time
is that kernel's average launch duration, which the roofline entry uses.

`cpu_baseline`: the oracle as it stands (single-threaded C) on a bounded
sample of each configuration, on this host; `host` names its CPU.

Beside each workload, `ceilings` gives references measured the same way in
the same run: for memory-bound calls a plain streaming read of the same byte
count and, where the bytes fit the Infinity Cache, the same call on one
reused operand copy (labelled MALL-resident; never the headline); for the
W4A16 shapes the same product through the vendor library with 16-bit
weights (torch.mm); for MoE stage 1 a dense bf16 GEMM of the same FLOPs.

Other workloads of the pages (tiny GEMV, small batch, prefill, MoE stage 1,
the zero-point page's qkv / down decode shapes and batch-4 g = 128 shapes, the
grouped GEMM on an MoE-like configuration) are measured the same way and
reported under "others".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as wl  # noqa: E402

METRIC = ("µs/call + achieved HBM GB/s (M≤8) / TFLOP/s (M≥16), % of roofline")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA, published
MALL_BYTES = 256 << 20         # Infinity Cache
REUSE_BYTES = 2 * MALL_BYTES   # bytes touched between two uses of one operand copy
MAX_COPIES = 512               # tiny calls: the cache cannot be defeated; labelled hot
SETTLE_S = 0.3                 # untimed replays before each timed series (clock ramp)
COVER_CYCLES = 400_000         # spin ahead of each timed replay (~0.2 ms) to cover its submission
_settle_s = SETTLE_S           # --settle-s
FETCH_FACTOR_DEFAULT = 2.0     # FETCH_SIZE reads half of a device copy's bytes on this part
TRAFFIC_SOURCE = ("committed rocprofv3 counters (profiles/traffic.json: FETCH_SIZE x fetch "
                  "factor + WRITE_SIZE per dispatch); null when the kernel sources changed "
                  "since they were taken")

# Sources of the kernel each workload's roofline entry describes: a committed
# counter summary counts only while these are unchanged.
KERNEL_SOURCES = {
    "skinny": ["weight_only_bit_amd/csrc/skinny.hip", "weight_only_bit_amd/csrc/wob_device.hpp"],
    "tiled": ["weight_only_bit_amd/csrc/tiled.hip", "weight_only_bit_amd/csrc/wob_tile.hpp",
              "weight_only_bit_amd/csrc/wob_device.hpp"],
    "moe": ["weight_only_bit_amd/csrc/moe.hip", "weight_only_bit_amd/csrc/wob_tile.hpp",
            "weight_only_bit_amd/csrc/wob_device.hpp"],
}


def source_sha(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(key: str, kind: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE in KiB per dispatch of the
    dominant kernel, and the FETCH_SIZE scale measured on a plain device copy),
    if the kernel sources are unchanged since the counters were taken; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(kind):
        return None
    factor = rec.get("fetch_factor", FETCH_FACTOR_DEFAULT)
    return int(round((rec["fetch_kib"] * factor + rec["write_kib"]) * 1024))


def _torch():
    import torch
    return torch


def _to_dev(d):
    torch = _torch()
    act = torch.float16 if d["dtype"] == wl.F16 else torch.bfloat16

    def a(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(act).cuda()

    return dict(x=a(d["x"]), qweight=torch.from_numpy(d["qweight"]).cuda(), scales=a(d["scales"]),
                qzeros=None if d["qzeros"] is None else torch.from_numpy(d["qzeros"]).cuda())


def copies_for(bytes_per_call: int, max_copies: int = MAX_COPIES) -> int:
    """Operand copies n with (n - 1) * bytes_per_call >= 2 x the Infinity Cache
    (capped at max_copies: a call that small is cache-resident whatever)."""
    n = -(-REUSE_BYTES // max(bytes_per_call, 1)) + 1
    return max(2, min(n, max_copies))


class Timing:
    """R timed graph replays of K steps each over a rotation of n copies."""

    def __init__(self, reps_ms, copies, graphs, steps):
        self.reps_ms = reps_ms
        self.copies = copies
        self.graphs = graphs
        self.steps = steps

    @property
    def ms(self):
        return statistics.median(self.reps_ms)

    @property
    def min_ms(self):
        return min(self.reps_ms)

    def summary(self):
        return dict(us_per_call=round(self.ms * 1e3, 3), us_per_call_min=round(self.min_ms * 1e3, 3),
                    reps_us=[round(r * 1e3, 3) for r in self.reps_ms], copies=self.copies,
                    graphs=self.graphs)


def rotation_graphs(copies: int, steps: int):
    """Copy index of every step of every graph: graph j holds rotation
    positions j*steps .. j*steps + steps - 1 (copy = position mod copies), and
    copies / gcd(copies, steps) graphs replayed in order close the cycle."""
    ngraphs = copies // math.gcd(copies, steps)
    return [[(j * steps + i) % copies for i in range(steps)] for j in range(ngraphs)]


def time_steps(step, steps: int, warmup: int, copies: int, reps: int) -> Timing:
    """Time R replays of exactly `steps` steps; step(c) runs one call on copy c.

    Graph j captures the steps at rotation positions j*steps .. j*steps +
    steps - 1 (copy = position mod copies); copies / gcd(copies, steps)
    graphs close the cycle, so replaying them in order keeps the rotation
    continuous.  Every graph is replayed once untimed (upload), which ends on
    a cycle boundary; the timed replays then start the cycle again."""
    torch = _torch()
    for i in range(warmup):
        step(i % copies)
    torch.cuda.synchronize()
    plan = rotation_graphs(copies, steps)
    ngraphs = len(plan)
    graphs = []
    for seq in plan:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in seq:
                step(c)
        graphs.append(g)
    for g in graphs:  # untimed: the first replay of a graph uploads it
        g.replay()
    torch.cuda.synchronize()
    # untimed: whole cycles until the clocks have settled (the first replays
    # after an idle period run up to a quarter slower while they ramp)
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < _settle_s:
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    reps_ms = []
    for r in range(reps):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        # A spin kernel ahead of the start event keeps the GPU busy while the
        # host submits the graph, so the timed span holds the K calls back to
        # back and not the submission latency (which a model's graph of many
        # layers amortizes over all of them, not over K calls).
        torch.cuda._sleep(COVER_CYCLES)
        start.record(stream)
        graphs[r % ngraphs].replay()
        end.record(stream)
        torch.cuda.synchronize()
        reps_ms.append(start.elapsed_time(end) / steps)
    del graphs
    return Timing(reps_ms, copies, ngraphs, steps)


def stream_read_ceiling(nbytes: int, steps: int, warmup: int, reps: int):
    """The device's streaming-read reference for this byte count: the
    library's plain read kernel over the same number of bytes, rotated over
    copies like the operands (HBM, not cache), timed the same way."""
    import weight_only_bit_amd as wob
    torch = _torch()
    nb = (nbytes + 15) // 16 * 16
    copies = copies_for(nb)
    pool = torch.empty(copies * nb, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.empty(1024, dtype=torch.uint8, device="cuda")
    views = [pool[i * nb:(i + 1) * nb] for i in range(copies)]

    def step(c):
        wob.stream_read(views[c], nb, sink)

    t = time_steps(step, steps, warmup, copies, reps)
    del pool, views
    torch.cuda.empty_cache()
    return dict(what=f"plain streaming read of {nb:,} bytes", us=round(t.ms * 1e3, 3),
                gbs=round(nb / (t.ms * 1e-3) / 1e9, 1), copies=copies)


def library_gemm(M: int, N: int, K: int, act, steps: int, warmup: int, reps: int, what: str):
    """The same product through the vendor library (torch.mm -> hipBLASLt /
    rocBLAS) with 16-bit weights: y[M][N] = x[M][K] w[N][K]^T, rotated over
    weight copies like the operands."""
    torch = _torch()
    wbytes = N * K * 2
    copies = copies_for(wbytes, max_copies=64)
    ws = [torch.empty((N, K), dtype=act, device="cuda").normal_() for _ in range(copies)]
    x = torch.empty((M, K), dtype=act, device="cuda").normal_()
    y = torch.empty((M, N), dtype=act, device="cuda")

    def step(c):
        torch.mm(x, ws[c].t(), out=y)

    t = time_steps(step, steps, warmup, copies, reps)
    del ws, x, y
    torch.cuda.empty_cache()
    nbytes = wbytes + 2 * M * K + 2 * M * N
    return dict(what=what, us=round(t.ms * 1e3, 3), gbs=round(nbytes / (t.ms * 1e-3) / 1e9, 1),
                tflops=round(2 * M * N * K / (t.ms * 1e-3) / 1e12, 2), copies=copies)


def _ceilings(entries):
    """Run each reference; a failure is reported in its entry, not raised."""
    out = {}
    for name, fn in entries:
        try:
            out[name] = fn()
        except Exception as e:  # noqa: BLE001 - reported in the JSON line
            out[name] = dict(error=f"{type(e).__name__}: {e}")
    return out


def _roofline_hbm(nbytes, t, traffic):
    achieved = nbytes / (t.ms * 1e-3) / 1e9
    return dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                traffic_source=TRAFFIC_SOURCE)


def _roofline_mfma(flops, t, traffic):
    achieved = flops / (t.ms * 1e-3) / 1e12
    return dict(bound="mfma", achieved=round(achieved, 2), peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                frac=round(achieved / MFMA_PEAK_TFLOPS, 4), traffic=traffic,
                traffic_source=TRAFFIC_SOURCE)


def bench_w4a16(wkey: str, steps: int, warmup: int, reps: int):
    import weight_only_bit_amd as wob
    torch = _torch()
    w = wl.BY_KEY[wkey]
    d = w.make(seed=0)
    M, N, K, g = d["M"], d["N"], d["K"], d["g"]
    nbytes = wl.w4a16_bytes(M, N, K, g)
    flops = 2 * M * N * K
    copies = copies_for(nbytes)
    bufs = [_to_dev(d) for _ in range(copies)]
    act = bufs[0]["x"].dtype
    ys = [torch.empty((M, N), dtype=act, device="cuda") for _ in range(copies)]

    def step(c):
        b = bufs[c]
        wob.gemm(b["x"], b["qweight"], b["scales"], b["qzeros"], g, out=ys[c])

    t = time_steps(step, steps, warmup, copies, reps)
    skinny = M <= 8
    mall = None
    if skinny and nbytes < MALL_BYTES // 2:
        # the same call on one operand copy: after the first call its bytes sit
        # in the Infinity Cache (a labelled side figure, never the headline)
        th = time_steps(step, steps, warmup, 1, reps)
        mall = dict(what="MALL-resident: one operand copy reused (Infinity Cache hits)",
                    us=round(th.ms * 1e3, 3), gbs=round(nbytes / (th.ms * 1e-3) / 1e9, 1))
    res = dict(workload=w.desc, M=M, N=N, K=K, g=g, dtype=wl.DTYPE_NAMES[d["dtype"]],
               bytes_per_call=nbytes, flops_per_call=flops, **t.summary())
    if nbytes * (copies - 1) < REUSE_BYTES:
        res["cache"] = "hot: the rotation cannot exceed the Infinity Cache at this call size"
    if skinny:
        res["gbs"] = round(nbytes / (t.ms * 1e-3) / 1e9, 1)
        res["roofline"] = _roofline_hbm(nbytes, t, committed_traffic(wkey, "skinny"))
    else:
        res["tflops"] = round(flops / (t.ms * 1e-3) / 1e12, 2)
        res["roofline"] = _roofline_mfma(flops, t, committed_traffic(wkey, "tiled"))
    del bufs, ys
    torch.cuda.empty_cache()
    act_name = wl.DTYPE_NAMES[d["dtype"]]
    refs = [("library_16bit", lambda: library_gemm(
        M, N, K, act, steps, warmup, reps,
        f"torch.mm {M}x{N}x{K} {act_name} with 16-bit weights ({N * K * 2:,} weight bytes)"))]
    if skinny:
        refs.insert(0, ("stream_read", lambda: stream_read_ceiling(nbytes, steps, warmup, reps)))
    res["ceilings"] = _ceilings(refs)
    if mall is not None:
        res["ceilings"]["mall_resident"] = mall
    return res, d


def bench_grouped(wkey: str, steps: int, warmup: int, reps: int):
    import weight_only_bit_amd as wob
    torch = _torch()
    w = wl.BY_KEY[wkey]
    d = w.make(seed=0)
    off = d["m_offsets"]
    total_m, E, N, K, g = int(off[-1]), len(off) - 1, d["N"], d["K"], d["g"]
    nbytes = wl.grouped_bytes(total_m, E, N, K, g)
    flops = 2 * total_m * N * K
    copies = copies_for(nbytes)
    act = torch.float16 if d["dtype"] == wl.F16 else torch.bfloat16

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    bufs = [dict(x=dev(d["x"].view(np.int16)).view(act), off=dev(off), q=dev(d["qweight"]),
                 s=dev(d["scales"].view(np.int16)).view(act), z=dev(d["qzeros"]))
            for _ in range(copies)]
    ys = [torch.empty((total_m, N), dtype=act, device="cuda") for _ in range(copies)]

    def step(c):
        b = bufs[c]
        wob.gemm_grouped(b["x"], b["off"], b["q"], b["s"], b["z"], g, out=ys[c])

    t = time_steps(step, steps, warmup, copies, reps)
    res = dict(workload=w.desc, groups=E, total_M=total_m, N=N, K=K, g=g,
               dtype=wl.DTYPE_NAMES[d["dtype"]], bytes_per_call=nbytes, flops_per_call=flops,
               **t.summary(), tflops=round(flops / (t.ms * 1e-3) / 1e12, 2))
    res["roofline"] = _roofline_mfma(flops, t, committed_traffic(wkey, "tiled"))
    del bufs, ys
    torch.cuda.empty_cache()
    return res, d


def bench_moe(wkey: str, steps: int, warmup: int, reps: int, act: int = 0):
    import weight_only_bit_amd as wob
    torch = _torch()
    w = wl.BY_KEY[wkey]
    d = w.make(seed=0)
    T, E, topk, N, K = d["T"], d["E"], d["topk"], d["N"], d["K"]
    if T <= 8:  # decode batch: only the experts the ids name are streamed
        nbytes = wl.moe_decode_bytes(d["ids"], E, N, K)
    else:
        nbytes = wl.moe_bytes(T, E, topk, N, K)
    copies = copies_for(nbytes)
    flops = 2 * T * topk * N * K

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    bufs = []
    for _ in range(copies):
        bufs.append(dict(x=dev(d["x"].view(np.int16)).view(torch.bfloat16), ids=dev(d["ids"]),
                         w=dev(d["w_fp4"]), s=dev(d["w_scale"])))
    nout = N // 2 if act else N
    ys = [torch.empty((T, topk, nout), dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
    ws = torch.empty(max(wob.moe_workspace_size(T, topk, E, N, K), 16), dtype=torch.uint8,
                     device="cuda")

    def step(c):
        b = bufs[c]
        wob.mxfp4_moe_gemm(b["x"], b["ids"], b["w"], b["s"], out=ys[c], workspace=ws, act=act)

    t = time_steps(step, steps, warmup, copies, reps)
    res = dict(workload=w.desc + (" + fused silu(gate)*up" if act else ""), T=T, E=E, topk=topk,
               N=N, K=K, dtype="bf16 x mxfp4", bytes_per_call=nbytes, flops_per_call=flops,
               **t.summary(), tflops=round(flops / (t.ms * 1e-3) / 1e12, 2))
    traffic = committed_traffic(wkey + ("_silu" if act else ""), "moe")
    if T <= 8:  # decode batch: memory-bound, bytes of the experts the ids name
        res["gbs"] = round(nbytes / (t.ms * 1e-3) / 1e9, 1)
        res["roofline"] = _roofline_hbm(nbytes, t, traffic)
    else:
        # a step is the routing kernel plus the GEMM: the rate is conservative
        # for the GEMM kernel alone
        res["roofline"] = _roofline_mfma(flops, t, traffic)
    del bufs, ys
    torch.cuda.empty_cache()
    if T <= 8:
        res["ceilings"] = _ceilings([("stream_read",
                                      lambda: stream_read_ceiling(nbytes, steps, warmup, reps))])
    elif not act:
        P = T * topk
        res["ceilings"] = _ceilings([("library_dense_bf16", lambda: library_gemm(
            P, N, K, torch.bfloat16, steps, warmup, reps,
            f"torch.mm {P}x{N}x{K} bf16: the same FLOPs as one dense GEMM (one weight "
            "matrix, no routing, no dequantization)"))])
    return res, d


def bench_moe2(wkey: str, steps: int, warmup: int, reps: int):
    import weight_only_bit_amd as wob
    torch = _torch()
    w = wl.BY_KEY[wkey]
    d = w.make(seed=0)
    T, E, topk, H, I = d["T"], d["E"], d["topk"], d["H"], d["I"]
    nbytes = wl.moe_stage2_bytes(T, E, topk, H, I)
    copies = copies_for(nbytes)
    flops = 2 * T * topk * H * I

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    bufs = [dict(a=dev(d["a"].view(np.int16)).view(torch.bfloat16), ids=dev(d["ids"]),
                 w=dev(d["w"]), w2=dev(d["w2_fp4"]), s2=dev(d["w2_scale"]))
            for _ in range(copies)]
    ys = [torch.empty((T, H), dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
    ws = torch.empty(max(wob.moe_stage2_workspace_size(T, topk, E, H, I), 16), dtype=torch.uint8,
                     device="cuda")

    def step(c):
        b = bufs[c]
        wob.mxfp4_moe_stage2(b["a"], b["ids"], b["w"], b["w2"], b["s2"], out=ys[c], workspace=ws)

    t = time_steps(step, steps, warmup, copies, reps)
    res = dict(workload=w.desc, T=T, E=E, topk=topk, H=H, I=I, dtype="bf16 x mxfp4",
               bytes_per_call=nbytes, flops_per_call=flops, **t.summary(),
               tflops=round(flops / (t.ms * 1e-3) / 1e12, 2))
    # a step is routing + GEMM + combine: conservative for the GEMM alone
    res["roofline"] = _roofline_mfma(flops, t, committed_traffic(wkey, "moe"))
    del bufs, ys
    torch.cuda.empty_cache()
    return res, d


# --- CPU baseline: the oracle as it stands, one host thread ----------------------

def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _host():
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return dict(cpu_model=_cpu_model(), nproc=os.cpu_count(), cpus_available=avail)


def _median_runs(fn, budget_s, max_runs=5):
    times = []
    t_start = time.perf_counter()
    while not times or (time.perf_counter() - t_start < budget_s and len(times) < max_runs):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return statistics.median(times), len(times)


def cpu_baseline(key: str, d, budget_s: float = 12.0):
    """The oracle (single-threaded C, fp64 accumulation) on this host: the
    whole call for the GEMV configurations (median of up to 5 runs), a slice
    of the weight rows with every activation row for prefill and MoE stage 1
    (one run), scaled to the workload's unit."""
    import oracle
    base = dict(cores=1, kind="oracle", host=_host())
    if key in ("tiny_gemv", "decode_gemv", "small_batch"):
        M, N, K, g = d["M"], d["N"], d["K"], d["g"]
        nbytes = wl.w4a16_bytes(M, N, K, g)
        t, n = _median_runs(lambda: oracle.w4a16_gemm(d["x"], d["dtype"], d["qweight"],
                                                      d["scales"], d["qzeros"], M, N, K, g),
                            budget_s)
        return dict(value=round(nbytes / t / 1e9, 4), unit="GB/s", seconds=round(t, 4),
                    sample=f"full {M}x{N}x{K} g={g} call, median of {n} runs", **base)
    if key == "prefill":
        M, N, K, g = d["M"], d["N"], d["K"], d["g"]
        ns = 64
        G = K // g
        t, _ = _median_runs(lambda: oracle.w4a16_gemm(d["x"], d["dtype"], d["qweight"][:ns],
                                                      d["scales"][:ns], d["qzeros"][:ns // 8],
                                                      M, ns, K, g), 0.0, 1)
        flops = 2 * M * ns * K
        return dict(value=round(flops / t / 1e9, 4), unit="GFLOP/s", seconds=round(t, 4),
                    sample=f"weight rows 0..{ns - 1} of {N} with all {M} activation rows "
                           f"(2*{M}*{ns}*{K} FLOP), one run; G={G}", **base)
    if key == "moe_stage1":
        T, E, topk, N, K = d["T"], d["E"], d["topk"], d["N"], d["K"]
        ns = 64
        w = np.ascontiguousarray(d["w_fp4"][:, :ns])
        s = np.ascontiguousarray(d["w_scale"][:, :ns])
        t, _ = _median_runs(lambda: oracle.mxfp4_moe_gemm(d["x"], d["ids"], w, s, T, topk, E, ns,
                                                          K), 0.0, 1)
        flops = 2 * T * topk * ns * K
        return dict(value=round(flops / t / 1e9, 4), unit="GFLOP/s", seconds=round(t, 4),
                    sample=f"weight rows 0..{ns - 1} of {N} of every expert with all "
                           f"{T}x{topk} routed rows (2*{T * topk}*{ns}*{K} FLOP), one run",
                    **base)
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="steps per timed replay (K)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=5, help="timed replays; the median is reported")
    ap.add_argument("--workload", default="decode_gemv", choices=[w.key for w in wl.WORKLOADS])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="seconds of untimed whole-cycle replays before each timed series")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, run three device-to-device copies of this many MiB "
                         "(untimed): the known-size reference for the profiler's byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported (each "
              "GEMM call runs on one GPU: a sharded layer would run it on each GPU's N- or "
              "K-slice of the weights)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.reps < 1 or args.warmup < 0:
        print("bench.py: --steps and --reps must be >= 1, --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    global _settle_s
    _settle_s = max(0.0, args.settle_s)
    torch = _torch()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import weight_only_bit_amd as wob
    wob.device_check()
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    run = {"w4a16": bench_w4a16, "grouped": bench_grouped, "moe": bench_moe, "moe2": bench_moe2}
    head = wl.BY_KEY[args.workload]
    res, d = run[head.kind](head.key, args.steps, args.warmup, args.reps)
    print(f"bench.py: {head.key} {res['us_per_call']} us", file=sys.stderr, flush=True)
    skinny = head.kind == "w4a16" and d["M"] <= 8
    line = dict(
        metric=METRIC,
        value=res["gbs"] if skinny else res["tflops"],
        unit="GB/s" if skinny else "TFLOP/s",
        n_gpus=1, steps=args.steps, warmup=args.warmup, reps=args.reps,
        ms_per_step=round(res["us_per_call"] / 1e3, 6),
        higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype=res["dtype"], data="synthetic",
        config=dict(workload=res["workload"], **{k: res[k] for k in ("M", "N", "K", "g", "T", "E",
                                                                     "topk") if k in res},
                    copies=res["copies"], bytes_per_call=res["bytes_per_call"],
                    flops_per_call=res["flops_per_call"]),
        us_per_call=res["us_per_call"],
        us_per_call_min=res["us_per_call_min"],
        reps_us=res["reps_us"],
        timing=(f"median of {args.reps} timed graph replays of {args.steps} steps each "
                f"(minimum beside it), operands rotated over {res['copies']} copies"),
        roofline=res["roofline"],
        ceilings=res.get("ceilings"),
    )
    line["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(head.key, d)
    if not args.no_others:
        others = {}
        for w in wl.WORKLOADS + wl.EXTRA_WORKLOADS:
            if w.key == head.key:
                continue
            try:
                r, dd = run[w.kind](w.key, args.steps, args.warmup, args.reps)
                if not args.no_cpu_baseline and w in wl.WORKLOADS:
                    r["cpu_baseline"] = cpu_baseline(w.key, dd)
                others[w.key] = r
                print(f"bench.py: {w.key} {r['us_per_call']} us", file=sys.stderr, flush=True)
            except Exception as e:  # report, do not hide: the entry says what failed
                others[w.key] = dict(workload=w.desc, error=f"{type(e).__name__}: {e}")
        try:
            others["moe_stage1_silu"], _ = bench_moe("moe_stage1", args.steps, args.warmup,
                                                     args.reps, act=1)
        except Exception as e:
            others["moe_stage1_silu"] = dict(workload="moe_stage1 + silu",
                                             error=f"{type(e).__name__}: {e}")
        line["others"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
