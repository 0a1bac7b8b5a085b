#!/usr/bin/env python3
"""Benchmark of the weight-only 4-bit GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_gemv]

Prints ONE JSON line.  A step is one call of the library on one batch of
synthetic operands of the named workload (default: the decode GEMV
1x43008x5376, g=32, fp16 -- the gate_up decode shape of the zero-point page,
section Results).  Operands are rotated over enough device copies that the
bytes touched between two uses of a copy exceed the 256 MB Infinity Cache, so
the timing sees HBM, not cache.

Timed region: K steps captured in one HIP graph and replayed once, bracketed
by torch.cuda.synchronize(), with HIP events on the launch stream around the
replay; `value` = algorithmic bytes (or FLOPs) per step / step time.  In the
graph the kernels run back to back, so the step time is the kernel's average
launch duration and the roofline entry uses it.  The CPU baseline is the
oracle (single-threaded C) on the full decode call.

Beside each workload, `ceilings` gives references measured the same way in
the same run: for memory-bound calls a plain streaming read of the same byte
count (what a kernel that only reads achieves on this device) and, where the
bytes fit the Infinity Cache, the same call on one reused operand copy
(labelled MALL-resident; never the headline); for the
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
import os
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
FETCH_FACTOR_DEFAULT = 2.0     # FETCH_SIZE reads half of a device copy's bytes on this part

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


def _copies_for(bytes_per_call: int, max_copies: int = 256) -> int:
    n = 1
    while n * bytes_per_call < 2 * MALL_BYTES and n < max_copies:
        n *= 2
    return max(n, 2)


def _time_steps(step, steps: int, warmup: int):
    """Time exactly `steps` steps: captured into one HIP graph, replayed once
    between two synchronizations, with HIP events recorded on the launch
    stream around the replay.  Returns the average step time in ms (in the
    graph the kernels run back to back, so this is the kernel's average
    launch duration plus the command processor's gap between nodes, which
    is zero for kernels longer than a few microseconds)."""
    torch = _torch()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step(i)
    g.replay()  # untimed: first replay uploads the graph
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    del g
    return ms


def stream_read_ceiling(nbytes: int, steps: int, warmup: int):
    """The device's streaming-read reference for this byte count: the
    library's plain read kernel over the same number of bytes, rotated over
    copies like the operands (HBM, not cache), timed the same way."""
    import weight_only_bit_amd as wob
    torch = _torch()
    nb = (nbytes + 15) // 16 * 16
    copies = _copies_for(nb)
    pool = torch.empty(copies * nb, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.empty(1024, dtype=torch.uint8, device="cuda")
    views = [pool[i * nb:(i + 1) * nb] for i in range(copies)]

    def step(i):
        wob.stream_read(views[i % copies], nb, sink)

    ms = _time_steps(step, steps, warmup)
    del pool, views
    torch.cuda.empty_cache()
    return dict(what=f"plain streaming read of {nb:,} bytes", us=round(ms * 1e3, 3),
                gbs=round(nb / (ms * 1e-3) / 1e9, 1))


def library_gemm(M: int, N: int, K: int, act, steps: int, warmup: int, what: str):
    """The same product through the vendor library (torch.mm -> hipBLASLt /
    rocBLAS) with 16-bit weights: y[M][N] = x[M][K] w[N][K]^T, rotated over
    weight copies like the operands."""
    torch = _torch()
    wbytes = N * K * 2
    copies = _copies_for(wbytes, max_copies=64)
    ws = [torch.empty((N, K), dtype=act, device="cuda").normal_() for _ in range(copies)]
    x = torch.empty((M, K), dtype=act, device="cuda").normal_()
    y = torch.empty((M, N), dtype=act, device="cuda")

    def step(i):
        torch.mm(x, ws[i % copies].t(), out=y)

    ms = _time_steps(step, steps, warmup)
    del ws, x, y
    torch.cuda.empty_cache()
    nbytes = wbytes + 2 * M * K + 2 * M * N
    return dict(what=what, us=round(ms * 1e3, 3), gbs=round(nbytes / (ms * 1e-3) / 1e9, 1),
                tflops=round(2 * M * N * K / (ms * 1e-3) / 1e12, 2))


def _ceilings(entries):
    """Run each reference; a failure is reported in its entry, not raised."""
    out = {}
    for name, fn in entries:
        try:
            out[name] = fn()
        except Exception as e:  # noqa: BLE001 - reported in the JSON line
            out[name] = dict(error=f"{type(e).__name__}: {e}")
    return out


def bench_w4a16(wkey: str, steps: int, warmup: int):
    import weight_only_bit_amd as wob
    torch = _torch()
    w = wl.BY_KEY[wkey]
    d = w.make(seed=0)
    M, N, K, g = d["M"], d["N"], d["K"], d["g"]
    nbytes = wl.w4a16_bytes(M, N, K, g)
    flops = 2 * M * N * K
    copies = _copies_for(nbytes)
    bufs = [_to_dev(d) for _ in range(copies)]
    act = bufs[0]["x"].dtype
    ys = [torch.empty((M, N), dtype=act, device="cuda") for _ in range(copies)]

    def step(i):
        b = bufs[i % copies]
        wob.gemm(b["x"], b["qweight"], b["scales"], b["qzeros"], g, out=ys[i % copies])

    graph_ms = kern_ms = _time_steps(step, steps, warmup)
    skinny = M <= 8
    mall = None
    if skinny and nbytes < MALL_BYTES // 2:
        # the same call on one operand copy: after the first call its bytes sit
        # in the Infinity Cache (a labelled side figure, never the headline)
        def step_hot(i):
            b = bufs[0]
            wob.gemm(b["x"], b["qweight"], b["scales"], b["qzeros"], g, out=ys[0])

        hot_ms = _time_steps(step_hot, steps, warmup)
        mall = dict(what="MALL-resident: one operand copy reused (Infinity Cache hits)",
                    us=round(hot_ms * 1e3, 3), gbs=round(nbytes / (hot_ms * 1e-3) / 1e9, 1))
    res = dict(workload=w.desc, M=M, N=N, K=K, g=g, dtype=wl.DTYPE_NAMES[d["dtype"]],
               copies=copies, bytes_per_call=nbytes, flops_per_call=flops,
               us_per_call=round(graph_ms * 1e3, 3))
    if skinny:
        res["gbs"] = round(nbytes / (graph_ms * 1e-3) / 1e9, 1)
        achieved = nbytes / (kern_ms * 1e-3) / 1e9
        res["roofline"] = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                               unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                               traffic=committed_traffic(wkey, "skinny"))
    else:
        res["tflops"] = round(flops / (graph_ms * 1e-3) / 1e12, 2)
        achieved = flops / (kern_ms * 1e-3) / 1e12
        res["roofline"] = dict(bound="mfma", achieved=round(achieved, 2), peak=MFMA_PEAK_TFLOPS,
                               unit="TFLOP/s", frac=round(achieved / MFMA_PEAK_TFLOPS, 4),
                               traffic=committed_traffic(wkey, "tiled"))
    del bufs, ys
    torch.cuda.empty_cache()
    act_name = wl.DTYPE_NAMES[d["dtype"]]
    refs = [("library_16bit", lambda: library_gemm(
        M, N, K, act, steps, warmup,
        f"torch.mm {M}x{N}x{K} {act_name} with 16-bit weights ({N * K * 2:,} weight bytes)"))]
    if skinny:
        refs.insert(0, ("stream_read", lambda: stream_read_ceiling(nbytes, steps, warmup)))
    res["ceilings"] = _ceilings(refs)
    if mall is not None:
        res["ceilings"]["mall_resident"] = mall
    return res, d


def bench_grouped(wkey: str, steps: int, warmup: int):
    import weight_only_bit_amd as wob
    torch = _torch()
    w = wl.BY_KEY[wkey]
    d = w.make(seed=0)
    off = d["m_offsets"]
    total_m, E, N, K, g = int(off[-1]), len(off) - 1, d["N"], d["K"], d["g"]
    nbytes = wl.grouped_bytes(total_m, E, N, K, g)
    flops = 2 * total_m * N * K
    copies = _copies_for(nbytes, max_copies=4)
    act = torch.float16 if d["dtype"] == wl.F16 else torch.bfloat16

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    bufs = [dict(x=dev(d["x"].view(np.int16)).view(act), off=dev(off), q=dev(d["qweight"]),
                 s=dev(d["scales"].view(np.int16)).view(act), z=dev(d["qzeros"]))
            for _ in range(copies)]
    ys = [torch.empty((total_m, N), dtype=act, device="cuda") for _ in range(copies)]

    def step(i):
        b = bufs[i % copies]
        wob.gemm_grouped(b["x"], b["off"], b["q"], b["s"], b["z"], g, out=ys[i % copies])

    graph_ms = kern_ms = _time_steps(step, steps, warmup)
    res = dict(workload=w.desc, groups=E, total_M=total_m, N=N, K=K, g=g,
               dtype=wl.DTYPE_NAMES[d["dtype"]], copies=copies, bytes_per_call=nbytes,
               flops_per_call=flops, us_per_call=round(graph_ms * 1e3, 3),
               tflops=round(flops / (graph_ms * 1e-3) / 1e12, 2))
    achieved = flops / (kern_ms * 1e-3) / 1e12
    res["roofline"] = dict(bound="mfma", achieved=round(achieved, 2), peak=MFMA_PEAK_TFLOPS,
                           unit="TFLOP/s", frac=round(achieved / MFMA_PEAK_TFLOPS, 4),
                           traffic=committed_traffic(wkey, "tiled"))
    del bufs, ys
    torch.cuda.empty_cache()
    return res, d


def bench_moe(wkey: str, steps: int, warmup: int, act: int = 0):
    import weight_only_bit_amd as wob
    torch = _torch()
    w = wl.BY_KEY[wkey]
    d = w.make(seed=0)
    T, E, topk, N, K = d["T"], d["E"], d["topk"], d["N"], d["K"]
    if T <= 8:  # decode batch: only the experts the ids name are streamed
        nbytes = wl.moe_decode_bytes(d["ids"], E, N, K)
        copies = _copies_for(nbytes, max_copies=8)
    else:
        nbytes = wl.moe_bytes(T, E, topk, N, K)
        copies = _copies_for(nbytes, max_copies=4)
    flops = 2 * T * topk * N * K

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    bufs = []
    for _ in range(copies):
        bufs.append(dict(x=dev(d["x"].view(np.int16)).view(torch.bfloat16), ids=dev(d["ids"]),
                         w=dev(d["w_fp4"]), s=dev(d["w_scale"])))
    nout = N // 2 if act else N
    ys = [torch.empty((T, topk, nout), dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
    ws = torch.empty(max(wob.moe_workspace_size(T, topk, E), 16), dtype=torch.uint8, device="cuda")

    def step(i):
        b = bufs[i % copies]
        wob.mxfp4_moe_gemm(b["x"], b["ids"], b["w"], b["s"], out=ys[i % copies], workspace=ws,
                           act=act)

    graph_ms = kern_ms = _time_steps(step, steps, warmup)
    res = dict(workload=w.desc + (" + fused silu(gate)*up" if act else ""), T=T, E=E, topk=topk,
               N=N, K=K, dtype="bf16 x mxfp4",
               copies=copies, bytes_per_call=nbytes, flops_per_call=flops,
               us_per_call=round(graph_ms * 1e3, 3),
               tflops=round(flops / (graph_ms * 1e-3) / 1e12, 2))
    traffic = committed_traffic(wkey + ("_silu" if act else ""), "moe")
    if T <= 8:  # decode batch: memory-bound, bytes of the experts the ids name
        achieved = nbytes / (kern_ms * 1e-3) / 1e9
        res["gbs"] = round(achieved, 1)
        res["roofline"] = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                               unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                               traffic=traffic)
    else:
        achieved = flops / (kern_ms * 1e-3) / 1e12
        res["roofline"] = dict(bound="mfma", achieved=round(achieved, 2), peak=MFMA_PEAK_TFLOPS,
                               unit="TFLOP/s", frac=round(achieved / MFMA_PEAK_TFLOPS, 4),
                               traffic=traffic)
    del bufs, ys
    torch.cuda.empty_cache()
    if T <= 8:
        res["ceilings"] = _ceilings([("stream_read",
                                      lambda: stream_read_ceiling(nbytes, steps, warmup))])
    elif not act:
        P = T * topk
        res["ceilings"] = _ceilings([("library_dense_bf16", lambda: library_gemm(
            P, N, K, torch.bfloat16, steps, warmup,
            f"torch.mm {P}x{N}x{K} bf16: the same FLOPs as one dense GEMM (one weight "
            "matrix, no routing, no dequantization)"))])
    return res, d


def cpu_baseline_decode(d, budget_s: float = 10.0):
    """The oracle as it stands, single-threaded, on the full decode call."""
    import oracle
    M, N, K, g = d["M"], d["N"], d["K"], d["g"]
    nbytes = wl.w4a16_bytes(M, N, K, g)
    times = []
    t_start = time.perf_counter()
    while not times or (time.perf_counter() - t_start < budget_s and len(times) < 5):
        t0 = time.perf_counter()
        oracle.w4a16_gemm(d["x"], d["dtype"], d["qweight"], d["scales"], d["qzeros"], M, N, K, g)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return dict(value=round(nbytes / t / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                sample=f"full {M}x{N}x{K} g={g} call, median of {len(times)} runs "
                       f"({t:.2f} s each) on one host thread")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_gemv", choices=[w.key for w in wl.WORKLOADS])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, run three device-to-device copies of this many MiB "
                         "(untimed): the known-size reference for the profiler's byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(the weight-only GEMM path is single-GPU; see the sharding notes in DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

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

    head = wl.BY_KEY[args.workload]
    if head.kind == "w4a16":
        res, d = bench_w4a16(head.key, args.steps, args.warmup)
    else:
        res, d = bench_moe(head.key, args.steps, args.warmup)
    skinny = head.kind == "w4a16" and d["M"] <= 8
    line = dict(
        metric=METRIC,
        value=res["gbs"] if skinny else res["tflops"],
        unit="GB/s" if skinny else "TFLOP/s",
        n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(res["us_per_call"] / 1e3, 6),
        higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype=res["dtype"], data="synthetic",
        config=dict(workload=res["workload"], **{k: res[k] for k in ("M", "N", "K", "g", "T", "E",
                                                                     "topk") if k in res},
                    copies=res["copies"], bytes_per_call=res["bytes_per_call"],
                    flops_per_call=res["flops_per_call"]),
        us_per_call=res["us_per_call"],
        roofline=res["roofline"],
        ceilings=res.get("ceilings"),
    )
    if not args.no_cpu_baseline and head.key == "decode_gemv":
        line["cpu_baseline"] = cpu_baseline_decode(d)
    else:
        line["cpu_baseline"] = None
    if not args.no_others:
        others = {}
        for w in wl.WORKLOADS + wl.EXTRA_WORKLOADS:
            if w.key == head.key:
                continue
            try:
                fn = {"w4a16": bench_w4a16, "grouped": bench_grouped, "moe": bench_moe}[w.kind]
                r, _ = fn(w.key, args.steps, args.warmup)
                others[w.key] = r
            except Exception as e:  # report, do not hide: the entry says what failed
                others[w.key] = dict(workload=w.desc, error=f"{type(e).__name__}: {e}")
        try:
            others["moe_stage1_silu"], _ = bench_moe("moe_stage1", args.steps, args.warmup, act=1)
        except Exception as e:
            others["moe_stage1_silu"] = dict(workload="moe_stage1 + silu", error=f"{type(e).__name__}: {e}")
        line["others"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
