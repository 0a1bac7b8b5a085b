"""The tile kernels' span-end waits cover every LDS copy (CPU: compiles to gfx950 assembly).

Each K-loop span of the tile pipeline issues its LDS copies
(`global_load_lds_dwordx4`, inline asm the compiler does not count), then the
next scale / zero-point loads, then waits with `s_waitcnt vmcnt(N)` before
the span barrier, N being the number of those scale loads.  Vector-memory
operations complete in issue order, so the wait covers every copy only if at
least N vector-memory operations follow the span's last copy.  A refill the
compiler finds dead (the last span of an odd span count) is deleted, and the
same N then left N copies in flight past the barrier, landing in LDS the
epilogue had already reused for staged outputs and row indices.

The check reads the assembly of the real kernels in text order: for every
`s_waitcnt vmcnt(N)` followed by `s_barrier`, the vector-memory operations
after the last preceding LDS copy must number at least N.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_only_bit_amd", "csrc")
HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)

VMEM = re.compile(r"(global_load|global_store|global_atomic|buffer_load|buffer_store|flat_load|flat_store)\w*\s")
WAIT = re.compile(r"s_waitcnt\s.*vmcnt\((\d+)\)")
KERNEL = re.compile(r"^(_ZN3wob\S*):\s*;")


def span_end_waits(asm):
    """[(kernel, line, N, vector-memory ops after the last LDS copy)] for each
    `s_waitcnt vmcnt(N)` that a `s_barrier` follows within five lines."""
    lines = asm.split("\n")
    out = []
    kernel, since = None, None
    for i, raw in enumerate(lines):
        m = KERNEL.match(raw)
        if m:
            kernel, since = m.group(1), None
            continue
        t = raw.strip()
        if t.startswith("global_load_lds"):
            since = 0
            continue
        if VMEM.match(t + " "):
            if since is not None:
                since += 1
            continue
        w = WAIT.match(t)
        if w and kernel and since is not None:
            if any(x.strip().startswith("s_barrier") for x in lines[i + 1:i + 6]):
                out.append((kernel, i + 1, int(w.group(1)), since))
    return out


def test_span_end_waits_parser():
    """The scan on a hand-written fragment: one covered wait, one short."""
    asm = "\n".join([
        "_ZN3wob1kEv: ; @k",
        "global_load_lds_dwordx4 v1, s[0:1]",
        "global_load_dword v2, v[4:5], off",
        "global_load_dword v3, v[4:5], off",
        "s_waitcnt vmcnt(2)",
        "s_barrier",
        "global_load_lds_dwordx4 v1, s[0:1]",
        "s_waitcnt vmcnt(2)",
        "s_barrier",
    ])
    assert span_end_waits(asm) == [("_ZN3wob1kEv", 5, 2, 2), ("_ZN3wob1kEv", 8, 2, 0)]


@pytest.mark.skipif(HIPCC is None, reason="hipcc not found")
def test_tile_kernels_wait_for_every_copy():
    flags = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "--cuda-device-only", "-S"]
    with tempfile.TemporaryDirectory() as td:
        procs = {}
        for src in ("tiled.hip", "moe.hip"):
            out = os.path.join(td, src + ".s")
            procs[src] = (out, subprocess.Popen([HIPCC] + flags + ["-o", out, os.path.join(CSRC, src)],
                                                stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
        checked = {}
        for src, (out, p) in procs.items():
            log = p.communicate(timeout=600)[0].decode(errors="replace")
            assert p.returncode == 0, log[-2000:]
            waits = span_end_waits(open(out).read())
            short = [w for w in waits if w[3] < w[2]]
            assert not short, "span-end waits short of their copies: %s" % short[:5]
            checked[src] = {w[0] for w in waits}
    # not vacuous: every tile kernel has span-end waits
    assert sum("w4a16_tiled_kernel" in k for k in checked["tiled.hip"]) >= 12
    assert any("moe_gemm_kernel" in k for k in checked["moe.hip"])
    assert any("moe_stage2_kernel" in k for k in checked["moe.hip"])
