"""bench.py's command-line contract on the host (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    """The measured path is single-GPU: --gpus N > 1 ends with status 2 and says
    why, before any device is touched."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_operand_rotation_keeps_its_reuse_distance():
    """The timed replays walk the operand copies in one continuous cycle: the
    untimed pass over every graph ends where the cycle starts again, and any
    sequence of replays in graph order never reuses a copy before all the
    others (so (copies - 1) calls' bytes, >= 2 x the Infinity Cache, separate
    two uses of one copy)."""
    sys.path.insert(0, ROOT)
    import bench
    for nbytes in (77_312, 2_211_840, 133_765_632, 134_889_472, 335_110_144):
        n = bench.copies_for(nbytes)
        if n < bench.MAX_COPIES:
            assert (n - 1) * nbytes >= bench.REUSE_BYTES
        for steps in (1, 7, 20, 50, 200):
            plan = bench.rotation_graphs(n, steps)
            warm = [c for seq in plan for c in seq]
            assert len(warm) % n == 0  # the untimed pass ends on a cycle boundary
            timed = [c for r in range(5) for c in plan[r % len(plan)]]
            seq = warm + timed
            assert seq == [i % n for i in range(len(seq))]
