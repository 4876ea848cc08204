"""Host-side facts the kernels rely on, and the benchmark's command-line
contract (CPU only)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_partition_by_multiply_high_is_exact():
    """The layout kernels compute an expert's partition e // Ep as
    (e * ceil(2^32 / Ep)) >> 32; check it for every expert id and every
    experts-per-partition count this build allows (E <= 1024)."""
    for ep in range(1, 1025):
        magic = -(-(1 << 32) // ep)
        for e in range(1024):
            assert (e * magic) >> 32 == e // ep, (e, ep)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 (or a multi-rank launch) must
    exit with a message before touching a device."""
    for args, env in [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "4"})]:
        proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                              capture_output=True, text=True, timeout=120,
                              env=dict(os.environ, **env))
        assert proc.returncode == 2, (args, proc.returncode, proc.stderr)
        assert "one GPU" in proc.stderr
        assert proc.stdout == ""
