"""Host-side facts the kernels rely on, and the benchmark's command-line
contract (CPU only)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_partition_by_multiply_high_is_exact():
    """The layout kernels compute an expert's partition e // Ep as
    (e * ceil(2^32 / Ep)) >> 32; check it for every expert id and every
    experts-per-partition count the library allows (E <= 1024)."""
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


def test_bench_byte_model_matches_the_published_table():
    """bench.py's algorithmic bytes per step (what `value` divides by the step
    time) reproduce the byte model's table of the five workloads: layout,
    dispatch and combine bytes as printed there, each within one unit of its
    last printed digit."""
    sys.path.insert(0, ROOT)
    import bench
    from combine_ep_get_dispatch_amd import workloads as wl
    # config -> (layout, dispatch, combine) bytes and the rounding step of each figure
    table = {
        "tiny": ((1.4e3, 100.4e3, 99.3e3), (0.1e3, 0.1e3, 0.1e3)),
        "decode": ((14e3, 9.42e6, 16.52e6), (1e3, 0.01e6, 0.01e6)),
        "prefill": ((0.53e6, 301.47e6, 528.74e6), (0.01e6, 0.01e6, 0.01e6)),
        "skewed": ((1.05e6, 1058.0e6, 1057.5e6), (0.01e6, 0.1e6, 0.1e6)),
        "coarse": ((0.79e6, 806.4e6, 805.8e6), (0.01e6, 0.1e6, 0.1e6)),
    }
    for name, (want, step) in table.items():
        c = wl.CONFIGS[name]
        got = bench.algorithmic_bytes(c["T"], c["H"], c["E"], c["P"], c["K"], c["fp8"])
        for part, w, s in zip(("layout", "dispatch", "combine"), want, step):
            assert abs(got[part] - w) < s, (name, part, got[part], w)
        assert got["total"] == got["layout"] + got["dispatch"] + got["combine"]
    assert bench.algorithmic_bytes(4096, 7168, 256, 64, 8, True)["total"] == 830_736_904


def test_cpu_baseline_runs_the_path_being_timed():
    """bench.py's CPU baseline times the oracle of the same path as the GPU
    step: offsets, de-duplicated, aligned or fixed capacity."""
    sys.path.insert(0, ROOT)
    import bench
    from combine_ep_get_dispatch_amd import workloads as wl
    case = wl.make("tiny")
    for kw, words in [({}, "layout+dispatch+combine"), ({"dedup": True}, "de-duplicated"),
                      ({"align": 8}, "aligned (8 rows)"), ({"capacity": 16}, "fixed-capacity (C=16)")]:
        r = bench.cpu_baseline(case, 1000, 0.0, **kw)
        assert r["kind"] == "oracle" and r["cores"] == 1 and r["value"] > 0
        assert words in r["sample"], (kw, r["sample"])


def test_bench_refuses_paths_it_cannot_time_together():
    """One path per run, and the CU budget only on the one-call path: other
    combinations exit with a message before touching a device."""
    for args in (["--two-calls", "--cu-budget", "8"], ["--dedup", "--align", "8"],
                 ["--low-latency", "--two-calls"], ["--align", "64", "--cu-budget", "4"]):
        proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                              capture_output=True, text=True, timeout=120)
        assert proc.returncode == 2, (args, proc.returncode, proc.stderr)
        assert "one path at a time" in proc.stderr
        assert proc.stdout == ""
