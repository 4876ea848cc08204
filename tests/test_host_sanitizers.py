"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two host-side parts are rebuilt with both sanitizers and exercised in a child
process that preloads the sanitizer runtime:
  * the CPU oracle (plain C, gcc): every path -- offsets, fixed capacity,
    de-duplicated, aligned, the scalar encoders -- over random inputs with
    masked, invalid and repeated ids, one token and no tokens;
  * the host side of the HIP library (argument validation, workspace sizing,
    status strings; hipcc, only the host pass instrumented): the C-ABI
    checks of test_abi_cpu.py, which launch nothing.
A report from either sanitizer ends the child with a non-zero status.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from combine_ep_get_dispatch_amd import build as hip_build  # noqa: E402

SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0",
    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
}

ORACLE_SCRIPT = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np
import oracle
from combine_ep_get_dispatch_amd import workloads as wl
oracle.use_library(sys.argv[2])
cases = [(300, 256, 16, 4, 3, dict()),
         (200, 512, 64, 8, 6, dict(fp8=True, masked_frac=0.1, invalid_frac=0.05)),
         (65, 128, 40, 5, 7, dict(allow_dup=True, fp8=True)),
         (1, 128, 4, 2, 2, dict()),
         (0, 128, 8, 4, 2, dict(fp8=True))]
for i, (T, H, E, P, K, kw) in enumerate(cases):
    c = wl.random_case(T, H, E, P, K, 900 + i, with_y=True, **kw)
    oracle.run(c.topk_idx, c.x_bits, E, P, c.fp8, c.y_bits, c.topk_weights)
    C = max(1, T // 4)
    oracle.run_ll(c.topk_idx, c.x_bits, E, C, c.fp8, wl.normal_bf16(5, (E * C, H)),
                  c.topk_weights)
    oracle.run_dedup(c.topk_idx, c.x_bits, E, P, c.fp8)
    R = oracle.aligned_rows(T, K, E, 8)
    oracle.run_aligned(c.topk_idx, c.x_bits, E, P, 8, c.fp8, wl.normal_bf16(6, (R, H)),
                       c.topk_weights)
v = np.random.default_rng(7).standard_normal(4096).astype(np.float32) * 300
oracle.bf16_rne(v)
oracle.e4m3(v)
print("oracle paths done")
"""

ABI_SCRIPT = r"""
import sys
sys.path.insert(0, sys.argv[1])
import pytest
from combine_ep_get_dispatch_amd import binding
binding.LIB_PATH = sys.argv[2]
sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider",
                      sys.argv[1] + "/tests/test_abi_cpu.py"]))
"""


def _runtime(compiler, name):
    out = subprocess.run([compiler, "-print-file-name=" + name], capture_output=True,
                         text=True).stdout.strip()
    if not out or not os.path.isabs(out) or not os.path.exists(out):
        pytest.skip("%s has no %s" % (compiler, name))
    return out


def _run_child(script, lib, preload):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    proc = subprocess.run([sys.executable, "-c", script, ROOT, lib], capture_output=True,
                          text=True, timeout=600, env=env, cwd=ROOT)
    assert proc.returncode == 0, (proc.stdout[-4000:], proc.stderr[-4000:])
    for marker in ("ERROR: AddressSanitizer", "runtime error:"):
        assert marker not in proc.stdout + proc.stderr, proc.stderr[-4000:]
    return proc


def test_oracle_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libep_oracle_san.so")
    cmd = ["gcc", "-O1", "-g", "-fPIC", "-shared", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           os.path.join(ROOT, "oracle", "ep_oracle.c"), "-o", lib, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    proc = _run_child(ORACLE_SCRIPT, lib, _runtime("gcc", "libasan.so"))
    assert "oracle paths done" in proc.stdout


def test_library_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(hip_build.HIPCC):
        pytest.skip("no hipcc")
    lib = str(tmp_path / "libep_san.so")
    flags = [f for f in hip_build.FLAGS if f not in ("-O3", "-Wall")]
    cmd = [hip_build.HIPCC, *flags, "-O1", "-g",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           *hip_build.sources(), "-o", lib]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    proc = _run_child(ABI_SCRIPT, lib, _runtime(hip_build.HIPCC, "libclang_rt.asan-x86_64.so"))
    assert " passed" in proc.stdout and "failed" not in proc.stdout, proc.stdout[-4000:]
