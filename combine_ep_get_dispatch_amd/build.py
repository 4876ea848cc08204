"""Build libep_mi355x.so (the HIP kernels + C ABI) in-tree with hipcc for gfx950.

    python -m combine_ep_get_dispatch_amd.build

Packed-fp32 instructions are switched off for the device code (the feature
``-packed-fp32-ops``); hipcc's host pass does not know that feature and warns,
which is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libep_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into ``libep_mi355x.so`` next to this file."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *sources(), "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if noise not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
