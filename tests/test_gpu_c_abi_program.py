"""The C ABI used from C++ alone (GPU): tests/c_abi_check.cpp allocates with
hipMalloc, calls ep_get_dispatch_layout -> ep_dispatch and, separately,
ep_layout_dispatch (bf16 and FP8 each), then ep_combine and
ep_get_device_error, and checks the results (expert counts against a count on
the host, the one invalid id reported, offsets, distinct in-run rows in token
order, recv_src_token inverting dst_row, bf16 rows as token copies, FP8 group
maxima at 448 with scale max|x|/448, combine of identity experts returning x)
and that bad arguments are refused.  It runs as a child process."""
import os
import subprocess

import pytest

from parity import announce

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")


def test_c_abi_program():
    assert os.path.exists(EXE), "tests/c_abi_check is not built: run __graft_entry__.build()"
    announce("c_abi_check program")
    proc = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert proc.returncode == 0, proc.stdout + proc.stderr
    assert "c_abi_check ok" in proc.stdout
