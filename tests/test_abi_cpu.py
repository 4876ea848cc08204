"""The C ABI without a GPU: the library loads, exports every function that
include/ep.h declares, sizes workspaces, and rejects bad arguments on the host
before anything is enqueued.

No call here reaches a kernel: each one must fail host validation.  When a
GPU is present the pointers are real (tiny) device buffers, so that even a
validation bug could not hand a kernel a bogus address; without one they are
aligned placeholders that are never dereferenced.
"""
import ctypes
import os
import re

import pytest
import torch

from combine_ep_get_dispatch_amd import binding as b
from combine_ep_get_dispatch_amd import build as build_mod

HEADER = os.path.join(build_mod.INCLUDE, "ep.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"ep_get_dispatch_layout", "ep_dispatch", "ep_combine"} <= set(names)
    lib = ctypes.CDLL(b.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding declares a signature for each of them
    assert set(names) == set(b.SIGNATURES), set(names) ^ set(b.SIGNATURES)


def test_status_strings():
    for code, name in [(0, "EP_OK"), (1, "EP_ERR_INVALID_ARG"), (2, "EP_ERR_UNSUPPORTED"),
                       (3, "EP_ERR_WORKSPACE"), (4, "EP_ERR_HIP"), (99, "EP_ERR_UNKNOWN")]:
        assert b.status_string(code) == name


def test_workspace_bytes():
    L = b.lib()
    # header + cnt [nb][E] + pcnt [nb][P] + inv [nb] + pre [nb][E+1] + ppre [nb][P+1]
    # + prank [T*K] + rows [T*K], each rounded up to 256 bytes
    tb = 2048 // 8
    nb = -(-4096 // tb)
    r256 = lambda v: -(-v // 256) * 256
    want = 256 + r256(4 * 256 * nb) + r256(4 * 64 * nb) + r256(4 * nb) + r256(4 * 257 * nb) \
        + r256(4 * 65 * nb) + r256(4 * 4096 * 8) + r256(4 * 4096 * 8)
    assert L.ep_workspace_bytes(4096, 8, 256, 64) == want
    assert L.ep_workspace_bytes(0, 8, 256, 64) == 256
    for bad in [(-1, 2, 4, 2), (4, 0, 4, 2), (4, 2, 0, 1), (4, 2, 4, 0), (4, 2, 6, 4),
                (4, 5, 4, 2), (1 << 28, 8, 256, 64), (4, 2, 2048, 2), (4, 65, 128, 2)]:
        assert L.ep_workspace_bytes(*bad) == 0, bad


class Bufs:
    """Device buffers (GPU present) or never-dereferenced placeholders."""

    def __init__(self):
        self.keep = []
        self.gpu = torch.cuda.is_available()

    def __call__(self, nbytes=4096):
        if self.gpu:
            t = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device="cuda")
            self.keep.append(t)
            return ctypes.c_void_p(t.data_ptr())
        return ctypes.c_void_p(0x100000)


@pytest.fixture
def buf():
    return Bufs()


def test_layout_rejects_bad_arguments(buf):
    L = b.lib()
    ws = buf(1 << 16)
    p = [buf() for _ in range(6)]

    def call(idx=p[0], T=4, K=2, E=4, P=2, ce=p[1], cp=p[2], ip=p[3], oe=p[4], op=p[5],
             w=ws, wsz=1 << 16):
        return L.ep_get_dispatch_layout(idx, T, K, E, P, ce, cp, ip, oe, op, w, wsz, None)

    assert call(idx=None) == INVALID
    assert call(ce=None) == INVALID
    assert call(cp=None) == INVALID
    assert call(ip=None) == INVALID
    assert call(oe=None) == INVALID
    assert call(op=None) == INVALID
    assert call(w=None) == INVALID
    assert call(T=-1) == INVALID
    assert call(K=0) == INVALID
    assert call(E=0) == INVALID
    assert call(P=0) == INVALID
    assert call(E=6, P=4) == INVALID          # E % P != 0
    assert call(K=5) == INVALID               # K > E
    assert call(T=1 << 28, K=8, E=8) == INVALID   # T*K >= 2^31
    assert call(E=2048, P=2) == UNSUPPORTED
    assert call(K=65, E=128) == UNSUPPORTED
    assert call(wsz=255) == WORKSPACE
    assert call(T=4096, K=8, E=256, P=64, wsz=1 << 16) == WORKSPACE


def test_dispatch_rejects_bad_arguments(buf):
    L = b.lib()
    ws = buf(1 << 16)
    x, idx, rx, rs, src, dst = (buf() for _ in range(6))

    def call(x=x, T=4, H=256, idx=idx, K=2, E=4, P=2, dt=0, rx=rx, rs=rs, src=src, dst=dst,
             w=ws, wsz=1 << 16):
        return L.ep_dispatch(x, T, H, idx, K, E, P, dt, rx, rs, src, dst, w, wsz, None)

    for kw in [dict(x=None), dict(idx=None), dict(rx=None), dict(src=None), dict(dst=None),
               dict(w=None), dict(H=0), dict(H=12), dict(dt=2), dict(dt=1, H=136),
               dict(dt=1, rs=None), dict(E=6, P=4), dict(K=5), dict(T=-3),
               dict(x=ctypes.c_void_p(0x100008)), dict(rx=ctypes.c_void_p(0x100004))]:
        assert call(**kw) == INVALID, kw
    assert call(E=2048, P=2) == UNSUPPORTED
    assert call(wsz=128) == WORKSPACE


def test_layout_dispatch_rejects_bad_arguments(buf):
    L = b.lib()
    ws = buf(1 << 16)
    x, idx, ce, cp, ip, oe, op, rx, rs, src, dst = (buf() for _ in range(11))

    def call(x=x, T=4, H=256, idx=idx, K=2, E=4, P=2, dt=0, ce=ce, cp=cp, ip=ip, oe=oe, op=op,
             rx=rx, rs=rs, src=src, dst=dst, w=ws, wsz=1 << 16):
        return L.ep_layout_dispatch(x, T, H, idx, K, E, P, dt, ce, cp, ip, oe, op, rx, rs, src,
                                    dst, w, wsz, None)

    for kw in [dict(x=None), dict(idx=None), dict(ce=None), dict(cp=None), dict(ip=None),
               dict(oe=None), dict(op=None), dict(rx=None), dict(src=None), dict(dst=None),
               dict(w=None), dict(H=0), dict(H=12), dict(dt=2), dict(dt=1, H=136),
               dict(dt=1, rs=None), dict(E=6, P=4), dict(K=5), dict(T=-3),
               dict(x=ctypes.c_void_p(0x100008)), dict(rx=ctypes.c_void_p(0x100004))]:
        assert call(**kw) == INVALID, kw
    assert call(E=2048, P=2) == UNSUPPORTED
    assert call(wsz=128) == WORKSPACE


def test_layout_dispatch_static_rejects_bad_arguments(buf):
    """The no-allocation entry point checks its arguments like
    ep_layout_dispatch and refuses shapes whose workspace would not fit its
    static scratch -- all before touching the device."""
    L = b.lib()
    x, idx, ce, cp, ip, oe, op, rx, rs, src, dst = (buf() for _ in range(11))

    def call(x=x, T=4, H=256, idx=idx, K=2, E=4, P=2, dt=0, ce=ce, cp=cp, ip=ip, oe=oe, op=op,
             rx=rx, rs=rs, src=src, dst=dst):
        return L.ep_layout_dispatch_static(x, T, H, idx, K, E, P, dt, ce, cp, ip, oe, op, rx, rs,
                                           src, dst, None)

    for kw in [dict(x=None), dict(idx=None), dict(ce=None), dict(cp=None), dict(ip=None),
               dict(oe=None), dict(op=None), dict(rx=None), dict(src=None), dict(dst=None),
               dict(H=0), dict(H=12), dict(dt=2), dict(dt=1, H=136),
               dict(dt=1, rs=None), dict(E=6, P=4), dict(K=5), dict(T=-3),
               dict(x=ctypes.c_void_p(0x100008)), dict(rx=ctypes.c_void_p(0x100004))]:
        assert call(**kw) == INVALID, kw
    assert call(E=2048, P=2) == UNSUPPORTED
    # 8 MiB of scratch: T = 65536 tokens at top-8 of 256 experts fit, 2^18 do not
    assert L.ep_workspace_bytes(65536, 8, 256, 64) <= 8 << 20
    assert L.ep_workspace_bytes(1 << 18, 8, 256, 64) > 8 << 20
    assert call(T=1 << 18, K=8, E=256, P=64) == UNSUPPORTED


def test_dispatch_dedup_rejects_bad_arguments(buf):
    L = b.lib()
    ws = buf(1 << 16)
    args = {n: buf() for n in ["x", "idx", "ce", "cp", "ip", "oe", "op", "pto", "rx", "rs", "src",
                               "rti", "ssr", "dst"]}

    def call(T=4, H=256, K=2, E=4, P=2, dt=0, w=ws, wsz=1 << 16, **kw):
        a = dict(args)
        a.update(kw)
        return L.ep_dispatch_dedup(a["x"], T, H, a["idx"], K, E, P, dt, a["ce"], a["cp"], a["ip"],
                                   a["oe"], a["op"], a["pto"], a["rx"], a["rs"], a["src"],
                                   a["rti"], a["ssr"], a["dst"], w, wsz, None)

    for name in args:
        if name == "rs":
            continue
        assert call(**{name: None}) == INVALID, name
    for kw in [dict(w=None), dict(H=0), dict(H=12), dict(dt=2), dict(dt=1, H=136),
               dict(dt=1, rs=None), dict(E=6, P=4), dict(K=5), dict(T=-3),
               dict(x=ctypes.c_void_p(0x100008)), dict(rx=ctypes.c_void_p(0x100004))]:
        assert call(**kw) == INVALID, kw
    assert call(E=2048, P=2) == UNSUPPORTED
    assert call(wsz=128) == WORKSPACE


def test_aligned_rows():
    L = b.lib()
    assert L.ep_aligned_rows(4096, 8, 256, 128) == 4096 * 8 + 256 * 127
    assert L.ep_aligned_rows(4096, 8, 256, 1) == 4096 * 8
    assert L.ep_aligned_rows(0, 8, 256, 64) == 256 * 63
    for bad in [(4, 2, 4, 0), (4, 2, 4, 1025), (-1, 2, 4, 8), (4, 0, 4, 8), (4, 5, 4, 8),
                (2147482648, 1, 1024, 1024), (4, 2, 2048, 8)]:
        assert L.ep_aligned_rows(*bad) == 0, bad


def test_layout_dispatch_aligned_rejects_bad_arguments(buf):
    L = b.lib()
    ws = buf(1 << 16)
    args = {n: buf() for n in ["x", "idx", "ce", "cp", "ip", "oe", "op", "rx", "rs", "src", "dst"]}

    def call(T=4, H=256, K=2, E=4, P=2, A=8, dt=0, w=ws, wsz=1 << 16, **kw):
        a = dict(args)
        a.update(kw)
        return L.ep_layout_dispatch_aligned(a["x"], T, H, a["idx"], K, E, P, A, dt, a["ce"],
                                            a["cp"], a["ip"], a["oe"], a["op"], a["rx"], a["rs"],
                                            a["src"], a["dst"], w, wsz, None)

    for name in args:
        if name == "rs":
            continue
        assert call(**{name: None}) == INVALID, name
    for kw in [dict(w=None), dict(H=0), dict(H=12), dict(dt=2), dict(dt=1, H=136),
               dict(dt=1, rs=None), dict(E=6, P=4), dict(K=5), dict(T=-3), dict(A=0),
               dict(A=1025), dict(A=-4), dict(T=2147482648, K=1, E=1024, P=1, A=1024),
               dict(x=ctypes.c_void_p(0x100008)), dict(rx=ctypes.c_void_p(0x100004))]:
        assert call(**kw) == INVALID, kw
    assert call(T=0, A=0) == INVALID
    assert call(E=2048, P=2) == UNSUPPORTED
    assert call(wsz=128) == WORKSPACE


def test_cu_budget_entry_points_reject_negative_budgets(buf):
    L = b.lib()
    ws = buf(1 << 16)
    p = [buf() for _ in range(12)]
    assert L.ep_layout_dispatch_cu(p[0], 4, 256, p[1], 2, 4, 2, 0, p[2], p[3], p[4], p[5], p[6],
                                   p[7], None, p[8], p[9], ws, 1 << 16, -1, None) == INVALID
    assert L.ep_combine_cu(p[0], 8, p[1], p[2], 4, 2, 256, p[3], -1, None) == INVALID
    # the other checks are those of the calls without a budget
    assert L.ep_combine_cu(None, 8, p[1], p[2], 4, 2, 256, p[3], 4, None) == INVALID
    assert L.ep_layout_dispatch_cu(p[0], 4, 256, p[1], 2, 6, 4, 0, p[2], p[3], p[4], p[5], p[6],
                                   p[7], None, p[8], p[9], ws, 1 << 16, 4, None) == INVALID


def test_low_latency_dispatch_rejects_bad_arguments(buf):
    L = b.lib()
    x, idx, cnt, rx, rs, src, dst = (buf() for _ in range(7))

    def call(x=x, T=4, H=256, idx=idx, K=2, E=4, C=4, dt=0, cnt=cnt, rx=rx, rs=rs, src=src,
             dst=dst, inv=None):
        return L.ep_low_latency_dispatch(x, T, H, idx, K, E, C, dt, cnt, rx, rs, src, dst, inv,
                                         None)

    for kw in [dict(x=None), dict(idx=None), dict(cnt=None), dict(rx=None), dict(src=None),
               dict(dst=None), dict(H=0), dict(H=12), dict(dt=2), dict(dt=1, H=136),
               dict(dt=1, rs=None), dict(K=5), dict(K=0), dict(E=0), dict(T=-3), dict(C=0),
               dict(C=-1), dict(E=1024, C=1 << 21),
               dict(x=ctypes.c_void_p(0x100008)), dict(rx=ctypes.c_void_p(0x100004))]:
        assert call(**kw) == INVALID, kw
    # T = 0 needs no token buffers, but the counts and the row map still
    assert call(T=0, cnt=None) == INVALID and call(T=0, src=None) == INVALID
    assert call(E=2048) == UNSUPPORTED
    assert call(K=65, E=128) == UNSUPPORTED
    assert call(T=1025, K=8, E=16) == UNSUPPORTED     # T*K > EP_LL_MAX_SLOTS
    assert b.LL_MAX_SLOTS == 8192


def test_combine_rejects_bad_arguments(buf):
    L = b.lib()
    y, dst, w, out = (buf() for _ in range(4))

    def call(y=y, rows=8, dst=dst, w=w, T=4, K=2, H=256, out=out):
        return L.ep_combine(y, rows, dst, w, T, K, H, out, None)

    for kw in [dict(y=None), dict(rows=-1), dict(dst=None), dict(w=None), dict(out=None),
               dict(T=-1),
               dict(K=0), dict(H=0), dict(H=20), dict(T=1 << 28, K=8),
               dict(y=ctypes.c_void_p(0x100002)), dict(out=ctypes.c_void_p(0x10000c))]:
        assert call(**kw) == INVALID, kw
    assert call(K=65) == UNSUPPORTED


def test_diagnostics_reject_bad_arguments(buf):
    L = b.lib()
    a, o = buf(), buf()
    assert L.ep_convert_e4m3(None, o, 4, 0, None) == INVALID
    assert L.ep_convert_e4m3(a, o, -1, 0, None) == INVALID
    assert L.ep_convert_e4m3(a, o, 4, 2, None) == INVALID
    assert L.ep_convert_bf16(a, None, 4, None) == INVALID
    assert L.ep_copy(a, o, 17, None) == INVALID
    assert L.ep_copy(None, o, 16, None) == INVALID
    assert L.ep_copy(ctypes.c_void_p(0x100004), o, 16, None) == INVALID
    n = ctypes.c_int64(0)
    assert L.ep_get_device_error(None, 256, ctypes.byref(n), None) == INVALID
    assert L.ep_get_device_error(a, 16, ctypes.byref(n), None) == INVALID
    assert L.ep_get_device_error(a, 256, None, None) == INVALID


def test_binding_rejects_cpu_tensors():
    idx = torch.zeros((4, 2), dtype=torch.int64)
    with pytest.raises(ValueError):
        b.get_dispatch_layout(idx, 4, 2)
    with pytest.raises((ValueError, TypeError)):
        b.combine(torch.zeros((8, 16), dtype=torch.bfloat16),
                  torch.zeros((4, 2), dtype=torch.int32), torch.zeros((4, 2)))


class _NoLaunch:
    """Stands in for the library: any call into it fails the test."""
    def __getattr__(self, name):
        raise AssertionError("the binding called %s before rejecting its arguments" % name)


@pytest.mark.parametrize("field,bad", [
    ("num_tokens_per_expert", lambda E, P, T: torch.zeros(E - 1, dtype=torch.int32)),
    ("num_tokens_per_partition", lambda E, P, T: torch.zeros(P, dtype=torch.int64)),
    ("is_token_in_partition", lambda E, P, T: torch.zeros((T + 1, P), dtype=torch.uint8)),
    ("expert_offsets", lambda E, P, T: torch.zeros(E, dtype=torch.int32)),
    ("partition_offsets", lambda E, P, T: torch.zeros(2 * (P + 1), dtype=torch.int32)[::2]),
])
def test_get_dispatch_layout_checks_a_caller_layout(monkeypatch, field, bad):
    """A Layout passed in as ``out`` (for instance one built for another T or
    P) is checked before anything is launched: the C ABI cannot see buffer
    sizes, so a wrong one would let the layout kernels write past it."""
    monkeypatch.setattr(b, "_is_gpu", lambda t: True)     # CPU tensors stand in for GPU ones
    monkeypatch.setattr(b, "lib", lambda: _NoLaunch())
    T, K, E, P = 6, 2, 8, 4
    idx = torch.zeros((T, K), dtype=torch.int64)
    ws = torch.zeros(4096, dtype=torch.uint8)
    lay = b.Layout(torch.zeros(E, dtype=torch.int32), torch.zeros(P, dtype=torch.int32),
                   torch.zeros((T, P), dtype=torch.uint8), torch.zeros(E + 1, dtype=torch.int32),
                   torch.zeros(P + 1, dtype=torch.int32), ws)
    setattr(lay, field, bad(E, P, T))
    with pytest.raises((ValueError, TypeError)):
        b.get_dispatch_layout(idx, E, P, workspace=ws, out=lay)


def test_binding_rejects_tensors_on_another_device(monkeypatch):
    """Every tensor of a call must be on the device of its first input."""
    monkeypatch.setattr(b, "_is_gpu", lambda t: True)
    monkeypatch.setattr(b, "lib", lambda: _NoLaunch())
    x = torch.zeros((4, 16), dtype=torch.bfloat16)
    idx = torch.zeros((4, 2), dtype=torch.int64, device="meta")
    with pytest.raises(ValueError, match="must be on"):
        b.dispatch(x, idx, 4, 2, torch.zeros(4096, dtype=torch.uint8))
