"""CPU oracle for MoE token dispatch and combine -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
does, and nothing here is shared with it.

The arithmetic lives in ``ep_oracle.c`` (plain single-threaded C, built with
``-ffp-contract=off``); this module only builds that file with gcc and
marshals numpy arrays into it.  Every function returns fresh numpy arrays.

The method (expert-parallel dispatch and combine, with FP8 dispatch) is the
one described in "DeepSeek releases DeepEP, an efficient communication library
for MoE models" (section "DeepEP: Optimizing MoE Communication") and in the
feature list of "DeepSeek Open Source Weekly Review - 2"; the readings taken
where those pages are silent are stated at the top of ``ep_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libep_oracle.so")

CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile ``ep_oracle.c`` into ``libep_oracle.so`` with gcc."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


def _bind(lib):
    lib.oracle_bf16_rne.argtypes = [ctypes.c_float]
    lib.oracle_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_e4m3.argtypes = [ctypes.c_float]
    lib.oracle_e4m3.restype = ctypes.c_uint8
    lib.oracle_bf16_rne_array.argtypes = [_f32p, _u16p, _i64]
    lib.oracle_e4m3_array.argtypes = [_f32p, _u8p, _i64]
    lib.oracle_layout.argtypes = [_i64p, _i32, _i32, _i32, _i32,
                                  _i32p, _i32p, _u8p, _i32p, _i32p]
    lib.oracle_layout.restype = ctypes.c_int64
    lib.oracle_permutation.argtypes = [_i64p, _i32, _i32, _i32, _i32p, _i32p, _i32p]
    lib.oracle_dispatch_bf16.argtypes = [_u16p, _i32, _i32, _i32p, _i32, _u16p]
    lib.oracle_quantize.argtypes = [_u16p, _i32, _i32, _u8p, _f32p]
    lib.oracle_dispatch_fp8.argtypes = [_u16p, _i32, _i32, _i32p, _i32, _u8p, _f32p]
    lib.oracle_combine.argtypes = [_u16p, _i32p, _f32p, _i32, _i32, _i32, _u16p]
    lib.oracle_ll_layout.argtypes = [_i64p, _i32, _i32, _i32, _i32, _i32p, _i32p, _i32p]
    lib.oracle_ll_layout.restype = _i64
    lib.oracle_dispatch_rows_bf16.argtypes = [_u16p, _i32, _i32, _i32p, _i64, _u16p]
    lib.oracle_dispatch_rows_fp8.argtypes = [_u16p, _i32, _i32, _i32p, _i64, _u8p, _f32p]
    lib.oracle_dedup_layout.argtypes = [_i64p, _i32, _i32, _i32, _i32, _i32p, _i32p, _i32p,
                                        _i32p, _i32p, _i32p, _i32p]
    lib.oracle_dedup_layout.restype = _i32
    lib.oracle_aligned_layout.argtypes = [_i64p, _i32, _i32, _i32, _i32, _i32, _i32p, _i32p,
                                          _u8p, _i32p, _i32p, _i32p, _i32p]
    lib.oracle_aligned_layout.restype = _i64
    return lib


_default_lib = None
_lib_override = None


def _load():
    """The oracle library in use: the override set by ``use_library`` if any,
    else ``libep_oracle.so`` (rebuilt first if it is missing or stale)."""
    global _default_lib
    if _lib_override is not None:
        return _lib_override
    if _default_lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build(force=True)
        _default_lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _default_lib


def use_library(path: str | None):
    """Route every call below to another build of ``ep_oracle.c`` (the tests
    use this to check that deliberately broken builds fail the pins); ``None``
    restores the default library."""
    global _lib_override
    _lib_override = None if path is None else _bind(ctypes.CDLL(path))


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ---------------------------------------------------------------------------
# scalar formats
# ---------------------------------------------------------------------------

def bf16_rne(v) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float32)).reshape(-1)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_bf16_rne_array(_ptr(a, ctypes.c_float), _ptr(out, ctypes.c_uint16), a.size)
    return out.reshape(np.shape(v))


def e4m3(v) -> np.ndarray:
    """fp32 -> OCP E4M3 codes (uint8), round to nearest even, saturating."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float32)).reshape(-1)
    out = np.empty(a.shape, dtype=np.uint8)
    _load().oracle_e4m3_array(_ptr(a, ctypes.c_float), _ptr(out, ctypes.c_uint8), a.size)
    return out.reshape(np.shape(v))


# ---------------------------------------------------------------------------
# the path
# ---------------------------------------------------------------------------

def layout(topk_idx: np.ndarray, E: int, P: int) -> dict:
    """Counts and offsets of the dispatch layout (see ``oracle_layout``)."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    cnt_e = np.empty(E, np.int32)
    cnt_p = np.empty(P, np.int32)
    in_part = np.empty((T, P), np.uint8)
    off_e = np.empty(E + 1, np.int32)
    off_p = np.empty(P + 1, np.int32)
    nerr = _load().oracle_layout(_ptr(idx, ctypes.c_int64), T, K, E, P,
                                 _ptr(cnt_e, ctypes.c_int32), _ptr(cnt_p, ctypes.c_int32),
                                 _ptr(in_part, ctypes.c_uint8), _ptr(off_e, ctypes.c_int32),
                                 _ptr(off_p, ctypes.c_int32))
    return dict(num_tokens_per_expert=cnt_e, num_tokens_per_partition=cnt_p,
                is_token_in_partition=in_part, expert_offsets=off_e,
                partition_offsets=off_p, num_invalid=int(nerr))


def permutation(topk_idx: np.ndarray, E: int, expert_offsets: np.ndarray):
    """(dst_row [T,K] int32, recv_src_token [T*K] int32)."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    off = np.ascontiguousarray(expert_offsets, dtype=np.int32)
    dst = np.empty((T, K), np.int32)
    src = np.empty(T * K, np.int32)
    _load().oracle_permutation(_ptr(idx, ctypes.c_int64), T, K, E,
                               _ptr(off, ctypes.c_int32), _ptr(dst, ctypes.c_int32),
                               _ptr(src, ctypes.c_int32))
    return dst, src


def dispatch_bf16(x_bits: np.ndarray, recv_src_token: np.ndarray, n_rows: int,
                  total_rows: int) -> np.ndarray:
    """bf16 receive buffer [total_rows, H] (uint16 bits); rows >= n_rows stay 0."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    src = np.ascontiguousarray(recv_src_token, dtype=np.int32)
    out = np.zeros((total_rows, H), np.uint16)
    _load().oracle_dispatch_bf16(_ptr(x, ctypes.c_uint16), T, H, _ptr(src, ctypes.c_int32),
                                 n_rows, _ptr(out, ctypes.c_uint16))
    return out


def quantize(x_bits: np.ndarray):
    """Per-token FP8 codes [T,H] uint8 and per-128-channel scales [T,H/128] fp32."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    assert H % 128 == 0
    q = np.empty((T, H), np.uint8)
    s = np.empty((T, H // 128), np.float32)
    _load().oracle_quantize(_ptr(x, ctypes.c_uint16), T, H, _ptr(q, ctypes.c_uint8),
                            _ptr(s, ctypes.c_float))
    return q, s


def dispatch_fp8(x_bits: np.ndarray, recv_src_token: np.ndarray, n_rows: int,
                 total_rows: int):
    """FP8 receive buffer [total_rows, H] uint8 and scales [total_rows, H/128]."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    assert H % 128 == 0
    src = np.ascontiguousarray(recv_src_token, dtype=np.int32)
    rx = np.zeros((total_rows, H), np.uint8)
    rs = np.zeros((total_rows, H // 128), np.float32)
    _load().oracle_dispatch_fp8(_ptr(x, ctypes.c_uint16), T, H, _ptr(src, ctypes.c_int32),
                                n_rows, _ptr(rx, ctypes.c_uint8), _ptr(rs, ctypes.c_float))
    return rx, rs


def combine(y_bits: np.ndarray, dst_row: np.ndarray, topk_weights: np.ndarray) -> np.ndarray:
    """Weighted top-k combine -> out [T,H] bf16 bits (uint16)."""
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    H = y.shape[1]
    dst = np.ascontiguousarray(dst_row, dtype=np.int32)
    w = np.ascontiguousarray(topk_weights, dtype=np.float32)
    T, K = dst.shape
    assert w.shape == (T, K)
    if T > 0 and K > 0 and dst.max(initial=-1) >= y.shape[0]:
        raise ValueError("dst_row points past the end of y")
    out = np.empty((T, H), np.uint16)
    _load().oracle_combine(_ptr(y, ctypes.c_uint16), _ptr(dst, ctypes.c_int32),
                           _ptr(w, ctypes.c_float), T, K, H, _ptr(out, ctypes.c_uint16))
    return out


def ll_layout(topk_idx: np.ndarray, E: int, C: int) -> dict:
    """Fixed-capacity layout (see ``oracle_ll_layout``): expert e owns rows
    [e*C, (e+1)*C)."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    cnt_e = np.empty(E, np.int32)
    dst = np.empty((T, K), np.int32)
    src = np.empty(E * C, np.int32)
    nerr = _load().oracle_ll_layout(_ptr(idx, ctypes.c_int64), T, K, E, C,
                                    _ptr(cnt_e, ctypes.c_int32), _ptr(dst, ctypes.c_int32),
                                    _ptr(src, ctypes.c_int32))
    return dict(num_tokens_per_expert=cnt_e, dst_row=dst, recv_src_token=src,
                num_invalid=int(nerr))


def dispatch_rows_bf16(x_bits: np.ndarray, recv_src_token: np.ndarray, fill: int = 0):
    """bf16 rows [R, H] for a source map with -1 holes; holes hold ``fill``."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    src = np.ascontiguousarray(recv_src_token, dtype=np.int32)
    out = np.full((src.size, H), fill, np.uint16)
    _load().oracle_dispatch_rows_bf16(_ptr(x, ctypes.c_uint16), T, H, _ptr(src, ctypes.c_int32),
                                      src.size, _ptr(out, ctypes.c_uint16))
    return out


def dispatch_rows_fp8(x_bits: np.ndarray, recv_src_token: np.ndarray, fill: int = 0):
    """FP8 rows [R, H] uint8 and scales [R, H/128] for a source map with -1
    holes; hole bytes hold ``fill`` and hole scales 0."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x.shape
    assert H % 128 == 0
    src = np.ascontiguousarray(recv_src_token, dtype=np.int32)
    rx = np.full((src.size, H), fill, np.uint8)
    rs = np.zeros((src.size, H // 128), np.float32)
    _load().oracle_dispatch_rows_fp8(_ptr(x, ctypes.c_uint16), T, H, _ptr(src, ctypes.c_int32),
                                     src.size, _ptr(rx, ctypes.c_uint8), _ptr(rs, ctypes.c_float))
    return rx, rs


def run_ll(topk_idx, x_bits, E, C, fp8, y_bits=None, topk_weights=None) -> dict:
    """The decode path: fixed-capacity layout, dispatch and (optionally)
    combine of expert outputs y [E*C, H] laid out like the receive rows."""
    res = ll_layout(topk_idx, E, C)
    src = res["recv_src_token"]
    if fp8:
        res["recv_x"], res["recv_scales"] = dispatch_rows_fp8(x_bits, src)
    else:
        res["recv_x"] = dispatch_rows_bf16(x_bits, src)
    if y_bits is not None:
        res["out"] = combine(y_bits, res["dst_row"], topk_weights)
    return res


def dedup_layout(topk_idx: np.ndarray, E: int, P: int) -> dict:
    """De-duplicated per-partition rows (see ``oracle_dedup_layout``), with
    the offsets layout and permutation it builds on."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    lay = layout(idx, E, P)
    dst, src = permutation(idx, E, lay["expert_offsets"])
    Kp = min(K, P)
    ptok_off = np.empty(P + 1, np.int32)
    dd_row = np.empty((T, P), np.int32)
    dd_src = np.empty(T * Kp, np.int32)
    dd_idx = np.empty((T * Kp, K), np.int32)
    slot_src = np.empty(T * K, np.int32)
    cnt_p = np.ascontiguousarray(lay["num_tokens_per_partition"], dtype=np.int32)
    n = _load().oracle_dedup_layout(_ptr(idx, ctypes.c_int64), T, K, E, P,
                                    _ptr(cnt_p, ctypes.c_int32), _ptr(dst, ctypes.c_int32),
                                    _ptr(ptok_off, ctypes.c_int32), _ptr(dd_row, ctypes.c_int32),
                                    _ptr(dd_src, ctypes.c_int32), _ptr(dd_idx, ctypes.c_int32),
                                    _ptr(slot_src, ctypes.c_int32))
    res = dict(lay)
    res.update(dst_row=dst, recv_src_token=src, partition_token_offsets=ptok_off,
               dedup_row=dd_row, dedup_src_token=dd_src, dedup_topk_idx=dd_idx,
               slot_src_row=slot_src, num_dedup_rows=int(n))
    return res


def aligned_rows(T: int, K: int, E: int, align: int) -> int:
    """Receive rows an aligned layout may use: T*K + E*(align-1)."""
    return T * K + E * (align - 1)


def aligned_layout(topk_idx: np.ndarray, E: int, P: int, align: int) -> dict:
    """Expert-major layout with every expert's run padded to a multiple of
    ``align`` rows (see ``oracle_aligned_layout``)."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    cnt_e = np.empty(E, np.int32)
    cnt_p = np.empty(P, np.int32)
    in_part = np.empty((T, P), np.uint8)
    off_e = np.empty(E + 1, np.int32)
    off_p = np.empty(P + 1, np.int32)
    dst = np.empty((T, K), np.int32)
    src = np.empty(aligned_rows(T, K, E, align), np.int32)
    nerr = _load().oracle_aligned_layout(
        _ptr(idx, ctypes.c_int64), T, K, E, P, align, _ptr(cnt_e, ctypes.c_int32),
        _ptr(cnt_p, ctypes.c_int32), _ptr(in_part, ctypes.c_uint8), _ptr(off_e, ctypes.c_int32),
        _ptr(off_p, ctypes.c_int32), _ptr(dst, ctypes.c_int32), _ptr(src, ctypes.c_int32))
    return dict(num_tokens_per_expert=cnt_e, num_tokens_per_partition=cnt_p,
                is_token_in_partition=in_part, expert_offsets=off_e, partition_offsets=off_p,
                dst_row=dst, recv_src_token=src, num_invalid=int(nerr))


def run_aligned(topk_idx, x_bits, E, P, align, fp8, y_bits=None, topk_weights=None) -> dict:
    """The aligned path: layout, dispatch into the padded rows and
    (optionally) combine of expert outputs laid out like the receive rows."""
    res = aligned_layout(topk_idx, E, P, align)
    src = res["recv_src_token"]
    if fp8:
        res["recv_x"], res["recv_scales"] = dispatch_rows_fp8(x_bits, src)
    else:
        res["recv_x"] = dispatch_rows_bf16(x_bits, src)
    if y_bits is not None:
        res["out"] = combine(y_bits, res["dst_row"], topk_weights)
    return res


def run_dedup(topk_idx, x_bits, E, P, fp8) -> dict:
    """The de-duplicated dispatch: layout, dedup rows and their data."""
    res = dedup_layout(topk_idx, E, P)
    src = res["dedup_src_token"]
    if fp8:
        res["dedup_x"], res["dedup_scales"] = dispatch_rows_fp8(x_bits, src)
    else:
        res["dedup_x"] = dispatch_rows_bf16(x_bits, src)
    return res


def run(topk_idx, x_bits, E, P, fp8, y_bits=None, topk_weights=None) -> dict:
    """The whole path: layout, permutation, dispatch and (optionally) combine."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    res = layout(idx, E, P)
    dst, src = permutation(idx, E, res["expert_offsets"])
    res["dst_row"] = dst
    res["recv_src_token"] = src
    n = int(res["expert_offsets"][E])
    if fp8:
        res["recv_x"], res["recv_scales"] = dispatch_fp8(x_bits, src, n, T * K)
    else:
        res["recv_x"] = dispatch_bf16(x_bits, src, n, T * K)
    if y_bits is not None:
        res["out"] = combine(y_bits, dst, topk_weights)
    return res
