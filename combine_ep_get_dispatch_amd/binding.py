"""Thin ctypes binding of libep_mi355x.so (include/ep.h) for torch tensors.

Argument marshalling only: every step of dispatch and combine runs in the HIP
kernels behind the C ABI; torch provides device memory and the current
stream.  The functions allocate their outputs with ``torch.empty`` unless
``out``-style arguments are passed (the benchmark passes them so that nothing
is allocated in its timed loop).  If the library is not built the first call
raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep_mi355x.so")

EP_OK = 0
EP_DTYPE_BF16 = 0
EP_DTYPE_FP8_E4M3 = 1
MAX_EXPERTS = 1024
MAX_TOPK = 64
LL_MAX_SLOTS = 8192
MAX_EXPERT_ALIGNMENT = 1024


class EpError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s" % (what, status_string(status)))


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

SIGNATURES = {
    "ep_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "ep_get_dispatch_layout": (ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                              _vp, _vp, _sz, _vp]),
    "ep_dispatch": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _i32, _i32, ctypes.c_int, _vp,
                                   _vp, _vp, _vp, _vp, _sz, _vp]),
    "ep_combine": (ctypes.c_int, [_vp, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "ep_combine_cu": (ctypes.c_int, [_vp, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp]),
    "ep_layout_dispatch_cu": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _i32, _i32, ctypes.c_int,
                                             _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _sz, _i32, _vp]),
    "ep_layout_dispatch": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _i32, _i32, ctypes.c_int,
                                          _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                          _vp]),
    "ep_layout_dispatch_static": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _i32, _i32,
                                                 ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                 _vp, _vp, _vp]),
    "ep_aligned_rows": (_i64, [_i32, _i32, _i32, _i32]),
    "ep_layout_dispatch_aligned": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _i32, _i32, _i32,
                                                  ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                  _vp, _vp, _vp, _sz, _vp]),
    "ep_dispatch_dedup": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _i32, _i32, ctypes.c_int,
                                         _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _vp, _vp, _sz, _vp]),
    "ep_low_latency_dispatch": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _i32, _i32,
                                               ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "ep_get_device_error": (ctypes.c_int, [_vp, _sz, ctypes.POINTER(_i64), _vp]),
    "ep_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ep_convert_e4m3": (ctypes.c_int, [_vp, _vp, _i64, _i32, _vp]),
    "ep_convert_bf16": (ctypes.c_int, [_vp, _vp, _i64, _vp]),
    "ep_copy": (ctypes.c_int, [_vp, _vp, _sz, _vp]),
}


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libep_mi355x.so is not built: run `python -m combine_ep_get_dispatch_amd.build`"
                " (or __graft_entry__.build()) first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().ep_status_string(status).decode()


def _check(status: int, what: str):
    if status != EP_OK:
        raise EpError(status, what)


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor):
    """torch's current stream on t's device, as a hipStream_t."""
    if _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(t.device.index))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _is_gpu(t: torch.Tensor) -> bool:
    return t.device.type == "cuda"


def _need(t: torch.Tensor, dtype, name: str, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not _is_gpu(t):
        raise ValueError("%s must be a GPU tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


# ---------------------------------------------------------------------------
# layout
# ---------------------------------------------------------------------------

def workspace_bytes(num_tokens: int, num_topk: int, num_experts: int, num_partitions: int) -> int:
    n = lib().ep_workspace_bytes(num_tokens, num_topk, num_experts, num_partitions)
    if n == 0:
        raise ValueError("invalid shape T=%d K=%d E=%d P=%d" % (
            num_tokens, num_topk, num_experts, num_partitions))
    return int(n)


def new_workspace(num_tokens, num_topk, num_experts, num_partitions, device="cuda"):
    """A workspace for this shape.  It needs no initialisation (every layout
    call writes all that later calls read from it); it is zero-filled only so
    that its contents are defined before the first call."""
    return torch.zeros(workspace_bytes(num_tokens, num_topk, num_experts, num_partitions),
                       dtype=torch.uint8, device=device)


@dataclass
class Layout:
    num_tokens_per_expert: torch.Tensor     # [E] int32
    num_tokens_per_partition: torch.Tensor  # [P] int32
    is_token_in_partition: torch.Tensor     # [T, P] uint8
    expert_offsets: torch.Tensor            # [E+1] int32
    partition_offsets: torch.Tensor         # [P+1] int32
    workspace: torch.Tensor                 # uint8, consumed by dispatch


def get_dispatch_layout(topk_idx: torch.Tensor, num_experts: int, num_partitions: int,
                        workspace: torch.Tensor | None = None,
                        out: Layout | None = None) -> Layout:
    """ep_get_dispatch_layout on ``topk_idx`` [T, K] int64."""
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [T, K]")
    T, K = topk_idx.shape
    dev = topk_idx.device
    _need(topk_idx, torch.int64, "topk_idx", device=dev)
    E, P = int(num_experts), int(num_partitions)
    if workspace is None:
        workspace = new_workspace(T, K, E, P, dev)
    _need(workspace, torch.uint8, "workspace", device=dev)
    if out is None:
        out = Layout(torch.empty(E, dtype=torch.int32, device=dev),
                     torch.empty(P, dtype=torch.int32, device=dev),
                     torch.empty((T, P), dtype=torch.uint8, device=dev),
                     torch.empty(E + 1, dtype=torch.int32, device=dev),
                     torch.empty(P + 1, dtype=torch.int32, device=dev), workspace)
    else:
        out.workspace = workspace
    _need(out.num_tokens_per_expert, torch.int32, "num_tokens_per_expert", (E,), device=dev)
    _need(out.num_tokens_per_partition, torch.int32, "num_tokens_per_partition", (P,), device=dev)
    _need(out.is_token_in_partition, torch.uint8, "is_token_in_partition", (T, P), device=dev)
    _need(out.expert_offsets, torch.int32, "expert_offsets", (E + 1,), device=dev)
    _need(out.partition_offsets, torch.int32, "partition_offsets", (P + 1,), device=dev)
    _check(lib().ep_get_dispatch_layout(
        _ptr(topk_idx), T, K, E, P, _ptr(out.num_tokens_per_expert),
        _ptr(out.num_tokens_per_partition), _ptr(out.is_token_in_partition),
        _ptr(out.expert_offsets), _ptr(out.partition_offsets), _ptr(workspace),
        workspace.numel(), _stream(topk_idx)), "ep_get_dispatch_layout")
    return out


def get_device_error(workspace: torch.Tensor) -> int:
    """Invalid topk_idx entries met by the last layout call (synchronises)."""
    n = _i64(0)
    _check(lib().ep_get_device_error(_ptr(workspace), workspace.numel(), ctypes.byref(n),
                                     _stream(workspace)), "ep_get_device_error")
    return int(n.value)


# ---------------------------------------------------------------------------
# dispatch / combine
# ---------------------------------------------------------------------------

@dataclass
class Dispatched:
    recv_x: torch.Tensor                 # [T*K, H] bf16, or uint8 E4M3 codes
    recv_scales: torch.Tensor | None     # [T*K, H/128] float32 (FP8 only)
    recv_src_token: torch.Tensor         # [T*K] int32
    dst_row: torch.Tensor                # [T, K] int32


def dispatch(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int, num_partitions: int,
             workspace: torch.Tensor, fp8: bool = False,
             out: Dispatched | None = None) -> Dispatched:
    """ep_dispatch: x [T, H] bf16 -> receive rows grouped by expert."""
    if x.dim() != 2 or topk_idx.dim() != 2:
        raise ValueError("x must be [T, H] and topk_idx [T, K]")
    T, H = x.shape
    K = topk_idx.shape[1]
    dev = x.device
    _need(x, torch.bfloat16, "x", device=dev)
    _need(topk_idx, torch.int64, "topk_idx", (T, K), device=dev)
    _need(workspace, torch.uint8, "workspace", device=dev)
    R = T * K
    if out is None:
        out = Dispatched(
            torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev),
            torch.empty((R, H // 128), dtype=torch.float32, device=dev) if fp8 else None,
            torch.empty(R, dtype=torch.int32, device=dev),
            torch.empty((T, K), dtype=torch.int32, device=dev))
    _need(out.recv_x, torch.uint8 if fp8 else torch.bfloat16, "recv_x", (R, H), device=dev)
    if fp8:
        _need(out.recv_scales, torch.float32, "recv_scales", (R, H // 128), device=dev)
    _need(out.recv_src_token, torch.int32, "recv_src_token", (R,), device=dev)
    _need(out.dst_row, torch.int32, "dst_row", (T, K), device=dev)
    _check(lib().ep_dispatch(
        _ptr(x), T, H, _ptr(topk_idx), K, int(num_experts), int(num_partitions),
        EP_DTYPE_FP8_E4M3 if fp8 else EP_DTYPE_BF16, _ptr(out.recv_x),
        _ptr(out.recv_scales) if fp8 else None, _ptr(out.recv_src_token), _ptr(out.dst_row),
        _ptr(workspace), workspace.numel(), _stream(x)), "ep_dispatch")
    return out


def layout_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int,
                    num_partitions: int, workspace: torch.Tensor | None = None,
                    fp8: bool = False, out_layout: Layout | None = None,
                    out: Dispatched | None = None, num_cus: int = 0):
    """ep_layout_dispatch: the outputs of get_dispatch_layout + dispatch from
    one call (one kernel launch fewer).  num_cus > 0 confines the dispatch
    launch to that many CUs (ep_layout_dispatch_cu).  Returns (Layout,
    Dispatched)."""
    if x.dim() != 2 or topk_idx.dim() != 2:
        raise ValueError("x must be [T, H] and topk_idx [T, K]")
    T, H = x.shape
    K = topk_idx.shape[1]
    E, P = int(num_experts), int(num_partitions)
    dev = x.device
    _need(x, torch.bfloat16, "x", device=dev)
    _need(topk_idx, torch.int64, "topk_idx", (T, K), device=dev)
    if workspace is None:
        workspace = new_workspace(T, K, E, P, dev)
    _need(workspace, torch.uint8, "workspace", device=dev)
    if out_layout is None:
        out_layout = Layout(torch.empty(E, dtype=torch.int32, device=dev),
                            torch.empty(P, dtype=torch.int32, device=dev),
                            torch.empty((T, P), dtype=torch.uint8, device=dev),
                            torch.empty(E + 1, dtype=torch.int32, device=dev),
                            torch.empty(P + 1, dtype=torch.int32, device=dev), workspace)
    else:
        out_layout.workspace = workspace
    R = T * K
    if out is None:
        out = Dispatched(
            torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev),
            torch.empty((R, H // 128), dtype=torch.float32, device=dev) if fp8 else None,
            torch.empty(R, dtype=torch.int32, device=dev),
            torch.empty((T, K), dtype=torch.int32, device=dev))
    lo = out_layout
    _need(lo.num_tokens_per_expert, torch.int32, "num_tokens_per_expert", (E,), device=dev)
    _need(lo.num_tokens_per_partition, torch.int32, "num_tokens_per_partition", (P,), device=dev)
    _need(lo.is_token_in_partition, torch.uint8, "is_token_in_partition", (T, P), device=dev)
    _need(lo.expert_offsets, torch.int32, "expert_offsets", (E + 1,), device=dev)
    _need(lo.partition_offsets, torch.int32, "partition_offsets", (P + 1,), device=dev)
    _need(out.recv_x, torch.uint8 if fp8 else torch.bfloat16, "recv_x", (R, H), device=dev)
    if fp8:
        _need(out.recv_scales, torch.float32, "recv_scales", (R, H // 128), device=dev)
    _need(out.recv_src_token, torch.int32, "recv_src_token", (R,), device=dev)
    _need(out.dst_row, torch.int32, "dst_row", (T, K), device=dev)
    _check(lib().ep_layout_dispatch_cu(
        _ptr(x), T, H, _ptr(topk_idx), K, E, P, EP_DTYPE_FP8_E4M3 if fp8 else EP_DTYPE_BF16,
        _ptr(lo.num_tokens_per_expert), _ptr(lo.num_tokens_per_partition),
        _ptr(lo.is_token_in_partition), _ptr(lo.expert_offsets), _ptr(lo.partition_offsets),
        _ptr(out.recv_x), _ptr(out.recv_scales) if fp8 else None, _ptr(out.recv_src_token),
        _ptr(out.dst_row), _ptr(workspace), workspace.numel(), int(num_cus), _stream(x)),
        "ep_layout_dispatch_cu")
    return out_layout, out


def layout_dispatch_static(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int,
                           num_partitions: int, fp8: bool = False,
                           out_layout: Layout | None = None, out: Dispatched | None = None):
    """ep_layout_dispatch_static: the outputs of layout_dispatch, with the
    library's static per-GPU scratch as the workspace (the C call allocates
    nothing; outputs not given are allocated here).  The Layout's workspace
    is None: the invalid-id count is not reported.  Returns (Layout,
    Dispatched)."""
    if x.dim() != 2 or topk_idx.dim() != 2:
        raise ValueError("x must be [T, H] and topk_idx [T, K]")
    T, H = x.shape
    K = topk_idx.shape[1]
    E, P = int(num_experts), int(num_partitions)
    dev = x.device
    _need(x, torch.bfloat16, "x", device=dev)
    _need(topk_idx, torch.int64, "topk_idx", (T, K), device=dev)
    if out_layout is None:
        out_layout = Layout(torch.empty(E, dtype=torch.int32, device=dev),
                            torch.empty(P, dtype=torch.int32, device=dev),
                            torch.empty((T, P), dtype=torch.uint8, device=dev),
                            torch.empty(E + 1, dtype=torch.int32, device=dev),
                            torch.empty(P + 1, dtype=torch.int32, device=dev), None)
    R = T * K
    if out is None:
        out = Dispatched(
            torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev),
            torch.empty((R, H // 128), dtype=torch.float32, device=dev) if fp8 else None,
            torch.empty(R, dtype=torch.int32, device=dev),
            torch.empty((T, K), dtype=torch.int32, device=dev))
    lo = out_layout
    _need(lo.num_tokens_per_expert, torch.int32, "num_tokens_per_expert", (E,), device=dev)
    _need(lo.num_tokens_per_partition, torch.int32, "num_tokens_per_partition", (P,), device=dev)
    _need(lo.is_token_in_partition, torch.uint8, "is_token_in_partition", (T, P), device=dev)
    _need(lo.expert_offsets, torch.int32, "expert_offsets", (E + 1,), device=dev)
    _need(lo.partition_offsets, torch.int32, "partition_offsets", (P + 1,), device=dev)
    _need(out.recv_x, torch.uint8 if fp8 else torch.bfloat16, "recv_x", (R, H), device=dev)
    if fp8:
        _need(out.recv_scales, torch.float32, "recv_scales", (R, H // 128), device=dev)
    _need(out.recv_src_token, torch.int32, "recv_src_token", (R,), device=dev)
    _need(out.dst_row, torch.int32, "dst_row", (T, K), device=dev)
    _check(lib().ep_layout_dispatch_static(
        _ptr(x), T, H, _ptr(topk_idx), K, E, P, EP_DTYPE_FP8_E4M3 if fp8 else EP_DTYPE_BF16,
        _ptr(lo.num_tokens_per_expert), _ptr(lo.num_tokens_per_partition),
        _ptr(lo.is_token_in_partition), _ptr(lo.expert_offsets), _ptr(lo.partition_offsets),
        _ptr(out.recv_x), _ptr(out.recv_scales) if fp8 else None, _ptr(out.recv_src_token),
        _ptr(out.dst_row), _stream(x)), "ep_layout_dispatch_static")
    return out_layout, out


def aligned_rows(num_tokens: int, num_topk: int, num_experts: int, expert_alignment: int) -> int:
    """ep_aligned_rows: receive rows of layout_dispatch_aligned (0 if rejected)."""
    return int(lib().ep_aligned_rows(num_tokens, num_topk, num_experts, expert_alignment))


def layout_dispatch_aligned(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int,
                            num_partitions: int, expert_alignment: int,
                            workspace: torch.Tensor | None = None, fp8: bool = False,
                            out_layout: Layout | None = None, out: Dispatched | None = None):
    """ep_layout_dispatch_aligned: layout and dispatch with every expert's run
    of receive rows padded to a multiple of expert_alignment rows (recv_x,
    recv_scales and recv_src_token have aligned_rows(...) rows).  Returns
    (Layout, Dispatched)."""
    if x.dim() != 2 or topk_idx.dim() != 2:
        raise ValueError("x must be [T, H] and topk_idx [T, K]")
    T, H = x.shape
    K = topk_idx.shape[1]
    E, P, A = int(num_experts), int(num_partitions), int(expert_alignment)
    dev = x.device
    _need(x, torch.bfloat16, "x", device=dev)
    _need(topk_idx, torch.int64, "topk_idx", (T, K), device=dev)
    R = aligned_rows(T, K, E, A)
    if R == 0 and T > 0:
        raise ValueError("expert_alignment %d rejected for T=%d K=%d E=%d" % (A, T, K, E))
    if workspace is None:
        workspace = new_workspace(T, K, E, P, dev)
    _need(workspace, torch.uint8, "workspace", device=dev)
    if out_layout is None:
        out_layout = Layout(torch.empty(E, dtype=torch.int32, device=dev),
                            torch.empty(P, dtype=torch.int32, device=dev),
                            torch.empty((T, P), dtype=torch.uint8, device=dev),
                            torch.empty(E + 1, dtype=torch.int32, device=dev),
                            torch.empty(P + 1, dtype=torch.int32, device=dev), workspace)
    else:
        out_layout.workspace = workspace
    if out is None:
        out = Dispatched(
            torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev),
            torch.empty((R, H // 128), dtype=torch.float32, device=dev) if fp8 else None,
            torch.empty(R, dtype=torch.int32, device=dev),
            torch.empty((T, K), dtype=torch.int32, device=dev))
    lo = out_layout
    _need(lo.num_tokens_per_expert, torch.int32, "num_tokens_per_expert", (E,), device=dev)
    _need(lo.num_tokens_per_partition, torch.int32, "num_tokens_per_partition", (P,), device=dev)
    _need(lo.is_token_in_partition, torch.uint8, "is_token_in_partition", (T, P), device=dev)
    _need(lo.expert_offsets, torch.int32, "expert_offsets", (E + 1,), device=dev)
    _need(lo.partition_offsets, torch.int32, "partition_offsets", (P + 1,), device=dev)
    _need(out.recv_x, torch.uint8 if fp8 else torch.bfloat16, "recv_x", (R, H), device=dev)
    if fp8:
        _need(out.recv_scales, torch.float32, "recv_scales", (R, H // 128), device=dev)
    _need(out.recv_src_token, torch.int32, "recv_src_token", (R,), device=dev)
    _need(out.dst_row, torch.int32, "dst_row", (T, K), device=dev)
    _check(lib().ep_layout_dispatch_aligned(
        _ptr(x), T, H, _ptr(topk_idx), K, E, P, A, EP_DTYPE_FP8_E4M3 if fp8 else EP_DTYPE_BF16,
        _ptr(lo.num_tokens_per_expert), _ptr(lo.num_tokens_per_partition),
        _ptr(lo.is_token_in_partition), _ptr(lo.expert_offsets), _ptr(lo.partition_offsets),
        _ptr(out.recv_x), _ptr(out.recv_scales) if fp8 else None, _ptr(out.recv_src_token),
        _ptr(out.dst_row), _ptr(workspace), workspace.numel(), _stream(x)),
        "ep_layout_dispatch_aligned")
    return out_layout, out


@dataclass
class DedupDispatched:
    partition_token_offsets: torch.Tensor  # [P+1] int32
    recv_x: torch.Tensor                   # [T*Kp, H] bf16, or uint8 E4M3 codes
    recv_scales: torch.Tensor | None       # [T*Kp, H/128] float32 (FP8 only)
    recv_src_token: torch.Tensor           # [T*Kp] int32, -1 past the rows used
    recv_topk_idx: torch.Tensor            # [T*Kp, K] int32 local expert ids or -1
    slot_src_row: torch.Tensor             # [T*K] int32
    dst_row: torch.Tensor                  # [T, K] int32


def dispatch_dedup(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int,
                   num_partitions: int, workspace: torch.Tensor | None = None,
                   fp8: bool = False, out_layout: Layout | None = None,
                   out: DedupDispatched | None = None):
    """ep_dispatch_dedup: one copy of each token per partition it reaches.
    Returns (Layout, DedupDispatched)."""
    if x.dim() != 2 or topk_idx.dim() != 2:
        raise ValueError("x must be [T, H] and topk_idx [T, K]")
    T, H = x.shape
    K = topk_idx.shape[1]
    E, P = int(num_experts), int(num_partitions)
    Kp = min(K, P)
    RD = T * Kp
    dev = x.device
    _need(x, torch.bfloat16, "x", device=dev)
    _need(topk_idx, torch.int64, "topk_idx", (T, K), device=dev)
    if workspace is None:
        workspace = new_workspace(T, K, E, P, dev)
    _need(workspace, torch.uint8, "workspace", device=dev)
    if out_layout is None:
        out_layout = Layout(torch.empty(E, dtype=torch.int32, device=dev),
                            torch.empty(P, dtype=torch.int32, device=dev),
                            torch.empty((T, P), dtype=torch.uint8, device=dev),
                            torch.empty(E + 1, dtype=torch.int32, device=dev),
                            torch.empty(P + 1, dtype=torch.int32, device=dev), workspace)
    else:
        out_layout.workspace = workspace
    if out is None:
        out = DedupDispatched(
            torch.empty(P + 1, dtype=torch.int32, device=dev),
            torch.empty((RD, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev),
            torch.empty((RD, H // 128), dtype=torch.float32, device=dev) if fp8 else None,
            torch.empty(RD, dtype=torch.int32, device=dev),
            torch.empty((RD, K), dtype=torch.int32, device=dev),
            torch.empty(T * K, dtype=torch.int32, device=dev),
            torch.empty((T, K), dtype=torch.int32, device=dev))
    lo = out_layout
    _need(lo.num_tokens_per_expert, torch.int32, "num_tokens_per_expert", (E,), device=dev)
    _need(lo.num_tokens_per_partition, torch.int32, "num_tokens_per_partition", (P,), device=dev)
    _need(lo.is_token_in_partition, torch.uint8, "is_token_in_partition", (T, P), device=dev)
    _need(lo.expert_offsets, torch.int32, "expert_offsets", (E + 1,), device=dev)
    _need(lo.partition_offsets, torch.int32, "partition_offsets", (P + 1,), device=dev)
    _need(out.partition_token_offsets, torch.int32, "partition_token_offsets", (P + 1,), device=dev)
    _need(out.recv_x, torch.uint8 if fp8 else torch.bfloat16, "recv_x", (RD, H), device=dev)
    if fp8:
        _need(out.recv_scales, torch.float32, "recv_scales", (RD, H // 128), device=dev)
    _need(out.recv_src_token, torch.int32, "recv_src_token", (RD,), device=dev)
    _need(out.recv_topk_idx, torch.int32, "recv_topk_idx", (RD, K), device=dev)
    _need(out.slot_src_row, torch.int32, "slot_src_row", (T * K,), device=dev)
    _need(out.dst_row, torch.int32, "dst_row", (T, K), device=dev)
    _check(lib().ep_dispatch_dedup(
        _ptr(x), T, H, _ptr(topk_idx), K, E, P, EP_DTYPE_FP8_E4M3 if fp8 else EP_DTYPE_BF16,
        _ptr(lo.num_tokens_per_expert), _ptr(lo.num_tokens_per_partition),
        _ptr(lo.is_token_in_partition), _ptr(lo.expert_offsets), _ptr(lo.partition_offsets),
        _ptr(out.partition_token_offsets), _ptr(out.recv_x),
        _ptr(out.recv_scales) if fp8 else None, _ptr(out.recv_src_token),
        _ptr(out.recv_topk_idx), _ptr(out.slot_src_row), _ptr(out.dst_row), _ptr(workspace),
        workspace.numel(), _stream(x)), "ep_dispatch_dedup")
    return out_layout, out


@dataclass
class LowLatencyDispatched:
    num_tokens_per_expert: torch.Tensor  # [E] int32 (dropped slots included)
    recv_x: torch.Tensor                 # [E*C, H] bf16, or uint8 E4M3 codes
    recv_scales: torch.Tensor | None     # [E*C, H/128] float32 (FP8 only)
    recv_src_token: torch.Tensor         # [E*C] int32, -1 for unfilled rows
    dst_row: torch.Tensor                # [T, K] int32
    num_invalid: torch.Tensor            # [1] int64


def low_latency_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int,
                         capacity: int, fp8: bool = False,
                         out: LowLatencyDispatched | None = None) -> LowLatencyDispatched:
    """ep_low_latency_dispatch: x [T, H] bf16 -> fixed-capacity rows, expert
    e owning rows [e*C, (e+1)*C), in one launch."""
    if x.dim() != 2 or topk_idx.dim() != 2:
        raise ValueError("x must be [T, H] and topk_idx [T, K]")
    T, H = x.shape
    K = topk_idx.shape[1]
    E, C = int(num_experts), int(capacity)
    dev = x.device
    _need(x, torch.bfloat16, "x", device=dev)
    _need(topk_idx, torch.int64, "topk_idx", (T, K), device=dev)
    R = E * C
    if out is None:
        out = LowLatencyDispatched(
            torch.empty(E, dtype=torch.int32, device=dev),
            torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev),
            torch.empty((R, H // 128), dtype=torch.float32, device=dev) if fp8 else None,
            torch.empty(R, dtype=torch.int32, device=dev),
            torch.empty((T, K), dtype=torch.int32, device=dev),
            torch.empty(1, dtype=torch.int64, device=dev))
    _need(out.num_tokens_per_expert, torch.int32, "num_tokens_per_expert", (E,), device=dev)
    _need(out.recv_x, torch.uint8 if fp8 else torch.bfloat16, "recv_x", (R, H), device=dev)
    if fp8:
        _need(out.recv_scales, torch.float32, "recv_scales", (R, H // 128), device=dev)
    _need(out.recv_src_token, torch.int32, "recv_src_token", (R,), device=dev)
    _need(out.dst_row, torch.int32, "dst_row", (T, K), device=dev)
    _need(out.num_invalid, torch.int64, "num_invalid", (1,), device=dev)
    _check(lib().ep_low_latency_dispatch(
        _ptr(x), T, H, _ptr(topk_idx), K, E, C, EP_DTYPE_FP8_E4M3 if fp8 else EP_DTYPE_BF16,
        _ptr(out.num_tokens_per_expert), _ptr(out.recv_x),
        _ptr(out.recv_scales) if fp8 else None, _ptr(out.recv_src_token), _ptr(out.dst_row),
        _ptr(out.num_invalid), _stream(x)), "ep_low_latency_dispatch")
    return out


def combine(y: torch.Tensor, dst_row: torch.Tensor, topk_weights: torch.Tensor,
            out: torch.Tensor | None = None, num_cus: int = 0) -> torch.Tensor:
    """ep_combine: y [R, H] bf16 expert outputs -> out [T, H] bf16.  num_cus >
    0 confines it to that many CUs (ep_combine_cu)."""
    if y.dim() != 2 or dst_row.dim() != 2:
        raise ValueError("y must be [R, H] and dst_row [T, K]")
    T, K = dst_row.shape
    H = y.shape[1]
    dev = y.device
    _need(y, torch.bfloat16, "y", device=dev)
    _need(dst_row, torch.int32, "dst_row", device=dev)
    _need(topk_weights, torch.float32, "topk_weights", (T, K), device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _need(out, torch.bfloat16, "out", (T, H), device=dev)
    _check(lib().ep_combine_cu(_ptr(y), y.shape[0], _ptr(dst_row), _ptr(topk_weights), T, K, H,
                               _ptr(out), int(num_cus), _stream(y)), "ep_combine_cu")
    return out


# ---------------------------------------------------------------------------
# diagnostics
# ---------------------------------------------------------------------------

def convert_e4m3(v: torch.Tensor, mode: int = 0) -> torch.Tensor:
    """E4M3 codes of fp32 ``v`` with the dispatch kernel's conversion (mode 0)
    or the software conversion (mode 1)."""
    _need(v, torch.float32, "v")
    out = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _check(lib().ep_convert_e4m3(_ptr(v), _ptr(out), v.numel(), mode, _stream(v)),
           "ep_convert_e4m3")
    return out


def convert_bf16(v: torch.Tensor) -> torch.Tensor:
    """bf16 bits (as int16) of fp32 ``v`` with the combine kernel's rounding."""
    _need(v, torch.float32, "v")
    out = torch.empty(v.shape, dtype=torch.int16, device=v.device)
    _check(lib().ep_convert_bf16(_ptr(v), _ptr(out), v.numel(), _stream(v)), "ep_convert_bf16")
    return out


def copy(src: torch.Tensor, dst: torch.Tensor):
    """ep_copy of all of ``src``'s bytes into ``dst``."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    _check(lib().ep_copy(_ptr(src), _ptr(dst), nbytes, _stream(src)), "ep_copy")
