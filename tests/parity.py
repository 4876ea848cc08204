"""Helpers for the GPU parity tests: run one case through the HIP path (via the
C ABI binding) and through the CPU oracle, and compare them.

Bars: bit-exact for every integer output (counts, offsets, partition mask,
dst_row, recv_src_token), for the receive rows (bf16 bits or E4M3 bytes) and
the fp32 scales; combine within 2 bf16 ulp (the same fp32 FMA order is used on
both sides, so 0 is expected and reported).
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from combine_ep_get_dispatch_amd import binding as ep

MAX_COMBINE_ULP = 2


def announce(msg: str):
    """Name the case on the real stderr before its GPU work starts."""
    sys.__stderr__.write("[gpu-case] %s\n" % msg)
    sys.__stderr__.flush()


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|m(a) - m(b)| with bf16 bits mapped to ordered integers (+0 == -0)."""
    def m(x):
        x = x.astype(np.int32)
        return np.where(x < 0x8000, x, -(x & 0x7FFF))
    return np.abs(m(a) - m(b))


def run_gpu(case, with_combine=True, workspace=None, one_call=False, num_cus=0):
    """The whole path on cuda:0 (layout and dispatch as two calls, or as the
    one ep_layout_dispatch call, optionally with a CU budget for it and for
    combine); returns numpy copies of every output."""
    idx = torch.from_numpy(case.topk_idx).cuda()
    x = to_dev_bf16(case.x_bits)
    if one_call:
        lay, d = ep.layout_dispatch(x, idx, case.E, case.P, workspace=workspace, fp8=case.fp8,
                                    num_cus=num_cus)
    else:
        lay = ep.get_dispatch_layout(idx, case.E, case.P, workspace=workspace)
        d = ep.dispatch(x, idx, case.E, case.P, lay.workspace, fp8=case.fp8)
    res = dict(
        num_tokens_per_expert=lay.num_tokens_per_expert.cpu().numpy(),
        num_tokens_per_partition=lay.num_tokens_per_partition.cpu().numpy(),
        is_token_in_partition=lay.is_token_in_partition.cpu().numpy(),
        expert_offsets=lay.expert_offsets.cpu().numpy(),
        partition_offsets=lay.partition_offsets.cpu().numpy(),
        dst_row=d.dst_row.cpu().numpy(),
        recv_src_token=d.recv_src_token.cpu().numpy(),
    )
    res["num_invalid"] = ep.get_device_error(lay.workspace)
    if case.fp8:
        res["recv_x"] = d.recv_x.cpu().numpy()
        res["recv_scales"] = d.recv_scales.cpu().numpy()
    else:
        res["recv_x"] = bf16_bits(d.recv_x)
    if with_combine:
        y = to_dev_bf16(case.y_bits)
        w = torch.from_numpy(case.topk_weights).cuda()
        res["out"] = bf16_bits(ep.combine(y, d.dst_row, w, num_cus=num_cus))
    torch.cuda.synchronize()
    return res


def run_oracle(case, with_combine=True):
    return oracle.run(case.topk_idx, case.x_bits, case.E, case.P, case.fp8,
                      case.y_bits if with_combine else None,
                      case.topk_weights if with_combine else None)


def compare(g: dict, o: dict, case, with_combine=True) -> dict:
    """Assert parity; return a few statistics."""
    for k in ["num_tokens_per_expert", "num_tokens_per_partition", "is_token_in_partition",
              "expert_offsets", "partition_offsets", "dst_row", "recv_src_token"]:
        np.testing.assert_array_equal(g[k], o[k], err_msg=k)
    assert g["num_invalid"] == o["num_invalid"]
    N = int(o["expert_offsets"][case.E])
    np.testing.assert_array_equal(g["recv_x"][:N], o["recv_x"][:N], err_msg="recv_x")
    if case.fp8:
        np.testing.assert_array_equal(g["recv_scales"][:N].view(np.uint32),
                                      o["recv_scales"][:N].view(np.uint32), err_msg="recv_scales")
    stats = {"N": N}
    if with_combine:
        u = ulp_distance(g["out"], o["out"])
        stats["combine_max_ulp"] = int(u.max(initial=0))
        stats["combine_mismatches"] = int((u > 0).sum())
        assert stats["combine_max_ulp"] <= MAX_COMBINE_ULP, stats
    return stats


def check_case(case, with_combine=True, label="", one_call=False, num_cus=0):
    label = (label or case.name) + (" (one call)" if one_call else "") + \
        (" (%d CUs)" % num_cus if num_cus else "")
    announce("%s T=%d H=%d E=%d P=%d K=%d fp8=%s" % (label, case.T, case.H, case.E,
                                                     case.P, case.K, case.fp8))
    t0 = time.time()
    g = run_gpu(case, with_combine, one_call=one_call, num_cus=num_cus)
    t1 = time.time()
    o = run_oracle(case, with_combine)
    t2 = time.time()
    stats = compare(g, o, case, with_combine)
    stats.update(gpu_s=round(t1 - t0, 2), oracle_s=round(t2 - t1, 2))
    announce("%s ok %s" % (label, stats))
    return stats
