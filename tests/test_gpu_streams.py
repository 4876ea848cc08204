"""Concurrent calls on several streams (GPU).

The library keeps no global state besides per-device launch attributes, so
calls with separate workspaces and outputs may run at the same time on
different streams.  Each case enqueues several different paths on their own
default-priority streams without waiting in between, then checks every result
against the oracle (bit-exact layout, rows and scales; combine within 2 bf16
ulp) -- and against the same calls run one at a time.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_get_dispatch_amd import binding as ep
from combine_ep_get_dispatch_amd import workloads as wl
from parity import MAX_COMBINE_ULP, announce, bf16_bits, to_dev_bf16, ulp_distance

pytestmark = pytest.mark.gpu


def _inputs(case, dev):
    return (torch.from_numpy(np.ascontiguousarray(case.topk_idx)).to(dev),
            to_dev_bf16(case.x_bits), to_dev_bf16(case.y_bits),
            torch.from_numpy(np.ascontiguousarray(case.topk_weights)).to(dev))


def _enqueue(kind, case, tensors):
    """Enqueue one path on the current stream; return a function that reads
    its results back (after a synchronisation)."""
    idx, x, y, w = tensors
    E, P = case.E, case.P
    if kind == "one_call":
        lay, d = ep.layout_dispatch(x, idx, E, P, fp8=case.fp8)
    elif kind == "two_calls":
        lay = ep.get_dispatch_layout(idx, E, P)
        d = ep.dispatch(x, idx, E, P, lay.workspace, fp8=case.fp8)
    elif kind == "budget":
        lay, d = ep.layout_dispatch(x, idx, E, P, fp8=case.fp8, num_cus=24)
    else:
        raise ValueError(kind)
    out = ep.combine(y, d.dst_row, w, num_cus=24 if kind == "budget" else 0)

    def read():
        n = int(lay.expert_offsets[-1].item())
        res = dict(expert_offsets=lay.expert_offsets.cpu().numpy(),
                   num_tokens_per_expert=lay.num_tokens_per_expert.cpu().numpy(),
                   num_tokens_per_partition=lay.num_tokens_per_partition.cpu().numpy(),
                   is_token_in_partition=lay.is_token_in_partition.cpu().numpy(),
                   partition_offsets=lay.partition_offsets.cpu().numpy(),
                   dst_row=d.dst_row.cpu().numpy(), recv_src_token=d.recv_src_token.cpu().numpy(),
                   out=bf16_bits(out), n=n)
        if case.fp8:
            res["recv_x"] = d.recv_x[:n].cpu().numpy()
            res["recv_scales"] = d.recv_scales[:n].cpu().numpy().view(np.uint32)
        else:
            res["recv_x"] = bf16_bits(d.recv_x[:n])
        return res
    return read


def _check_against_oracle(case, got, label):
    o = oracle.run(case.topk_idx, case.x_bits, case.E, case.P, case.fp8, case.y_bits,
                   case.topk_weights)
    n = got["n"]
    for key in ["expert_offsets", "num_tokens_per_expert", "num_tokens_per_partition",
                "is_token_in_partition", "partition_offsets", "dst_row", "recv_src_token"]:
        np.testing.assert_array_equal(got[key], np.asarray(o[key]), err_msg="%s %s" % (label, key))
    np.testing.assert_array_equal(got["recv_x"], np.asarray(o["recv_x"])[:n], err_msg=label)
    if case.fp8:
        np.testing.assert_array_equal(got["recv_scales"],
                                      np.asarray(o["recv_scales"])[:n].view(np.uint32),
                                      err_msg=label)
    assert int(ulp_distance(got["out"], o["out"]).max(initial=0)) <= MAX_COMBINE_ULP, label


def test_paths_on_concurrent_streams():
    dev = torch.device("cuda:0")
    jobs = [("one_call", wl.random_case(3000, 2048, 256, 64, 8, 301, fp8=True)),
            ("two_calls", wl.random_case(2000, 1032, 64, 8, 6, 302, masked_frac=0.05)),
            ("budget", wl.random_case(1500, 1024, 32, 4, 4, 303, fp8=True, skew=2.0)),
            ("one_call", wl.random_case(700, 520, 16, 16, 2, 304, invalid_frac=0.02))]
    announce("concurrent streams: %d jobs" % len(jobs))
    tensors = [_inputs(case, dev) for _, case in jobs]
    streams = [torch.cuda.Stream() for _ in jobs]
    torch.cuda.synchronize()
    readers = []
    for (kind, case), ts, st in zip(jobs, tensors, streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            readers.append(_enqueue(kind, case, ts))
    torch.cuda.synchronize()
    concurrent = [r() for r in readers]
    for (kind, case), got in zip(jobs, concurrent):
        _check_against_oracle(case, got, "concurrent %s T=%d" % (kind, case.T))

    # the same calls one at a time on the default stream give the same bits
    for (kind, case), ts, got in zip(jobs, tensors, concurrent):
        alone = _enqueue(kind, case, ts)
        torch.cuda.synchronize()
        ref = alone()
        for key, val in ref.items():
            np.testing.assert_array_equal(np.asarray(got[key]), np.asarray(val),
                                          err_msg="%s %s alone vs concurrent" % (kind, key))
    announce("concurrent streams ok")
