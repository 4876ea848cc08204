"""The path captured in a HIP graph and replayed (GPU).

Layout, dispatch and combine are captured once with preallocated outputs and
replayed several times, with eager work and synchronisations between the
replays; every replay must reproduce the eager results bit for bit.  The
two-call path, the one-call path (with and without a CU budget), the
de-duplicated path and the aligned path are each captured.
"""
import numpy as np
import pytest
import torch

from combine_ep_get_dispatch_amd import binding as ep
from combine_ep_get_dispatch_amd import workloads as wl
from parity import announce

pytestmark = pytest.mark.gpu


PATHS = [("decode", None, "two_calls"), ("prefill", 1024, "two_calls"),
         ("coarse", 3000, "two_calls"), ("prefill", 1024, "one_call"),
         ("skewed", 3000, "one_call"), ("prefill", 2048, "budget"), ("prefill", 1024, "dedup"),
         ("coarse", 3000, "dedup"), ("prefill", 1024, "aligned"), ("decode", None, "aligned")]
ALIGN = 128


@pytest.mark.parametrize("name,T,path", PATHS, ids=["%s-%s-%s" % p for p in PATHS])
def test_graph_replays_match_eager(name, T, path):
    case = wl.make(name, T=T)
    announce("graph replay %s T=%d %s" % (name, case.T, path))
    dev = torch.device("cuda:0")
    idx = torch.from_numpy(case.topk_idx).to(dev)
    x = torch.from_numpy(case.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.from_numpy(case.y_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(case.topk_weights).to(dev)
    T, K, E, P, H = case.T, case.K, case.E, case.P, case.H
    R = T * K
    if path == "aligned":
        # expert outputs laid out like the aligned receive rows
        R = ep.aligned_rows(T, K, E, ALIGN)
        y = torch.from_numpy(wl.normal_bf16(960, (R, H)).view(np.int16)).to(dev).view(
            torch.bfloat16)

    def outputs():
        lay = ep.Layout(torch.empty(E, dtype=torch.int32, device=dev),
                        torch.empty(P, dtype=torch.int32, device=dev),
                        torch.empty((T, P), dtype=torch.uint8, device=dev),
                        torch.empty(E + 1, dtype=torch.int32, device=dev),
                        torch.empty(P + 1, dtype=torch.int32, device=dev),
                        ep.new_workspace(T, K, E, P, dev))
        if path == "dedup":
            RD = T * min(K, P)
            d = ep.DedupDispatched(
                torch.empty(P + 1, dtype=torch.int32, device=dev),
                torch.empty((RD, H), dtype=torch.uint8 if case.fp8 else torch.bfloat16,
                            device=dev),
                torch.empty((RD, H // 128), dtype=torch.float32, device=dev) if case.fp8 else None,
                torch.empty(RD, dtype=torch.int32, device=dev),
                torch.empty((RD, K), dtype=torch.int32, device=dev),
                torch.empty(T * K, dtype=torch.int32, device=dev),
                torch.empty((T, K), dtype=torch.int32, device=dev))
        else:
            d = ep.Dispatched(
                torch.empty((R, H), dtype=torch.uint8 if case.fp8 else torch.bfloat16, device=dev),
                torch.empty((R, H // 128), dtype=torch.float32, device=dev) if case.fp8 else None,
                torch.empty(R, dtype=torch.int32, device=dev),
                torch.empty((T, K), dtype=torch.int32, device=dev))
        return lay, d, torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    budget = 37 if path == "budget" else 0

    def step(lay, d, out):
        if path == "two_calls":
            ep.get_dispatch_layout(idx, E, P, workspace=lay.workspace, out=lay)
            ep.dispatch(x, idx, E, P, lay.workspace, fp8=case.fp8, out=d)
        elif path == "dedup":
            ep.dispatch_dedup(x, idx, E, P, workspace=lay.workspace, fp8=case.fp8, out_layout=lay,
                              out=d)
        elif path == "aligned":
            ep.layout_dispatch_aligned(x, idx, E, P, ALIGN, workspace=lay.workspace, fp8=case.fp8,
                                       out_layout=lay, out=d)
        else:
            ep.layout_dispatch(x, idx, E, P, workspace=lay.workspace, fp8=case.fp8,
                               out_layout=lay, out=d, num_cus=budget)
        ep.combine(y, d.dst_row, w, out=out, num_cus=budget)

    def snapshot(lay, d, out):
        tensors = [lay.num_tokens_per_expert, lay.num_tokens_per_partition,
                   lay.is_token_in_partition, lay.expert_offsets, lay.partition_offsets,
                   d.recv_src_token, d.dst_row, out.view(torch.int16)]
        if path == "dedup":
            n = int(d.partition_token_offsets[-1].item())
            tensors += [d.partition_token_offsets, d.recv_topk_idx, d.slot_src_row]
        else:
            n = int(lay.expert_offsets[-1].item())
        # rows holding a token (an aligned layout's padding rows are never written)
        held = (d.recv_src_token[:n] >= 0).nonzero().flatten()
        tensors.append(d.recv_x[held].view(torch.uint8))
        if case.fp8:
            tensors.append(d.recv_scales[held])
        return [t.cpu().numpy().copy() for t in tensors]

    ref = outputs()
    step(*ref)
    torch.cuda.synchronize()
    want = snapshot(*ref)

    bufs = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(*bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(*bufs)
    for rep in range(3):
        # eager work between replays, and scribble over the outputs
        bufs[2].fill_(0)
        bufs[1].dst_row.fill_(-7)
        step(*ref)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(*bufs)
        for a, b in zip(got, want):
            np.testing.assert_array_equal(a, b, err_msg="replay %d" % rep)


_FIRST_CALL_CAPTURED = r'''
import sys
import numpy as np
import torch
from combine_ep_get_dispatch_amd import binding as ep
from combine_ep_get_dispatch_amd import workloads as wl

T, H, K, R = 4096, 7168, 8, 4096 * 8      # tiles of 8 tokens: 112 KiB of LDS per workgroup
y_bits, dst, w = wl.combine_inputs(T, H, K, R, 311, masked_frac=0.01)
dev = torch.device("cuda:0")
y = torch.from_numpy(y_bits.view(np.int16)).to(dev).view(torch.bfloat16)
d_dst = torch.from_numpy(dst).to(dev)
d_w = torch.from_numpy(w).to(dev)
out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
side = torch.cuda.Stream()
side.wait_stream(torch.cuda.current_stream())
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g, stream=side):      # the process's first combine call
    ep.combine(y, d_dst, d_w, out=out)
results = []
for _ in range(3):
    out.fill_(0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    results.append(out.clone())
eager = ep.combine(y, d_dst, d_w)
torch.cuda.synchronize()
ok = all(torch.equal(r.view(torch.int16), eager.view(torch.int16)) for r in results)
print("first-call capture ok" if ok else "first-call capture MISMATCH", flush=True)
sys.exit(0 if ok else 1)
'''


def test_first_combine_call_inside_a_capture():
    """A process whose first combine is made under graph capture, at a shape
    whose tiles need more than 64 KiB of LDS (so the kernel's LDS cap is
    raised during the capture): every replay equals an eager call."""
    import os
    import subprocess
    import sys
    announce("first combine call inside a capture (subprocess)")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _FIRST_CALL_CAPTURED], cwd=root,
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])
    assert "first-call capture ok" in r.stdout
