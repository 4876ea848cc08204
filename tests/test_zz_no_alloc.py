"""ep_layout_dispatch_static, the entry point that allocates nothing (GPU).

Its workspace is the library's static per-GPU scratch array instead of a
caller's buffer.  Two calls in a row -- the second with a smaller input, so
that it runs over what the first left in the array -- must give exactly the
outputs of ep_layout_dispatch with a workspace of its own (bit-exact: counts,
offsets, partition rows, receive rows, FP8 scales, source tokens, dst_row).
"""
import numpy as np
import pytest
import torch

from combine_ep_get_dispatch_amd import binding as ep
from combine_ep_get_dispatch_amd import workloads as wl
from parity import announce, to_dev_bf16

pytestmark = pytest.mark.gpu

LAYOUT_FIELDS = ("num_tokens_per_expert", "num_tokens_per_partition", "is_token_in_partition",
                 "expert_offsets", "partition_offsets")


def _outputs(lay, d, fp8):
    res = {f: getattr(lay, f) for f in LAYOUT_FIELDS}
    res.update(recv_x=d.recv_x, recv_src_token=d.recv_src_token, dst_row=d.dst_row)
    if fp8:
        res["recv_scales"] = d.recv_scales
    return {k: v.contiguous().view(torch.uint8).cpu().numpy() for k, v in res.items()}


@pytest.mark.parametrize("first,second", [("prefill", "decode"), ("skewed", "tiny")])
def test_static_scratch_matches_workspace_path(first, second):
    for name in (first, second):
        case = wl.make(name)
        announce("no-alloc entry point: %s (T=%d H=%d E=%d P=%d K=%d fp8=%s)"
                 % (name, case.T, case.H, case.E, case.P, case.K, case.fp8))
        idx = torch.from_numpy(case.topk_idx).cuda()
        x = to_dev_bf16(case.x_bits)
        lay_s, d_s = ep.layout_dispatch_static(x, idx, case.E, case.P, fp8=case.fp8)
        lay_w, d_w = ep.layout_dispatch(x, idx, case.E, case.P, fp8=case.fp8)
        torch.cuda.synchronize()
        a = _outputs(lay_s, d_s, case.fp8)
        b = _outputs(lay_w, d_w, case.fp8)
        for k in b:
            np.testing.assert_array_equal(a[k], b[k], err_msg="%s: %s" % (name, k))


def test_static_scratch_refuses_oversized_shapes():
    idx = torch.zeros((1 << 18, 8), dtype=torch.int64, device="cuda")
    x = torch.zeros((1 << 18, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ep.EpError):
        ep.layout_dispatch_static(x, idx, 256, 64)
