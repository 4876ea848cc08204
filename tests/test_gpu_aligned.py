"""Parity of the aligned layout + dispatch (every expert's run padded to a
multiple of the alignment) with the CPU oracle (GPU).

Each case runs ep_layout_dispatch_aligned and then ep_combine on expert outputs
laid out like its receive rows, through the C ABI on cuda:0, and compares with
the oracle's aligned layout, row dispatch and combine on the same seeded
inputs: the five layout outputs, dst_row, recv_src_token (including the -1 of
every padding and unused row) and the invalid count bit for bit; the receive
rows holding a token (bf16 bits or E4M3 bytes and scales) bit for bit, with
padding and unused rows pre-set to a sentinel that must survive; combine within
2 bf16 ulp.  Cases: the five configurations at full size with the alignments a
grouped GEMM would use, alignments 1 (equal to ep_layout_dispatch), 2, 3, 7,
64, 128 and 1024, ragged token blocks and channel chunks, masked, invalid and
repeated ids, skew, every slot on one expert, T = 0, one token, the largest E
and K, and a workspace shared with the other paths.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_get_dispatch_amd import binding as ep
from combine_ep_get_dispatch_amd import workloads as wl
from parity import (MAX_COMBINE_ULP, announce, bf16_bits, compare, run_gpu, run_oracle,
                    to_dev_bf16, ulp_distance)

pytestmark = pytest.mark.gpu

SENTINEL_BF16 = 0x7FBF          # a NaN pattern no copy of a finite token produces
SENTINEL_FP8 = 0x7F             # E4M3 NaN: the quantiser never writes it


def _outputs(T, K, E, P, R, H, fp8, dev):
    if fp8:
        rx = torch.full((R, H), SENTINEL_FP8, dtype=torch.uint8, device=dev)
        rs = torch.full((R, H // 128), -1.0, dtype=torch.float32, device=dev)
    else:
        rx = torch.full((R, H), SENTINEL_BF16, dtype=torch.int16, device=dev).view(torch.bfloat16)
        rs = None
    lay = ep.Layout(torch.full((E,), -7, dtype=torch.int32, device=dev),
                    torch.full((P,), -7, dtype=torch.int32, device=dev),
                    torch.full((T, P), 7, dtype=torch.uint8, device=dev),
                    torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
                    torch.full((P + 1,), -7, dtype=torch.int32, device=dev), None)
    d = ep.Dispatched(rx, rs, torch.full((R,), -7, dtype=torch.int32, device=dev),
                      torch.full((T, K), -7, dtype=torch.int32, device=dev))
    return lay, d


def check_aligned(case, align, label, workspace=None, y_seed=950):
    T, K, E, P, H = case.T, case.K, case.E, case.P, case.H
    R = ep.aligned_rows(T, K, E, align)
    announce("aligned %s T=%d H=%d E=%d P=%d K=%d align=%d fp8=%s" %
             (label, T, H, E, P, K, align, case.fp8))
    dev = torch.device("cuda:0")
    idx = torch.from_numpy(np.ascontiguousarray(case.topk_idx)).to(dev)
    x = to_dev_bf16(case.x_bits)
    lay, d = _outputs(T, K, E, P, R, H, case.fp8, dev)
    if workspace is None:
        workspace = ep.new_workspace(T, K, E, P, dev)
    ep.layout_dispatch_aligned(x, idx, E, P, align, workspace=workspace, fp8=case.fp8,
                               out_layout=lay, out=d)
    y_bits = wl.normal_bf16(y_seed, (R, H))
    y = to_dev_bf16(y_bits)
    w = torch.from_numpy(np.ascontiguousarray(case.topk_weights, dtype=np.float32)).to(dev)
    comb = bf16_bits(ep.combine(y, d.dst_row, w)) if T > 0 else None
    nerr = ep.get_device_error(workspace)
    torch.cuda.synchronize()

    o = oracle.aligned_layout(case.topk_idx, E, P, align)
    for key, got in [("num_tokens_per_expert", lay.num_tokens_per_expert),
                     ("num_tokens_per_partition", lay.num_tokens_per_partition),
                     ("is_token_in_partition", lay.is_token_in_partition),
                     ("expert_offsets", lay.expert_offsets),
                     ("partition_offsets", lay.partition_offsets),
                     ("dst_row", d.dst_row), ("recv_src_token", d.recv_src_token)]:
        np.testing.assert_array_equal(got.cpu().numpy(), np.asarray(o[key]), err_msg=key)
    assert nerr == o["num_invalid"]
    src = o["recv_src_token"]
    held = src >= 0
    if case.fp8:
        want_x, want_s = oracle.dispatch_rows_fp8(case.x_bits, src, fill=SENTINEL_FP8)
        got_s = d.recv_scales.cpu().numpy()
        np.testing.assert_array_equal(d.recv_x.cpu().numpy(), want_x, err_msg="recv_x")
        np.testing.assert_array_equal(got_s[held].view(np.uint32), want_s[held].view(np.uint32),
                                      err_msg="recv_scales")
        assert np.all(got_s[~held] == -1.0), "padding or unused scale rows were written"
    else:
        want_x = oracle.dispatch_rows_bf16(case.x_bits, src, fill=SENTINEL_BF16)
        np.testing.assert_array_equal(bf16_bits(d.recv_x), want_x, err_msg="recv_x")
    stats = dict(rows=R, used=int(o["expert_offsets"][E]), padding=int(o["expert_offsets"][E]) -
                 int(held.sum()))
    if T > 0:
        want = oracle.combine(y_bits, o["dst_row"], np.asarray(case.topk_weights, np.float32))
        u = ulp_distance(comb, want)
        stats["combine_max_ulp"] = int(u.max(initial=0))
        assert stats["combine_max_ulp"] <= MAX_COMBINE_ULP
    announce("aligned %s ok %s" % (label, stats))
    return stats


@pytest.mark.parametrize("name,align", [("tiny", 8), ("decode", 64), ("prefill", 128),
                                        ("skewed", 128), ("coarse", 256)])
def test_configuration_full_size(name, align):
    case = wl.make(name)
    stats = check_aligned(case, align, "config " + name)
    assert stats["used"] % align == 0


CASES = [
    # T, H, E, P, K, align, seed, kwargs
    (1000, 264, 16, 4, 3, 2, 71, dict()),
    (777, 1032, 64, 8, 6, 3, 72, dict(masked_frac=0.1)),
    (513, 384, 32, 4, 4, 7, 73, dict(fp8=True)),
    (300, 1152, 256, 64, 8, 64, 74, dict(fp8=True, masked_frac=0.05)),
    (2500, 520, 8, 8, 2, 128, 75, dict(skew=2.0)),
    (130, 136, 12, 3, 5, 1024, 76, dict(allow_dup=True)),
    (257, 2048, 128, 16, 16, 32, 77, dict(fp8=True)),
    (65, 512, 40, 5, 7, 5, 78, dict(masked_frac=0.3, invalid_frac=0.1)),
    (4097, 128, 1024, 1024, 64, 16, 79, dict()),
    (1, 8, 4, 2, 2, 128, 80, dict()),
    (50, 256, 1, 1, 1, 64, 81, dict()),
    (9000, 128, 256, 64, 8, 128, 82, dict(masked_frac=0.02, invalid_frac=0.01)),
    (70, 17536, 64, 8, 8, 64, 87, dict(fp8=True, masked_frac=0.05)),   # waves loop over chunks
    (66, 18440, 32, 4, 6, 3, 88, dict(allow_dup=True)),
]


@pytest.mark.parametrize("T,H,E,P,K,align,seed,kw", CASES,
                         ids=["T%d_H%d_E%d_P%d_K%d_A%d" % c[:6] for c in CASES])
def test_generic_case(T, H, E, P, K, align, seed, kw):
    case = wl.random_case(T, H, E, P, K, seed, **kw)
    check_aligned(case, align, "random seed=%d" % seed)


def test_align_one_equals_layout_dispatch():
    case = wl.random_case(3000, 1024, 64, 8, 6, 83, masked_frac=0.05, invalid_frac=0.01,
                          fp8=True)
    announce("aligned align=1 vs ep_layout_dispatch")
    check_aligned(case, 1, "align 1")
    g = run_gpu(case, one_call=True)
    compare(g, run_oracle(case), case)


def test_all_slots_on_one_expert():
    case = wl.random_case(3000, 256, 32, 8, 2, 84)
    case.topk_idx[:, 0] = 17
    case.topk_idx[:, 1] = -1
    stats = check_aligned(case, 128, "one hot expert")
    assert stats["used"] == 3072 and stats["padding"] == 72


def test_zero_tokens():
    announce("aligned zero tokens")
    dev = torch.device("cuda:0")
    idx = torch.zeros((0, 4), dtype=torch.int64, device=dev)
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=dev)
    R = ep.aligned_rows(0, 4, 16, 64)
    lay, d = _outputs(0, 4, 16, 4, R, 256, True, dev)
    ep.layout_dispatch_aligned(x, idx, 16, 4, 64, fp8=True, out_layout=lay, out=d)
    torch.cuda.synchronize()
    assert R == 16 * 63
    assert lay.expert_offsets.cpu().tolist() == [0] * 17
    assert lay.partition_offsets.cpu().tolist() == [0] * 5
    assert lay.num_tokens_per_expert.cpu().tolist() == [0] * 16
    assert bool((d.recv_src_token == -1).all())
    assert ep.get_device_error(lay.workspace) == 0


def test_workspace_shared_with_other_paths():
    big = wl.random_case(5000, 256, 64, 16, 8, 85, invalid_frac=0.01, with_y=True)
    small = wl.random_case(600, 512, 16, 4, 4, 86, fp8=True)
    ws = ep.new_workspace(5000, 8, 64, 16)
    for case, how in [(big, "aligned"), (big, "one"), (small, "aligned"), (big, "two"),
                      (big, "aligned")]:
        announce("shared workspace T=%d %s" % (case.T, how))
        if how == "aligned":
            check_aligned(case, 64, "shared workspace", workspace=ws)
        else:
            g = run_gpu(case, workspace=ws, one_call=(how == "one"))
            compare(g, run_oracle(case), case)
