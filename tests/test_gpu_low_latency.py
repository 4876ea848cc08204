"""Parity of the single-launch fixed-capacity (decode) dispatch with the CPU
oracle (GPU).

Each case runs ep_low_latency_dispatch and then ep_combine on expert outputs
laid out like its receive rows, through the C ABI on cuda:0, and compares
with the oracle's fixed-capacity layout, row dispatch and combine on the same
seeded inputs: counts, dst_row, recv_src_token, the invalid count, the filled
receive rows and FP8 scales bit for bit, combine within 2 bf16 ulp.  Unfilled
rows are pre-set to a sentinel and must keep it.  Cases cover the decode
configuration (with and without drops), ragged channel chunks, masked,
invalid and repeated ids, skewed routing, T = 0, one token, the largest E, K
and T*K, and agreement with the offsets path when nothing drops; a graph
capture of dispatch + combine is replayed and checked against eager runs.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_get_dispatch_amd import binding as ep
from combine_ep_get_dispatch_amd import workloads as wl
from parity import MAX_COMBINE_ULP, announce, bf16_bits, to_dev_bf16, ulp_distance

pytestmark = pytest.mark.gpu

SENTINEL_BF16 = 0x7FBF          # a NaN pattern no copy of a finite token produces
SENTINEL_FP8 = 0x7F             # E4M3 NaN: the quantiser never writes it


def _outputs(T, K, E, C, H, fp8, dev):
    R = E * C
    if fp8:
        rx = torch.full((R, H), SENTINEL_FP8, dtype=torch.uint8, device=dev)
        rs = torch.full((R, H // 128), -1.0, dtype=torch.float32, device=dev)
    else:
        rx = torch.full((R, H), SENTINEL_BF16, dtype=torch.int16, device=dev).view(torch.bfloat16)
        rs = None
    return ep.LowLatencyDispatched(
        torch.full((E,), -7, dtype=torch.int32, device=dev), rx, rs,
        torch.full((R,), -7, dtype=torch.int32, device=dev),
        torch.full((T, K), -7, dtype=torch.int32, device=dev),
        torch.full((1,), -7, dtype=torch.int64, device=dev))


def check_ll(topk_idx, x_bits, topk_weights, E, C, fp8, label, y_seed=900):
    T, K = topk_idx.shape
    H = x_bits.shape[1]
    announce("ll %s T=%d H=%d E=%d C=%d K=%d fp8=%s" % (label, T, H, E, C, K, fp8))
    dev = torch.device("cuda:0")
    idx = torch.from_numpy(np.ascontiguousarray(topk_idx)).to(dev)
    x = to_dev_bf16(x_bits)
    out = _outputs(T, K, E, C, H, fp8, dev)
    ep.low_latency_dispatch(x, idx, E, C, fp8=fp8, out=out)
    y_bits = wl.normal_bf16(y_seed, (E * C, H))
    y = to_dev_bf16(y_bits)
    w = torch.from_numpy(np.ascontiguousarray(topk_weights, dtype=np.float32)).to(dev)
    comb = bf16_bits(ep.combine(y, out.dst_row, w))
    torch.cuda.synchronize()

    o = oracle.ll_layout(topk_idx, E, C)
    np.testing.assert_array_equal(out.num_tokens_per_expert.cpu().numpy(),
                                  o["num_tokens_per_expert"], err_msg="num_tokens_per_expert")
    np.testing.assert_array_equal(out.dst_row.cpu().numpy(), o["dst_row"], err_msg="dst_row")
    src = o["recv_src_token"]
    np.testing.assert_array_equal(out.recv_src_token.cpu().numpy(), src, err_msg="recv_src")
    assert int(out.num_invalid.item()) == o["num_invalid"]
    filled = src >= 0
    if fp8:
        want_x, want_s = oracle.dispatch_rows_fp8(x_bits, src, fill=SENTINEL_FP8)
        got_x = out.recv_x.cpu().numpy()
        got_s = out.recv_scales.cpu().numpy()
        np.testing.assert_array_equal(got_x, want_x, err_msg="recv_x")
        np.testing.assert_array_equal(got_s[filled].view(np.uint32),
                                      want_s[filled].view(np.uint32), err_msg="recv_scales")
        assert np.all(got_s[~filled] == -1.0), "unfilled scale rows were written"
    else:
        want_x = oracle.dispatch_rows_bf16(x_bits, src, fill=SENTINEL_BF16)
        np.testing.assert_array_equal(bf16_bits(out.recv_x), want_x, err_msg="recv_x")
    want_out = oracle.combine(y_bits, o["dst_row"], np.asarray(topk_weights, np.float32))
    u = ulp_distance(comb, want_out)
    assert int(u.max(initial=0)) <= MAX_COMBINE_ULP
    stats = dict(filled=int(filled.sum()), dropped=int(np.maximum(
        o["num_tokens_per_expert"] - C, 0).sum()), combine_max_ulp=int(u.max(initial=0)))
    announce("ll %s ok %s" % (label, stats))
    return stats


@pytest.mark.parametrize("C,drops", [(32, False), (4, True)])
def test_decode_configuration(C, drops):
    case = wl.make("decode")
    stats = check_ll(case.topk_idx, case.x_bits, case.topk_weights, case.E, C, case.fp8,
                     "decode")
    assert (stats["dropped"] > 0) == drops


def test_decode_configuration_bf16():
    case = wl.make("decode")
    check_ll(case.topk_idx, case.x_bits, case.topk_weights, case.E, 16, False, "decode-bf16")


def test_tiny_configuration():
    case = wl.make("tiny")
    check_ll(case.topk_idx, case.x_bits, case.topk_weights, case.E, case.T, case.fp8, "tiny")


LL_CASES = [
    # T, H, E, K, C, seed, kwargs
    (128, 7168, 256, 8, 128, 1, dict(fp8=True)),                     # capacity = T
    (100, 264, 16, 3, 9, 2, dict(masked_frac=0.1)),                  # ragged H, drops
    (77, 1032, 64, 6, 12, 3, dict(fp8=False, allow_dup=True)),       # repeated experts
    (200, 384, 32, 4, 40, 4, dict(fp8=True, skew=2.0)),
    (65, 512, 40, 7, 20, 5, dict(masked_frac=0.3, invalid_frac=0.1)),
    (1, 7168, 256, 8, 1, 6, dict(fp8=True)),                         # one token
    (128, 128, 1024, 64, 8, 7, dict()),                              # largest E and K
    (1024, 128, 256, 8, 64, 8, dict(fp8=True, masked_frac=0.02)),    # T*K at the limit
    (40, 8, 4, 2, 3, 9, dict(skew=3.0)),                             # smallest H
    (33, 2048, 1, 1, 40, 10, dict()),                                # one expert
    (70, 17536, 64, 8, 16, 11, dict(fp8=True, masked_frac=0.05)),    # waves loop over chunks
    (66, 18440, 32, 6, 20, 12, dict(allow_dup=True)),
    (96, 2048, 64, 6, 24, 13, dict(fp8=True, nonfinite_frac=0.01)),   # infinities and NaNs in x
    (96, 2048, 64, 6, 24, 14, dict(nonfinite_frac=0.01)),
]


@pytest.mark.parametrize("T,H,E,K,C,seed,kw", LL_CASES,
                         ids=["T%d_H%d_E%d_K%d_C%d" % g[:5] for g in LL_CASES])
def test_random_case(T, H, E, K, C, seed, kw):
    case = wl.random_case(T, H, E, 1, K, 700 + seed, **kw)
    check_ll(case.topk_idx, case.x_bits, case.topk_weights, E, C, case.fp8,
             "random seed=%d" % (700 + seed), y_seed=800 + seed)


def test_zero_tokens():
    announce("ll zero tokens")
    dev = torch.device("cuda:0")
    E, C, K, H = 16, 5, 2, 256
    out = _outputs(0, K, E, C, H, True, dev)
    ep.low_latency_dispatch(torch.empty((0, H), dtype=torch.bfloat16, device=dev),
                            torch.empty((0, K), dtype=torch.int64, device=dev), E, C, fp8=True,
                            out=out)
    torch.cuda.synchronize()
    assert np.all(out.num_tokens_per_expert.cpu().numpy() == 0)
    assert np.all(out.recv_src_token.cpu().numpy() == -1)
    assert int(out.num_invalid.item()) == 0
    assert np.all(out.recv_x.cpu().numpy() == SENTINEL_FP8)


def test_matches_offsets_path_when_nothing_drops():
    """With capacity >= every count, each slot's row inside its expert and the
    row contents are those of layout + dispatch."""
    case = wl.make("decode")
    announce("ll vs offsets path decode")
    dev = torch.device("cuda:0")
    idx = torch.from_numpy(case.topk_idx).to(dev)
    x = to_dev_bf16(case.x_bits)
    lay = ep.get_dispatch_layout(idx, case.E, case.P)
    d = ep.dispatch(x, idx, case.E, case.P, lay.workspace, fp8=True)
    C = int(lay.num_tokens_per_expert.max().item())
    ll = ep.low_latency_dispatch(x, idx, case.E, C, fp8=True)
    torch.cuda.synchronize()
    dst, lld = d.dst_row.cpu().numpy(), ll.dst_row.cpu().numpy()
    off = lay.expert_offsets.cpu().numpy()
    e = case.topk_idx
    np.testing.assert_array_equal(lld - e * C, dst - off[e])
    np.testing.assert_array_equal(ll.recv_x.cpu().numpy()[lld.reshape(-1)],
                                  d.recv_x.cpu().numpy()[dst.reshape(-1)])
    np.testing.assert_array_equal(ll.recv_scales.cpu().numpy()[lld.reshape(-1)],
                                  d.recv_scales.cpu().numpy()[dst.reshape(-1)])


def test_graph_replays_match_eager():
    """Dispatch + combine captured once and replayed with eager work and
    synchronisations in between; every replay reproduces the eager outputs."""
    case = wl.make("decode")
    announce("ll graph replay decode")
    dev = torch.device("cuda:0")
    T, K, E, H = case.T, case.K, case.E, case.H
    C = 32
    idx = torch.from_numpy(case.topk_idx).to(dev)
    x = to_dev_bf16(case.x_bits)
    y = to_dev_bf16(wl.normal_bf16(901, (E * C, H)))
    w = torch.from_numpy(case.topk_weights).to(dev)

    def step(o, comb):
        ep.low_latency_dispatch(x, idx, E, C, fp8=True, out=o)
        ep.combine(y, o.dst_row, w, out=comb)

    def snapshot(o, comb):
        src = o.recv_src_token
        filled = torch.nonzero(src >= 0).flatten()
        return [t.cpu().numpy().copy() for t in
                (o.num_tokens_per_expert, src, o.dst_row, o.num_invalid,
                 o.recv_x[filled], o.recv_scales[filled], comb.view(torch.int16))]

    ref_o = _outputs(T, K, E, C, H, True, dev)
    ref_c = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    step(ref_o, ref_c)
    torch.cuda.synchronize()
    ref = snapshot(ref_o, ref_c)

    g_o = _outputs(T, K, E, C, H, True, dev)
    g_c = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(g_o, g_c)                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_o, g_c)
    for rep in range(3):
        g_o.dst_row.fill_(-5)
        g_c.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot(g_o, g_c)
        for a, b in zip(got, ref):
            np.testing.assert_array_equal(a, b, err_msg="replay %d" % rep)
        step(ref_o, ref_c)               # eager work between replays
        torch.cuda.synchronize()
