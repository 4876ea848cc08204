"""Parity of the HIP path with the CPU oracle (GPU).

Every case runs layout -> dispatch -> combine through the C ABI on cuda:0 and
through the oracle on the same seeded inputs, and compares element by element
(bit-exact layout, permutation, receive rows and FP8 scales; combine within
2 bf16 ulp).  The five workload configurations run at their full sizes, in
the same launch configuration the benchmark times; the generic cases cover
ragged token blocks (T not a multiple of the layout block), ragged channel
chunks (H not a multiple of 512/1024), masked, invalid and repeated expert
ids, and the degenerate shapes (T = 0, one token, one expert, P = 1, P = E,
K = E, everything routed to one expert, the largest E and K).
"""
import numpy as np
import pytest
import torch

from combine_ep_get_dispatch_amd import binding as ep
from combine_ep_get_dispatch_amd import workloads as wl
from parity import announce, check_case, run_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("one_call", [False, True], ids=["two_calls", "one_call"])
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed", "coarse"])
def test_configuration_full_size(name, one_call):
    case = wl.make(name)
    stats = check_case(case, label="config " + name, one_call=one_call)
    assert stats["N"] == case.T * case.K


GENERIC = [
    # T, H, E, P, K, seed, kwargs
    (1000, 264, 16, 4, 3, 1, dict()),                       # ragged T and H (bf16)
    (777, 1032, 64, 8, 6, 2, dict(masked_frac=0.1)),
    (513, 384, 32, 4, 4, 3, dict(fp8=True)),                 # FP8, ragged T
    (300, 1152, 256, 64, 8, 4, dict(fp8=True, masked_frac=0.05)),
    (2500, 520, 8, 8, 2, 5, dict(skew=2.0)),
    (96, 7168, 256, 32, 8, 6, dict(fp8=True, skew=1.5)),
    (130, 136, 12, 3, 5, 7, dict(allow_dup=True)),           # repeated experts in a row
    (257, 2048, 128, 16, 16, 8, dict(fp8=True)),            # generic-K combine path
    (65, 512, 40, 5, 7, 9, dict(masked_frac=0.3, invalid_frac=0.1)),
    (4097, 128, 1024, 1024, 64, 10, dict()),                 # largest E, P = E, largest K
    (1, 8, 4, 2, 2, 11, dict()),                             # one token, smallest H
    (50, 256, 1, 1, 1, 12, dict()),                          # a single expert
    (200, 640, 16, 1, 16, 13, dict(fp8=True)),               # P = 1 and K = E
    (100_000, 16, 4, 2, 1, 14, dict()),                      # many tokens, K = 1
    # around the size where the layout switches from one launch (at most two
    # blocks of 2048 slots) to two launches: 512 x 8 slots take one, 520 x 8 two
    (512, 128, 256, 64, 8, 15, dict(masked_frac=0.02, invalid_frac=0.01)),
    (520, 128, 256, 64, 8, 16, dict(masked_frac=0.02, invalid_frac=0.01)),
    (9000, 128, 256, 64, 8, 17, dict(masked_frac=0.02, invalid_frac=0.01)),
    # few tokens and the largest E: the single-launch layout with more than 64 KiB of LDS
    (20, 256, 1024, 1024, 64, 20, dict(fp8=True, masked_frac=0.05)),
    (60, 136, 1024, 256, 32, 21, dict(invalid_frac=0.02)),
    # rows wider than 16 chunks (1024 channels FP8, 512 bf16): waves loop over chunks
    (70, 17536, 64, 8, 8, 18, dict(fp8=True, masked_frac=0.05)),   # 18 chunks, last 128 ch
    (66, 18440, 32, 4, 6, 19, dict(allow_dup=True)),               # 37 chunks, last 8 ch
    # the two-launch layout (more than two blocks of 2048 slots) with K a power of two
    # up to 16 and P a multiple of 16 (membership rows in 16-byte stores), several
    # slots of a token in one partition
    (3000, 256, 64, 64, 4, 22, dict(masked_frac=0.05, invalid_frac=0.01)),
    (5000, 128, 64, 32, 2, 23, dict(allow_dup=True)),
    (9000, 128, 32, 16, 1, 24, dict(masked_frac=0.1)),
    (600, 256, 256, 64, 16, 25, dict(allow_dup=True, invalid_frac=0.02)),
    (1000, 264, 96, 48, 8, 26, dict(masked_frac=0.1)),
]


@pytest.mark.parametrize("T,H,E,P,K,seed,kw", GENERIC,
                         ids=["T%d_H%d_E%d_P%d_K%d" % g[:5] for g in GENERIC])
def test_generic_case(T, H, E, P, K, seed, kw):
    case = wl.random_case(T, H, E, P, K, seed, **kw)
    check_case(case, label="random seed=%d" % seed)
    check_case(case, label="random seed=%d" % seed, one_call=True)


@pytest.mark.parametrize("one_call", [False, True], ids=["two_calls", "one_call"])
def test_all_tokens_to_one_expert(one_call):
    case = wl.random_case(5000, 256, 32, 8, 1, 21)     # 3 token blocks
    case.topk_idx[:] = 17
    check_case(case, label="one hot expert", one_call=one_call)


@pytest.mark.parametrize("one_call", [False, True], ids=["two_calls", "one_call"])
def test_every_slot_masked(one_call):
    case = wl.random_case(3000, 256, 16, 4, 4, 22)
    case.topk_idx[:] = -1
    stats = check_case(case, label="all masked", one_call=one_call)
    assert stats["N"] == 0


@pytest.mark.parametrize("one_call", [False, True], ids=["two_calls", "one_call"])
@pytest.mark.parametrize("fp8", [True, False], ids=["fp8", "bf16"])
def test_nonfinite_tokens(fp8, one_call):
    """Infinities and NaNs of both signs in x (1% of the values, an all-NaN
    group, groups with an infinity): FP8 codes and scales bit-exact with the
    oracle's reading (NaNs left out of the group maximum, an infinity giving
    scale +inf and signed zeros, S.1111.111 with the sign of x for every
    non-finite x), bf16 rows bitwise copies."""
    case = wl.random_case(700, 1024, 64, 8, 6, 31, fp8=fp8, nonfinite_frac=0.01)
    check_case(case, label="non-finite x", one_call=one_call)


def test_invalid_ids_are_counted():
    case = wl.random_case(900, 128, 64, 8, 4, 23, invalid_frac=0.05, masked_frac=0.05)
    n_bad = int(((case.topk_idx != -1) & ((case.topk_idx < 0) | (case.topk_idx >= 64))).sum())
    assert n_bad > 0
    g = run_gpu(case)
    assert g["num_invalid"] == n_bad
    check_case(case, label="invalid ids")
    assert run_gpu(case, one_call=True)["num_invalid"] == n_bad
    check_case(case, label="invalid ids", one_call=True)


def test_zero_tokens():
    announce("zero tokens")
    idx = torch.zeros((0, 4), dtype=torch.int64, device="cuda")
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    lay = ep.get_dispatch_layout(idx, 16, 4)
    d = ep.dispatch(x, idx, 16, 4, lay.workspace, fp8=True)
    out = ep.combine(torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda"), d.dst_row,
                     torch.zeros((0, 4), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert out.shape == (0, 256)
    assert lay.expert_offsets.cpu().tolist() == [0] * 17
    assert lay.partition_offsets.cpu().tolist() == [0] * 5
    assert lay.num_tokens_per_expert.sum().item() == 0
    assert ep.get_device_error(lay.workspace) == 0
    lay1, d1 = ep.layout_dispatch(x, idx, 16, 4, fp8=True)
    torch.cuda.synchronize()
    assert lay1.expert_offsets.cpu().tolist() == [0] * 17
    assert lay1.partition_offsets.cpu().tolist() == [0] * 5
    assert lay1.num_tokens_per_partition.sum().item() == 0
    assert ep.get_device_error(lay1.workspace) == 0


def test_workspace_reuse_across_shapes():
    """One workspace serves a large call, then smaller ones (its header must be
    left clean by every layout call), then the large one again."""
    big = wl.random_case(5000, 256, 64, 16, 8, 31, invalid_frac=0.01)
    small = wl.random_case(37, 512, 16, 4, 2, 32, fp8=True)
    ws = ep.new_workspace(5000, 8, 64, 16)
    from parity import compare, run_oracle
    for case, one_call in [(big, False), (small, False), (small, True), (big, True),
                           (big, False), (small, True)]:
        announce("workspace reuse T=%d one_call=%s" % (case.T, one_call))
        g = run_gpu(case, workspace=ws, one_call=one_call)
        compare(g, run_oracle(case), case)


def _step_outputs(case, fill):
    """The benchmark's step (ep_layout_dispatch -> ep_combine) on cuda:0 into
    outputs pre-filled with the byte ``fill``; returns the outputs (on the GPU)."""
    idx = torch.from_numpy(case.topk_idx).cuda()
    x = to_dev_bf16(case.x_bits)
    y = to_dev_bf16(case.y_bits)
    w = torch.from_numpy(case.topk_weights).cuda()
    T, H, E, P, K, R = case.T, case.H, case.E, case.P, case.K, case.T * case.K

    def filled(shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        return torch.full((n,), fill, dtype=torch.uint8, device="cuda").view(dtype).view(shape)
    ws = filled((ep.workspace_bytes(T, K, E, P),), torch.uint8)
    lay = ep.Layout(filled((E,), torch.int32), filled((P,), torch.int32),
                    filled((T, P), torch.uint8), filled((E + 1,), torch.int32),
                    filled((P + 1,), torch.int32), ws)
    d = ep.Dispatched(filled((R, H), torch.uint8 if case.fp8 else torch.bfloat16),
                      filled((R, H // 128), torch.float32) if case.fp8 else None,
                      filled((R,), torch.int32), filled((T, K), torch.int32))
    out = filled((T, H), torch.bfloat16)
    ep.layout_dispatch(x, idx, E, P, workspace=ws, fp8=case.fp8, out_layout=lay, out=d)
    ep.combine(y, d.dst_row, w, out=out)
    torch.cuda.synchronize()
    res = {f: getattr(lay, f) for f in ("num_tokens_per_expert", "num_tokens_per_partition",
                                        "is_token_in_partition", "expert_offsets",
                                        "partition_offsets")}
    res.update(recv_x=d.recv_x, recv_src_token=d.recv_src_token, dst_row=d.dst_row, out=out)
    if case.fp8:
        res["recv_scales"] = d.recv_scales
    return res


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed", "coarse"])
def test_deterministic_across_runs_full_size(name):
    """Run the benchmark's step twice on the same inputs at the configuration's
    full size, each time into outputs pre-filled with a different byte, and
    compare every output bitwise: nothing depends on scheduling order, and
    nothing is left over from the first run."""
    case = wl.make(name)
    announce("determinism %s" % name)
    a = _step_outputs(case, 0xA5)
    b = _step_outputs(case, 0x5A)
    for k in a:
        ua = a[k].contiguous().view(torch.uint8)
        ub = b[k].contiguous().view(torch.uint8)
        assert torch.equal(ua, ub), "%s differs between two runs of %s" % (k, name)
        assert ua.numel() == 0 or not bool((ua == 0xA5).all()), k   # the run wrote it


def test_rows_past_the_valid_ones_are_untouched():
    """Receive rows >= N are not written (dispatch leaves them as they were)."""
    case = wl.random_case(400, 256, 16, 4, 4, 41, masked_frac=0.25)
    announce("untouched rows")
    idx = torch.from_numpy(case.topk_idx).cuda()
    x = torch.from_numpy(case.x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    lay = ep.get_dispatch_layout(idx, case.E, case.P)
    R = case.T * case.K
    out = ep.Dispatched(torch.full((R, case.H), 0x1234, dtype=torch.int16,
                                   device="cuda").view(torch.bfloat16),
                        None, torch.empty(R, dtype=torch.int32, device="cuda"),
                        torch.empty((case.T, case.K), dtype=torch.int32, device="cuda"))
    ep.dispatch(x, idx, case.E, case.P, lay.workspace, out=out)
    N = int(lay.expert_offsets[-1].item())
    assert N < R
    tail = out.recv_x[N:].view(torch.int16).cpu().numpy()
    assert (tail == 0x1234).all()
    assert (out.recv_src_token[N:].cpu().numpy() == -1).all()
