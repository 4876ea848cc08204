"""The tiled combine (top-8 batches large enough to give every CU two tiles:
workgroups own tiles of consecutive tokens, stage the tile's outputs in LDS
and write them as one burst) against the oracle's combine, element by
element (the same fp32 FMA order in slot order, so bitwise in practice; the
bar is the parity bar of 2 bf16 ulp), and bitwise against the
one-wave-per-task form on the same inputs (ep_combine_cu with a CU budget,
which never tiles).  The shapes cover ragged tail tiles, channel counts that
are not a multiple of the 512-channel chunk, masked slots and rows past the
end of y (skipped like masked ones), a tile size limited by the LDS budget,
the batch sizes on both sides of where tiles start, and other top-k values,
which keep one wave per task.  The combine is the second half of the
all-to-all in "DeepSeek releases DeepEP, an efficient communication library
for MoE models", section "DeepEP: Optimizing MoE Communication".
"""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_get_dispatch_amd import binding as ep
from combine_ep_get_dispatch_amd import workloads as wl
from parity import MAX_COMBINE_ULP, announce, bf16_bits, to_dev_bf16, ulp_distance

pytestmark = pytest.mark.gpu

TILE_LDS = 112 * 1024          # bytes of one tile's outputs
TILE_MIN_BLOCKS = 512          # tiles only while T / tile >= this


def expected_tile(T, H, K):
    """The tile size the library picks (0: one wave per task)."""
    if K != 8:
        return 0
    tile = min(TILE_LDS // (2 * H), 64 // K, T // TILE_MIN_BLOCKS)
    return tile if tile >= 2 else 0


CASES = [
    # T, H, K, R, seed, masked_frac, past_frac
    (4101, 7168, 8, 4101 * 8, 301, 0.0, 0.0),      # tile 8, tail tile of 5
    (1029, 520, 8, 3000, 302, 0.05, 0.02),         # tile 2, tail of 1, ragged chunks
    (2055, 4096, 8, 5000, 303, 0.1, 0.05),         # tile 4, tail of 3
    (2000, 18440, 8, 4000, 306, 0.0, 0.0),         # tile 3, limited by LDS, tail of 2
    (1024, 7168, 8, 8192, 307, 0.0, 0.0),          # T / 512 = 2: the smallest tiles
    (1023, 7168, 8, 8184, 308, 0.0, 0.0),          # one token fewer: no tiles
    (8192, 136, 8, 8192 * 8, 309, 0.3, 0.0),       # many masked slots, tile 8
    (4096, 1024, 6, 9000, 305, 0.02, 0.01),        # other top-k: one wave per task
    (4096, 256, 2, 4096, 304, 0.0, 0.0),
]


@pytest.mark.parametrize("T,H,K,R,seed,masked,past", CASES,
                         ids=["T%d_H%d_K%d" % c[:3] for c in CASES])
def test_tiled_combine(T, H, K, R, seed, masked, past):
    announce("tiled combine T=%d H=%d K=%d tile=%d" % (T, H, K, expected_tile(T, H, K)))
    y_bits, dst, w = wl.combine_inputs(T, H, K, R, seed, masked_frac=masked, past_frac=past)
    y = to_dev_bf16(y_bits)
    d_dst = torch.from_numpy(dst).cuda()
    d_w = torch.from_numpy(w).cuda()
    got = bf16_bits(ep.combine(y, d_dst, d_w))
    per_task = bf16_bits(ep.combine(y, d_dst, d_w, num_cus=64))
    torch.cuda.synchronize()
    ref = oracle.combine(y_bits, np.where(dst >= R, -1, dst).astype(np.int32), w)
    u = ulp_distance(got, ref)
    assert int(u.max(initial=0)) <= MAX_COMBINE_ULP, (int(u.max()), int((u > 0).sum()))
    assert np.array_equal(got, per_task)


def test_tiled_combine_leaves_other_tokens_alone():
    """A tiled combine writes exactly out[0:T]: the rows of a larger out
    buffer past T keep their bytes."""
    T, H, K, R = 2050, 1024, 8, 9000        # tile 4, tail of 2
    y_bits, dst, w = wl.combine_inputs(T, H, K, R, 310)
    big = torch.full((T + 5, H), 1.5, dtype=torch.bfloat16, device="cuda")
    out = big[:T]
    ep.combine(to_dev_bf16(y_bits), torch.from_numpy(dst).cuda(), torch.from_numpy(w).cuda(),
               out=out)
    torch.cuda.synchronize()
    assert torch.equal(big[T:], torch.full((5, H), 1.5, dtype=torch.bfloat16, device="cuda"))
    ref = oracle.combine(y_bits, dst, w)
    assert int(ulp_distance(bf16_bits(out), ref).max(initial=0)) <= MAX_COMBINE_ULP
