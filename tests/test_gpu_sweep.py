"""Seeded randomized parity sweep over shapes and every path (GPU).

24 shapes drawn from a fixed generator -- ragged T and H, every kind of E, P
and K combination the limits allow, masked, invalid and repeated ids, skewed
routing, bf16 and FP8 -- each run through the two-call path, the one-call
path, the one-call path under a random CU budget, the de-duplicated path, the aligned path
with a random alignment and (when T*K allows) the fixed-capacity decode
path, and compared with the
oracle to the usual bars (bit-exact layout, rows and scales; combine within
2 bf16 ulp).  Six more draws are top-8 batches of 1024 to 5000 tokens with
ragged widths, where combine runs in tiles of consecutive tokens, through
the two-call, one-call and de-duplicated paths.  The draws are fixed by the
seed, so a failure names a reproducible case.
"""
import numpy as np
import pytest

from combine_ep_get_dispatch_amd import workloads as wl
from parity import check_case
from test_gpu_aligned import check_aligned
from test_gpu_dedup import check_dedup
from test_gpu_low_latency import check_ll

pytestmark = pytest.mark.gpu


def _draw(i):
    rng = np.random.default_rng(9000 + i)
    E = int(rng.choice([1, 2, 3, 8, 12, 32, 64, 96, 256, 512, 1024]))
    divisors = [d for d in range(1, E + 1) if E % d == 0]
    P = int(rng.choice(divisors))
    K = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.integers(1, 3000))
    fp8 = bool(rng.integers(0, 2))
    H = int(rng.choice([128, 256, 384, 1152, 2048, 3200])) if fp8 else \
        int(rng.choice([8, 72, 264, 520, 1024, 1544, 2056]))
    kw = dict(masked_frac=float(rng.choice([0.0, 0.0, 0.05, 0.3])),
              invalid_frac=float(rng.choice([0.0, 0.0, 0.02])),
              allow_dup=bool(rng.integers(0, 2)), skew=float(rng.choice([0.0, 1.0, 3.0])),
              fp8=fp8)
    budget = int(rng.choice([1, 5, 64, 200]))
    align = int(rng.choice([1, 2, 3, 16, 64, 128, 1000]))
    return T, H, E, P, K, 9100 + i, kw, budget, align


SWEEP = [_draw(i) for i in range(24)]


@pytest.mark.parametrize("T,H,E,P,K,seed,kw,budget,align", SWEEP,
                         ids=["s%d_T%d_H%d_E%d_P%d_K%d" % ((i,) + c[:5]) for i, c in enumerate(SWEEP)])
def test_sweep(T, H, E, P, K, seed, kw, budget, align):
    case = wl.random_case(T, H, E, P, K, seed, **kw)
    label = "sweep seed=%d" % seed
    check_case(case, label=label)
    check_case(case, label=label, one_call=True)
    check_case(case, label=label, one_call=True, num_cus=budget)
    check_dedup(case, label)
    check_aligned(case, align, label, y_seed=seed + 2)
    if T * K <= 8192:
        check_ll(case.topk_idx, case.x_bits, case.topk_weights, E, max(1, T // 3), case.fp8,
                 label, y_seed=seed + 1)


def _draw_top8(i):
    rng = np.random.default_rng(9500 + i)
    E = int(rng.choice([8, 32, 64, 256]))
    divisors = [d for d in range(1, E + 1) if E % d == 0]
    P = int(rng.choice(divisors))
    T = int(rng.integers(1024, 5000))
    fp8 = bool(rng.integers(0, 2))
    H = int(rng.choice([640, 1152, 3200, 7168])) if fp8 else \
        int(rng.choice([136, 520, 1032, 4104]))
    kw = dict(masked_frac=float(rng.choice([0.0, 0.05, 0.3])),
              invalid_frac=float(rng.choice([0.0, 0.02])),
              allow_dup=bool(rng.integers(0, 2)), skew=float(rng.choice([0.0, 1.0, 3.0])),
              fp8=fp8)
    return T, H, E, P, 8, 9600 + i, kw


SWEEP_TOP8 = [_draw_top8(i) for i in range(6)]


@pytest.mark.parametrize("T,H,E,P,K,seed,kw", SWEEP_TOP8,
                         ids=["t%d_T%d_H%d_E%d_P%d" % ((i,) + c[:4]) for i, c in enumerate(SWEEP_TOP8)])
def test_sweep_top8_batches(T, H, E, P, K, seed, kw):
    """Top-8 batches of 1024 tokens or more, where combine runs in tiles of
    consecutive tokens (ragged tails, ragged widths): the two-call, one-call
    and de-duplicated paths against the oracle."""
    case = wl.random_case(T, H, E, P, K, seed, **kw)
    label = "top-8 sweep seed=%d" % seed
    check_case(case, label=label)
    check_case(case, label=label, one_call=True)
    check_dedup(case, label)
