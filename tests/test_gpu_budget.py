"""The CU-budget entry points (GPU): ep_layout_dispatch_cu and ep_combine_cu
with at most num_cus workgroups looping over the work must give exactly the
results of the calls without a budget, i.e. the oracle's (bit-exact layout,
rows and scales; combine within 2 bf16 ulp).  Budgets from 1 CU to more than
the work, on the one-call path (count + layout-finishing dispatch) and on the
small-shape fallback (single-launch layout + plain dispatch), FP8 and bf16.
"""
import pytest

from combine_ep_get_dispatch_amd import workloads as wl
from parity import check_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("num_cus", [32, 100, 255])
def test_prefill_full_size(num_cus):
    case = wl.make("prefill")
    check_case(case, label="config prefill", one_call=True, num_cus=num_cus)


@pytest.mark.parametrize("num_cus", [1, 16])
def test_decode_fallback_path(num_cus):
    case = wl.make("decode")              # 2 token blocks or fewer: single-launch layout
    check_case(case, label="config decode", one_call=True, num_cus=num_cus)


BUDGET_CASES = [
    # T, H, E, P, K, seed, kwargs, num_cus
    (1000, 264, 16, 4, 3, 71, dict(), 3),
    (777, 1032, 64, 8, 6, 72, dict(masked_frac=0.1, invalid_frac=0.02), 7),
    (2500, 520, 8, 8, 2, 73, dict(skew=2.0), 64),
    (257, 2048, 128, 16, 16, 74, dict(fp8=True), 1),
    (9000, 128, 256, 64, 8, 75, dict(masked_frac=0.02), 200),
    (3000, 7168, 256, 64, 8, 76, dict(), 40),        # bf16 rows of the real width
    (50, 256, 16, 4, 2, 77, dict(), 1000),           # budget above the work: no budget
    (600, 17536, 64, 8, 8, 78, dict(fp8=True), 5),   # waves loop over 18 chunks
    (66, 18440, 32, 4, 6, 79, dict(), 3),            # the same on the plain dispatch
]


@pytest.mark.parametrize("T,H,E,P,K,seed,kw,num_cus", BUDGET_CASES,
                         ids=["T%d_H%d_K%d_cus%d" % (c[0], c[1], c[4], c[7]) for c in BUDGET_CASES])
def test_budget_case(T, H, E, P, K, seed, kw, num_cus):
    case = wl.random_case(T, H, E, P, K, seed, **kw)
    check_case(case, label="random seed=%d" % seed, one_call=True, num_cus=num_cus)
