"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case copies ``oracle/ep_oracle.c``, replaces one fragment with a plausible
slip (a wrong tie rule, index, order, term or sign), builds the copy with the
same flags into a temporary directory and, in a child process, routes the
``oracle`` module to it and runs the pins that cover that part.  At least one
pin must fail (a mutant that corrupts memory and crashes the child counts as
caught too).  The real oracle source is never modified.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ep_oracle.c")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

E4M3 = [lambda: pins.test_e4m3_golden_points(GOLDEN), pins.test_e4m3_dense_sweep_and_torch]
BF16 = [lambda: pins.test_bf16_golden_points(GOLDEN), pins.test_bf16_rne_against_torch]
LAYOUT = [lambda: pins.test_layout_hand_worked(GOLDEN),
          lambda: pins.test_layout_random_against_library_routines(1),
          lambda: pins.test_layout_random_against_library_routines(4),
          pins.test_layout_invalid_ids_are_masked_and_counted]
QUANT = [pins.test_quantize_matches_numpy_steps_and_invariants,
         pins.test_fp8_dispatch_rows_are_quantised_tokens]
# Non-finite tokens in the quantiser.
QUANT_NONFINITE = [lambda: pins.test_quantize_hand_worked_nonfinite_groups(GOLDEN),
                   pins.test_quantize_nonfinite_invariants]
# The quantiser's two divisions, pinned without the numpy restatement of its steps.
QUANT_EXACT = [lambda: pins.test_quantize_hand_worked_scale_groups(GOLDEN),
               pins.test_quantize_exact_rational]
COMBINE = [lambda: pins.test_combine_hand_worked(GOLDEN), pins.test_combine_exact_rational_small,
           pins.test_combine_closed_forms, pins.test_combine_identity_expert_and_fp64_bound,
           pins.test_combine_rounding_sensitive_cases]
DISPATCH = [pins.test_bf16_dispatch_rows_are_bitwise_copies,
            pins.test_fp8_dispatch_rows_are_quantised_tokens]
DEDUP = [lambda: pins.test_dedup_hand_worked(GOLDEN),
         lambda: pins.test_dedup_random_against_cumsum_and_invariants(1),
         lambda: pins.test_dedup_random_against_cumsum_and_invariants(4)]
ALIGNED = [lambda: pins.test_aligned_layout_hand_worked(GOLDEN),
           lambda: pins.test_aligned_layout_exhaustive_small(2, 2),
           lambda: pins.test_aligned_layout_random_against_library_routines(1),
           lambda: pins.test_aligned_layout_random_against_library_routines(4)]
LL = [lambda: pins.test_ll_layout_hand_worked(GOLDEN),
      lambda: pins.test_ll_layout_random_against_library_routines(1),
      lambda: pins.test_ll_layout_random_against_library_routines(4),
      pins.test_ll_layout_matches_offsets_layout_when_nothing_drops,
      pins.test_ll_dispatch_rows_are_copies_and_holes_untouched]

PERM_LOOP = """    for (int32_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int64_t v = idx[(int64_t)t * K + k];
            if (v >= 0 && v < E) {
                int32_t r"""
PERM_LOOP_SLOT_MAJOR = """    for (int32_t k = 0; k < K; ++k) {
        for (int32_t t = 0; t < T; ++t) {
            int64_t v = idx[(int64_t)t * K + k];
            if (v >= 0 && v < E) {
                int32_t r"""

# The row copies of the offsets-layout dispatch (the fixed-capacity dispatch
# has a hole test between these lines, so the anchors stay unique).
BF16_ROW_COPY = """        int64_t t = src[r];
        for (int64_t h = 0; h < H; ++h)
            recv_x[r * H + h] = x[t * H + h];"""
FP8_ROW_COPY = """        int64_t t = src[r];
        for (int64_t h = 0; h < H; ++h)
            recv_x[r * H + h] = q[t * H + h];
        for (int32_t g = 0; g < G; ++g)
            recv_scales[r * G + g] = s[t * G + g];"""

MUTANTS = [
    ("e4m3 ties away from zero", "double q = nearbyint(a / ldexp(1.0, E - 3));",
     "double q = round(a / ldexp(1.0, E - 3));", E4M3),
    ("e4m3 loses the sign of zero", "    if (a == 0.0)\n        return sign;",
     "    if (a == 0.0)\n        return 0;", E4M3),
    ("e4m3 wrong exponent bias", "code = ((E + 7) << 3) | ((int)q - 8);",
     "code = ((E + 8) << 3) | ((int)q - 8);", E4M3),
    ("e4m3 no subnormal range", "    if (E < -6)\n        E = -6;",
     "    if (E < -9)\n        E = -9;", E4M3),
    ("bf16 ties always up", "mag = (lo & 1u) ? hi : lo;", "mag = hi;", BF16),
    ("bf16 truncates", "if (dlo < dhi)\n        mag = lo;", "if (1)\n        mag = lo;", BF16),
    ("partition map by modulo", "in_part[(int64_t)t * P + v / Ep] = 1;",
     "in_part[(int64_t)t * P + v % P] = 1;", LAYOUT),
    ("partition offsets indexed by partition", "off_p[p] = off_e[p * Ep];",
     "off_p[p] = off_e[p];", LAYOUT),
    ("invalid ids not masked", "if (v >= 0 && v < E) {\n                cnt_e[v] += 1;",
     "if (v >= 0) {\n                cnt_e[v % E] += 1;", LAYOUT),
    ("offsets inclusive", "off_e[e + 1] = off_e[e] + cnt_e[e];",
     "off_e[e + 1] = off_e[e] + cnt_e[e] + (e == 0 ? cnt_e[0] : 0);", LAYOUT),
    ("permutation ordered slot-major", PERM_LOOP, PERM_LOOP_SLOT_MAJOR, LAYOUT),
    ("unused rows not marked", "        src[r] = -1;\n    free(next);", "    free(next);", LAYOUT),
    ("scale inverted", "s[t * G + g] = ac / 448.0f;", "s[t * G + g] = 448.0f / ac;", QUANT),
    ("quantiser multiplies by a reciprocal", "float inv = 448.0f / ac;",
     "float inv = 448.0f * (1.0f / ac);", QUANT_EXACT),
    ("scale multiplies by a reciprocal", "s[t * G + g] = ac / 448.0f;",
     "s[t * G + g] = ac * (1.0f / 448.0f);", QUANT_EXACT),
    ("non-finite codes lose the sign of x", "q[t * H + 128 * g + j] = signbit(xv) ? 0xFFu : 0x7Fu;",
     "q[t * H + 128 * g + j] = 0x7Fu;", QUANT_NONFINITE),
    ("NaN taken into the maximum", "                if (v > a)\n                    a = v;",
     "                if (v > a || isnan(v))\n                    a = v;", QUANT_NONFINITE),
    ("non-finite x encoded from the product", "                if (isnan(xv) || isinf(xv))",
     "                if (isnan(xv))", QUANT_NONFINITE),
    ("amax floor dropped", "float ac = (a > 1e-4f) ? a : 1e-4f;", "float ac = a;", QUANT),
    ("amax without abs", "float v = fabsf(bf16_to_f32(x[t * H + 128 * g + j]));",
     "float v = bf16_to_f32(x[t * H + 128 * g + j]);", QUANT),
    ("fp8 dispatch copies the wrong scale", FP8_ROW_COPY,
     FP8_ROW_COPY.replace("= s[t * G + g];", "= s[r % 1 * G + g];"), DISPATCH),
    ("bf16 dispatch copies by row index", BF16_ROW_COPY,
     BF16_ROW_COPY.replace("= x[t * H + h];", "= x[(r % T) * H + h];"), DISPATCH),
    ("combine ignores weights", "acc = fmaf(w[t * K + k], bf16_to_f32(y[r * H + h]), acc);",
     "acc = acc + bf16_to_f32(y[r * H + h]);", COMBINE),
    ("combine unfused", "acc = fmaf(w[t * K + k], bf16_to_f32(y[r * H + h]), acc);",
     "acc = w[t * K + k] * bf16_to_f32(y[r * H + h]) + acc;", COMBINE),
    ("combine reversed slot order", "for (int32_t k = 0; k < K; ++k) {\n                int64_t r = dst",
     "for (int32_t k = K - 1; k >= 0; --k) {\n                int64_t r = dst", COMBINE),
    ("combine truncates to bf16", "out[t * H + h] = oracle_bf16_rne(acc);",
     "{ uint32_t u_; memcpy(&u_, &acc, 4); out[t * H + h] = (uint16_t)(u_ >> 16); }", COMBINE),
    ("combine weight of the wrong slot", "acc = fmaf(w[t * K + k],",
     "acc = fmaf(w[t * K + (K - 1 - k)],", COMBINE),
    ("dedup offsets inclusive", "ptok_off[p + 1] = ptok_off[p] + cnt_p[p];",
     "ptok_off[p + 1] = ptok_off[p] + cnt_p[p] + (p == 0);", DEDUP),
    ("dedup partition by modulo", "if (v >= 0 && v < E && v / Ep == p)\n                    member = 1;",
     "if (v >= 0 && v < E && v % P == p)\n                    member = 1;", DEDUP),
    ("dedup global expert ids", "dd_idx[(int64_t)r * K + k] = (int32_t)(v - (int64_t)p * Ep);",
     "dd_idx[(int64_t)r * K + k] = (int32_t)v;", DEDUP),
    ("dedup slot map from the slot's token row in partition 0",
     "slot_src[r] = dd_row[(int64_t)t * P + v / Ep];", "slot_src[r] = dd_row[(int64_t)t * P + 0];", DEDUP),
    ("dedup unused rows keep a token", "    for (int64_t r = 0; r < RD; ++r) {\n        dd_src[r] = -1;",
     "    for (int64_t r = 0; r < RD; ++r) {\n        dd_src[r] = 0;", DEDUP),
    ("ll capacity off by one", "if (rank < C) {", "if (rank <= C) {", LL),
    ("ll rows strided by top-k", "row = (int32_t)v * C + rank;",
     "row = (int32_t)v * K + rank;", LL),
    ("ll count stops at capacity", "                cnt_e[v] += 1;\n                if (rank < C) {",
     "                if (rank < C) {\n                    cnt_e[v] += 1;", LL),
    ("ll holes not marked", "    for (int64_t r = 0; r < (int64_t)E * C; ++r)\n        src[r] = -1;\n", "", LL),
    ("ll dispatch fills holes",
     "if (t < 0)\n            continue;\n        for (int64_t h = 0; h < H; ++h)\n"
     "            recv_x[r * H + h] = x[t * H + h];",
     "if (t < 0)\n            t = 0;\n        for (int64_t h = 0; h < H; ++h)\n"
     "            recv_x[r * H + h] = x[t * H + h];", LL),
    ("aligned runs rounded down", "run += (cnt_e[e] + align - 1) / align * align;",
     "run += cnt_e[e] / align * align;", ALIGNED),
    ("aligned runs not padded", "run += (cnt_e[e] + align - 1) / align * align;",
     "run += cnt_e[e];", ALIGNED),
    ("aligned partition offsets left unpadded",
     "    off_e[E] = run;\n    for (int32_t p = 0; p <= P; ++p)\n        off_p[p] = off_e[Ep * p];\n",
     "    off_e[E] = run;\n", ALIGNED),
    ("aligned padding rows not marked", "    for (int64_t r = 0; r < R; ++r)\n        src[r] = -1;\n",
     "", ALIGNED),
    ("aligned source token from the slot index", "src[dst[i]] = (int32_t)(i / K);",
     "src[dst[i]] = (int32_t)(i % K);", ALIGNED),
]


GROUPS = {"E4M3": E4M3, "BF16": BF16, "LAYOUT": LAYOUT, "QUANT": QUANT, "QUANT_EXACT": QUANT_EXACT,
          "QUANT_NONFINITE": QUANT_NONFINITE,
          "COMBINE": COMBINE, "DISPATCH": DISPATCH, "LL": LL, "DEDUP": DEDUP,
          "ALIGNED": ALIGNED}


def _group_name(checks):
    return next(k for k, v in GROUPS.items() if v is checks)


def run_checks(lib_path, group):
    """Child-process entry: run one group of pins against ``lib_path``;
    print the number that failed."""
    oracle.use_library(lib_path)
    failures = 0
    with np.errstate(all="ignore"):
        for check in GROUPS[group]:
            try:
                check()
            except AssertionError:
                failures += 1
    print("FAILURES", failures)


@pytest.fixture(scope="module")
def source():
    return open(SRC).read()


@pytest.mark.parametrize("name,old,new,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, checks, source, tmp_path):
    assert source.count(old) == 1, "mutation anchor not found exactly once: %r" % old
    csrc = tmp_path / "ep_oracle_mutant.c"
    csrc.write_text(source.replace(old, new))
    lib = tmp_path / "libep_oracle_mutant.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(csrc), "-o", str(lib), "-lm"])
    here = os.path.dirname(os.path.abspath(__file__))
    code = ("import sys; sys.path[:0] = [%r, %r]; import test_oracle_mutants as m; "
            "m.run_checks(%r, %r)" % (here, os.path.dirname(here), str(lib), _group_name(checks)))
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=600)
    if proc.returncode != 0:
        return                       # the mutant crashed or raised: caught
    line = [ln for ln in proc.stdout.splitlines() if ln.startswith("FAILURES")][-1]
    assert int(line.split()[1]) > 0, "no pin caught the planted mistake: " + name
