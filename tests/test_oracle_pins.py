"""Pins of the CPU oracle against things other than itself (CPU only).

* hand-worked fixtures under tests/golden/ (format definitions, a worked layout
  and combine example);
* exhaustive search over the 256 E4M3 codes for every bf16 pattern and a dense
  fp32 sweep, plus torch's CPU float8_e4m3fn cast in range;
* torch's CPU bf16 cast for the bf16 rounding;
* library routines (stable argsort, bincount, cumsum) and pairwise brute force
  for the layout and permutation, exhaustively over every routing tensor with
  T*K <= 6 and ids in {-1, 0..3};
* invariants of the quantiser and exact rational arithmetic / closed forms for
  combine.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import bruteforce as bf
from combine_ep_get_dispatch_amd import workloads as wl


def _read_kv(path):
    out = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, *v = line.split()
        out[k] = v
    return out


def _read_points(path):
    rows = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        rows.append((float(parts[0]), int(parts[1], 16)))
    return rows


# ---------------------------------------------------------------------------
# scalar formats
# ---------------------------------------------------------------------------

def test_e4m3_golden_points(golden_dir):
    pts = _read_points(os.path.join(golden_dir, "e4m3_points.txt"))
    v = np.array([p[0] for p in pts], np.float32)
    want = np.array([p[1] for p in pts], np.uint8)
    np.testing.assert_array_equal(oracle.e4m3(v), want)
    np.testing.assert_array_equal(bf.e4m3_nearest(v), want)


def test_e4m3_all_bf16_patterns_times_scales():
    """Every finite bf16 value, times a set of scales, encoded by the oracle
    equals the exhaustive nearest-code search."""
    bits = np.arange(65536, dtype=np.uint32)
    vals = ((bits << 16).view(np.float32))
    vals = vals[np.isfinite(vals)]
    for mult in [1.0, 0.5, 3.0, 448.0 / 3.1, 1.0 / 7.0, 2.0 ** -8, 1.37e-3]:
        with np.errstate(over="ignore"):
            v = (vals * np.float32(mult)).astype(np.float32)
        v = v[np.isfinite(v)]
        np.testing.assert_array_equal(oracle.e4m3(v), bf.e4m3_nearest(v), err_msg=str(mult))


def test_e4m3_dense_sweep_and_torch():
    v = np.linspace(-464.0, 464.0, 400_001, dtype=np.float64).astype(np.float32)
    # add every midpoint between neighbouring codes and one fp32 step either side
    mags = bf.e4m3_decode_table()[:0x7F]
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(1000))])
    v = np.concatenate([v, near, -near])
    got = oracle.e4m3(v)
    np.testing.assert_array_equal(got, bf.e4m3_nearest(v))
    # torch's cast is round-to-nearest-even in range (it gives NaN beyond 464)
    inr = np.abs(v) <= 448
    t = torch.from_numpy(v[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got[inr], t)


def test_bf16_golden_points(golden_dir):
    pts = _read_points(os.path.join(golden_dir, "bf16_points.txt"))
    v = np.array([p[0] for p in pts], np.float32)
    want = np.array([p[1] for p in pts], np.uint16)
    np.testing.assert_array_equal(oracle.bf16_rne(v), want)


def test_bf16_rne_against_torch():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    v = v[np.isfinite(v)]
    # exact ties: a bf16 value plus half its step
    b = rng.integers(0, 0x7F7F, size=100_000).astype(np.uint32) << 16
    ties = (b | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties, np.float32([0.0, -0.0, 1e-45, -1e-45])])
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.bf16_rne(v), want)


# ---------------------------------------------------------------------------
# layout and permutation
# ---------------------------------------------------------------------------

def _check_against_bruteforce(idx, E, P):
    got = oracle.layout(idx, E, P)
    want = bf.layout(idx, E, P)
    for k in want:
        np.testing.assert_array_equal(np.asarray(got[k]), np.asarray(want[k]), err_msg=k)
    dst, src = oracle.permutation(idx, E, got["expert_offsets"])
    bdst, bsrc = bf.permutation(idx, E)
    np.testing.assert_array_equal(dst, bdst)
    np.testing.assert_array_equal(src, bsrc)
    return got, dst, src


def test_layout_hand_worked(golden_dir):
    g = _read_kv(os.path.join(golden_dir, "layout_hand_worked.txt"))
    T, K, E, P = (int(g[k][0]) for k in "TKEP")
    idx = np.array(g["topk_idx"], np.int64).reshape(T, K)
    lay = oracle.layout(idx, E, P)
    for key in ["num_tokens_per_expert", "expert_offsets", "num_tokens_per_partition",
                "partition_offsets"]:
        np.testing.assert_array_equal(lay[key], np.array(g[key], np.int32), err_msg=key)
    np.testing.assert_array_equal(lay["is_token_in_partition"].reshape(-1),
                                  np.array(g["is_token_in_partition"], np.uint8))
    dst, src = oracle.permutation(idx, E, lay["expert_offsets"])
    np.testing.assert_array_equal(dst.reshape(-1), np.array(g["dst_row"], np.int32))
    np.testing.assert_array_equal(src, np.array(g["recv_src_token"], np.int32))


def test_combine_hand_worked(golden_dir):
    g = _read_kv(os.path.join(golden_dir, "layout_hand_worked.txt"))
    T, K, H = int(g["T"][0]), int(g["K"][0]), int(g["H"][0])
    dst = np.array(g["dst_row"], np.int32).reshape(T, K)
    w = np.array(g["topk_weights"], np.float32).reshape(T, K)
    y = np.array([int(b, 16) for b in g["y_bits_hex"]], np.uint16).reshape(-1, H)
    want = np.array([int(b, 16) for b in g["out_bits_hex"]], np.uint16).reshape(T, H)
    np.testing.assert_array_equal(oracle.combine(y, dst, w), want)


@pytest.mark.parametrize("T,K", [(1, 6), (2, 3), (3, 2), (6, 1), (2, 2), (1, 1)])
def test_layout_exhaustive_small(T, K):
    """Every routing tensor of this shape with ids in {-1, 0, 1, 2, 3} (masked
    slots and repeated experts included), E = 4, P in {1, 2, 4}."""
    E = 4
    n = T * K
    grid = np.array(np.meshgrid(*[np.arange(-1, E)] * n, indexing="ij")).reshape(n, -1).T
    batch = grid.reshape(-1, T, K).astype(np.int64)
    dst_ref = None
    for P in (1, 2, 4):
        cnt_e, in_part, off_e, dst_b, nerr = bf.layout_batch(batch, E, P)
        for i in range(batch.shape[0]):
            got = oracle.layout(batch[i], E, P)
            assert np.array_equal(got["num_tokens_per_expert"], cnt_e[i])
            assert np.array_equal(got["is_token_in_partition"], in_part[i])
            assert np.array_equal(got["expert_offsets"], off_e[i])
            assert np.array_equal(got["num_tokens_per_partition"], in_part[i].sum(axis=0))
            assert np.array_equal(got["partition_offsets"], off_e[i][np.arange(P + 1) * (E // P)])
            assert got["num_invalid"] == 0 == nerr[i]
            if P == 1:
                dst, src = oracle.permutation(batch[i], E, got["expert_offsets"])
                assert np.array_equal(dst, dst_b[i]), (batch[i], dst, dst_b[i])
                N = off_e[i][E]
                # src is the inverse of dst on [0, N), and -1 beyond
                inv = np.full(T * K, -1, np.int32)
                for t in range(T):
                    for k in range(K):
                        if dst[t, k] >= 0:
                            inv[dst[t, k]] = t
                assert np.array_equal(src, inv) and (src[N:] == -1).all()


@pytest.mark.parametrize("seed", range(12))
def test_layout_random_against_library_routines(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    P = int(rng.choice([d for d in (1, 2, 4, 8, 16, 32) if E % d == 0]))
    K = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(0, 300))
    c = wl.random_case(T, 8, E, P, K, seed, masked_frac=0.1 * (seed % 3),
                       allow_dup=bool(seed % 2), skew=float(seed % 4), with_y=False)
    got, dst, src = _check_against_bruteforce(c.topk_idx, E, P)
    N = got["expert_offsets"][E]
    # invariants: bijection of valid slots onto [0, N), segment membership, order
    valid = dst >= 0
    assert sorted(dst[valid].tolist()) == list(range(N))
    assert np.all(src[dst[valid]] == np.nonzero(valid)[0])
    for e in range(E):
        seg = src[got["expert_offsets"][e]:got["expert_offsets"][e + 1]]
        assert np.all(np.diff(seg) >= 0)
    Tn = T
    assert Tn <= got["num_tokens_per_partition"].sum() + (~valid.any(axis=1)).sum() or T == 0
    assert got["num_tokens_per_partition"].sum() <= T * min(K, P)


def test_layout_invalid_ids_are_masked_and_counted():
    c = wl.random_case(200, 8, 32, 8, 4, 5, masked_frac=0.1, invalid_frac=0.1, with_y=False)
    got, dst, src = _check_against_bruteforce(c.topk_idx, 32, 8)
    bad = (c.topk_idx != -1) & ((c.topk_idx < 0) | (c.topk_idx >= 32))
    assert got["num_invalid"] == int(bad.sum()) > 0
    assert np.all(dst[bad] == -1) and np.all(dst[c.topk_idx == -1] == -1)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed", "coarse"])
def test_layout_of_each_configuration(name):
    cfg = wl.CONFIGS[name]
    idx, w, meta = wl.route(cfg)
    assert idx.shape == (cfg["T"], cfg["K"])
    got, dst, src = _check_against_bruteforce(idx, cfg["E"], cfg["P"])
    assert got["expert_offsets"][-1] == cfg["T"] * cfg["K"]          # every slot valid
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    if name == "prefill":
        assert meta["groups_per_token_max"] <= cfg["topk_groups"]
    if name == "skewed":
        assert meta["max_over_mean_load"] >= 10.0


# ---------------------------------------------------------------------------
# fixed-capacity (decode) layout
# ---------------------------------------------------------------------------

def test_ll_layout_hand_worked(golden_dir):
    g = _read_kv(os.path.join(golden_dir, "ll_layout_hand_worked.txt"))
    T, K, E = (int(g[k][0]) for k in "TKE")
    idx = np.array(g["topk_idx"], np.int64).reshape(T, K)
    for C in (1, 2):
        got = oracle.ll_layout(idx, E, C)
        np.testing.assert_array_equal(got["num_tokens_per_expert"],
                                      np.array(g["num_tokens_per_expert"], np.int32))
        np.testing.assert_array_equal(got["dst_row"].reshape(-1),
                                      np.array(g["C%d_dst_row" % C], np.int32))
        np.testing.assert_array_equal(got["recv_src_token"],
                                      np.array(g["C%d_recv_src_token" % C], np.int32))
        assert got["num_invalid"] == 0


@pytest.mark.parametrize("T,K", [(1, 5), (2, 2), (3, 2), (5, 1), (1, 1)])
def test_ll_layout_exhaustive_small(T, K):
    """Every routing tensor of this shape with ids in {-1, 0, 1, 2} (masked
    slots and repeated experts included), E = 3, capacities 1..3, against
    ranks from direct pairwise comparison."""
    E = 3
    n = T * K
    grid = np.array(np.meshgrid(*[np.arange(-1, E)] * n, indexing="ij")).reshape(n, -1).T
    batch = grid.reshape(-1, T, K).astype(np.int64)
    rank = bf.ll_rank_batch(batch, E)
    for C in (1, 2, 3):
        want_dst = np.where((rank >= 0) & (rank < C), batch * C + rank, -1)
        for i in range(batch.shape[0]):
            got = oracle.ll_layout(batch[i], E, C)
            assert np.array_equal(got["dst_row"], want_dst[i]), (batch[i], C)
            cnt = np.bincount(batch[i][batch[i] >= 0], minlength=E)
            assert np.array_equal(got["num_tokens_per_expert"], cnt)
            src = np.full(E * C, -1, np.int32)
            for t in range(T):
                for k in range(K):
                    if want_dst[i, t, k] >= 0:
                        src[want_dst[i, t, k]] = t
            assert np.array_equal(got["recv_src_token"], src)


@pytest.mark.parametrize("seed", range(10))
def test_ll_layout_random_against_library_routines(seed):
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 256]))
    K = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(0, 300))
    c = wl.random_case(T, 8, E, 1, K, seed, masked_frac=0.1 * (seed % 3),
                       invalid_frac=0.05 * (seed % 2), allow_dup=bool(seed % 2),
                       skew=float(seed % 4), with_y=False)
    cnt = np.bincount(c.topk_idx[(c.topk_idx >= 0) & (c.topk_idx < E)], minlength=E)
    for C in {1, max(1, int(cnt.max(initial=0)) // 2), max(1, int(cnt.max(initial=0))), T + 1}:
        got = oracle.ll_layout(c.topk_idx, E, C)
        want = bf.ll_layout(c.topk_idx, E, C)
        for k in want:
            np.testing.assert_array_equal(np.asarray(got[k]), np.asarray(want[k]), err_msg=k)
        # invariants: expert e's kept slots fill rows e*C .. e*C + min(cnt, C) - 1
        dst = got["dst_row"]
        kept = dst >= 0
        assert int(kept.sum()) == int(np.minimum(cnt, C).sum())
        filled = got["recv_src_token"].reshape(E, C) >= 0
        assert np.array_equal(filled.sum(axis=1), np.minimum(cnt, C))
        assert np.all(filled == (np.arange(C)[None, :] < np.minimum(cnt, C)[:, None]))
        assert np.all(dst[kept] // C == c.topk_idx[kept])


def test_ll_layout_matches_offsets_layout_when_nothing_drops():
    """With capacity >= every expert's count, a slot's row inside its expert
    is the same in both layouts."""
    c = wl.random_case(257, 8, 64, 8, 6, 21, masked_frac=0.1, invalid_frac=0.02,
                       allow_dup=True, skew=2.0, with_y=False)
    lay = oracle.layout(c.topk_idx, 64, 8)
    dst, _ = oracle.permutation(c.topk_idx, 64, lay["expert_offsets"])
    C = int(lay["num_tokens_per_expert"].max())
    ll = oracle.ll_layout(c.topk_idx, 64, C)
    assert ll["num_invalid"] == lay["num_invalid"] > 0
    np.testing.assert_array_equal(ll["num_tokens_per_expert"], lay["num_tokens_per_expert"])
    valid = dst >= 0
    e = c.topk_idx[valid]
    np.testing.assert_array_equal(ll["dst_row"][valid] - e * C,
                                  dst[valid] - lay["expert_offsets"][e])
    assert np.all(ll["dst_row"][~valid] == -1)


def test_ll_dispatch_rows_are_copies_and_holes_untouched():
    c = wl.random_case(60, 256, 16, 4, 4, 23, masked_frac=0.1, allow_dup=True)
    res_b = oracle.run_ll(c.topk_idx, c.x_bits, 16, 16, fp8=False)
    src = res_b["recv_src_token"]
    rx = oracle.dispatch_rows_bf16(c.x_bits, src, fill=0xABCD)
    rq, rs = oracle.dispatch_rows_fp8(c.x_bits, src, fill=0x5A)
    q, s = oracle.quantize(c.x_bits)
    hole = src < 0
    assert hole.any() and (~hole).any()
    assert np.all(rx[hole] == 0xABCD) and np.all(rq[hole] == 0x5A) and np.all(rs[hole] == 0)
    np.testing.assert_array_equal(rx[~hole], c.x_bits[src[~hole]])
    np.testing.assert_array_equal(rq[~hole], q[src[~hole]])
    np.testing.assert_array_equal(rs[~hole], s[src[~hole]])
    np.testing.assert_array_equal(res_b["recv_x"][~hole], rx[~hole])


# ---------------------------------------------------------------------------
# expert runs aligned for grouped GEMMs
# ---------------------------------------------------------------------------

def test_aligned_layout_hand_worked(golden_dir):
    g = _read_kv(os.path.join(golden_dir, "aligned_layout_hand_worked.txt"))
    T, K, E, P = (int(g[k][0]) for k in "TKEP")
    idx = np.array(g["topk_idx"], np.int64).reshape(T, K)
    for align in (1, 3):
        got = oracle.aligned_layout(idx, E, P, align)
        for key in ["num_tokens_per_expert", "num_tokens_per_partition", "is_token_in_partition"]:
            np.testing.assert_array_equal(np.asarray(got[key]).reshape(-1),
                                          np.array(g[key], np.int64), err_msg=key)
        for key in ["expert_offsets", "partition_offsets", "dst_row", "recv_src_token"]:
            np.testing.assert_array_equal(np.asarray(got[key]).reshape(-1),
                                          np.array(g["A%d_%s" % (align, key)], np.int32),
                                          err_msg="%s align=%d" % (key, align))
        assert got["num_invalid"] == int(g["num_invalid"][0])


@pytest.mark.parametrize("T,K", [(1, 4), (2, 2), (4, 1), (1, 3)])
def test_aligned_layout_exhaustive_small(T, K):
    """Every routing tensor of this shape with ids in {-1, 0, 1, 2, 3} (masked
    slots and repeated experts included), E = 4, P in {1, 2, 4}, alignments
    1..3, against ranks from direct pairwise comparison and runs from the
    counts rounded up by hand."""
    E = 4
    n = T * K
    grid = np.array(np.meshgrid(*[np.arange(-1, E)] * n, indexing="ij")).reshape(n, -1).T
    batch = grid.reshape(-1, T, K).astype(np.int64)
    rank = bf.ll_rank_batch(batch, E)
    for P in (1, 2, 4):
        for align in (1, 2, 3):
            for i in range(batch.shape[0]):
                idx = batch[i]
                got = oracle.aligned_layout(idx, E, P, align)
                cnt = np.bincount(idx[idx >= 0], minlength=E)
                off = [0]
                for e in range(E):
                    off.append(off[-1] + (cnt[e] + align - 1) // align * align)
                off = np.array(off)
                want_dst = np.where(idx >= 0, off[np.maximum(idx, 0)] + rank[i], -1)
                assert np.array_equal(got["expert_offsets"], off), (idx, P, align)
                assert np.array_equal(got["partition_offsets"], off[np.arange(P + 1) * (E // P)])
                assert np.array_equal(got["dst_row"], want_dst), (idx, P, align)
                src = np.full(n + E * (align - 1), -1, np.int32)
                for t in range(T):
                    for k in range(K):
                        if want_dst[t, k] >= 0:
                            src[want_dst[t, k]] = t
                assert np.array_equal(got["recv_src_token"], src), (idx, P, align)


@pytest.mark.parametrize("seed", range(10))
def test_aligned_layout_random_against_library_routines(seed):
    rng = np.random.default_rng(1500 + seed)
    E = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 256]))
    P = int(rng.choice([d for d in (1, 2, 4, 8) if E % d == 0]))
    K = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(0, 300))
    c = wl.random_case(T, 8, E, P, K, seed, masked_frac=0.1 * (seed % 3),
                       invalid_frac=0.05 * (seed % 2), allow_dup=bool(seed % 2),
                       skew=float(seed % 4), with_y=False)
    for align in (1, 2, 3, 64, 128):
        got = oracle.aligned_layout(c.topk_idx, E, P, align)
        want = bf.aligned_layout(c.topk_idx, E, P, align)
        for k in want:
            np.testing.assert_array_equal(np.asarray(got[k]), np.asarray(want[k]),
                                          err_msg="%s align=%d" % (k, align))
        # invariants: every run starts on a multiple of align and is the count
        # rounded up; its first cnt rows hold its tokens, the rest are padding
        off, cnt = got["expert_offsets"], got["num_tokens_per_expert"]
        assert np.all(off % align == 0)
        assert np.all(np.diff(off) == -(-cnt // align) * align)
        src = got["recv_src_token"]
        for e in range(E):
            run = src[off[e]:off[e + 1]]
            assert np.all(run[:cnt[e]] >= 0) and np.all(run[cnt[e]:] == -1)
        assert np.all(src[off[E]:] == -1)
        valid = got["dst_row"] >= 0
        tok = np.broadcast_to(np.arange(T)[:, None], (T, K))
        np.testing.assert_array_equal(src[got["dst_row"][valid]], tok[valid])


def test_aligned_layout_align_one_is_the_offsets_layout():
    c = wl.random_case(300, 8, 64, 8, 6, 31, masked_frac=0.1, invalid_frac=0.02,
                       allow_dup=True, skew=2.0, with_y=False)
    got = oracle.aligned_layout(c.topk_idx, 64, 8, 1)
    lay = oracle.layout(c.topk_idx, 64, 8)
    dst, src = oracle.permutation(c.topk_idx, 64, lay["expert_offsets"])
    for k in lay:
        np.testing.assert_array_equal(np.asarray(got[k]), np.asarray(lay[k]), err_msg=k)
    np.testing.assert_array_equal(got["dst_row"], dst)
    np.testing.assert_array_equal(got["recv_src_token"], src)


def test_aligned_dispatch_rows_are_copies_and_padding_untouched():
    c = wl.random_case(90, 256, 16, 4, 4, 33, masked_frac=0.1, allow_dup=True)
    res = oracle.run_aligned(c.topk_idx, c.x_bits, 16, 4, 8, fp8=True)
    src = res["recv_src_token"]
    q, s = oracle.quantize(c.x_bits)
    pad = src < 0
    assert pad.any() and (~pad).any()
    np.testing.assert_array_equal(res["recv_x"][~pad], q[src[~pad]])
    np.testing.assert_array_equal(res["recv_scales"][~pad], s[src[~pad]])
    assert np.all(res["recv_x"][pad] == 0) and np.all(res["recv_scales"][pad] == 0)


# ---------------------------------------------------------------------------
# de-duplicated per-partition dispatch
# ---------------------------------------------------------------------------

DEDUP_KEYS = ["partition_token_offsets", "dedup_row", "dedup_src_token", "dedup_topk_idx",
              "slot_src_row", "num_dedup_rows"]


def test_dedup_hand_worked(golden_dir):
    g = _read_kv(os.path.join(golden_dir, "dedup_hand_worked.txt"))
    T, K, E, P = (int(g[k][0]) for k in "TKEP")
    idx = np.array(g["topk_idx"], np.int64).reshape(T, K)
    got = oracle.dedup_layout(idx, E, P)
    for key in ["partition_token_offsets", "dedup_row", "dedup_src_token", "dedup_topk_idx",
                "slot_src_row"]:
        np.testing.assert_array_equal(np.asarray(got[key]).reshape(-1),
                                      np.array(g[key], np.int32), err_msg=key)
    assert got["num_dedup_rows"] == 4


@pytest.mark.parametrize("T,K", [(1, 4), (2, 2), (3, 1), (1, 2), (5, 1)])
def test_dedup_exhaustive_small(T, K):
    """Every routing tensor of this shape with ids in {-1, 0, 1, 2, 3} (E = 4),
    P in {1, 2, 4}, against the cumsum formulation."""
    E = 4
    n = T * K
    grid = np.array(np.meshgrid(*[np.arange(-1, E)] * n, indexing="ij")).reshape(n, -1).T
    batch = grid.reshape(-1, T, K).astype(np.int64)
    for P in (1, 2, 4):
        for i in range(batch.shape[0]):
            got = oracle.dedup_layout(batch[i], E, P)
            want = bf.dedup_layout(batch[i], E, P)
            for key in DEDUP_KEYS:
                assert np.array_equal(np.asarray(got[key]), np.asarray(want[key])), (key, batch[i], P)


@pytest.mark.parametrize("seed", range(8))
def test_dedup_random_against_cumsum_and_invariants(seed):
    rng = np.random.default_rng(2000 + seed)
    E = int(rng.choice([4, 8, 16, 64, 256]))
    P = int(rng.choice([d for d in (1, 2, 4, 8, 32, 64) if E % d == 0]))
    K = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(1, 300))
    c = wl.random_case(T, 8, E, P, K, 3000 + seed, masked_frac=0.1 * (seed % 3),
                       invalid_frac=0.05 * (seed % 2), allow_dup=bool(seed % 2),
                       skew=float(seed % 4), with_y=False)
    got = oracle.dedup_layout(c.topk_idx, E, P)
    want = bf.dedup_layout(c.topk_idx, E, P)
    for key in DEDUP_KEYS:
        np.testing.assert_array_equal(np.asarray(got[key]), np.asarray(want[key]), err_msg=key)
    # invariants: one row per (token, member partition); rows of p contiguous and token-ordered;
    # every valid slot's row holds its local expert id; slot_src agrees with recv_src_token
    Ep = E // P
    in_part = got["is_token_in_partition"]
    rows = got["dedup_row"]
    RD = got["num_dedup_rows"]
    assert RD == int(in_part.sum())
    assert sorted(rows[rows >= 0].tolist()) == list(range(RD))
    for p in range(P):
        seg = got["dedup_src_token"][got["partition_token_offsets"][p]:got["partition_token_offsets"][p + 1]]
        assert np.all(np.diff(seg) > 0)
    assert np.all(got["dedup_src_token"][RD:] == -1)
    dst = got["dst_row"]
    N = got["expert_offsets"][E]
    for t in range(T):
        for k in range(K):
            r = dst[t, k]
            if r < 0:
                continue
            e = int(c.topk_idx[t, k])
            d = got["slot_src_row"][r]
            assert d == rows[t, e // Ep] >= 0
            assert got["dedup_topk_idx"][d, k] == e - (e // Ep) * Ep
            assert got["dedup_src_token"][d] == got["recv_src_token"][r] == t
    assert np.all(got["slot_src_row"][N:] == -1)


def test_dedup_saves_copies_under_group_limited_gating():
    """At the prefill shape, group-limited routing sends fewer copies per token
    than slots (the point of de-duplication)."""
    cfg = wl.CONFIGS["prefill"]
    idx, _, _ = wl.route(cfg, T=512)
    got = oracle.dedup_layout(idx, cfg["E"], cfg["P"])
    per_token = got["num_dedup_rows"] / 512
    assert 6.0 < per_token < 8.0, per_token


def test_dedup_dispatch_rows_are_token_copies():
    c = wl.random_case(80, 384, 16, 4, 4, 41, masked_frac=0.1, allow_dup=True, fp8=True)
    res = oracle.run_dedup(c.topk_idx, c.x_bits, 16, 4, fp8=True)
    q, s = oracle.quantize(c.x_bits)
    src = res["dedup_src_token"]
    live = src >= 0
    np.testing.assert_array_equal(res["dedup_x"][live], q[src[live]])
    np.testing.assert_array_equal(res["dedup_scales"][live], s[src[live]])
    resb = oracle.run_dedup(c.topk_idx, c.x_bits, 16, 4, fp8=False)
    np.testing.assert_array_equal(resb["dedup_x"][live], c.x_bits[src[live]])


# ---------------------------------------------------------------------------
# FP8 quantiser
# ---------------------------------------------------------------------------

def _quant_numpy(x_bits):
    """The quantiser's steps in numpy fp32 arithmetic, with the exhaustive
    nearest-code encoder (numpy's fp32 division and product round correctly)."""
    x = bf.bf16_bits_to_f32(x_bits)
    T, H = x.shape
    g = x.reshape(T, H // 128, 128)
    a = np.abs(g).max(axis=2)
    ac = np.maximum(a, np.float32(1e-4)).astype(np.float32)
    inv = (np.float32(448.0) / ac).astype(np.float32)
    s = (ac / np.float32(448.0)).astype(np.float32)
    prod = (g * inv[:, :, None]).astype(np.float32)
    q = bf.e4m3_nearest(prod.reshape(-1)).reshape(T, H)
    return q, s


def test_quantize_matches_numpy_steps_and_invariants():
    rng = np.random.default_rng(3)
    T, H = 48, 1024
    xf = rng.standard_normal((T, H), dtype=np.float32)
    xf[0, :128] = 0.0                                  # all-zero group
    xf[1, 128:256] = -0.0                              # all negative zero
    xf[2, 256:384] *= 1e-6                             # amax below the 1e-4 floor
    xf[3, :] *= 1e4
    xf[4, 512:640] = 3.0                               # constant group
    xb = wl.bf16_bits_from_f32(xf)
    q, s = oracle.quantize(xb)
    nq, ns = _quant_numpy(xb)
    np.testing.assert_array_equal(q, nq)
    np.testing.assert_array_equal(s.view(np.uint32), ns.view(np.uint32))

    x = bf.bf16_bits_to_f32(xb).reshape(T, H // 128, 128)
    qg = q.reshape(T, H // 128, 128)
    amax = np.abs(x).max(axis=2)
    big = amax >= 1e-4
    # (i) the largest-magnitude element of a group encodes to +-448
    for t, g in zip(*np.nonzero(big)):
        j = np.argmax(np.abs(x[t, g]))
        assert qg[t, g, j] & 0x7F == 0x7E
    # (ii) reconstruction error bound: half a step of E4M3 relative to the value,
    # or half a subnormal step, times the scale, plus fp32 slack
    dec = bf.e4m3_decode_table()[qg].astype(np.float64) * s[:, :, None]
    err = np.abs(dec - x)
    bound = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * s[:, :, None] + 4 * 2.0 ** -24 * np.abs(x)
    assert np.all(err <= bound)
    # (iii) zero groups: codes are signed zeros and the scale is 1e-4/448
    zs = np.float32(np.float32(1e-4) / np.float32(448.0))
    assert s[0, 0] == zs and s[1, 1] == zs
    assert np.all(qg[0, 0] == 0x00) and np.all(qg[1, 1] == 0x80)


def _f32_bits(v) -> int:
    return int(np.array([v], np.float32).view(np.uint32)[0])


_FLOOR = Fraction(float(np.float32(1e-4)))        # a_c = max(a, 1e-4f): the fp32 value of 1e-4


def test_quantize_hand_worked_scale_groups(golden_dir):
    """Groups whose codes and scales were worked out by hand with exact arithmetic
    (tests/golden/fp8_scale_hand_worked.txt): inv = RN32(448 / a_c) and
    s = RN32(a_c / 448) computed any other way -- for instance as products with a
    rounded reciprocal -- change a code or a scale there.  The fixture's own inv,
    scale and codes are re-derived from exact rationals, so a slip in the hand
    arithmetic fails too."""
    groups = {}
    for line in open(os.path.join(golden_dir, "fp8_scale_hand_worked.txt")):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        g = groups.setdefault(int(f[1]), {"ch": [], "inv": None, "scale": None})
        if f[2] == "ch":
            g["ch"].append((int(f[3]), int(f[5], 16), int(f[7], 16)))
        else:
            g["inv"], g["scale"] = int(f[3], 16), int(f[5], 16)
    ng = len(groups)
    xb = np.zeros((1, 128 * ng), np.uint16)
    want_q = np.zeros((1, 128 * ng), np.uint8)
    want_s = np.zeros(ng, np.uint32)
    for gi, g in groups.items():
        for ch, xbits, code in g["ch"]:
            xb[0, 128 * gi + ch] = xbits
            want_q[0, 128 * gi + ch] = code
        want_s[gi] = g["scale"]
        # the hand arithmetic, redone with exact rationals
        xs = [Fraction(float(bf.bf16_bits_to_f32([xbits])[0])) for _, xbits, _ in g["ch"]]
        ac = max(max(abs(v) for v in xs), _FLOOR)
        inv = bf.f32_round(Fraction(448) / ac)
        assert _f32_bits(inv) == g["inv"]
        assert _f32_bits(bf.f32_round(ac / 448)) == g["scale"]
        for v, (_, _, code) in zip(xs, g["ch"]):
            assert int(bf.e4m3_nearest([bf.f32_round(v * Fraction(inv))])[0]) == code
    q, s = oracle.quantize(xb)
    np.testing.assert_array_equal(q, want_q)
    np.testing.assert_array_equal(s.reshape(-1).view(np.uint32), want_s)


def test_quantize_exact_rational():
    """Scales and codes of many groups against exact arithmetic: the two
    divisions as correctly rounded quotients of exact rationals, each code from
    the product x * inv (exact in float64: an 8-bit times a 24-bit significand)
    rounded once to fp32, then the exhaustive nearest-code encoder.  The group
    maxima span seven decades, with many just above and below the 1e-4 floor."""
    rng = np.random.default_rng(17)
    T = 192
    xf = rng.standard_normal((T, 128), dtype=np.float32)
    mag = np.where(np.arange(T) % 2 == 0,
                   10.0 ** rng.uniform(-6.0, 2.0, T),            # anywhere
                   10.0 ** rng.uniform(-4.3, -3.7, T))           # around the floor
    xf *= (mag / np.abs(xf).max(axis=1))[:, None].astype(np.float32)
    xb = wl.bf16_bits_from_f32(xf)
    q, s = oracle.quantize(xb)
    x = bf.bf16_bits_to_f32(xb)
    n_floor = 0
    for t in range(T):
        a = Fraction(float(np.abs(x[t]).max()))
        n_floor += a < _FLOOR
        ac = max(a, _FLOOR)
        assert _f32_bits(s[t, 0]) == _f32_bits(bf.f32_round(ac / 448)), t
        inv = bf.f32_round(Fraction(448) / ac)
        prod = (x[t].astype(np.float64) * inv).astype(np.float32)
        np.testing.assert_array_equal(q[t], bf.e4m3_nearest(prod), err_msg="group %d" % t)
    assert 10 < n_floor < T - 10


def _read_nonfinite_groups(golden_dir):
    """x [1, 384] bf16 bits, expected codes [1, 384] and scale bits [3] from
    tests/golden/fp8_nonfinite_hand_worked.txt."""
    x = np.zeros((1, 384), np.uint16)
    want_q = np.zeros((1, 384), np.uint8)
    want_s = np.zeros(3, np.uint32)
    for line in open(os.path.join(golden_dir, "fp8_nonfinite_hand_worked.txt")):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        g = int(f[1])
        if f[2] == "ch":
            x[0, 128 * g + int(f[3])] = int(f[5], 16)
            want_q[0, 128 * g + int(f[3])] = int(f[7], 16)
        elif f[2] == "nan_even":
            even, odd = int(f[3], 16), int(f[5], 16)
            x[0, 128 * g:128 * g + 128] = np.where(np.arange(128) % 2 == 0, even, odd)
            want_q[0, 128 * g:128 * g + 128] = np.where(
                np.arange(128) % 2 == 0, 0x7F | ((even >> 8) & 0x80), 0x7F | ((odd >> 8) & 0x80))
        else:
            want_s[g] = int(f[3], 16)
    return x, want_q, want_s


def test_quantize_hand_worked_nonfinite_groups(golden_dir):
    """Infinities and NaNs in a group, worked by hand
    (tests/golden/fp8_nonfinite_hand_worked.txt): NaNs left out of the maximum,
    an infinity giving s = +inf and signed-zero codes for the finite values,
    and S.1111.111 with the sign of x for every non-finite x."""
    x, want_q, want_s = _read_nonfinite_groups(golden_dir)
    q, s = oracle.quantize(x)
    np.testing.assert_array_equal(q, want_q)
    np.testing.assert_array_equal(s.reshape(-1).view(np.uint32), want_s)


def test_quantize_nonfinite_invariants():
    """Random groups with infinities and NaNs of both signs (quiet and
    signalling) dropped in: (i) the code of every non-finite x is 0x7F with
    the sign of x; (ii) a group with a NaN but no infinity quantises its
    finite values exactly as the same group with the NaNs replaced by zeros
    (a NaN takes no part in the maximum); (iii) a group with an infinity has
    s = +inf and signed zeros for its finite values."""
    rng = np.random.default_rng(23)
    T, H = 40, 1024
    xb = wl.bf16_bits_from_f32(rng.standard_normal((T, H), dtype=np.float32))
    specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0xFFFF, 0x7FA5], np.uint16)
    hit = rng.random((T, H)) < 0.01
    hit[:, :128] = False                                   # group 0 of every token stays finite
    xb[hit] = specials[rng.integers(0, specials.size, hit.sum())]
    q, s = oracle.quantize(xb)
    nonfin = (xb & 0x7F80) == 0x7F80
    sign = (xb >> 8) & 0x80
    np.testing.assert_array_equal(q[nonfin], (0x7F | sign[nonfin]).astype(np.uint8))
    xg = xb.reshape(T, H // 128, 128)
    qg = q.reshape(T, H // 128, 128)
    is_inf = ((xg & 0x7FFF) == 0x7F80).any(axis=2)
    is_nan = ((xg & 0x7FFF) > 0x7F80).any(axis=2)
    assert is_inf.any() and (is_nan & ~is_inf).any()
    zeroed = np.where((xb & 0x7FFF) > 0x7F80, np.uint16(0), xb)
    qz, sz = oracle.quantize(zeroed)
    qzg = qz.reshape(T, H // 128, 128)
    for t, g in zip(*np.nonzero(is_nan & ~is_inf)):
        fin = (xg[t, g] & 0x7F80) != 0x7F80
        np.testing.assert_array_equal(qg[t, g][fin], qzg[t, g][fin])
        assert s[t, g] == sz[t, g]
    for t, g in zip(*np.nonzero(is_inf)):
        fin = (xg[t, g] & 0x7F80) != 0x7F80
        assert np.isposinf(s[t, g])
        np.testing.assert_array_equal(qg[t, g][fin], ((xg[t, g][fin] >> 8) & 0x80).astype(np.uint8))


def test_fp8_dispatch_rows_are_quantised_tokens():
    c = wl.random_case(70, 384, 16, 4, 3, 11, masked_frac=0.1)
    res = oracle.run(c.topk_idx, c.x_bits, 16, 4, fp8=True)
    q, s = oracle.quantize(c.x_bits)
    N = res["expert_offsets"][16]
    src = res["recv_src_token"][:N]
    np.testing.assert_array_equal(res["recv_x"][:N], q[src])
    np.testing.assert_array_equal(res["recv_scales"][:N], s[src])


def test_bf16_dispatch_rows_are_bitwise_copies():
    c = wl.random_case(90, 264, 12, 3, 4, 12, masked_frac=0.05, allow_dup=True)
    res = oracle.run(c.topk_idx, c.x_bits, 12, 3, fp8=False)
    T, K = c.topk_idx.shape
    for t in range(T):
        for k in range(K):
            r = res["dst_row"][t, k]
            if r >= 0:
                assert np.array_equal(res["recv_x"][r], c.x_bits[t])


# ---------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------

def test_combine_exact_rational_small():
    """Exact rational evaluation of each fused step on small random cases,
    including masked slots and weights of both signs."""
    rng = np.random.default_rng(5)
    for trial in range(6):
        T, K, H = 5, int(rng.integers(1, 5)), 7
        R = T * K
        dst = rng.permutation(R).reshape(T, K).astype(np.int32)
        dst[rng.random((T, K)) < 0.2] = -1
        w = (rng.standard_normal((T, K)) * 3).astype(np.float32)
        y = wl.bf16_bits_from_f32(rng.standard_normal((R, H), dtype=np.float32) * 10)
        np.testing.assert_array_equal(oracle.combine(y, dst, w), bf.combine_exact(y, dst, w))


def test_combine_closed_forms():
    rng = np.random.default_rng(9)
    T, K, H = 40, 4, 96
    R = T * K
    dst = rng.permutation(R).reshape(T, K).astype(np.int32)
    # powers of two times small integers: every step is exact
    w = rng.choice(np.float32([0.5, 1.0, 2.0, -1.0]), size=(T, K)).astype(np.float32)
    yi = rng.integers(-4, 5, size=(R, H)).astype(np.float32)
    y = wl.bf16_bits_from_f32(yi)
    want = (w[:, :, None] * yi[dst]).sum(axis=1)
    got = bf.bf16_bits_to_f32(oracle.combine(y, dst, w))
    np.testing.assert_array_equal(got, want.astype(np.float32))
    # K = 1, w = 1: combine returns the rows themselves
    d1 = rng.permutation(R)[:T].reshape(T, 1).astype(np.int32)
    y2 = wl.bf16_bits_from_f32(rng.standard_normal((R, H), dtype=np.float32))
    out = oracle.combine(y2, d1, np.ones((T, 1), np.float32))
    np.testing.assert_array_equal(out, y2[d1[:, 0]])


def test_combine_identity_expert_and_fp64_bound():
    """y = the bf16 dispatch output (identity experts): out ~ (sum_k w) * x;
    and everywhere within the fp32 FMA-chain bound of the exact float64 sum."""
    c = wl.random_case(64, 512, 16, 4, 4, 21)
    w = c.topk_weights / c.topk_weights.sum(axis=1, keepdims=True)
    res = oracle.run(c.topk_idx, c.x_bits, 16, 4, fp8=False)
    out = bf.bf16_bits_to_f32(oracle.combine(res["recv_x"], res["dst_row"], w))
    x = bf.bf16_bits_to_f32(c.x_bits).astype(np.float64)
    exact = w.astype(np.float64).sum(axis=1, keepdims=True) * x
    K = 4
    bound = 2.0 ** -8 * np.abs(exact) + K * 2.0 ** -24 * np.abs(x) * 1.01 + 1e-38
    assert np.all(np.abs(out - exact) <= bound)
    # general weights: float64 sum of the products
    y = bf.bf16_bits_to_f32(c.y_bits).astype(np.float64)
    dst = res["dst_row"]
    prod = c.topk_weights.astype(np.float64)[:, :, None] * y[dst]
    exact = prod.sum(axis=1)
    out = bf.bf16_bits_to_f32(oracle.combine(c.y_bits, dst, c.topk_weights))
    bound = 2.0 ** -8 * np.abs(exact) + (K + 1) * 2.0 ** -24 * np.abs(prod).sum(axis=1)
    assert np.all(np.abs(out - exact) <= bound)


def test_combine_rounding_sensitive_cases():
    """Cases built to land next to a bf16 rounding boundary, where the fused
    multiply-add, the slot order and the single final rounding decide the last
    bit: acc = 1 from slot 0, then a slot-1 product of about 2^-8 + 2^-24 with
    random low bits.  The exact rational evaluation of the fused chain is the
    reference; the test also checks that an unfused or reversed evaluation
    would differ on a good share of these cases, so they do discriminate."""
    from fractions import Fraction
    rng = np.random.default_rng(17)
    n = 256
    y2 = wl.bf16_bits_from_f32(rng.uniform(2.0 ** -9, 2.0 ** -7, n).astype(np.float32))
    y2f = bf.bf16_bits_to_f32(y2).astype(np.float64)
    target = 2.0 ** -8 + 2.0 ** -24 + rng.uniform(-1, 1, n) * 2.0 ** -32
    w2 = (target / y2f).astype(np.float32)
    T, K, H = n, 2, 1
    y = np.empty((2 * n, 1), np.uint16)
    y[0::2, 0] = 0x3F80                      # 1.0
    y[1::2, 0] = y2
    dst = np.stack([np.arange(0, 2 * n, 2), np.arange(1, 2 * n, 2)], axis=1).astype(np.int32)
    w = np.stack([np.ones(n, np.float32), w2], axis=1)
    want = bf.combine_exact(y, dst, w)
    np.testing.assert_array_equal(oracle.combine(y, dst, w), want)
    # discrimination: evaluate the unfused chain exactly and count differences
    differ = 0
    for i in range(n):
        p = bf.f32_round(Fraction(float(w2[i])) * Fraction(float(y2f[i])))
        unfused = bf.bf16_round_bits(Fraction(bf.f32_round(Fraction(1) + Fraction(p))))
        differ += int(unfused != want[i, 0])
    assert differ >= n // 8, differ
