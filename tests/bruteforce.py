"""Independent brute-force formulations used to pin the CPU oracle.

Nothing here is derived from the oracle's C code: every function is a
different formulation of the same definition -- a library routine (stable
argsort, bincount, cumsum), an exhaustive search over a format's code points,
or exact rational arithmetic -- so that a slip in the oracle (a wrong index,
sign, tie rule, order or term) shows up as a mismatch.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


# ---------------------------------------------------------------------------
# E4M3 by exhaustive search over the 256 codes
# ---------------------------------------------------------------------------

def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 OCP E4M3 codes (NaN for S.1111.111), float64."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = e4m3_decode_table()
_MAGS = _E4M3[:0x7F]          # codes 0x00..0x7E: every finite magnitude, ascending


def e4m3_nearest(v) -> np.ndarray:
    """Nearest finite E4M3 code to each fp32 value (saturating), ties to the
    even code, sign kept (so -tiny -> 0x80).  Finite inputs only."""
    v = np.asarray(v, dtype=np.float32).reshape(-1)
    assert np.all(np.isfinite(v))
    # Beyond 448 the nearest finite code is 448 itself; clamping far-away
    # magnitudes to 1000 keeps the distances below distinguishable in float64.
    a = np.minimum(np.abs(v.astype(np.float64)), 1000.0)
    out = np.empty(v.shape, np.uint8)
    codes = np.arange(0x7F)
    for i0 in range(0, a.size, 1 << 15):
        blk = a[i0:i0 + (1 << 15)]
        d = np.abs(blk[:, None] - _MAGS[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        even = cand & (codes[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        out[i0:i0 + blk.size] = pick
    out |= np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    return out


# ---------------------------------------------------------------------------
# exact rational rounding
# ---------------------------------------------------------------------------

def _round_fraction(q: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Round a rational to the nearest value with ``mant_bits`` significand
    bits (including the leading one) and minimum normal exponent ``emin``,
    ties to even, unbounded exponent range above."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (mant_bits - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def f32_round(q: Fraction) -> float:
    """Exact rational -> nearest fp32 (ties to even) as a Python float."""
    return float(_round_fraction(q, 24, -126))


def bf16_round_bits(q: Fraction) -> int:
    """Exact rational -> nearest bf16 (ties to even) -> 16-bit pattern."""
    r = _round_fraction(q, 8, -126)
    if abs(r) >= Fraction(2) ** 128:
        return 0xFF80 if r < 0 else 0x7F80
    f = np.float32(float(r))
    return int(np.array([f], np.float32).view(np.uint32)[0] >> 16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def combine_exact(y_bits, dst, w) -> np.ndarray:
    """Combine by exact rational arithmetic: each fused multiply-add is the
    exact value w*y + acc rounded once to fp32; the result rounded to bf16."""
    y = bf16_bits_to_f32(y_bits)
    T, K = dst.shape
    H = y.shape[1]
    out = np.empty((T, H), np.uint16)
    for t in range(T):
        for h in range(H):
            acc = Fraction(0)
            for k in range(K):
                r = int(dst[t, k])
                if r < 0:
                    continue
                acc = Fraction(f32_round(Fraction(float(w[t, k])) * Fraction(float(y[r, h])) + acc))
            out[t, h] = bf16_round_bits(acc)
    return out


# ---------------------------------------------------------------------------
# layout and permutation
# ---------------------------------------------------------------------------

def layout(idx: np.ndarray, E: int, P: int) -> dict:
    """Counts, partition mask and offsets via bincount / unique / cumsum."""
    idx = np.asarray(idx, np.int64)
    T, K = idx.shape
    Ep = E // P
    valid = (idx >= 0) & (idx < E)
    cnt_e = np.bincount(idx[valid], minlength=E).astype(np.int32)
    in_part = np.zeros((T, P), np.uint8)
    for t in range(T):
        parts = np.unique(idx[t][valid[t]] // Ep)
        in_part[t, parts] = 1
    cnt_p = in_part.sum(axis=0).astype(np.int32)
    off_e = np.concatenate([[0], np.cumsum(cnt_e)]).astype(np.int32)
    off_p = off_e[np.arange(P + 1) * Ep].astype(np.int32)
    nerr = int((~valid & (idx != -1)).sum())
    return dict(num_tokens_per_expert=cnt_e, num_tokens_per_partition=cnt_p,
                is_token_in_partition=in_part, expert_offsets=off_e,
                partition_offsets=off_p, num_invalid=nerr)


def permutation(idx: np.ndarray, E: int):
    """dst_row / recv_src_token from a stable sort of the flattened expert ids:
    flattening row-major lists the (token, slot) pairs in (token, slot) order,
    so a stable sort by expert gives each expert's rows in that order."""
    idx = np.asarray(idx, np.int64)
    T, K = idx.shape
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    key = np.where(valid, flat, E)          # masked/invalid slots sort last
    order = np.argsort(key, kind="stable")[: int(valid.sum())]
    dst = np.full(T * K, -1, np.int32)
    dst[order] = np.arange(order.size, dtype=np.int32)
    src = np.full(T * K, -1, np.int32)
    src[: order.size] = order // K
    return dst.reshape(T, K), src


def layout_batch(idx_batch: np.ndarray, E: int, P: int):
    """Vectorised brute force over a batch of small [T,K] tensors: returns
    (cnt_e [B,E], in_part [B,T,P], off_e [B,E+1], dst [B,T,K], nerr [B])."""
    B, T, K = idx_batch.shape
    Ep = E // P
    flat = idx_batch.reshape(B, T * K)
    valid = (flat >= 0) & (flat < E)
    onehot = (flat[:, :, None] == np.arange(E)[None, None, :]) & valid[:, :, None]
    cnt_e = onehot.sum(axis=1).astype(np.int32)
    off_e = np.concatenate([np.zeros((B, 1), np.int64), np.cumsum(cnt_e, axis=1)], axis=1)
    # rank of (t,k) among earlier equal experts, by direct pairwise comparison
    n = T * K
    earlier = np.tril(np.ones((n, n), bool), k=-1)          # [j, j'] : j' < j
    same = (flat[:, :, None] == flat[:, None, :]) & valid[:, None, :]
    rank = (same & earlier[None]).sum(axis=2)
    e_safe = np.where(valid, flat, 0)
    dst = np.where(valid, np.take_along_axis(off_e, e_safe, axis=1) + rank, -1)
    part = np.where(valid, flat // Ep, -1).reshape(B, T, K)
    in_part = (part[:, :, :, None] == np.arange(P)[None, None, None, :]).any(axis=2)
    nerr = (~valid & (flat != -1)).sum(axis=1)
    return cnt_e, in_part.astype(np.uint8), off_e.astype(np.int32), \
        dst.reshape(B, T, K).astype(np.int32), nerr


def ll_layout(idx: np.ndarray, E: int, C: int) -> dict:
    """Fixed-capacity layout from the stable-sort permutation above: a slot's
    rank inside its expert is its sorted position minus the expert's start."""
    idx = np.asarray(idx, np.int64)
    T, K = idx.shape
    lay = layout(idx, E, 1)
    dst, _ = permutation(idx, E)
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    e_safe = np.where(valid, flat, 0)
    rank = dst.reshape(-1) - lay["expert_offsets"][e_safe]
    keep = valid & (rank < C)
    ll = np.where(keep, e_safe * C + rank, -1).astype(np.int32)
    src = np.full(E * C, -1, np.int32)
    src[ll[keep]] = np.nonzero(keep)[0] // K
    return dict(num_tokens_per_expert=lay["num_tokens_per_expert"], dst_row=ll.reshape(T, K),
                recv_src_token=src, num_invalid=lay["num_invalid"])


def ll_rank_batch(idx_batch: np.ndarray, E: int) -> np.ndarray:
    """Rank of each slot among the earlier valid slots of the same expert, by
    direct pairwise comparison over a batch of small [T,K] tensors; -1 for
    slots that are not valid."""
    B, T, K = idx_batch.shape
    flat = idx_batch.reshape(B, T * K)
    valid = (flat >= 0) & (flat < E)
    n = T * K
    earlier = np.tril(np.ones((n, n), bool), k=-1)
    same = (flat[:, :, None] == flat[:, None, :]) & valid[:, None, :]
    rank = (same & earlier[None]).sum(axis=2)
    return np.where(valid, rank, -1).reshape(B, T, K)


def dedup_layout(idx: np.ndarray, E: int, P: int) -> dict:
    """De-duplicated per-partition rows from the partition mask with cumsum:
    a token's row in partition p is the partition's offset plus the number of
    earlier member tokens (an exclusive running sum down the mask column)."""
    idx = np.asarray(idx, np.int64)
    T, K = idx.shape
    Ep = E // P
    Kp = min(K, P)
    lay = layout(idx, E, P)
    in_part = lay["is_token_in_partition"].astype(np.int64)
    cnt_p = in_part.sum(axis=0)
    ptok_off = np.concatenate([[0], np.cumsum(cnt_p)]).astype(np.int32)
    before = np.cumsum(in_part, axis=0) - in_part          # earlier member tokens
    dd_row = np.where(in_part == 1, ptok_off[:-1][None, :] + before, -1).astype(np.int32)
    dd_src = np.full(T * Kp, -1, np.int32)
    dd_idx = np.full((T * Kp, K), -1, np.int32)
    tt, pp = np.nonzero(dd_row >= 0)
    dd_src[dd_row[tt, pp]] = tt
    valid = (idx >= 0) & (idx < E)
    for t, p in zip(tt, pp):
        r = dd_row[t, p]
        local = valid[t] & (idx[t] // Ep == p)
        dd_idx[r, local] = idx[t, local] - p * Ep
    dst, _ = permutation(idx, E)
    slot_src = np.full(T * K, -1, np.int32)
    vt, vk = np.nonzero(valid)
    slot_src[dst[vt, vk]] = dd_row[vt, idx[vt, vk] // Ep]
    return dict(partition_token_offsets=ptok_off, dedup_row=dd_row, dedup_src_token=dd_src,
                dedup_topk_idx=dd_idx, slot_src_row=slot_src, num_dedup_rows=int(ptok_off[-1]))


def aligned_layout(idx: np.ndarray, E: int, P: int, align: int) -> dict:
    """Aligned expert runs from the stable-sort permutation: a slot keeps its
    rank inside its expert, and the runs start at the cumulative sum of the
    counts rounded up to a multiple of ``align``."""
    idx = np.asarray(idx, np.int64)
    T, K = idx.shape
    Ep = E // P
    lay = layout(idx, E, P)
    dst, _ = permutation(idx, E)
    cnt = lay["num_tokens_per_expert"].astype(np.int64)
    padded = -(-cnt // align) * align
    off = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    e_safe = np.where(valid, flat, 0)
    rank = dst.reshape(-1) - lay["expert_offsets"][e_safe]
    rows = np.where(valid, off[e_safe] + rank, -1).astype(np.int32)
    src = np.full(T * K + E * (align - 1), -1, np.int32)
    src[rows[valid]] = np.nonzero(valid)[0] // K
    res = dict(lay)
    res.update(expert_offsets=off, partition_offsets=off[np.arange(P + 1) * Ep].astype(np.int32),
               dst_row=rows.reshape(T, K), recv_src_token=src)
    return res
