"""Seeded synthetic inputs for MoE dispatch/combine.

This module only draws inputs: router logits, the router's top-k choice and
gate weights, token activations ``x`` and expert outputs ``y``.  It holds none
of the dispatch/combine arithmetic, and both the HIP path's tests/benchmark and
the CPU oracle's checks take their inputs from here.

Shapes follow DeepSeek-V3-style MoE layers (hidden 7168, 256 routed experts,
top-8, 8 expert groups with 4 groups per token); group-limited gating is
named in "DeepSeek releases DeepEP, an efficient communication library for MoE
models" (section "DeepEP: Optimizing MoE Communication") without a formula, so
the gating below is this module's plain reading of it (sigmoid scores, group
score = sum of the group's two best scores, top-4 groups, top-8 experts among
them).  No dataset or trained weights are involved.

Random numbers: ``numpy.random.Generator(PCG64(seed))`` with seeds
100+c (logits), 200+c (x), 300+c (y) and 400+c (Zipf popularity order) for
configuration number c.  ``x`` and ``y`` are fp32 N(0,1) draws rounded to bf16
by torch's CPU cast (round to nearest even); the bf16 values are returned as
their uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# name -> parameters.  c is the configuration number that picks the seeds.
CONFIGS = {
    "tiny": dict(c=1, T=64, H=256, E=16, P=4, K=2, gating="softmax", fp8=False),
    "decode": dict(c=2, T=128, H=7168, E=256, P=32, K=8, gating="sigmoid", fp8=True),
    "prefill": dict(c=3, T=4096, H=7168, E=256, P=64, K=8, gating="group_limited",
                    n_groups=8, topk_groups=4, fp8=True),
    "skewed": dict(c=4, T=8192, H=7168, E=256, P=64, K=8, gating="zipf_softmax",
                   zipf_s=1.2, fp8=False),
    "coarse": dict(c=5, T=32768, H=4096, E=8, P=8, K=2, gating="softmax", fp8=False),
}

# The configuration the headline throughput is quoted on.
HEADLINE = "prefill"


@dataclass
class Workload:
    name: str
    T: int
    H: int
    E: int
    P: int
    K: int
    fp8: bool
    topk_idx: np.ndarray          # [T, K] int64, descending router score
    topk_weights: np.ndarray      # [T, K] float32
    x_bits: np.ndarray            # [T, H] uint16 (bf16 bit patterns)
    y_bits: np.ndarray | None     # [T*K, H] uint16 (bf16), expert outputs
    meta: dict = field(default_factory=dict)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (torch CPU cast, nearest even) -> uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_bf16(seed: int, shape) -> np.ndarray:
    """N(0,1) fp32 draws rounded to bf16 bits, generated in row blocks."""
    rng = _rng(seed)
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, np.uint16)
    if out.size == 0:
        return out
    flat = out.reshape(shape[0], -1)
    step = max(1, (1 << 24) // max(1, flat.shape[1]))
    for r0 in range(0, flat.shape[0], step):
        r1 = min(flat.shape[0], r0 + step)
        blk = rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32)
        flat[r0:r1] = bf16_bits_from_f32(blk)
    return out


def _topk(score: np.ndarray, K: int) -> np.ndarray:
    """Top-k indices in descending score, ties to the lower expert id."""
    return np.argsort(-score, axis=1, kind="stable")[:, :K].astype(np.int64)


def route(cfg: dict, T: int | None = None):
    """Router: (topk_idx [T,K] int64, topk_weights [T,K] fp32, meta)."""
    c, E, K = cfg["c"], cfg["E"], cfg["K"]
    T = cfg["T"] if T is None else T
    logits = _rng(100 + c).standard_normal((T, E))  # float64
    meta = {}
    g = cfg["gating"]
    if g in ("softmax", "zipf_softmax"):
        if g == "zipf_softmax":
            ranks = 1 + _rng(400 + c).permutation(E)
            logits = logits - cfg["zipf_s"] * np.log(ranks.astype(np.float64))[None, :]
        z = logits - logits.max(axis=1, keepdims=True)
        score = np.exp(z)
        score /= score.sum(axis=1, keepdims=True)
        idx = _topk(score, K)
    elif g == "sigmoid":
        score = 1.0 / (1.0 + np.exp(-logits))
        idx = _topk(score, K)
    elif g == "group_limited":
        score = 1.0 / (1.0 + np.exp(-logits))
        G, TG = cfg["n_groups"], cfg["topk_groups"]
        per = E // G
        grouped = score.reshape(T, G, per)
        top2 = np.sort(grouped, axis=2)[:, :, -2:].sum(axis=2)       # [T, G]
        gsel = np.argsort(-top2, axis=1, kind="stable")[:, :TG]      # [T, TG]
        allowed = np.zeros((T, G), bool)
        np.put_along_axis(allowed, gsel, True, axis=1)
        masked = np.where(np.repeat(allowed, per, axis=1), score, -np.inf)
        idx = _topk(masked, K)
        meta["groups_per_token_max"] = int(
            max((len(np.unique(r // per)) for r in idx), default=0))
    else:
        raise ValueError(g)
    sel = np.take_along_axis(score, idx, axis=1)
    w = (sel / sel.sum(axis=1, keepdims=True)).astype(np.float32)
    if T > 0:
        load = np.bincount(idx.ravel(), minlength=E)
        meta["max_over_mean_load"] = float(load.max() / load.mean())
        meta["empty_experts"] = int((load == 0).sum())
    return idx, w, meta


def make(name: str, T: int | None = None, with_y: bool = True) -> Workload:
    """Build configuration ``name``; ``T`` (optional) keeps only the first T tokens'
    worth of routing and activations (the same seeds, so a prefix sample of
    the routing when T is smaller; x and y are drawn at the reduced shape)."""
    cfg = CONFIGS[name]
    T = cfg["T"] if T is None else int(T)
    H, K = cfg["H"], cfg["K"]
    idx, w, meta = route(cfg, T)
    x = normal_bf16(200 + cfg["c"], (T, H))
    y = normal_bf16(300 + cfg["c"], (T * K, H)) if with_y else None
    return Workload(name, T, H, cfg["E"], cfg["P"], K, cfg["fp8"], idx, w, x, y, meta)


# Non-finite bf16 patterns: +-inf, quiet NaNs and NaNs whose fp32 widening is
# signalling, of both signs and several payloads.
NONFINITE_BF16 = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0xFF81, 0x7FA5, 0xFFFF],
                          np.uint16)


def combine_inputs(T: int, H: int, K: int, R: int, seed: int, *, masked_frac: float = 0.0,
                   past_frac: float = 0.0):
    """Seeded inputs of a combine alone: y [R, H] bf16 bits, dst_row [T, K]
    int32 with rows drawn from [0, R) (repeats allowed), ``masked_frac`` of
    them -1 and ``past_frac`` of them in [R, R + 100) (past the end of y),
    and topk_weights [T, K] fp32 in [0, 1)."""
    rng = _rng(seed)
    y = normal_bf16(seed + 1, (R, H))
    dst = rng.integers(0, max(R, 1), (T, K)).astype(np.int32)
    if masked_frac > 0:
        dst[rng.random((T, K)) < masked_frac] = -1
    if past_frac > 0:
        past = rng.random((T, K)) < past_frac
        dst[past] = (R + rng.integers(0, 100, (T, K))).astype(np.int32)[past]
    w = rng.random((T, K)).astype(np.float32)
    return y, dst, w


def random_case(T: int, H: int, E: int, P: int, K: int, seed: int, *,
                masked_frac: float = 0.0, invalid_frac: float = 0.0,
                allow_dup: bool = False, skew: float = 0.0, fp8: bool = False,
                with_y: bool = True, nonfinite_frac: float = 0.0) -> Workload:
    """A generic seeded case for edge and ragged-shape tests.

    Experts are drawn without replacement per token unless ``allow_dup``;
    ``skew`` > 0 biases the draw towards low expert ids (weights 1/(e+1)^skew);
    ``masked_frac`` of the slots become -1 and ``invalid_frac`` become
    out-of-range ids (E + j or -2 - j).  ``nonfinite_frac`` of the values of x
    become infinities or NaNs (NONFINITE_BF16), and then token 0's first 128
    channels are all NaNs (alternating signs) and token 1's first channel is
    +inf.
    """
    rng = _rng(seed)
    p = 1.0 / np.arange(1, E + 1, dtype=np.float64) ** skew
    p /= p.sum()
    idx = np.empty((T, K), np.int64)
    for t in range(T):
        idx[t] = rng.choice(E, size=K, replace=allow_dup or K > E, p=p)
    if masked_frac > 0:
        idx[rng.random((T, K)) < masked_frac] = -1
    if invalid_frac > 0:
        bad = rng.random((T, K)) < invalid_frac
        vals = np.where(rng.random((T, K)) < 0.5, E + rng.integers(0, 5, (T, K)),
                        -2 - rng.integers(0, 5, (T, K)))
        idx[bad] = vals[bad]
    w = rng.random((T, K)).astype(np.float32)
    x = bf16_bits_from_f32(rng.standard_normal((T, H), dtype=np.float32))
    y = (bf16_bits_from_f32(rng.standard_normal((T * K, H), dtype=np.float32))
         if with_y else None)
    if nonfinite_frac > 0:
        hit = rng.random((T, H)) < nonfinite_frac
        x[hit] = NONFINITE_BF16[rng.integers(0, NONFINITE_BF16.size, int(hit.sum()))]
        x[0, :min(128, H)] = np.where(np.arange(min(128, H)) % 2 == 0, 0x7FC1, 0xFFA0)
        if T > 1:
            x[1, 0] = 0x7F80
    return Workload("random", T, H, E, P, K, fp8, idx, w, x, y, {"seed": seed})
