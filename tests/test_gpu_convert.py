"""The device conversions, value by value, against the oracle (GPU).

E4M3: the dispatch kernel's hardware conversion (v_cvt_pk_fp8_f32) over the
inputs the quantiser hands it (finite, |v| < 464: every bf16 value times a set
of scales, a dense sweep, every midpoint between codes and its fp32
neighbours) -- the quantiser never converts a non-finite product, it writes
the NaN code of an infinite or NaN x itself (tests/test_gpu_parity.py covers
those tokens) -- and the software conversion over every finite value plus
infinities and NaNs of both signs and several payloads.  bf16: the combine
kernel's rounding over random bit patterns and exact ties.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_get_dispatch_amd import binding as ep
from parity import announce

pytestmark = pytest.mark.gpu


def _e4m3_inputs(limit=None):
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals)]
    parts = []
    with np.errstate(over="ignore"):
        for mult in [1.0, 0.5, 3.0, 448.0 / 3.1, 1.0 / 7.0, 2.0 ** -8, 1.37e-3, 1.0e3]:
            parts.append((vals * np.float32(mult)).astype(np.float32))
    parts.append(np.linspace(-470.0, 470.0, 2_000_001).astype(np.float32))
    # midpoints between adjacent codes and their fp32 neighbours
    mags = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        mags.append((m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    mags = np.array(mags)
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(1e9))])
    parts += [near, -near, np.float32([0.0, -0.0, 448.0, -448.0, 463.99997, -463.99997])]
    v = np.concatenate(parts)
    v = v[np.isfinite(v)]
    if limit is not None:
        v = v[np.abs(v) < limit]
    return np.ascontiguousarray(v)


def test_e4m3_hardware_conversion_matches_oracle():
    v = _e4m3_inputs(limit=464.0)
    announce("convert_e4m3 hw n=%d" % v.size)
    got = ep.convert_e4m3(torch.from_numpy(v).cuda(), mode=0).cpu().numpy()
    want = oracle.e4m3(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_e4m3_software_conversion_matches_oracle():
    v = _e4m3_inputs()
    rng = np.random.default_rng(1)
    rnd = rng.integers(0, 2 ** 32, 1_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    nonfinite = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7F800001,
                          0xFF800001, 0x7FA5A5A5, 0xFFFFFFFF], np.uint32).view(np.float32)
    v = np.concatenate([v, rnd[np.isfinite(rnd)], nonfinite])
    announce("convert_e4m3 sw n=%d" % v.size)
    got = ep.convert_e4m3(torch.from_numpy(v).cuda(), mode=1).cpu().numpy()
    want = oracle.e4m3(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_bf16_conversion_matches_oracle():
    rng = np.random.default_rng(2)
    u = rng.integers(0, 2 ** 32, 4_000_000, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    b = rng.integers(0, 0x7F7F, 200_000).astype(np.uint32) << 16
    ties = (b | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties, np.float32([0.0, -0.0, 3.4028234e38, -3.4028234e38])])
    v = np.ascontiguousarray(v[np.isfinite(v)])
    announce("convert_bf16 n=%d" % v.size)
    got = ep.convert_bf16(torch.from_numpy(v).cuda()).cpu().numpy().view(np.uint16)
    want = oracle.bf16_rne(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


@pytest.mark.parametrize("nbytes", [16, 4096, 4096 + 16, 3 * 4096 - 16, (1 << 20) + 48,
                                    (64 << 20) + 4080, 1 << 30])
def test_copy_is_exact_and_stays_in_bounds(nbytes):
    """ep_copy (the counters' reference kernel and the copy ceiling) copies
    every byte, whole 4 KiB spans and the partial last one alike, and writes
    nothing past the end."""
    announce("ep_copy %d bytes" % nbytes)
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.full((nbytes + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    ep.copy(src, dst[:nbytes])
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all())
