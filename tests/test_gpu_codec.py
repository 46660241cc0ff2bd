"""GPU: the device E2M1 encoders (through the nvfp4_debug_e2m1_pack hook)
against the CPU oracle, bit for bit, on chosen values and random words.

Stochastic rounding is tested where it can go wrong: for every value, the
16-bit random numbers at and next to its threshold 65536 * f (f = the
value's position between its two grid neighbours), over every binade from
denormals up, both signs, zeros and saturating values. Both device forms are
covered (four pairs per word, and one pair at a time).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_05_amd as nv
import oracle as O
from gpu_helpers import DEV, host

pytestmark = pytest.mark.gpu

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def sample_values(rng, per_exponent=160):
    """FP32 values from every binade between the smallest denormal and 8,
    both signs, plus zeros and large values."""
    out = []
    for e in range(-149, 3):
        if e < -126:
            m = rng.integers(1, 2 ** 23, per_exponent // 4)
            v = (m.astype(np.float64) * 2.0 ** -149).astype(np.float32)
        else:
            m = rng.integers(0, 2 ** 23, per_exponent)
            v = ((1.0 + m / 2.0 ** 23) * 2.0 ** e).astype(np.float32)
        out.append(v)
    # grid values, their FP32 neighbours and midpoints
    g = GRID.astype(np.float32)
    out += [g, np.nextafter(g, np.float32(0)), np.nextafter(g, np.float32(8)),
            ((GRID[1:] + GRID[:-1]) / 2).astype(np.float32)]
    out.append(np.array([0.0, 6.5, 7.99, 8.0, 100.0, 1e30, 3.4e38], np.float32))
    v = np.concatenate(out)
    sign = np.where(rng.random(v.size) < 0.5, -1.0, 1.0).astype(np.float32)
    return np.concatenate([v, v * sign, np.array([-0.0], np.float32)])


def thresholds(v):
    """65536 * f for each value (exact in binary64), or -1 where |v| >= 6."""
    a = np.abs(v.astype(np.float64))
    i = np.clip(np.searchsorted(GRID, a, side="right") - 1, 0, 6)
    lo, hi = GRID[i], GRID[np.minimum(i + 1, 7)]
    t = (a - lo) / (hi - lo) * 65536.0
    return np.where(a >= 6.0, -1.0, t)


def cases(seed):
    """(values [2n], r16 [2n]) with r16 around each value's threshold."""
    rng = np.random.default_rng(seed)
    v = sample_values(rng)
    t = thresholds(v)
    vals, rs = [], []
    for d in (-1, 0, 1):
        for base in (np.floor(t), np.ceil(t)):
            r = base + d
            ok = (r >= 0) & (r <= 65535) & (t >= 0)
            vals.append(v[ok])
            rs.append(r[ok])
    vals.append(v)  # plus random words for every value
    rs.append(rng.integers(0, 65536, v.size).astype(np.float64))
    vals = np.concatenate(vals).astype(np.float32)
    rs = np.concatenate(rs).astype(np.uint16)
    perm = rng.permutation(vals.size)  # mix cases within pairs and words
    vals, rs = vals[perm], rs[perm]
    if vals.size % 2:
        vals, rs = vals[:-1], rs[:-1]
    return vals, rs


def run_hook(vals, words, flags):
    n = vals.size // 2
    out = torch.empty(n, dtype=torch.uint8, device=DEV)
    vd = torch.from_numpy(vals).to(DEV)
    rd = None if words is None else torch.from_numpy(words.view(np.int32)).to(DEV)
    nv.nvfp4_debug_e2m1_pack(vd, rd, out, flags)
    torch.cuda.synchronize()
    return host(out)


def packed(codes):
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("pairwise", [False, True])
def test_stochastic_rounding_at_every_threshold(pairwise):
    vals, r16 = cases(123)
    words = (r16[0::2].astype(np.uint32) | (r16[1::2].astype(np.uint32) << 16))
    got = run_hook(vals, words, nv.NVFP4_DEBUG_SR | (nv.NVFP4_DEBUG_PAIRWISE if pairwise else 0))
    want = packed(O.e2m1_sr(vals, r16))
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(vals[2 * k]), float(vals[2 * k + 1]), hex(int(words[k])), int(got[k]), int(want[k]))
                           for k in bad[:5]]
    assert vals.size > 200_000


@pytest.mark.parametrize("pairwise", [False, True])
def test_nearest_even_on_sampled_values(pairwise):
    vals, _ = cases(124)
    got = run_hook(vals, None, nv.NVFP4_DEBUG_PAIRWISE if pairwise else 0)
    want = packed(O.e2m1_rne(vals))
    assert np.array_equal(got, want)


def test_stochastic_rounding_up_rate_matches_fraction():
    # at a fixed value the share of random words that round up is
    # ceil(65536 f) / 65536 exactly when every r16 is used once
    v = np.float32(0.3 + 2.0 ** -20)  # below 1/2: f has bits beyond 2^-22
    f = thresholds(np.array([v]))[0]
    r16 = np.arange(65536, dtype=np.uint32)
    words = r16 | (r16 << 16)
    vals = np.full(2 * 65536, v, np.float32)
    got = run_hook(vals, words, nv.NVFP4_DEBUG_SR)
    ups = int(np.count_nonzero((got & 7) == 1))
    assert ups == int(np.ceil(f))
