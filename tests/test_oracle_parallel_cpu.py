"""The OpenMP build of the oracle (used only to time the CPU baseline on all
cores) gives the single-threaded checker's results bit for bit, on every
option path: per-tensor 1x16 and 16x16, stochastic rounding, the RHT pair
(binary32 and BF16 values), row scaling of both orientations, UE5M3."""

from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import workloads as W

CASES = {
    "1d_bf16": (lambda: W.randn_bf16(96, 160, 3), {}),
    "2d_fp32": (lambda: (np.random.default_rng(4).standard_normal((64, 96)) * 7).astype(np.float32),
                dict(block_2d=True)),
    "1d_sr": (lambda: W.randn_bf16(64, 128, 5), dict(stochastic=True, sr_seed=77)),
    "rht_sr": (lambda: W.randn_bf16(64, 64, 6), dict(rht=True, sign_mask=0x6B1D, stochastic=True, sr_seed=3)),
    "rht_bf16": (lambda: W.randn_bf16(48, 80, 7), dict(rht=True, sign_mask=0x0F0F, rht_bf16=True)),
    "row_scaled_both": (lambda: W.c4(rows=48, cols=64, seed=8), dict(row_scaled=True)),
    "ue5m3": (lambda: W.randn_bf16(32, 64, 9), dict(scale_fmt=O.SCALE_UE5M3)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_all_cores_build_equals_the_checker(name):
    make, kw = CASES[name]
    x = make()
    want = O.quantize(x, **kw)
    with O.all_cores() as threads:
        assert threads >= 1
        got = O.quantize(x, **kw)
    for k, v in want.items():
        if v is None:
            assert got[k] is None, k
        else:
            assert np.array_equal(got[k], v), (name, k)
