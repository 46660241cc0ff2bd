"""GPU: seeded random cases over shapes and options, bit for bit against the
oracle. Shapes are small and often ragged (any multiple of 16, down to a
single 16 x 16 block); options are drawn from every combination the
deterministic paths accept (the RHT column side, held to tolerances, is
covered elsewhere)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import run_quantize

pytestmark = pytest.mark.gpu

N_CASES = 60


def _case(i):
    rng = np.random.default_rng(1000 + i)
    rows = int(rng.integers(1, 25)) * 16
    cols = int(rng.integers(1, 41)) * 16
    row_scaled = bool(rng.random() < 0.2)
    block_2d = (not row_scaled) and bool(rng.random() < 0.4)
    if row_scaled:
        rw, cw = True, False
        rows = int(rng.integers(1, 300))  # row-wise only: any row count
    else:
        rw, cw = [(True, True), (True, False), (False, True)][int(rng.integers(0, 3))]
    swizzled = (not row_scaled) and bool(rng.random() < 0.35)
    if swizzled:  # whole 128 x 128 tiles
        rows, cols = int(rng.integers(1, 4)) * 128, int(rng.integers(1, 6)) * 128
    kw = dict(block_2d=block_2d, row_scaled=row_scaled, stochastic=bool(rng.random() < 0.5),
              sr_seed=int(rng.integers(0, 2 ** 32)), scale_fmt=int(rng.random() < 0.3))
    fp32 = bool(rng.random() < 0.4)
    scale = float(2.0 ** rng.integers(-20, 20))
    x = (W.gaussian_fp32(rows, cols, 2000 + i, scale) if fp32
         else W.c2(rows=rows, cols=cols, seed=2000 + i))
    return x, rw, cw, swizzled, kw


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    x, rw, cw, swizzled, kw = _case(i)
    got = run_quantize(x, rowwise=rw, columnwise=cw, swizzled=swizzled, **kw)
    ref = O.quantize(x, rowwise=rw, columnwise=cw, **kw)
    for side in ("row", "col"):
        if ref[f"{side}_data"] is None:
            assert got[f"{side}_data"] is None
            continue
        assert np.array_equal(got[f"{side}_data"], ref[f"{side}_data"]), (i, side, x.shape, kw)
        want = O.swizzle_scales(ref[f"{side}_scales"]) if swizzled else ref[f"{side}_scales"].ravel()
        assert np.array_equal(got[f"{side}_scales"].ravel(), want), (i, side, x.shape, kw)
        assert np.array_equal(got[f"amax_{side}"], ref[f"amax_{side}"]), (i, side, x.shape, kw)
