"""GPU: the swizzle-fusion check that the "Fuse NVFP4 scale swizzling on
SM120 and SM121" page lists among its tests (Changes). Over every
combination of quantizer (1x16, 16x16, RHT), requested outputs, rounding
mode, block-scale format and input type, a call that writes GEMM-swizzled
scales must produce the FP4 bytes and amaxes of the compact call, and its
scale bytes must be the compact ones moved by an independent statement of
the tile permutation (the oracle's reshape). The compact call itself is
checked against the oracle in the option-matrix tests."""

from __future__ import annotations

import zlib

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import run_quantize

pytestmark = pytest.mark.gpu

ORIENT = {"row": (True, False), "col": (False, True), "both": (True, True)}
ROWS, COLS = 256, 384  # whole 128 x 128 tiles, as swizzled scales require


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3"])
@pytest.mark.parametrize("rounding", ["rne", "sr"])
@pytest.mark.parametrize("orient", ["row", "col", "both"])
@pytest.mark.parametrize("quantizer", ["1d", "2d", "rht"])
def test_swizzled_scales_are_the_compact_scales_permuted(quantizer, orient, rounding, fmt, dtype):
    seed = zlib.crc32(f"{quantizer}/{orient}/{rounding}/{fmt}/{dtype}".encode()) % 1000
    x = W.c2(rows=ROWS, cols=COLS, seed=seed) if dtype == "bf16" else W.gaussian_fp32(ROWS, COLS, seed, 3.0)
    rw, cw = ORIENT[orient]
    kw = dict(block_2d=quantizer == "2d", rht=quantizer == "rht", rht_sign_mask=W.rht_sign_mask(seed),
              stochastic=rounding == "sr", sr_seed=seed, scale_fmt=1 if fmt == "ue5m3" else 0)
    compact = run_quantize(x, rowwise=rw, columnwise=cw, swizzled=False, **kw)
    swz = run_quantize(x, rowwise=rw, columnwise=cw, swizzled=True, **kw)
    for side, n, k in (("row", ROWS, COLS), ("col", COLS, ROWS)):
        if compact[f"{side}_data"] is None:
            assert swz[f"{side}_data"] is None
            continue
        assert np.array_equal(swz[f"{side}_data"], compact[f"{side}_data"]), side
        assert np.array_equal(swz[f"amax_{side}"], compact[f"amax_{side}"]), side
        permuted = O.swizzle_scales(compact[f"{side}_scales"].reshape(n, k // 16))
        assert np.array_equal(swz[f"{side}_scales"].ravel(), permuted), side
