"""GPU parity over the option matrix of nvfp4_quantize: input dtype x block
shape x rounding x scale layout x orientations (bit-exact against the
oracle), and the RHT column-wise side x dtype x rounding x layout x
binary32 or BF16 transformed values (to the stated tolerances). Shapes have ragged edge tiles where the layout allows
(compact), and whole 128x128 tiles where it requires them (swizzled)."""

from __future__ import annotations

import zlib

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import codes, e2m1_step_distance, run_quantize

pytestmark = pytest.mark.gpu

ORIENT = {"both": (True, True), "row": (True, False), "col": (False, True)}


def make_input(dtype, rows, cols, seed):
    if dtype == "bf16":
        return W.c2(rows=rows, cols=cols, seed=seed)  # per-column magnitudes over 5 decades
    return W.gaussian_fp32(rows, cols, seed, scale=3.0)


@pytest.mark.parametrize("orient", ["both", "row", "col"])
@pytest.mark.parametrize("layout", ["compact", "swizzled"])
@pytest.mark.parametrize("rounding", ["rne", "sr"])
@pytest.mark.parametrize("block", ["1d", "2d"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_option_matrix(dtype, block, rounding, layout, orient):
    rows, cols = (384, 640) if layout == "swizzled" else (272, 400)
    seed = zlib.crc32(f"{dtype}/{block}/{rounding}/{layout}/{orient}".encode()) % 1000
    x = make_input(dtype, rows, cols, seed)
    rowwise, columnwise = ORIENT[orient]
    kw = dict(block_2d=block == "2d", stochastic=rounding == "sr", sr_seed=seed)
    got = run_quantize(x, rowwise=rowwise, columnwise=columnwise, swizzled=layout == "swizzled", **kw)
    ref = O.quantize(x, rowwise=rowwise, columnwise=columnwise, **kw)
    for side, on in (("row", rowwise), ("col", columnwise)):
        if not on:
            assert got[f"{side}_data"] is None
            continue
        assert np.array_equal(got[f"{side}_data"], ref[f"{side}_data"]), side
        want = O.swizzle_scales(ref[f"{side}_scales"]) if layout == "swizzled" else ref[f"{side}_scales"].ravel()
        assert np.array_equal(got[f"{side}_scales"].ravel(), want), side
        assert np.array_equal(got[f"amax_{side}"], ref[f"amax_{side}"]), side


@pytest.mark.parametrize("tvals", ["fp32", "bf16"])
@pytest.mark.parametrize("orient", ["both", "col"])
@pytest.mark.parametrize("layout", ["compact", "swizzled"])
@pytest.mark.parametrize("rounding", ["rne", "sr"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rht_option_matrix(dtype, rounding, layout, orient, tvals):
    rows, cols = (384, 640) if layout == "swizzled" else (272, 400)
    seed = zlib.crc32(f"rht/{dtype}/{rounding}/{layout}/{orient}/{tvals}".encode()) % 1000
    x = make_input(dtype, rows, cols, seed)
    mask = W.rht_sign_mask(seed)
    rowwise, columnwise = ORIENT[orient]
    bf16 = tvals == "bf16"
    kw = dict(stochastic=rounding == "sr", sr_seed=seed)
    got = run_quantize(x, rowwise=rowwise, columnwise=columnwise, swizzled=layout == "swizzled", rht=True,
                       rht_sign_mask=mask, rht_bf16=bf16, **kw)
    a_row, a_col = O.compute_amax(x, O.AMAX_RHT_BF16 if bf16 else O.AMAX_RHT, mask)
    g_col = float(got["amax_col"][0])
    if bf16:
        # BF16 values: a one-step difference is possible when the binary32
        # transform lands next to a rounding midpoint; the rest is then
        # checked against the oracle given the GPU's amax
        assert abs(g_col - float(a_col[0])) <= 2.0 ** (np.frexp(np.float32(a_col[0]))[1] - 8)
        a_col = got["amax_col"]
    else:
        assert abs(g_col - float(a_col[0])) <= 1e-5 * float(a_col[0])
    ref = O.quantize(x, rowwise=rowwise, columnwise=columnwise, rht=True, rht_bf16=bf16, sign_mask=mask,
                     amax_row=a_row, amax_col=a_col, **kw)
    if rowwise:  # plain side: bit-exact
        assert np.array_equal(got["row_data"], ref["row_data"])
        want = O.swizzle_scales(ref["row_scales"]) if layout == "swizzled" else ref["row_scales"].ravel()
        assert np.array_equal(got["row_scales"].ravel(), want)
        assert got["amax_row"][0] == a_row[0]
    # column-wise RHT side: codes and scales may differ by one step in at
    # most 0.01% of places (transform rounding)
    d = e2m1_step_distance(codes(got["col_data"]), codes(ref["col_data"]))
    assert d.max() <= 1 and np.count_nonzero(d) <= max(1, 1e-4 * d.size)
    want = O.swizzle_scales(ref["col_scales"]) if layout == "swizzled" else ref["col_scales"].ravel()
    gs, rs = got["col_scales"].ravel().astype(np.int32), want.astype(np.int32)
    assert np.abs(gs - rs).max() <= 1 and np.count_nonzero(gs != rs) <= max(1, 1e-4 * gs.size)
