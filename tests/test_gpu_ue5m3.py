"""GPU: UE5M3 block scales (scale_fmt = NVFP4_SCALE_UE5M3) against the
oracle's UE5M3 option. The format is the library's reading of a name the
pages use without a definition, so this checks the GPU path against that
reading (bit for bit on the deterministic paths, to the RHT tolerances on
the RHT column side); parity with the pages themselves is unpinned."""

from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_05_amd as nv
import oracle as O
import workloads as W
from gpu_helpers import DEV, codes, e2m1_step_distance, host, run_quantize, to_device

pytestmark = pytest.mark.gpu

UE = nv.NVFP4_SCALE_UE5M3


def _input(dtype, rows, cols, seed):
    if dtype == "bf16":
        return W.c2(rows=rows, cols=cols, seed=seed)  # per-column magnitudes over 5 decades
    return W.gaussian_fp32(rows, cols, seed, scale=3.0)


@pytest.mark.parametrize("layout", ["compact", "swizzled"])
@pytest.mark.parametrize("rounding", ["rne", "sr"])
@pytest.mark.parametrize("block", ["1d", "2d"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_ue5m3_option_matrix(dtype, block, rounding, layout):
    rows, cols = (384, 640) if layout == "swizzled" else (272, 400)
    seed = zlib.crc32(f"ue5m3/{dtype}/{block}/{rounding}/{layout}".encode()) % 1000
    x = _input(dtype, rows, cols, seed)
    kw = dict(block_2d=block == "2d", stochastic=rounding == "sr", sr_seed=seed)
    got = run_quantize(x, swizzled=layout == "swizzled", scale_fmt=UE, **kw)
    ref = O.quantize(x, scale_fmt=O.SCALE_UE5M3, **kw)
    for side in ("row", "col"):
        assert np.array_equal(got[f"{side}_data"], ref[f"{side}_data"]), side
        want = O.swizzle_scales(ref[f"{side}_scales"]) if layout == "swizzled" else ref[f"{side}_scales"].ravel()
        assert np.array_equal(got[f"{side}_scales"].ravel(), want), side
        assert np.array_equal(got[f"amax_{side}"], ref[f"amax_{side}"]), side


def test_ue5m3_full_bench_shape():
    x = W.c2()
    got = run_quantize(x, block_2d=True, swizzled=True, scale_fmt=UE)
    ref = O.quantize(x, block_2d=True, scale_fmt=O.SCALE_UE5M3)
    assert np.array_equal(got["row_data"], ref["row_data"]) and np.array_equal(got["col_data"], ref["col_data"])
    assert np.array_equal(got["row_scales"], O.swizzle_scales(ref["row_scales"]))
    # the wider exponent range: c2's five decades of column scale leave no
    # zero block scale with UE5M3
    assert np.count_nonzero(ref["row_scales"] == 0) <= np.count_nonzero(O.quantize(x, block_2d=True)["row_scales"] == 0)


@pytest.mark.parametrize("stochastic", [False, True])
def test_ue5m3_rht(stochastic):
    x, mask, _ = W.c5(rows=256, cols=512)
    kw = dict(stochastic=stochastic, sr_seed=3)
    got = run_quantize(x, rht=True, rht_sign_mask=mask, scale_fmt=UE, **kw)
    a_row, a_col = O.compute_amax(x, O.AMAX_RHT, mask)
    ref = O.quantize(x, rht=True, sign_mask=mask, amax_row=a_row, amax_col=a_col, scale_fmt=O.SCALE_UE5M3, **kw)
    assert np.array_equal(got["row_data"], ref["row_data"])
    assert np.array_equal(got["row_scales"], ref["row_scales"].ravel())
    assert abs(float(got["amax_col"][0]) - float(a_col[0])) <= 1e-5 * float(a_col[0])
    d = e2m1_step_distance(codes(got["col_data"]), codes(ref["col_data"]))
    assert d.max() <= 1 and np.count_nonzero(d) <= max(1, 1e-4 * d.size)
    gs, rs = got["col_scales"].astype(np.int32), ref["col_scales"].ravel().astype(np.int32)
    assert np.abs(gs - rs).max() <= 1 and np.count_nonzero(gs != rs) <= max(1, 1e-4 * gs.size)


@pytest.mark.parametrize("stochastic", [False, True])
def test_ue5m3_rowscaled(stochastic):
    x = W.c4(rows=64, cols=8208, seed=93)  # a row longer than the register-resident part
    got = run_quantize(x, columnwise=False, row_scaled=True, stochastic=stochastic, sr_seed=4, scale_fmt=UE)
    ref = O.quantize(x, columnwise=False, row_scaled=True, stochastic=stochastic, sr_seed=4,
                     scale_fmt=O.SCALE_UE5M3)
    for k in ("row_data", "amax_row"):
        assert np.array_equal(got[k], ref[k]), k
    assert np.array_equal(got["row_scales"], ref["row_scales"].ravel())


def test_ue5m3_grouped():
    x = W.randn_bf16(400, 256, 94)
    groups = [128, 0, 16, 256]
    row, col = nv.quantize_grouped(to_device(x), groups, cfg=nv.make_config(scale_fmt=UE, stochastic=True,
                                                                           sr_seed=8))
    torch.cuda.synchronize()
    ref = O.quantize_grouped(x, groups, stochastic=True, sr_seed=8, scale_fmt=O.SCALE_UE5M3)
    for k, t in (("row_data", row.data), ("row_scales", row.scales), ("amax_row", row.amax),
                 ("col_data", col.data), ("col_scales", col.scales), ("amax_col", col.amax)):
        assert np.array_equal(host(t).ravel(), ref[k].ravel()), k


@pytest.mark.parametrize("swizzled", [False, True])
def test_ue5m3_dequantize(swizzled):
    x = W.c2(rows=256, cols=512, seed=95)
    row, col = nv.quantize(to_device(x), cfg=nv.make_config(swizzled=swizzled, scale_fmt=UE))
    layout = nv.NVFP4_SCALES_GEMM_SWIZZLED if swizzled else nv.NVFP4_SCALES_COMPACT
    y = torch.empty((256, 512), dtype=torch.float32, device=DEV)
    yc = torch.empty((512, 256), dtype=torch.float32, device=DEV)
    nv.nvfp4_dequantize(row, 256, 512, layout, False, y, scale_fmt=UE)
    nv.nvfp4_dequantize(col, 512, 256, layout, False, yc, scale_fmt=UE)
    torch.cuda.synchronize()
    ref = O.quantize(x, scale_fmt=O.SCALE_UE5M3)
    np.testing.assert_array_equal(host(y), O.dequantize(ref["row_data"], ref["row_scales"], ref["amax_row"], 256, 512,
                                                        scale_fmt=O.SCALE_UE5M3))
    np.testing.assert_array_equal(host(yc), O.dequantize(ref["col_data"], ref["col_scales"], ref["amax_col"], 512,
                                                         256, scale_fmt=O.SCALE_UE5M3))


def test_ue5m3_every_code_decodes_and_encodes():
    # blocks whose maxima walk through every UE5M3 value: with amax 61440 * 6 / 6
    # = 61440 the global scale is 6, so block max m gets sd = fl(m / 6) * 6 ~ m
    vals = np.array([O.ue5m3_value(c) for c in range(1, 0xF8)], np.float32)
    x = np.zeros((16, 16 * vals.size), np.float32)
    x[0, ::16] = vals
    x[0, 0] = 61440.0  # the tensor amax
    got = run_quantize(x, scale_fmt=UE)
    ref = O.quantize(x, scale_fmt=O.SCALE_UE5M3)
    assert np.array_equal(got["row_scales"], ref["row_scales"].ravel())
    assert np.array_equal(got["row_data"], ref["row_data"])
    assert np.array_equal(got["col_scales"], ref["col_scales"].ravel())
    assert len(set(ref["row_scales"][0].tolist())) > 200  # most codes are exercised
