"""GPU parity for the column-wise side of a row-scaled quantize: one amax per
input column, the column-wise tensor (the transpose) scaled along its own
rows (the quantizer prototype in the review thread of "Write both NVFP4
amax buffers" gives that amax buffer one float per input column). Bit-exact against the oracle:
per-column amax, scales, FP4 bytes, dequantized values."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_05_amd as nv
import oracle as O
import workloads as W
from gpu_helpers import DEV, host, run_quantize, to_device
from test_gpu_parity import assert_matches

pytestmark = pytest.mark.gpu


def check(x, *, rowwise=True, what="", **kw):
    got = run_quantize(x, rowwise=rowwise, columnwise=True, row_scaled=True, **kw)
    ref_kw = {k: v for k, v in kw.items() if k in ("stochastic", "sr_seed", "scale_fmt")}
    ref = O.quantize(x, rowwise=rowwise, columnwise=True, row_scaled=True, **ref_kw)
    assert_matches(got, ref, what=what)
    return got, ref


def test_c4_4096x8192_both_orientations():
    check(W.c4(), what="c4 both")


@pytest.mark.parametrize("shape,dtype", [((16, 16), "bf16"), ((48, 80), "fp32"), ((528, 1040), "bf16"),
                                         ((4112, 48), "fp32"), ((272, 4096), "bf16"), ((1024, 1056), "fp32")])
def test_ragged_shapes(shape, dtype):
    # partial column strips, partial row chunks, reduction tails
    x = W.c4(rows=shape[0], cols=shape[1], seed=81) if dtype == "bf16" else W.gaussian_fp32(*shape, 81, scale=4.0)
    print(f"rowscaled colwise {shape} {dtype}", flush=True)
    check(x, what=f"{shape} {dtype}")


def test_columnwise_only():
    check(W.c4(rows=256, cols=384, seed=82), rowwise=False, what="col only")


def test_column_magnitudes_spread_and_zero_columns():
    x = W.gaussian_fp32(160, 256, 83)
    x *= (2.0 ** np.linspace(-40, 40, 256)).astype(np.float32)[None, :]
    x[:, 7] = 0.0
    x[:, 200] = 0.0
    got, ref = check(x, what="spread")
    assert ref["amax_col"][7] == 0.0 and got["amax_col"][200] == 0.0


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_stochastic_rounding(dtype):
    x = W.c4(rows=320, cols=528, seed=84) if dtype == "bf16" else W.gaussian_fp32(320, 528, 84, scale=2.0)
    check(x, stochastic=True, sr_seed=17, what=f"sr {dtype}")


def test_ue5m3_scales():
    check(W.gaussian_fp32(96, 160, 85, scale=1e-3), scale_fmt=nv.NVFP4_SCALE_UE5M3, what="ue5m3")


def test_given_amax_is_used():
    x = W.c4(rows=64, cols=96, seed=86)
    a_row, a_col = O.compute_amax(x, O.AMAX_PER_ROW)
    a_row, a_col = a_row * 2, a_col * np.float32(0.75)  # the latter saturates some blocks
    xd = to_device(x)
    row = nv.empty_orientation(64, 96, DEV, 64)
    col = nv.empty_orientation(96, 64, DEV, 96)
    row.amax.copy_(torch.from_numpy(a_row))
    col.amax.copy_(torch.from_numpy(a_col))
    nv.nvfp4_quantize(xd, row, col, nv.make_config(row_scaled=True, compute_amax=False))
    torch.cuda.synchronize()
    ref = O.quantize(x, row_scaled=True, amax_row=a_row, amax_col=a_col)
    got = {"row_data": host(row.data), "row_scales": host(row.scales), "amax_row": host(row.amax),
           "col_data": host(col.data), "col_scales": host(col.scales), "amax_col": host(col.amax)}
    assert_matches(got, ref, what="given amax")


def test_noop_writes_nothing():
    x = W.c4(rows=64, cols=96, seed=87)
    col = nv.empty_orientation(96, 64, DEV, 96)
    col.data.fill_(0x5A)
    col.scales.fill_(0x33)
    col.amax.fill_(-1.0)
    noop = torch.ones((1,), device=DEV)
    nv.nvfp4_quantize(to_device(x), None, col, nv.make_config(row_scaled=True, noop=noop))
    torch.cuda.synchronize()
    assert np.all(host(col.data) == 0x5A) and np.all(host(col.scales) == 0x33) and np.all(host(col.amax) == -1.0)


def test_compute_amax_per_row_and_per_column():
    x = W.c4(rows=400, cols=1040, seed=88)
    xd = to_device(x)
    r = torch.full((400,), 5.0, device=DEV)
    c = torch.full((1040,), 5.0, device=DEV)
    nv.nvfp4_compute_amax(xd, r, c, nv.make_config(row_scaled=True))
    torch.cuda.synchronize()
    ra, ca = O.compute_amax(x, O.AMAX_PER_ROW)
    np.testing.assert_array_equal(host(r), ra)
    np.testing.assert_array_equal(host(c), ca)
    c.fill_(5.0)
    nv.nvfp4_compute_amax(xd, None, c, nv.make_config(row_scaled=True))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(c), ca)


def test_empty_input_zeroes_column_amax():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    c = torch.full((64,), 5.0, device=DEV)
    nv.nvfp4_compute_amax(x, None, c, nv.make_config(row_scaled=True))
    col = nv.empty_orientation(64, 0, DEV, 64)
    col.amax.fill_(5.0)
    nv.nvfp4_quantize(x, None, col, nv.make_config(row_scaled=True))
    torch.cuda.synchronize()
    assert np.all(host(c) == 0.0) and np.all(host(col.amax) == 0.0)


def test_dequantize_columnwise():
    x = W.c4(rows=128, cols=320, seed=89)
    _, col = nv.quantize(to_device(x), rowwise=False, cfg=nv.make_config(row_scaled=True))
    y = torch.empty((320, 128), dtype=torch.float32, device=DEV)
    nv.nvfp4_dequantize(col, 320, 128, nv.NVFP4_SCALES_COMPACT, True, y)
    torch.cuda.synchronize()
    ref = O.quantize(x, rowwise=False, row_scaled=True)
    np.testing.assert_array_equal(host(y), O.dequantize(ref["col_data"], ref["col_scales"], ref["amax_col"], 320, 128,
                                                        row_scaled=True))
