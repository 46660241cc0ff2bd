"""Non-finite inputs: every amax the library computes follows the policy in
include/nvfp4.h (NaN when the covered values include a NaN, else +inf when
they include an infinity), matching the oracle, on the per-tensor (zeroing +
atomics, workspace two-pass, single-pass), per-row, per-column and RHT
paths, for BF16 and FP32 input. The data and scales of such inputs are
unspecified and not compared."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_05_amd as nv
import oracle as O
from gpu_helpers import DEV, host, to_device

pytestmark = pytest.mark.gpu

BAD = {"nan": np.nan, "inf": np.inf, "-inf": -np.inf}


def _input(dtype, bad, rows=256, cols=384):
    x = (np.random.default_rng(5).standard_normal((rows, cols)) * 2).astype(np.float32)
    x[131, 77] = BAD[bad]
    x[7, 300] = 50.0  # a large finite value elsewhere
    if dtype == "bf16":
        import workloads as W
        return W.bf16_bits(torch.from_numpy(x))
    return x


def _same(got, want):
    got, want = np.asarray(got, np.float32), np.asarray(want, np.float32)
    assert got.shape == want.shape
    assert np.array_equal(np.isnan(got), np.isnan(want)), (got, want)
    assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)]), (got, want)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("bad", sorted(BAD))
def test_per_tensor_amax(dtype, bad):
    x = _input(dtype, bad)
    want = O.compute_amax(x)[0]
    xd = to_device(x)
    a, b = torch.empty(1, device=DEV), torch.empty(1, device=DEV)
    nv.nvfp4_compute_amax(xd, a, b)
    torch.cuda.synchronize()
    _same(host(a), want)
    _same(host(b), want)
    for path in ("atomic", nv.NVFP4_AMAX_PATH_TWO_PASS, nv.NVFP4_AMAX_PATH_SINGLE_PASS):
        ws = None if path == "atomic" else nv.empty_workspace(DEV)
        cfg = nv.make_config(workspace=ws, amax_path=0 if path == "atomic" else path)
        row, col = nv.quantize(xd, cfg=cfg, use_workspace=False)
        torch.cuda.synchronize()
        _same(host(row.amax), want)
        _same(host(col.amax), want)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("bad", sorted(BAD))
def test_per_row_and_per_column_amax(dtype, bad):
    x = _input(dtype, bad)
    want_r, want_c = O.compute_amax(x, O.AMAX_PER_ROW)
    xd = to_device(x)
    rows, cols = x.shape
    a, b = torch.empty(rows, device=DEV), torch.empty(cols, device=DEV)
    nv.nvfp4_compute_amax(xd, a, b, nv.make_config(row_scaled=True))
    torch.cuda.synchronize()
    _same(host(a), want_r)
    _same(host(b), want_c)
    row, col = nv.quantize(xd, cfg=nv.make_config(row_scaled=True))
    torch.cuda.synchronize()
    _same(host(row.amax), want_r)
    _same(host(col.amax), want_c)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("bad", sorted(BAD))
@pytest.mark.parametrize("unit", [nv.RHT_UNIT_DEFAULT, nv.RHT_UNIT_VALU, nv.RHT_UNIT_MATRIX])
def test_rht_amax_pair(dtype, bad, unit):
    x = _input(dtype, bad)
    want_r, want_c = O.compute_amax(x, O.AMAX_RHT, 0x6A95)
    xd = to_device(x)
    nv.nvfp4_debug_set_rht_unit(unit)
    try:
        a, b = torch.empty(1, device=DEV), torch.empty(1, device=DEV)
        nv.nvfp4_compute_amax(xd, a, b, nv.make_config(rht=True, rht_sign_mask=0x6A95))
        row, col = nv.quantize(xd, cfg=nv.make_config(rht=True, rht_sign_mask=0x6A95))
        torch.cuda.synchronize()
    finally:
        nv.nvfp4_debug_set_rht_unit(nv.RHT_UNIT_DEFAULT)
    for r, c in ((a, b), (row.amax, col.amax)):
        _same(host(r), want_r)
        _same(host(c), want_c)
