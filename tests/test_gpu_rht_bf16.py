"""GPU: the RHT variant whose transformed values are rounded to BF16
(rht_bf16), against the oracle's same option.

The transformed values themselves differ from the oracle's binary64 sums by
a few binary32 ulps, so the BF16 rounding of a single value can land one
BF16 step apart (test_rht_bf16_values bounds how often); the column side is
held to the RHT tolerances. The column amax is the rounding of one maximum,
which lands a step apart only when the oracle's binary32 maximum lies within
a few ulps of a BF16 rounding boundary (about 6 in 10^5 per tensor), so it
must equal the oracle's: at the full c5 shape, and on 64 seeded tensors
under every transform unit. The codes are then compared against the oracle
with the oracle's own amaxes. The device rounding itself is compared bit for
bit with the oracle's rounding of the device's own binary32 values."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_05_amd as nv
import oracle as O
import workloads as W
from gpu_helpers import DEV, codes, e2m1_step_distance, host, run_quantize, to_device

pytestmark = pytest.mark.gpu

BF16_BIT = 1 << 16


def _bf16_step(a: float) -> float:
    """Spacing of BF16 values at magnitude a (normal range)."""
    e = np.frexp(np.float32(a))[1]
    return float(2.0 ** (e - 8))


def test_rht_bf16_values():
    x, mask, _ = W.c5(rows=512, cols=1024)
    xd = to_device(x)
    t32 = torch.empty((1024, 512), dtype=torch.float32, device=DEV)
    t16 = torch.empty_like(t32)
    nv.nvfp4_debug_rht_colwise(xd, mask, t32)
    nv.nvfp4_debug_rht_colwise(xd, mask | BF16_BIT, t16)
    torch.cuda.synchronize()
    g32, g16 = host(t32), host(t16)
    # the device rounding is the oracle's rounding of the device's own values
    assert np.array_equal(g16.view(np.uint32), O.round_bf16(g32).view(np.uint32))
    assert np.all(g16.view(np.uint32) & 0xFFFF == 0)
    # and within one BF16 step (plus the binary32 tolerance) of the oracle's BF16 values
    r16 = O.rht_colwise(x, mask, bf16=True)
    gmax = np.abs(O.rht_colwise(x, mask)).reshape(1024, 32, 16).max(-1, keepdims=True)
    err = np.abs(g16 - r16).reshape(1024, 32, 16)
    step = np.exp2(np.frexp(np.abs(r16))[1] - 8).reshape(1024, 32, 16)
    assert np.all(err <= step + 1e-5 * gmax)
    assert np.count_nonzero(err) <= 1e-3 * err.size


def _compare(x, mask, stochastic, sr_seed, use_workspace=True):
    got = run_quantize(x, rht=True, rht_bf16=True, rht_sign_mask=mask, stochastic=stochastic, sr_seed=sr_seed,
                       use_workspace=use_workspace)
    a_row, a_col = O.compute_amax(x, O.AMAX_RHT_BF16, mask)
    assert got["amax_row"][0] == a_row[0]
    g_col = float(got["amax_col"][0])
    assert np.float32(g_col).view(np.uint32) & 0xFFFF == 0
    assert g_col == float(a_col[0]), (g_col, float(a_col[0]), _bf16_step(float(a_col[0])))
    ref = O.quantize(x, rht=True, rht_bf16=True, sign_mask=mask, stochastic=stochastic, sr_seed=sr_seed,
                     amax_row=a_row, amax_col=a_col)
    assert np.array_equal(got["row_data"], ref["row_data"])
    assert np.array_equal(got["row_scales"], ref["row_scales"].ravel())
    d = e2m1_step_distance(codes(got["col_data"]), codes(ref["col_data"]))
    assert d.max() <= 1 and np.count_nonzero(d) <= 1e-4 * d.size, np.count_nonzero(d)
    gs, rs = got["col_scales"].astype(np.int32), ref["col_scales"].ravel().astype(np.int32)
    assert np.abs(gs - rs).max() <= 1 and np.count_nonzero(gs != rs) <= 1e-4 * gs.size
    return got


@pytest.mark.parametrize("use_workspace", [True, False], ids=["workspace", "atomic"])
def test_rht_bf16_rne(use_workspace):
    x, mask, _ = W.c5(rows=256, cols=512)
    _compare(x, mask, False, 0, use_workspace)


def test_rht_bf16_sr_fp32_input_ragged():
    x = W.gaussian_fp32(272, 400, 81, 3.0)
    _compare(x, W.rht_sign_mask(81), True, 6)


def test_rht_bf16_full_c5_shape():
    x, mask, seed = W.c5()
    got = _compare(x, mask, True, seed)
    assert got["amax_row"][0] == 200.0


@pytest.mark.parametrize("unit", [nv.RHT_UNIT_DEFAULT, nv.RHT_UNIT_VALU, nv.RHT_UNIT_MATRIX])
def test_rht_bf16_column_amax_agrees_on_64_tensors(unit):
    # one amax per tensor: count the tensors whose GPU column amax is not the
    # oracle's (BF16-rounded max|t|); expected about 0.004 of 64
    nv.nvfp4_debug_set_rht_unit(unit)
    try:
        differ = []
        for seed in range(64):
            x, _, _ = W.c5(rows=128, cols=256, seed=1000 + seed)
            mask = W.rht_sign_mask(2000 + seed)
            a = torch.empty(1, device=DEV)
            b = torch.empty(1, device=DEV)
            nv.nvfp4_compute_amax(to_device(x), a, b, nv.make_config(rht=True, rht_bf16=True, rht_sign_mask=mask))
            torch.cuda.synchronize()
            _, ref = O.compute_amax(x, O.AMAX_RHT_BF16, mask)
            if host(b)[0] != ref[0]:
                differ.append(seed)
    finally:
        nv.nvfp4_debug_set_rht_unit(nv.RHT_UNIT_DEFAULT)
    print(f"unit {unit}: column amax differs from the oracle on {len(differ)} of 64 tensors {differ}")
    assert differ == []


def test_rht_bf16_differs_from_fp32_only_on_the_column_side():
    x, mask, _ = W.c5(rows=256, cols=512)
    a = run_quantize(x, rht=True, rht_sign_mask=mask)
    b = run_quantize(x, rht=True, rht_bf16=True, rht_sign_mask=mask)
    for k in ("row_data", "row_scales", "amax_row"):
        assert np.array_equal(a[k], b[k]), k
    assert not np.array_equal(a["col_data"], b["col_data"])


def test_rht_bf16_grouped():
    x, _, _ = W.c5(rows=320, cols=512)
    mask = W.rht_sign_mask(82)
    groups = [64, 0, 128, 128]
    xd = to_device(x)
    row, col = nv.quantize_grouped(xd, groups, cfg=nv.make_config(rht=True, rht_bf16=True, rht_sign_mask=mask))
    torch.cuda.synchronize()
    s = 0
    for g, m in enumerate(groups):
        if m:
            r1, c1 = nv.quantize(xd[s:s + m], cfg=nv.make_config(rht=True, rht_bf16=True, rht_sign_mask=mask))
            torch.cuda.synchronize()
            assert torch.equal(col.amax[g], c1.amax[0]) and torch.equal(row.amax[g], r1.amax[0])
            assert torch.equal(col.data[s * 256:(s + m) * 256], c1.data.reshape(-1))
            assert torch.equal(col.scales[s * 32:(s + m) * 32], c1.scales)
        s += m
