"""The RHT path under each transform unit setting (nvfp4_debug_set_rht_unit:
0 default, 1 vector ALU everywhere, 2 matrix cores everywhere): parity with
the oracle within the RHT tolerances (row side bit-exact), the same bytes on
repeated calls and with or without a workspace, the grouped form included.
Values of the transform may differ between the units in the last bits, so
only the row-wise side is compared across units byte for byte."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_05_amd as nv
import workloads as W
from gpu_helpers import DEV, host, run_quantize, to_device
from test_gpu_parity import _rht_compare

pytestmark = pytest.mark.gpu

UNITS = [nv.RHT_UNIT_DEFAULT, nv.RHT_UNIT_VALU, nv.RHT_UNIT_MATRIX]


@pytest.fixture
def unit(request):
    nv.nvfp4_debug_set_rht_unit(request.param)
    yield request.param
    nv.nvfp4_debug_set_rht_unit(nv.RHT_UNIT_DEFAULT)


@pytest.mark.parametrize("unit", UNITS, indirect=True)
@pytest.mark.parametrize("stochastic", [False, True], ids=["rne", "sr"])
@pytest.mark.parametrize("use_workspace", [True, False], ids=["workspace", "atomic"])
def test_rht_parity_per_unit(unit, stochastic, use_workspace):
    print(f"rht unit {unit} stochastic {stochastic} workspace {use_workspace}", flush=True)
    x, mask, seed = W.c5(rows=512, cols=1024)
    _rht_compare(x, mask, stochastic, seed, use_workspace=use_workspace)


@pytest.mark.parametrize("unit", UNITS, indirect=True)
def test_rht_repeated_calls_give_the_same_bytes(unit):
    x, mask, seed = W.c5(rows=1024, cols=768)
    outs = [run_quantize(x, rht=True, rht_sign_mask=mask, stochastic=True, sr_seed=seed, use_workspace=ws)
            for ws in (True, True, False)]
    for k in ("row_data", "row_scales", "col_data", "col_scales", "amax_row", "amax_col"):
        assert np.array_equal(outs[0][k], outs[1][k]), k
        assert np.array_equal(outs[0][k], outs[2][k]), k


@pytest.mark.parametrize("unit", UNITS, indirect=True)
def test_grouped_rht_workspace_and_atomic_agree(unit):
    rng = np.random.default_rng(91)
    groups = [int(m) for m in rng.integers(0, 9, 48) * 16]
    R, C = sum(groups), 1024
    g = torch.Generator(device=DEV).manual_seed(92)
    x = (torch.randn((R, C), generator=g, device=DEV) * 3).to(torch.bfloat16)
    kw = dict(rht=True, rht_sign_mask=0x3C5A, stochastic=True, sr_seed=7)
    res = []
    for cfg in (nv.make_config(workspace=nv.empty_workspace(DEV), **kw), nv.make_config(**kw),
                nv.make_config(workspace=nv.empty_workspace(DEV), **kw)):
        res.append(nv.quantize_grouped(x, groups, cfg=cfg, use_workspace=False))
    torch.cuda.synchronize()
    for other in res[1:]:
        for a, b in zip(res[0], other):
            assert torch.equal(a.amax, b.amax) and torch.equal(a.data, b.data) and torch.equal(a.scales, b.scales)


def test_row_side_is_the_same_under_every_unit():
    x, mask, seed = W.c5(rows=512, cols=512)
    outs = []
    try:
        for u in UNITS:
            nv.nvfp4_debug_set_rht_unit(u)
            outs.append(run_quantize(x, rht=True, rht_sign_mask=mask, stochastic=True, sr_seed=seed))
    finally:
        nv.nvfp4_debug_set_rht_unit(nv.RHT_UNIT_DEFAULT)
    for o in outs[1:]:
        for k in ("row_data", "row_scales", "amax_row"):
            assert np.array_equal(o[k], outs[0][k]), k


def test_unknown_unit_is_rejected():
    with pytest.raises(nv.NVFP4Error) as e:
        nv.nvfp4_debug_set_rht_unit(3)
    assert e.value.status == nv.NVFP4_ERR_UNSUPPORTED
