"""GPU: the dual-amax check that the "Write both NVFP4 amax buffers" page
lists among its tests (Changes). A single set of output buffers is used for
a sequence of inputs with maxima 8, 2, 0.5, 0 and 32 (falling, then zero,
then up again); after each call every requested amax buffer must hold the
input's maximum. The cases span the three output choices (rows, columns,
both), both block shapes, both input types and a 128-aligned and a ragged
shape; here also with and without a workspace, with every output byte
compared with the oracle."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_05_amd as nv
import oracle as O
import workloads as W
from gpu_helpers import DEV, host, to_device

pytestmark = pytest.mark.gpu

ORIENT = {"row": (True, False), "col": (False, True), "both": (True, True)}


@pytest.mark.parametrize("ws", [False, True], ids=["atomic", "workspace"])
@pytest.mark.parametrize("orient", ["row", "col", "both"])
@pytest.mark.parametrize("block", ["1d", "2d"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", [(256, 512), (1088, 1024)], ids=["aligned", "tail"])
def test_reused_output_across_falling_zero_rising_maxima(shape, dtype, block, orient, ws):
    rows, cols = shape
    xs = W.c3(rows, cols, seed=3)
    if dtype == "bf16":
        xs = [W.bf16_bits(torch.from_numpy(x)) for x in xs]  # the maxima are powers of two: exact in BF16
    rw, cw = ORIENT[orient]
    row = nv.empty_orientation(rows, cols, DEV) if rw else None
    col = nv.empty_orientation(cols, rows, DEV) if cw else None
    workspace = nv.empty_workspace(DEV) if ws else None
    cfg = nv.make_config(block_2d=block == "2d", workspace=workspace)
    for m, x in zip(W.C3_MAXIMA, xs):
        nv.nvfp4_quantize(to_device(x), row, col, cfg)
        torch.cuda.synchronize()
        ref = O.quantize(x, rowwise=rw, columnwise=cw, block_2d=block == "2d")
        for side, o in (("row", row), ("col", col)):
            if o is None:
                continue
            assert host(o.amax)[0] == np.float32(m), (side, m)
            assert np.array_equal(host(o.data), ref[f"{side}_data"]), (side, m)
            assert np.array_equal(host(o.scales), ref[f"{side}_scales"].ravel()), (side, m)
