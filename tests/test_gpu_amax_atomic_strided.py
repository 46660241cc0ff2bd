"""GPU: the amax passes without a workspace at sizes where their grids are
capped and each workgroup walks several parts of the input.

Without a workspace every amax workgroup publishes its maximum by an atomic
max on the amax buffers, so the passes run fewer, larger workgroups (at most
320 of 1024 threads for the plain amax, at most 512 for the RHT pair) and
stride over the input. A maximum must be found wherever it lies: each case
plants one value far above the rest (|x| < 8 elsewhere) at the first element,
the last one, the middle, or the first element of the last row, and the
per-tensor (and per-group) amax must be that value exactly. The RHT pair's
column-wise amax is compared with the oracle's (within 1e-5, as the other
RHT amax tests). Inputs are drawn on the GPU from a seeded generator.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_05_amd as nv
import oracle as O
import workloads as W
from gpu_helpers import DEV, host

pytestmark = pytest.mark.gpu

PLANT = 1000.0  # exact in BF16 and FP32, far above the clipped normal values


def _base(rows, cols, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.randn(rows, cols, generator=g, device=DEV).clamp_(-7.5, 7.5)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def _positions(rows, cols):
    n = rows * cols
    return {"first": 0, "last": n - 1, "middle": n // 2 + 7, "last_row": (rows - 1) * cols}


@pytest.mark.parametrize("where", ["first", "last", "middle", "last_row"])
@pytest.mark.parametrize("dtype,shape", [("bf16", (8192, 5120)), ("fp32", (4096, 5120)), ("bf16", (16368, 4112))],
                         ids=["bf16_c2", "fp32", "bf16_ragged"])
def test_plain_amax_without_workspace_finds_the_maximum(dtype, shape, where):
    rows, cols = shape
    x = _base(rows, cols, dtype, seed=701)
    sign = -1.0 if where in ("last", "last_row") else 1.0
    x.view(-1)[_positions(rows, cols)[where]] = sign * PLANT
    a = torch.full((1,), -1.0, device=DEV)
    b = torch.full((1,), -1.0, device=DEV)
    nv.nvfp4_compute_amax(x, a, b)
    torch.cuda.synchronize()
    assert host(a)[0] == np.float32(PLANT) and host(b)[0] == np.float32(PLANT), (where, host(a), host(b))


@pytest.mark.parametrize("where", ["first", "last", "middle"])
def test_rht_amax_pair_without_workspace(where):
    # 4096 x 6144: 1,536 units of 16 rows x 1024 columns, three per workgroup
    # at the 512-workgroup cap
    rows, cols = 4096, 6144
    x = _base(rows, cols, "bf16", seed=702)
    x.view(-1)[_positions(rows, cols)[where]] = PLANT
    mask = W.rht_sign_mask(702)
    a = torch.full((1,), -1.0, device=DEV)
    b = torch.full((1,), -1.0, device=DEV)
    nv.nvfp4_compute_amax(x, a, b, nv.make_config(rht=True, rht_sign_mask=mask))
    torch.cuda.synchronize()
    ra, rb = O.compute_amax(W.bf16_bits(x.cpu()), O.AMAX_RHT, mask)
    assert host(a)[0] == np.float32(PLANT) == ra[0]
    assert abs(host(b)[0] - rb[0]) <= 1e-5 * rb[0], (host(b)[0], rb[0])


@pytest.mark.parametrize("rht", [False, True], ids=["plain", "rht"])
def test_grouped_amax_without_workspace_finds_each_groups_maximum(rht):
    # MoE-like split of 16384 x 4096 BF16 (multiples of 16 rows, some empty);
    # each group gets its own planted maximum at a different place in it
    groups = [2048, 0, 5120, 16, 4080 + 16, 0, 1024, 4080]
    assert sum(groups) == 16384
    rows, cols = 16384, 4096
    x = _base(rows, cols, "bf16", seed=703)
    starts = np.concatenate([[0], np.cumsum(groups)])
    planted = []
    for g, n in enumerate(groups):
        if n == 0:
            planted.append(0.0)
            continue
        v = PLANT + 8.0 * g
        r = starts[g] + (n - 1 if g % 2 else n // 3)
        c = (cols - 1) if g % 3 == 0 else (g * 37) % cols
        x[r, c] = -v if g % 2 else v
        planted.append(v)
    mask = W.rht_sign_mask(703)
    kw = dict(rht=True, rht_sign_mask=mask) if rht else {}
    row, col = nv.quantize_grouped(x, groups, cfg=nv.make_config(workspace=None, **kw), use_workspace=False)
    torch.cuda.synchronize()
    ra = host(row.amax)
    ca = host(col.amax)
    for g, n in enumerate(groups):
        assert ra[g] == np.float32(planted[g]), (g, ra[g], planted[g])
        if not rht:
            assert ca[g] == np.float32(planted[g]), (g, ca[g], planted[g])
    if rht:
        xb = W.bf16_bits(x.cpu())
        for g, n in enumerate(groups):
            if n == 0:
                assert ca[g] == 0.0
                continue
            _, rb = O.compute_amax(xb[starts[g]:starts[g + 1]], O.AMAX_RHT, mask)
            assert abs(ca[g] - rb[0]) <= 1e-5 * rb[0], (g, ca[g], rb[0])
