"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Deterministic paths (amax, scales, FP4 bytes, swizzle permutation, dequant)
must match bit for bit. The column-wise RHT side is held to the stated
tolerances: transformed values within 1e-5 of the group's max|t|, the
column amax within 1e-5 relative, and at most 0.01% of codes or scales
different, each by one grid step.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_05_amd as nv
import oracle as O
import workloads as W
from gpu_helpers import DEV, codes, e2m1_step_distance, host, run_quantize, to_device

pytestmark = pytest.mark.gpu


def assert_matches(got, ref, *, swizzled=False, what=""):
    for side in ("row", "col"):
        if ref[f"{side}_data"] is None:
            assert got[f"{side}_data"] is None
            continue
        gd, rd = got[f"{side}_data"], ref[f"{side}_data"]
        assert gd.shape == rd.shape
        bad = np.flatnonzero(gd.ravel() != rd.ravel())
        assert bad.size == 0, f"{what} {side} data: {bad.size} bytes differ, first at {bad[:5]}"
        rs = O.swizzle_scales(ref[f"{side}_scales"]) if swizzled else ref[f"{side}_scales"].ravel()
        bad = np.flatnonzero(got[f"{side}_scales"].ravel() != rs)
        assert bad.size == 0, f"{what} {side} scales: {bad.size} differ, first at {bad[:5]}"
        np.testing.assert_array_equal(got[f"amax_{side}"], ref[f"amax_{side}"], err_msg=f"{what} {side} amax")


def check(x, *, rowwise=True, columnwise=True, swizzled=False, block_2d=False, stochastic=False, sr_seed=0,
          row_scaled=False, use_workspace=True, amax_path=0, what=""):
    got = run_quantize(x, rowwise=rowwise, columnwise=columnwise, swizzled=swizzled, block_2d=block_2d,
                       stochastic=stochastic, sr_seed=sr_seed, row_scaled=row_scaled, use_workspace=use_workspace,
                       amax_path=amax_path)
    ref = O.quantize(x, rowwise=rowwise, columnwise=columnwise, block_2d=block_2d, stochastic=stochastic,
                     sr_seed=sr_seed, row_scaled=row_scaled)
    assert_matches(got, ref, swizzled=swizzled, what=what)
    return got, ref


# ---------------------------------------------------------------------------
# 1D quantize, both orientations (workload c1 and ragged shapes)
# ---------------------------------------------------------------------------

def test_c1_1024x1024_bf16_1d_compact():
    check(W.c1(), what="c1")


@pytest.mark.parametrize("shape,dtype", [((272, 400), "bf16"), ((208, 336), "fp32"), ((16, 16), "bf16"),
                                         ((144, 1040), "fp32"), ((1040, 144), "bf16")])
def test_1d_ragged_tiles(shape, dtype):
    x = W.randn_bf16(*shape, 21) if dtype == "bf16" else W.gaussian_fp32(*shape, 21, scale=5.0)
    check(x, what=f"{shape} {dtype}")


@pytest.mark.parametrize("shape,dtype", [((100, 160), "bf16"), ((37, 48), "fp32"), ((1, 8192), "bf16")])
def test_rowwise_only_any_row_count(shape, dtype):
    x = W.randn_bf16(*shape, 22) if dtype == "bf16" else W.gaussian_fp32(*shape, 22)
    check(x, columnwise=False, what=f"row-only {shape}")


def test_columnwise_only():
    check(W.randn_bf16(176, 272, 23), rowwise=False, what="col-only")


# ---------------------------------------------------------------------------
# 2D (16x16) blocks, compact and GEMM-swizzled (workload c2)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("swizzled", [False, True])
def test_2d_small(swizzled):
    check(W.c2(rows=256, cols=384, seed=31), block_2d=True, swizzled=swizzled, what="2d small")


def test_2d_fp32_ragged():
    check(W.gaussian_fp32(208, 336, 32, scale=100.0), block_2d=True, what="2d fp32")


def test_c2_8192x5120_2d_swizzled_full():
    x = W.c2()
    got, ref = check(x, block_2d=True, swizzled=True, what="c2")
    # 16x16 blocks: the column-wise codes are the transpose of the row-wise ones
    assert np.array_equal(codes(got["col_data"]), codes(got["row_data"]).T)


def test_1d_swizzled():
    check(W.randn_bf16(256, 384, 33), swizzled=True, what="1d swizzled")


# ---------------------------------------------------------------------------
# Dual-amax sequence on the tail shape (workload c3): one output reused.
# ---------------------------------------------------------------------------

def test_c3_amax_sequence_reused_output():
    xs = W.c3()
    rows, cols = xs[0].shape
    row = nv.empty_orientation(rows, cols, DEV)
    col = nv.empty_orientation(cols, rows, DEV)
    for m, x in zip(W.C3_MAXIMA, xs):
        nv.nvfp4_quantize(to_device(x), row, col, nv.make_config())
        torch.cuda.synchronize()
        # both buffers hold exactly the input maximum after every call
        assert host(row.amax)[0] == m and host(col.amax)[0] == m, m
        ref = O.quantize(x)
        got = {"row_data": host(row.data), "row_scales": host(row.scales), "amax_row": host(row.amax),
               "col_data": host(col.data), "col_scales": host(col.scales), "amax_col": host(col.amax)}
        assert_matches(got, ref, what=f"c3 max {m}")


# ---------------------------------------------------------------------------
# Row-scaled (per-row amax, workload c4)
# ---------------------------------------------------------------------------

def test_c4_rowscaled_full():
    check(W.c4(), columnwise=False, row_scaled=True, what="c4")


@pytest.mark.parametrize("shape", [(5, 16), (3, 10000), (64, 8208)])
def test_rowscaled_row_lengths(shape):
    # rows shorter than a workgroup, and rows longer than the register-resident part
    check(W.c4(rows=shape[0], cols=shape[1], seed=41), columnwise=False, row_scaled=True, what=f"rowscaled {shape}")


def test_rowscaled_fp32_full():
    # c4's shape with FP32 input, every byte against the oracle
    x = W.gaussian_fp32(4096, 8192, 45, scale=2.0)
    x *= np.exp(2.0 * W.gaussian_fp32(4096, 1, 46)).astype(np.float32)  # per-row magnitudes, as c4
    check(x, columnwise=False, row_scaled=True, what="rowscaled fp32 4096x8192")


@pytest.mark.parametrize("stochastic", [False, True], ids=["rne", "sr"])
@pytest.mark.parametrize("shape", [(5, 16), (7, 784), (3, 10000), (64, 8208), (40, 8192)])
def test_rowscaled_fp32_row_lengths(shape, stochastic):
    # FP32 rows load as 16-byte pieces and are regrouped into whole blocks
    # by a transpose over lane quads: short rows, a partial last group of
    # scale codes, whole 8192-column rows and rows past the register part
    x = W.gaussian_fp32(shape[0], shape[1], 44, scale=3.0)
    check(x, columnwise=False, row_scaled=True, stochastic=stochastic, sr_seed=23, what=f"rowscaled fp32 {shape}")


@pytest.mark.parametrize("shape", [(48, 784), (8, 8240), (16, 4096)])
def test_rowscaled_bf16_sr(shape):
    # BF16 rows are loaded in 16-byte pieces and regrouped into whole blocks
    # between lane pairs: the stochastic-rounding byte index of every block,
    # a partial last group of scale codes and the part beyond 8192 columns
    check(W.c4(rows=shape[0], cols=shape[1], seed=43), columnwise=False, row_scaled=True, stochastic=True, sr_seed=21,
          what=f"rowscaled bf16 sr {shape}")


def test_rowscaled_fp32_sr():
    x = W.gaussian_fp32(33, 1024, 42, scale=3.0)
    check(x, columnwise=False, row_scaled=True, stochastic=True, sr_seed=9, what="rowscaled sr")


# ---------------------------------------------------------------------------
# Stochastic rounding (deterministic given the seed: bit-exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("block_2d", [False, True])
def test_sr_small(block_2d):
    check(W.randn_bf16(256, 384, 51), stochastic=True, sr_seed=5, block_2d=block_2d, what="sr")


# ---------------------------------------------------------------------------
# E2M1 encoding over every BF16 value: with amax 6 and a 6 in every block
# the block multiplier is exactly 1, so v' = v.
# ---------------------------------------------------------------------------

def _unit_multiplier_tensor(vals: np.ndarray):
    """Blocks [6, v0..v14], [6, v15..v29], ...; returns (x, number of such blocks)."""
    vals = vals[np.abs(vals) <= 6.0]
    n = (vals.size + 14) // 15
    blocks = np.zeros((n, 16), np.float32)
    blocks[:, 0] = 6.0
    flat = blocks[:, 1:].reshape(-1)
    flat[:vals.size] = vals
    blocks[:, 1:] = flat.reshape(n, 15)
    cols = 256
    rows = (n * 16 + cols - 1) // cols
    rows = (rows + 15) // 16 * 16
    x = np.zeros(rows * cols, np.float32)
    x[:blocks.size] = blocks.ravel()
    return x.reshape(rows, cols), n


@pytest.mark.parametrize("stochastic", [False, True])
def test_e2m1_every_bf16_value(stochastic):
    allv = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    allv = allv[np.isfinite(allv)]
    x, nblocks = _unit_multiplier_tensor(allv)
    got = run_quantize(x, columnwise=False, stochastic=stochastic, sr_seed=77)
    ref = O.quantize(x, columnwise=False, stochastic=stochastic, sr_seed=77)
    assert np.all(ref["row_scales"].ravel()[:nblocks] == 0x7E)  # e == 1 in every data block
    assert_matches(got, ref, what="e2m1 sweep")


def test_e2m1_fp32_near_decision_points():
    pts = np.array([0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0], np.float32)
    u = (pts.view(np.uint32)[:, None].astype(np.int64) + np.arange(-200, 201)[None, :]).ravel()
    v = u.astype(np.uint32).view(np.float32)
    v = np.concatenate([v, -v, np.float32([0.0, -0.0, 1e-40, -1e-40])])
    x, _ = _unit_multiplier_tensor(v)
    check(x, columnwise=False, what="fp32 decision points")
    check(x, columnwise=False, stochastic=True, sr_seed=3, what="fp32 decision points sr")


# ---------------------------------------------------------------------------
# RHT column-wise side (workload c5) and its transform values
# ---------------------------------------------------------------------------

def _rht_compare(x, mask, stochastic, sr_seed, use_workspace=True):
    got = run_quantize(x, rht=True, rht_sign_mask=mask, stochastic=stochastic, sr_seed=sr_seed,
                       use_workspace=use_workspace)
    a_row, a_col = O.compute_amax(x, O.AMAX_RHT, mask)
    ref = O.quantize(x, rht=True, sign_mask=mask, stochastic=stochastic, sr_seed=sr_seed, amax_row=a_row,
                     amax_col=a_col)
    # row-wise side: plain, bit-exact
    assert np.array_equal(got["row_data"], ref["row_data"])
    assert np.array_equal(got["row_scales"], ref["row_scales"].ravel())
    assert got["amax_row"][0] == ref["amax_row"][0]
    # column-wise side: tolerances
    assert abs(float(got["amax_col"][0]) - float(a_col[0])) <= 1e-5 * float(a_col[0])
    gc, rc = codes(got["col_data"]), codes(ref["col_data"])
    d = e2m1_step_distance(gc, rc)
    assert d.max() <= 1, "column-wise codes differ by more than one grid step"
    assert np.count_nonzero(d) <= 1e-4 * d.size, f"{np.count_nonzero(d)} of {d.size} codes differ"
    gs = got["col_scales"].astype(np.int32)
    rs = ref["col_scales"].ravel().astype(np.int32)
    assert np.abs(gs - rs).max() <= 1
    assert np.count_nonzero(gs != rs) <= 1e-4 * gs.size
    return got, ref


def test_rht_values_within_tolerance():
    x, mask, _ = W.c5(rows=512, cols=1024)
    t = torch.empty((1024, 512), dtype=torch.float32, device=DEV)
    nv.nvfp4_debug_rht_colwise(to_device(x), mask, t)
    torch.cuda.synchronize()
    tg = host(t)
    tr = O.rht_colwise(x, mask)
    gmax = np.abs(tr).reshape(1024, 32, 16).max(-1, keepdims=True)
    err = np.abs(tg - tr).reshape(1024, 32, 16)
    assert np.all(err <= 1e-5 * gmax)


def test_rht_small_rne():
    x, mask, _ = W.c5(rows=256, cols=512)
    _rht_compare(x, mask, False, 0)


def test_c5_rht_sr_full():
    x, mask, seed = W.c5()
    got, ref = _rht_compare(x, mask, True, seed)
    assert got["amax_row"][0] == 200.0


# ---------------------------------------------------------------------------
# Dequantize
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("swizzled", [False, True])
def test_dequantize_matches_oracle(swizzled):
    x = W.c2(rows=256, cols=512, seed=61)
    xd = to_device(x)
    row, col = nv.quantize(xd, cfg=nv.make_config(swizzled=swizzled))
    layout = nv.NVFP4_SCALES_GEMM_SWIZZLED if swizzled else nv.NVFP4_SCALES_COMPACT
    y = torch.empty((256, 512), dtype=torch.float32, device=DEV)
    yc = torch.empty((512, 256), dtype=torch.float32, device=DEV)
    nv.nvfp4_dequantize(row, 256, 512, layout, False, y)
    nv.nvfp4_dequantize(col, 512, 256, layout, False, yc)
    torch.cuda.synchronize()
    ref = O.quantize(x)
    np.testing.assert_array_equal(host(y), O.dequantize(ref["row_data"], ref["row_scales"], ref["amax_row"], 256, 512))
    np.testing.assert_array_equal(host(yc), O.dequantize(ref["col_data"], ref["col_scales"], ref["amax_col"], 512, 256))


def test_dequantize_rowscaled():
    x = W.c4(rows=64, cols=512, seed=62)
    row, _ = nv.quantize(to_device(x), columnwise=False, cfg=nv.make_config(row_scaled=True))
    y = torch.empty((64, 512), dtype=torch.float32, device=DEV)
    nv.nvfp4_dequantize(row, 64, 512, nv.NVFP4_SCALES_COMPACT, True, y)
    torch.cuda.synchronize()
    ref = O.quantize(x, columnwise=False, row_scaled=True)
    np.testing.assert_array_equal(host(y), O.dequantize(ref["row_data"], ref["row_scales"], ref["amax_row"], 64, 512,
                                                        row_scaled=True))


# ---------------------------------------------------------------------------
# Amax entry point, explicit amax, noop, empty input, guard bands, determinism
# ---------------------------------------------------------------------------

def test_compute_amax_modes():
    x = W.c4(rows=64, cols=256, seed=71)
    xd = to_device(x)
    a = torch.full((1,), 7.0, device=DEV)
    b = torch.full((1,), 7.0, device=DEV)
    nv.nvfp4_compute_amax(xd, a, b)
    ref_a, _ = O.compute_amax(x)
    torch.cuda.synchronize()
    assert host(a)[0] == ref_a[0] and host(b)[0] == ref_a[0]
    nv.nvfp4_compute_amax(xd, a, a)  # equal pointers: one buffer
    torch.cuda.synchronize()
    assert host(a)[0] == ref_a[0]
    r = torch.empty((64,), device=DEV)
    nv.nvfp4_compute_amax(xd, r, None, nv.make_config(row_scaled=True))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(r), O.compute_amax(x, O.AMAX_PER_ROW)[0])
    mask = 0x1234
    nv.nvfp4_compute_amax(xd, a, b, nv.make_config(rht=True, rht_sign_mask=mask))
    torch.cuda.synchronize()
    ra, rb = O.compute_amax(x, O.AMAX_RHT, mask)
    assert host(a)[0] == ra[0]
    assert abs(host(b)[0] - rb[0]) <= 1e-5 * rb[0]


def test_explicit_amax_is_used():
    x = W.gaussian_fp32(128, 256, 72)
    xd = to_device(x)
    row = nv.empty_orientation(128, 256, DEV)
    col = nv.empty_orientation(256, 128, DEV)
    row.amax.fill_(100.0)
    col.amax.fill_(3.0)
    nv.nvfp4_quantize(xd, row, col, nv.make_config(compute_amax=False))
    torch.cuda.synchronize()
    ref = O.quantize(x, amax_row=np.float32([100.0]), amax_col=np.float32([3.0]))
    got = {"row_data": host(row.data), "row_scales": host(row.scales), "amax_row": host(row.amax),
           "col_data": host(col.data), "col_scales": host(col.scales), "amax_col": host(col.amax)}
    assert_matches(got, ref, what="explicit amax")


@pytest.mark.parametrize("mode", ["plain", "2d", "rht", "rowscaled"])
def test_noop_writes_nothing(mode):
    x = to_device(W.randn_bf16(128, 256, 73))
    noop = torch.ones((1,), device=DEV)
    rs = mode == "rowscaled"
    row = nv.empty_orientation(128, 256, DEV, 128 if rs else 1)
    col = None if rs else nv.empty_orientation(256, 128, DEV)
    bufs = [row.data, row.scales, row.amax] + ([] if col is None else [col.data, col.scales, col.amax])
    for i, t in enumerate(bufs):
        t.view(torch.uint8).fill_(0xA5 - i)
    before = [host(t).copy() for t in bufs]
    cfg = nv.make_config(block_2d=mode == "2d", rht=mode == "rht", row_scaled=rs, noop=noop)
    nv.nvfp4_quantize(x, row, col, cfg)
    nv.nvfp4_compute_amax(x, row.amax, None if col is None else col.amax,
                          nv.make_config(row_scaled=rs, rht=mode == "rht", noop=noop))
    torch.cuda.synchronize()
    for b0, t in zip(before, bufs):
        assert np.array_equal(b0, host(t))
    noop.zero_()  # 0.0 is not the noop value: the call runs
    nv.nvfp4_quantize(x, row, col, cfg)
    torch.cuda.synchronize()
    assert not np.array_equal(before[0], host(row.data))


def test_empty_input_writes_zero_amax():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    row = nv.empty_orientation(0, 64, DEV)
    col = nv.empty_orientation(64, 0, DEV)
    row.amax.fill_(5.0)
    col.amax.fill_(5.0)
    nv.nvfp4_quantize(x, row, col)
    torch.cuda.synchronize()
    assert host(row.amax)[0] == 0.0 and host(col.amax)[0] == 0.0


def test_zero_and_tiny_inputs():
    check(np.zeros((64, 128), np.float32), what="zeros")
    tiny = (W.gaussian_fp32(64, 128, 74) * np.float32(1e-38)).astype(np.float32)
    check(tiny, what="tiny")
    huge = (W.gaussian_fp32(64, 128, 75) * np.float32(1e37)).astype(np.float32)
    check(huge, what="huge")


def test_outputs_stay_inside_their_buffers():
    rows, cols = 272, 400
    x = W.randn_bf16(rows, cols, 76)
    guard = 4096

    def guarded(n):
        t = torch.full((n + 2 * guard,), 0x5A, dtype=torch.uint8, device=DEV)
        return t, t[guard:guard + n]

    rd_all, rd = guarded(rows * cols // 2)
    rs_all, rs = guarded(rows * cols // 16)
    cd_all, cd = guarded(rows * cols // 2)
    cs_all, cs = guarded(rows * cols // 16)
    row = nv.Orientation(rd, rs, torch.empty(1, device=DEV))
    col = nv.Orientation(cd, cs, torch.empty(1, device=DEV))
    nv.nvfp4_quantize(to_device(x), row, col)
    torch.cuda.synchronize()
    for t_all in (rd_all, rs_all, cd_all, cs_all):
        h = host(t_all)
        assert np.all(h[:guard] == 0x5A) and np.all(h[-guard:] == 0x5A)
    ref = O.quantize(x)
    assert np.array_equal(host(rd), ref["row_data"].ravel())
    assert np.array_equal(host(cs), ref["col_scales"].ravel())


def test_deterministic_across_runs():
    x = W.c2(rows=512, cols=640, seed=77)
    outs = [run_quantize(x, block_2d=True, swizzled=True) for _ in range(3)]
    outs += [run_quantize(x, stochastic=True, sr_seed=1) for _ in range(2)]
    for k in ("row_data", "row_scales", "col_data", "col_scales", "amax_row", "amax_col"):
        assert np.array_equal(outs[0][k], outs[1][k]) and np.array_equal(outs[0][k], outs[2][k])
        assert np.array_equal(outs[3][k], outs[4][k])


# ---------------------------------------------------------------------------
# The two ways of reducing a computed per-tensor amax: zeroing pass + atomic
# max (no workspace) and per-workgroup maxima in a workspace reduced by the
# cast kernel. Both must give the oracle's bytes.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["1d", "2d_swizzled", "fp32_ragged", "row_only", "col_only", "sr"])
@pytest.mark.parametrize("use_workspace", [True, False, "two_pass", "single_pass"])
def test_amax_reduction_paths(case, use_workspace):
    if case == "1d":
        x, kw = W.c1(), {}
    elif case == "2d_swizzled":
        x, kw = W.c2(rows=640, cols=768, seed=90), dict(block_2d=True, swizzled=True)
    elif case == "fp32_ragged":
        x, kw = W.gaussian_fp32(208, 1040, 91), {}
    elif case == "row_only":
        x, kw = W.randn_bf16(100, 272, 92), dict(columnwise=False)
    elif case == "col_only":
        x, kw = W.randn_bf16(96, 272, 93), dict(rowwise=False)
    else:
        x, kw = W.randn_bf16(256, 512, 94), dict(stochastic=True, sr_seed=11)
    if use_workspace in ("two_pass", "single_pass"):
        path = nv.NVFP4_AMAX_PATH_TWO_PASS if use_workspace == "two_pass" else nv.NVFP4_AMAX_PATH_SINGLE_PASS
        use_workspace, kw = True, dict(kw, amax_path=path)
    check(x, use_workspace=use_workspace, what=f"{case} workspace={use_workspace}", **kw)


@pytest.mark.parametrize("use_workspace", [True, False])
def test_rht_amax_reduction_paths(use_workspace):
    _rht_compare(W.randn_bf16(512, 768, 95), W.rht_sign_mask(95), False, 0, use_workspace)


def _quantize_with(xd, cfg, rowwise=True, columnwise=True):
    rows, cols = xd.shape
    row = nv.empty_orientation(rows, cols, DEV) if rowwise else None
    col = nv.empty_orientation(cols, rows, DEV) if columnwise else None
    nv.nvfp4_quantize(xd, row, col, cfg)
    torch.cuda.synchronize()
    return [host(t) for o in (row, col) if o is not None for t in (o.data, o.scales, o.amax)]


def test_workspace_reuse_reads_only_this_calls_maxima():
    # A call that leaves many large maxima in the workspace, then a smaller
    # input with a smaller amax and fewer workgroups through the same workspace.
    ws = nv.empty_workspace(DEV)
    big = (W.randn_bf16(2048, 4096, 96), 2048, 4096)
    small = W.randn_bf16(128, 256, 97)
    cfg = nv.make_config(workspace=ws)
    _quantize_with(to_device(big[0]) * 100.0, cfg)
    got = _quantize_with(to_device(small), cfg)
    ref = O.quantize(small)
    for g, k in zip(got, ("row_data", "row_scales", "amax_row", "col_data", "col_scales", "amax_col")):
        assert np.array_equal(g.ravel(), ref[k].ravel()), k


@pytest.mark.parametrize("case", ["fp32_2112_chunks", "rht_2064_units"])
def test_workspace_when_workgroups_loop(case):
    # More reduction units than workspace entries (2048): workgroups of the
    # amax pass take several units. The largest magnitude sits in the last
    # unit. Compared with the atomic path (one unit per workgroup), bit for bit,
    # and the plain amax with torch's max.
    g = torch.Generator(device=DEV).manual_seed(98)
    if case == "fp32_2112_chunks":
        rows, cols = 8192, 8448  # 17.3M 16-byte vectors = 2112 chunks of 8192
        xd = torch.randn((rows, cols), generator=g, device=DEV, dtype=torch.float32)
        kw = {}
    else:
        rows, cols = 33024, 4096  # 2064 groups of 16 rows, several RHT amax units each
        xd = torch.randn((rows, cols), generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
        kw = dict(rht=True, rht_sign_mask=0x5A3C)
    xd[-1, -3] = -1000.0
    ws = nv.empty_workspace(DEV)
    with_ws = _quantize_with(xd, nv.make_config(workspace=ws, **kw))
    atomic = _quantize_with(xd, nv.make_config(**kw))
    for a, b in zip(with_ws, atomic):
        assert np.array_equal(a, b)
    assert with_ws[2][0] == 1000.0


SCRATCH_BYTES = 16384  # the workspace's partials arrays; the arrival counters follow


@pytest.mark.parametrize("mode", ["2d_swizzled", "1d_sr", "rht", "rowscaled", "2d_swizzled_ws", "rht_ws",
                                  "2d_swizzled_ws_two_pass", "1d_ws_single_pass"])
def test_graph_capture_replays_match_eager(mode):
    # The calls queue kernels only (no memset, no allocation, no sync), so a
    # captured graph must reproduce the eager result on every replay, with
    # other work and synchronizations between the replays.
    x = W.c2(rows=256, cols=384, seed=81)
    xd = to_device(x)
    ws = nv.empty_workspace(DEV)
    cfg = {"2d_swizzled": nv.make_config(block_2d=True, swizzled=True),
           "1d_sr": nv.make_config(stochastic=True, sr_seed=3),
           "rht": nv.make_config(rht=True, rht_sign_mask=0x9A5C),
           "rowscaled": nv.make_config(row_scaled=True),
           "2d_swizzled_ws": nv.make_config(block_2d=True, swizzled=True, workspace=ws),
           "rht_ws": nv.make_config(rht=True, rht_sign_mask=0x9A5C, workspace=ws),
           "2d_swizzled_ws_two_pass": nv.make_config(block_2d=True, swizzled=True, workspace=ws,
                                                     amax_path=nv.NVFP4_AMAX_PATH_TWO_PASS),
           "1d_ws_single_pass": nv.make_config(workspace=ws, amax_path=nv.NVFP4_AMAX_PATH_SINGLE_PASS)}[mode]
    rs = mode == "rowscaled"
    row = nv.empty_orientation(256, 384, DEV, 256 if rs else 1)
    col = None if rs else nv.empty_orientation(384, 256, DEV)
    outs = [row.data, row.scales, row.amax] + ([] if col is None else [col.data, col.scales, col.amax])
    nv.nvfp4_quantize(xd, row, col, cfg)
    torch.cuda.synchronize()
    eager = [host(t).copy() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        nv.nvfp4_quantize(xd, row, col, cfg, s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs + [ws[:SCRATCH_BYTES]]:  # the workspace's scratch part, not its arrival counters
            t.view(torch.uint8).fill_(0x33 + rep)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, t in zip(eager, outs):
            assert np.array_equal(e, host(t)), (mode, rep)


@pytest.mark.parametrize("mode", ["2d_ws", "rowscaled"])
def test_cast_events_bracket_the_cast_kernel(mode):
    import ctypes

    x = to_device(W.c2(rows=1024, cols=2048, seed=99))
    rs = mode == "rowscaled"
    ws = nv.empty_workspace(DEV)
    cfg = nv.make_config(row_scaled=True) if rs else nv.make_config(block_2d=True, workspace=ws)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * 2)(ev[0].cuda_event, ev[1].cuda_event)
    timed = nv.nvfp4_config_t.from_buffer_copy(cfg)
    timed.cast_events = ctypes.cast(handles, ctypes.c_void_p).value
    outs = []
    for c in (cfg, timed):
        row = nv.empty_orientation(1024, 2048, DEV, 1024 if rs else 1)
        col = None if rs else nv.empty_orientation(2048, 1024, DEV)
        nv.nvfp4_quantize(x, row, col, c)
        torch.cuda.synchronize()
        outs.append([host(t) for o in (row, col) if o is not None for t in (o.data, o.scales, o.amax)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    ms = ev[0].elapsed_time(ev[1])
    assert 0.0 < ms < 100.0


@pytest.mark.parametrize("stochastic", [False, True])
def test_rowscaled_zero_guard_rows(stochastic):
    # per-row zero guard ("Implement row-scaled NVFP4 fprop recipe",
    # changed-files table: the reference quantizer guards a zero amax): rows
    # of zeros (amax 0, S = 1), a row of denormals (2688 / amax overflows and
    # is clamped), huge rows and ordinary rows side by side
    x = W.gaussian_fp32(12, 256, 77, 2.0)
    x[1] = 0.0
    x[4] = -0.0
    x[5] = (W.gaussian_fp32(1, 256, 78)[0] * np.float32(1e-41)).astype(np.float32)
    x[7] = (W.gaussian_fp32(1, 256, 79)[0] * np.float32(3e37)).astype(np.float32)
    x[9, :] = 0.0
    x[9, 100] = np.float32(1.5e-45)  # a single smallest denormal
    check(x, columnwise=False, row_scaled=True, stochastic=stochastic, sr_seed=13,
          what=f"rowscaled zero guard sr={stochastic}")
