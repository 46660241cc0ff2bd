"""GPU: the one-launch grouped quantize (each group's tiles hand their
maxima to the group's head workgroup through the workspace and encode from
registers) gives the bytes
of the two-launch form and of the oracle, also when the handoff wait runs
out, with one group and empty groups, at the largest group it takes, across
many calls on one workspace and through the epoch wrap."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_05_amd as nv
import oracle as O
import workloads as W
from gpu_helpers import DEV, host, to_device

pytestmark = pytest.mark.gpu

AUTO, SINGLE, TWO = nv.NVFP4_AMAX_PATH_AUTO, nv.NVFP4_AMAX_PATH_SINGLE_PASS, nv.NVFP4_AMAX_PATH_TWO_PASS
EPOCH = 8256
SLOT = 4096  # first word of the tagged slots: workgroup i's at SLOT + 2 (i mod 2048)
GROUP_DONE = 12512  # group g's done slot (tag << 32 | maximum) at GROUP_DONE + 32 g
EPOCH_LIMIT = 0xFFFFFFFF - 256


def moe_groups(n, seed, unit=128, most=4):
    """n groups of 0 .. most * unit rows (multiples of unit)."""
    return [int(m) for m in np.random.default_rng(seed).integers(0, most + 1, n) * unit]


def run(xd, groups, ws, amax_path, rowwise=True, columnwise=True, **kw):
    row, col = nv.quantize_grouped(xd, groups, rowwise=rowwise, columnwise=columnwise,
                                   cfg=nv.make_config(workspace=ws, amax_path=amax_path, **kw), use_workspace=False)
    torch.cuda.synchronize()
    out = {}
    for side, o in (("row", row), ("col", col)):
        if o is not None:
            out[f"{side}_data"] = host(o.data)
            out[f"{side}_scales"] = host(o.scales)
            out[f"amax_{side}"] = host(o.amax)
    return out


def assert_same(a, b, what=""):
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{what} {k}"


def assert_oracle(got, x, groups, what="", **kw):
    ref = O.quantize_grouped(x, groups, **kw)
    for k in got:
        assert np.array_equal(got[k].ravel(), ref[k].ravel()), f"{what} {k}"


# (name, rows per group, cols, dtype, options): MoE-like splits with empty
# groups; 1x16 and 16x16 blocks, nearest even and stochastic rounding,
# swizzled scales, UE5M3, one orientation
CASES = [
    ("bf16_1d", moe_groups(24, 1), 1024, "bf16", {}),
    ("bf16_1d_sr", moe_groups(24, 2), 1024, "bf16", dict(stochastic=True, sr_seed=11)),
    ("bf16_2d", moe_groups(20, 3), 1536, "bf16", dict(block_2d=True)),
    ("bf16_2d_sr_swizzled", moe_groups(16, 4), 2048, "bf16",
     dict(block_2d=True, stochastic=True, sr_seed=12, swizzled=True)),
    ("bf16_ue5m3", moe_groups(16, 5), 1024, "bf16", dict(scale_fmt=nv.NVFP4_SCALE_UE5M3)),
    ("bf16_1d_swizzled", moe_groups(16, 10), 1536, "bf16", dict(swizzled=True)),
    ("fp32_1d_sr_swizzled", moe_groups(10, 11), 1024, "fp32", dict(swizzled=True, stochastic=True, sr_seed=14)),
    ("fp32_1d_ragged_cols", moe_groups(12, 6, unit=16, most=24), 1008, "fp32", {}),
    ("fp32_2d_sr", moe_groups(12, 7, unit=16, most=24), 528, "fp32", dict(block_2d=True, stochastic=True, sr_seed=3)),
    ("row_only", moe_groups(24, 8), 1024, "bf16", dict(rowwise_only=True)),
    ("col_only", moe_groups(24, 9), 1024, "bf16", dict(columnwise_only=True)),
    # 64 groups x 4096 columns, 4192 tiles: more workgroups than the 2048 slots
    ("laps_sr", moe_groups(64, 6), 4096, "bf16", dict(stochastic=True, sr_seed=13)),
]


def make_input(groups, cols, dtype, seed):
    rows = sum(groups)
    if dtype == "bf16":
        return W.randn_bf16(rows, cols, seed)
    return W.gaussian_fp32(rows, cols, seed, 3.0)


def split_opts(opts):
    kw = dict(opts)
    orient = dict(rowwise=not kw.pop("columnwise_only", False), columnwise=not kw.pop("rowwise_only", False))
    return kw, orient


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_one_launch_equals_two_launches(case):
    name, groups, cols, dtype, opts = case
    kw, orient = split_opts(opts)
    x = make_input(groups, cols, dtype, 100 + len(name))
    xd = to_device(x)
    ws = nv.empty_workspace(DEV)
    fused = run(xd, groups, ws, AUTO, **orient, **kw)
    # the call takes one tag per lap of its workgroups (a head per group, one
    # or two tiles per workgroup) over the 2048 slots
    tiles = sum(-(-m // 128) * -(-cols // 128) for m in groups)
    laps = int(host(ws).view(np.uint32)[EPOCH])
    assert 1 <= laps <= -(-(tiles + len(groups)) // 2048), "the one-launch form did not run"
    if name.startswith("laps"):
        assert laps >= 2, "the call did not take more than one lap over the slots"
    two = run(xd, groups, nv.empty_workspace(DEV), TWO, **orient, **kw)
    assert_same(fused, two, name)


def test_one_launch_matches_the_oracle():
    groups = [256, 0, 128, 384, 0, 512, 128]
    x = W.randn_bf16(sum(groups), 768, 120)
    kw = dict(stochastic=True, sr_seed=4)
    got = run(to_device(x), groups, nv.empty_workspace(DEV), AUTO, **kw)
    assert_oracle(got, x, groups, "one launch", **kw)


@pytest.mark.parametrize("block_2d", [False, True], ids=["1d", "2d"])
def test_wait_that_runs_out_gives_the_same_bytes(block_2d):
    # a wait bound of one tick: most tiles take their group's maximum from
    # the input itself
    groups = moe_groups(16, 21)
    x = W.randn_bf16(sum(groups), 1024, 121)
    xd = to_device(x)
    kw = dict(block_2d=block_2d, stochastic=True, sr_seed=6)
    normal = run(xd, groups, nv.empty_workspace(DEV), AUTO, **kw)
    nv.nvfp4_debug_set_wait_ticks(1)
    try:
        forced = run(xd, groups, nv.empty_workspace(DEV), AUTO, **kw)
    finally:
        nv.nvfp4_debug_set_wait_ticks(0)
    assert_same(normal, forced, "forced fallback")
    assert_oracle(forced, x, groups, "forced fallback", **kw)


def test_single_group_and_empty_groups():
    x = W.randn_bf16(640, 896, 122)
    xd = to_device(x)
    ws = nv.empty_workspace(DEV)
    one = run(xd, [640], ws, AUTO)
    assert int(host(ws).view(np.uint32)[EPOCH]) == 1
    padded = run(xd, [0, 640, 0], ws, AUTO)
    assert int(host(ws).view(np.uint32)[EPOCH]) == 2
    for k in ("row_data", "row_scales", "col_data", "col_scales"):
        assert np.array_equal(padded[k], one[k]), k
    assert list(padded["amax_row"]) == [0.0, one["amax_row"][0], 0.0]
    assert_oracle(one, x, [640], "one group")


@pytest.mark.parametrize("rows,one_launch", [(2048, True), (2176, False)], ids=["512_tiles", "544_tiles"])
def test_largest_group_for_one_launch(rows, one_launch):
    # a group of up to 512 tiles takes the one-launch form, a larger one the
    # two-launch form; both give the same bytes
    groups = [256, rows, 128]
    xd = to_device(W.randn_bf16(sum(groups), 4096, 123))
    ws = nv.empty_workspace(DEV)
    got = run(xd, groups, ws, AUTO, stochastic=True, sr_seed=1)
    assert int(host(ws).view(np.uint32)[EPOCH]) == (1 if one_launch else 0)
    want = run(xd, groups, nv.empty_workspace(DEV), TWO, stochastic=True, sr_seed=1)
    assert_same(got, want)


def test_many_calls_on_one_workspace():
    # one-launch grouped calls and single-tensor single-pass calls take turns
    # on one workspace; each tags its slots with the next epoch
    ws = nv.empty_workspace(DEV)
    groups = moe_groups(32, 31)
    single = W.randn_bf16(1024, 1024, 130)
    for i in range(4):
        x = W.randn_bf16(sum(groups), 512, 131 + i) if i % 2 else W.c2(rows=sum(groups), cols=512, seed=131 + i)
        xd = to_device(x)
        got = run(xd, groups, ws, AUTO, stochastic=bool(i & 1), sr_seed=i)
        want = run(xd, groups, nv.empty_workspace(DEV), TWO, stochastic=bool(i & 1), sr_seed=i)
        assert_same(got, want, f"grouped call {i}")
        row = nv.empty_orientation(1024, 1024, DEV)
        nv.nvfp4_quantize(to_device(single), row, None, nv.make_config(workspace=ws, amax_path=SINGLE))
        torch.cuda.synchronize()
        assert np.array_equal(host(row.data).ravel(), O.quantize(single)["row_data"].ravel()), i
    assert int(host(ws).view(np.uint32)[EPOCH]) == 8


def test_epoch_wrap_clears_stale_slots():
    # A done slot and a workgroup slot as a call 2^32 calls earlier would
    # have left them (tag 1, a huge maximum), for a group and a workgroup
    # that the call passing the epoch limit does not have: that call clears
    # them, so the call tagged 1 after it takes neither for its own.
    ws = nv.empty_workspace(DEV)
    words = ws.view(torch.int32)
    small = [128, 256, 0, 128]  # 4096 columns: 128 workgroups
    groups = moe_groups(24, 41)
    groups[20] = 256
    x0 = W.randn_bf16(sum(small), 4096, 141)
    x = W.randn_bf16(sum(groups), 4096, 140)
    stale = (1 << 32) | 0x7F000000  # tag 1, max 2^127
    for w in (GROUP_DONE + 32 * 20, SLOT + 2 * 600):
        words[w] = stale & 0xFFFFFFFF
        words[w + 1] = stale >> 32
    words[EPOCH] = EPOCH_LIMIT - (1 << 32)  # the next call passes the limit
    torch.cuda.synchronize()
    first = run(to_device(x0), small, ws, AUTO)
    assert_oracle(first, x0, small, "before the wrap")
    assert int(host(ws).view(np.uint32)[EPOCH]) == 0
    for w in (GROUP_DONE + 32 * 20, SLOT + 2 * 600):
        assert int(words[w + 1]) == 0, f"the stale word {w} was not cleared at the wrap"
    second = run(to_device(x), groups, ws, AUTO)
    assert int(host(ws).view(np.uint32)[EPOCH]) == 1
    assert_oracle(second, x, groups, "after the wrap")
    wv = host(ws).view(np.uint32)
    for g, m in enumerate(groups):  # every group's maximum went through its done slot, tagged 1
        if m:
            d = GROUP_DONE + 32 * g
            assert (wv[d + 1], wv[d]) == (1, second["amax_row"].view(np.uint32)[g]), g


def test_graph_replays_match_eager():
    groups = moe_groups(12, 51)
    xd = to_device(W.randn_bf16(sum(groups), 512, 150))
    ws = nv.empty_workspace(DEV)
    cfg = nv.make_config(workspace=ws, stochastic=True, sr_seed=9)
    row, col = nv.quantize_grouped(xd, groups, cfg=cfg, use_workspace=False)
    torch.cuda.synchronize()
    outs = [row.data, row.scales, row.amax, col.data, col.scales, col.amax]
    eager = [host(t).copy() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        nv.nvfp4_quantize_grouped(xd, groups, row, col, cfg, s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.view(torch.uint8).fill_(0x5A + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, t in zip(eager, outs):
            assert np.array_equal(e, host(t)), rep


@pytest.mark.parametrize("fill", ["uniform", "random"])
def test_workspace_not_zero_filled_still_gives_the_oracle_bytes(fill):
    # Uniform bytes leave the exit counters equal to their bases and no slot
    # with the next tags, so the handoff runs as usual; random words fail the
    # counters' check, and then the head reads every tile itself and the
    # tiles take their group's maximum from the input. Either way the bytes
    # are the oracle's, on this call and the next.
    groups = [128, 0, 256, 128, 384]
    x = W.randn_bf16(sum(groups), 640, 160)
    xd = to_device(x)
    ws = nv.empty_workspace(DEV)
    if fill == "uniform":
        ws.fill_(0xA5)
    else:
        g = torch.Generator(device=DEV).manual_seed(161)
        ws.copy_(torch.randint(0, 256, ws.shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8))
    kw = dict(stochastic=True, sr_seed=17)
    for i in range(2):
        got = run(xd, groups, ws, AUTO, **kw)
        assert_oracle(got, x, groups, f"{fill} call {i}", **kw)


def test_one_and_two_launch_calls_alternate_on_one_workspace():
    # the two-launch form writes its per-workgroup maxima into the scratch
    # part of the same workspace; the one-launch form's tags live elsewhere
    ws = nv.empty_workspace(DEV)
    groups = moe_groups(20, 170)
    x = W.randn_bf16(sum(groups), 768, 171)
    xd = to_device(x)
    ref = O.quantize_grouped(x, groups)
    for i, path in enumerate((AUTO, TWO, AUTO, TWO, AUTO)):
        got = run(xd, groups, ws, path)
        for k in got:
            assert np.array_equal(got[k].ravel(), ref[k].ravel()), (i, k)


def test_fp32_ue5m3_sr_one_launch():
    groups = [48, 0, 208, 16, 96]
    x = W.gaussian_fp32(sum(groups), 336, 180, 2.0)
    kw = dict(stochastic=True, sr_seed=23)
    ws = nv.empty_workspace(DEV)
    got = run(to_device(x), groups, ws, AUTO, scale_fmt=nv.NVFP4_SCALE_UE5M3, **kw)
    assert int(host(ws).view(np.uint32)[EPOCH]) == 1
    assert_oracle(got, x, groups, "fp32 ue5m3 sr", scale_fmt=O.SCALE_UE5M3, **kw)
