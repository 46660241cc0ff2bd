"""Single-pass quantize: one launch in which every workgroup holds its tiles
in registers across a grid-wide handoff of the per-tensor amax through the
workspace. Checked bit for bit against the oracle and against the two-pass
form (amax pass + cast), on shapes that give 1 to 4 tiles per workgroup
(the fourth held in LDS),
ragged edges, every output choice, one workspace reused across grid sizes,
the fast wait forced to run out (nearly every workgroup then takes the slow
path: it claims the tiles of workgroups that have not started and reduces
every slot itself), grids forced beyond what can be resident at once (the
slow path must complete them), and noop.

The workspace's exit counters and their bases (words 8416 + 64 x and
8448 + 64 x, x = 0..63; 8352 and 8384 over the lines) must be equal after
every call, and the epoch (word 8256) must have advanced by one per
single-pass call: that is what lets the next call start without a reset.
The done word (64 bits at word 8288: tag << 32 | amax bits) carries the
call's tag exactly when a workgroup took the slow path."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_05_amd as nv
import oracle as O
import workloads as W
from gpu_helpers import DEV, host, to_device

pytestmark = pytest.mark.gpu

SINGLE, TWO = nv.NVFP4_AMAX_PATH_SINGLE_PASS, nv.NVFP4_AMAX_PATH_TWO_PASS

EPOCH, DONE, EXIT_TOP, EXIT_TOP_BASE, EXIT, LINES = 8256, 8288, 8352, 8384, 8416, 64
EPOCH_LIMIT = 0xFFFFFFFF - 256  # past it the last workgroup clears the tagged words and restarts at 0


def handoff_words(ws):
    """(epoch, exit counters consistent with their bases)"""
    w = host(ws).view(np.uint32)
    ok = (np.array_equal(w[EXIT:EXIT + 64 * LINES:64], w[EXIT + 32:EXIT + 32 + 64 * LINES:64])
          and w[EXIT_TOP] == w[EXIT_TOP_BASE])
    return int(w[EPOCH]), bool(ok)


def done_word(ws):
    """(tag, amax bits) of the done word"""
    w = host(ws).view(np.uint32)
    return int(w[DONE + 1]), int(w[DONE])


def run(xd, cfg, rowwise=True, columnwise=True):
    rows, cols = xd.shape
    row = nv.empty_orientation(rows, cols, DEV) if rowwise else None
    col = nv.empty_orientation(cols, rows, DEV) if columnwise else None
    nv.nvfp4_quantize(xd, row, col, cfg)
    torch.cuda.synchronize()
    out = {}
    for side, o in (("row", row), ("col", col)):
        if o is not None:
            out[f"{side}_data"] = host(o.data)
            out[f"{side}_scales"] = host(o.scales)
            out[f"amax_{side}"] = host(o.amax)
    return out


def assert_oracle(got, x, *, swizzled=False, what="", **kw):
    ref = O.quantize(x, **kw)
    for side in ("row", "col"):
        if f"{side}_data" not in got:
            continue
        assert np.array_equal(got[f"{side}_data"].ravel(), ref[f"{side}_data"].ravel()), f"{what} {side} data"
        rs = O.swizzle_scales(ref[f"{side}_scales"]) if swizzled else ref[f"{side}_scales"].ravel()
        assert np.array_equal(got[f"{side}_scales"].ravel(), rs), f"{what} {side} scales"
        assert np.array_equal(got[f"amax_{side}"], ref[f"amax_{side}"]), f"{what} {side} amax"


def assert_same(a, b, what=""):
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{what} {k}"


# (name, rows, cols, dtype, options): tile counts 64 .. 2560, so that the
# library picks 1 to 3 register tiles per workgroup, or 3 register tiles
# and one LDS tile (BF16), and 1 (FP32)
CASES = [
    ("c1_1d", 1024, 1024, "bf16", dict()),
    ("ragged_1d_fp32", 1040, 1008, "fp32", dict()),
    ("2d_6144x4096", 6144, 4096, "bf16", dict(block_2d=True)),
    ("ragged_1d_6000x4000", 6000, 4000, "bf16", dict()),
    ("1d_sr_7168x4608", 7168, 4608, "bf16", dict(stochastic=True, sr_seed=21)),
    ("c2_2d_swizzled", 8192, 5120, "bf16", dict(block_2d=True, swizzled=True)),
    ("1d_ue5m3_8192x5120", 8192, 5120, "bf16", dict(scale_fmt=nv.NVFP4_SCALE_UE5M3)),
    ("2d_sr_7168x4608", 7168, 4608, "bf16", dict(block_2d=True, stochastic=True, sr_seed=5)),
    ("2d_sr_swizzled_8192x5120", 8192, 5120, "bf16", dict(block_2d=True, swizzled=True, stochastic=True, sr_seed=9)),
    # 2401 tiles: three register tiles and one LDS tile per workgroup, ragged edges
    ("lds_tile_ragged_1d_6256x6256", 6256, 6256, "bf16", dict()),
    ("lds_tile_ragged_2d_sr_6256x6256", 6256, 6256, "bf16", dict(block_2d=True, stochastic=True, sr_seed=3)),
    ("fp32_1d_3072x3072", 3072, 3072, "fp32", dict()),
    ("fp32_2d_swizzled_2048x4096", 2048, 4096, "fp32", dict(block_2d=True, swizzled=True)),
]


def _input(name, rows, cols, dtype, seed):
    if name.startswith("c2"):
        return W.c2(rows=rows, cols=cols, seed=1)
    if dtype == "fp32":
        return W.gaussian_fp32(rows, cols, seed, scale=3.0)
    return W.randn_bf16(rows, cols, seed)


def _oracle_kw(opts):
    kw = {k: v for k, v in opts.items() if k in ("block_2d", "stochastic", "sr_seed")}
    if opts.get("scale_fmt") == nv.NVFP4_SCALE_UE5M3:
        kw["scale_fmt"] = O.SCALE_UE5M3
    return kw


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_single_pass_matches_oracle_and_two_pass(case):
    name, rows, cols, dtype, opts = case
    print(f"single pass {name} {rows}x{cols} {dtype} {opts}", flush=True)
    x = _input(name, rows, cols, dtype, 300 + rows % 97)
    xd = to_device(x)
    ws = nv.empty_workspace(DEV)
    one = run(xd, nv.make_config(workspace=ws, amax_path=SINGLE, **opts))
    assert handoff_words(ws) == (1, True), "the single-pass kernel did not run, or left its counters"
    two = run(xd, nv.make_config(workspace=ws, amax_path=TWO, **opts))
    assert handoff_words(ws) == (1, True), "the two-pass form touched the handoff words"
    assert_same(one, two, name)
    assert_oracle(one, x, swizzled=opts.get("swizzled", False), what=name, **_oracle_kw(opts))


@pytest.mark.parametrize("rowwise,columnwise", [(True, False), (False, True)])
def test_single_pass_one_orientation(rowwise, columnwise):
    x = W.randn_bf16(7168, 4608, 41)
    xd = to_device(x)
    ws = nv.empty_workspace(DEV)
    got = run(xd, nv.make_config(workspace=ws, block_2d=True, amax_path=SINGLE), rowwise, columnwise)
    assert_oracle(got, x, what="one orientation", rowwise=rowwise, columnwise=columnwise, block_2d=True)
    assert handoff_words(ws)[1]


def test_workspace_reused_across_grid_sizes():
    # one workspace through calls whose grids differ (1 .. 5 tiles per
    # workgroup, 8 .. 512 workgroups), a smaller amax after a larger one,
    # and a two-pass call in between
    ws = nv.empty_workspace(DEV)
    seq = [(8192, 5120, 1.0, {}), (128, 256, 1.0, {}), (7168, 4608, 0.01, dict(block_2d=True)),
           (1024, 1024, 1e3, dict(amax_path=TWO)), (256, 384, 2.0, dict(swizzled=False)),
           (8192, 5120, 1e-3, dict(block_2d=True, swizzled=True))]
    for i, (rows, cols, scale, opts) in enumerate(seq):
        x = W.randn_bf16(rows, cols, 500 + i)
        xd = to_device(x) * scale
        xs = host(xd.view(torch.int16)).view(np.uint16)
        got = run(xd, nv.make_config(workspace=ws, **dict(dict(amax_path=SINGLE), **opts)))
        assert_oracle(got, xs, swizzled=opts.get("swizzled", False), what=f"call {i}",
                      block_2d=opts.get("block_2d", False))
        assert handoff_words(ws) == (i + (0 if i < 3 else -1) + 1, True), f"call {i}"


@pytest.mark.parametrize("rows,cols,opts", [(512, 768, dict(block_2d=True)), (7168, 4608, {}),
                                            (6256, 6256, dict(block_2d=True))])
def test_wait_that_runs_out_gives_the_same_bytes(rows, cols, opts):
    # a fast wait bound of one tick: nearly every workgroup takes the slow
    # path (claims, then reduces every slot itself)
    x = W.randn_bf16(rows, cols, 61)
    xd = to_device(x)
    ws = nv.empty_workspace(DEV)
    normal = run(xd, nv.make_config(workspace=ws, amax_path=SINGLE, **opts))
    nv.nvfp4_debug_set_wait_ticks(1)
    try:
        forced = run(xd, nv.make_config(workspace=ws, amax_path=SINGLE, **opts))
    finally:
        nv.nvfp4_debug_set_wait_ticks(0)
    assert_same(normal, forced, "forced slow path")
    assert handoff_words(ws) == (2, True)
    assert done_word(ws) == (2, int(forced["amax_row"].view(np.uint32)[0])), "the slow path did not run"
    after = run(xd, nv.make_config(workspace=ws, amax_path=SINGLE, **opts))  # the counters are ready for the next call
    assert_same(normal, after, "after the slow path")
    assert_oracle(normal, x, what="slow path shape", **opts)


# (variant, rows, cols, dtype, options): one workgroup per `variant` tiles
# gives grids of 1024 to 2048 workgroups, more than the variant's occupancy
# lets the GPU hold at once (its VGPRs or LDS allow 3 to 5 per CU on 256
# CUs), so part of the grid starts only after the rest has finished
OVERSUBSCRIBED = [
    (1, 8192, 4096, "bf16", dict(block_2d=True)),
    (1, 4096, 8192, "fp32", dict()),
    (2, 8192, 8192, "bf16", dict()),
    (3, 8192, 8192, "bf16", dict(block_2d=True, stochastic=True, sr_seed=13)),
    (6, 8192, 8192, "bf16", dict(swizzled=True)),
]


@pytest.mark.parametrize("case", OVERSUBSCRIBED, ids=[f"v{c[0]}_{c[1]}x{c[2]}_{c[3]}" for c in OVERSUBSCRIBED])
def test_grid_beyond_residency_completes_with_the_same_bytes(case):
    v, rows, cols, dtype, opts = case
    print(f"oversubscribed variant {v} {rows}x{cols} {dtype} {opts}", flush=True)
    x = W.gaussian_fp32(rows, cols, 77, scale=2.0) if dtype == "fp32" else W.randn_bf16(rows, cols, 77)
    xd = to_device(x)
    ws = nv.empty_workspace(DEV)
    two = run(xd, nv.make_config(workspace=ws, amax_path=TWO, **opts))
    nv.nvfp4_debug_set_resident_variant(v)
    try:
        for i in range(2):
            one = run(xd, nv.make_config(workspace=ws, amax_path=SINGLE, **opts))
            assert_same(one, two, f"call {i}")
            assert handoff_words(ws) == (i + 1, True), f"call {i}"
            assert done_word(ws) == (i + 1, int(one["amax_row"].view(np.uint32)[0])), f"call {i}: no slow path"
    finally:
        nv.nvfp4_debug_set_resident_variant(0)


def test_unknown_variant_is_rejected():
    with pytest.raises(nv.NVFP4Error) as e:
        nv.nvfp4_debug_set_resident_variant(7)
    assert e.value.status == nv.NVFP4_ERR_UNSUPPORTED


def test_noop_writes_nothing_and_leaves_the_counters():
    x = W.randn_bf16(1024, 2048, 71)
    xd = to_device(x)
    ws = nv.empty_workspace(DEV)
    run(xd, nv.make_config(workspace=ws, amax_path=SINGLE))
    words = host(ws).copy()
    noop = torch.ones(1, dtype=torch.float32, device=DEV)
    row = nv.empty_orientation(1024, 2048, DEV)
    col = nv.empty_orientation(2048, 1024, DEV)
    for o in (row, col):
        for t in (o.data, o.scales, o.amax):
            t.view(torch.uint8).fill_(0x5A)
    nv.nvfp4_quantize(xd, row, col, nv.make_config(workspace=ws, noop=noop, amax_path=SINGLE))
    torch.cuda.synchronize()
    for o in (row, col):
        for t in (o.data, o.scales, o.amax):
            assert bool((t.view(torch.uint8) == 0x5A).all())
    assert np.array_equal(host(ws)[16384:], words[16384:])


def test_graph_replays_of_the_bench_call():
    # The bench call (8192x5120 BF16, 16x16, swizzled; five tiles per
    # workgroup) captured in a HIP graph: every replay, with eager writes to
    # the outputs in between, gives the eager bytes and advances the epoch by
    # one with the exit counters consistent.
    x = W.c2(rows=8192, cols=5120, seed=1)
    xd = to_device(x)
    ws = nv.empty_workspace(DEV)
    cfg = nv.make_config(block_2d=True, swizzled=True, workspace=ws, amax_path=SINGLE)
    row = nv.empty_orientation(8192, 5120, DEV)
    col = nv.empty_orientation(5120, 8192, DEV)
    outs = [row.data, row.scales, row.amax, col.data, col.scales, col.amax]
    nv.nvfp4_quantize(xd, row, col, cfg)
    torch.cuda.synchronize()
    eager = [host(t).copy() for t in outs]
    assert handoff_words(ws) == (1, True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        nv.nvfp4_quantize(xd, row, col, cfg, s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.view(torch.uint8).fill_(0x33 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, t in zip(eager, outs):
            assert np.array_equal(e, host(t)), rep
        assert handoff_words(ws) == (2 + rep, True), rep


def test_epoch_wrap_clears_the_slots():
    # Drive the epoch through the point where 32-bit tags would repeat, with
    # a slot left as a call 2^32 calls earlier would have left it: tag 1 and
    # a huge maximum, in a slot that the small calls do not write. The call
    # that takes the epoch past its limit (which keeps the next call's tags
    # below 2^32) clears every slot, so the large call after it (tag 1
    # again) cannot take the stale slot for its own.
    ws = nv.empty_workspace(DEV)
    words = ws.view(torch.int32)
    small = W.randn_bf16(2048, 2048, 81)   # 256 tiles: 256 workgroups
    big = W.c2(rows=8192, cols=5120, seed=1)  # 768 workgroups
    stale = (1 << 32) | 0x7F000000  # tag 1, max 2^127
    slot = 4096 + 2 * 600
    words[EPOCH] = EPOCH_LIMIT - 1 - (1 << 32)  # the second call passes the limit
    for w in (slot, DONE):  # a slot and the done word, as such a call left them
        words[w] = stale & 0xFFFFFFFF
        words[w + 1] = stale >> 32
    torch.cuda.synchronize()
    for i in range(2):
        got = run(to_device(small), nv.make_config(workspace=ws, amax_path=SINGLE))
        assert_oracle(got, small, what=f"small call {i}")
    epoch, ok = handoff_words(ws)
    assert ok and epoch == 0
    assert int(words[slot + 1]) == 0, "the stale slot was not cleared at the wrap"
    assert int(words[DONE + 1]) == 0, "the stale done word was not cleared at the wrap"
    got = run(to_device(big), nv.make_config(workspace=ws, amax_path=SINGLE, block_2d=True, swizzled=True))
    assert_oracle(got, big, swizzled=True, what="after the wrap", block_2d=True)
    assert handoff_words(ws) == (1, True)


@pytest.mark.parametrize("fill", ["uniform", "random"])
def test_workspace_not_zero_filled_still_gives_the_oracle_bytes(fill):
    # A workspace that was not zero-filled: uniform bytes leave the counters
    # equal to their bases and no slot with the next tag, so the handoff runs
    # as usual; random words fail the counters' check and every workgroup
    # takes the maximum of the whole input itself. Either way the bytes are
    # the oracle's.
    x = W.randn_bf16(512, 768, 91)
    ws = nv.empty_workspace(DEV)
    if fill == "uniform":
        ws.fill_(0xA5)
    else:
        g = torch.Generator(device=DEV).manual_seed(92)
        ws.copy_(torch.randint(0, 256, ws.shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8))
    for i in range(2):
        got = run(to_device(x), nv.make_config(workspace=ws, amax_path=SINGLE, block_2d=True))
        assert_oracle(got, x, what=f"{fill} call {i}", block_2d=True)
