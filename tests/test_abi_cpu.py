"""C-ABI checks that need no GPU: the library loads, exports every function
include/nvfp4.h declares, and rejects bad arguments on the host before
queuing anything (all calls here fail validation, so no HIP call is made)."""

from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest
import torch

import nvfp4_block_scaled_05_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

# Fake, suitably aligned "device" addresses: validation never dereferences them.
X = 0x100000
D = 0x200000
S = 0x300000
A = 0x400000
A2 = 0x500000


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:nvfp4_status_t|const char \*|uint64_t)\s*(nvfp4_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(nv.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = nv.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def _out(data=D, scales=S, amax=A):
    return nv.nvfp4_out_t(data, scales, amax)


def _q(rows, cols, row=None, col=None, cfg=None, x=X, dtype=nv.NVFP4_IN_BF16):
    lib = nv.load()
    r = None if row is None else ctypes.byref(row)
    c = None if col is None else ctypes.byref(col)
    f = None if cfg is None else ctypes.byref(cfg)
    return lib.nvfp4_quantize(x, dtype, rows, cols, r, c, f, None)


@pytest.mark.parametrize("case,expected", [
    (dict(rows=64, cols=40, row=_out()), nv.NVFP4_ERR_SHAPE),                    # cols % 16
    (dict(rows=40, cols=64, col=_out()), nv.NVFP4_ERR_SHAPE),                    # col-wise needs rows % 16
    (dict(rows=-1, cols=64, row=_out()), nv.NVFP4_ERR_SHAPE),
    (dict(rows=1 << 17, cols=1 << 16, row=_out()), nv.NVFP4_ERR_SHAPE),          # 2^33 elements
    (dict(rows=64, cols=64), nv.NVFP4_ERR_NULL),                                 # no output at all
    (dict(rows=64, cols=64, row=_out(data=0)), nv.NVFP4_ERR_NULL),
    (dict(rows=64, cols=64, row=_out(), x=0), nv.NVFP4_ERR_NULL),
    (dict(rows=64, cols=64, row=_out(), x=X + 2), nv.NVFP4_ERR_ALIGN),
    (dict(rows=64, cols=64, row=_out(data=D + 4)), nv.NVFP4_ERR_ALIGN),
    (dict(rows=64, cols=64, row=_out(scales=S + 1)), nv.NVFP4_ERR_ALIGN),
    (dict(rows=64, cols=64, row=_out(), dtype=7), nv.NVFP4_ERR_UNSUPPORTED),
])
def test_quantize_rejects_bad_arguments(case, expected):
    assert _q(**case) == expected
    assert nv.nvfp4_last_error() != ""


def _q_noalloc(rows, cols, row=None, col=None, cfg=None, x=X):
    lib = nv.load()
    return lib.nvfp4_quantize_noalloc(x, nv.NVFP4_IN_BF16, rows, cols, None if row is None else ctypes.byref(row),
                                      None if col is None else ctypes.byref(col),
                                      None if cfg is None else ctypes.byref(cfg), None)


@pytest.mark.parametrize("case,expected", [
    (dict(rows=64, cols=40, row=_out()), nv.NVFP4_ERR_SHAPE),
    (dict(rows=40, cols=64, col=_out()), nv.NVFP4_ERR_SHAPE),
    (dict(rows=64, cols=64), nv.NVFP4_ERR_NULL),
    (dict(rows=64, cols=64, row=_out(), x=X + 2), nv.NVFP4_ERR_ALIGN),
])
def test_noalloc_quantize_rejects_bad_arguments(case, expected):
    # validation comes before the device is touched (no HIP call here)
    assert _q_noalloc(**case) == expected
    assert nv.nvfp4_last_error() != ""


def test_noalloc_quantize_refuses_a_workspace():
    cfg = nv.make_config()
    cfg.workspace = 0x600000
    assert _q_noalloc(64, 64, row=_out(), cfg=cfg) == nv.NVFP4_ERR_UNSUPPORTED
    assert "workspace" in nv.nvfp4_last_error()


def test_swizzled_scales_reject_partial_tiles():
    # "Fuse NVFP4 scale swizzling on SM120 and SM121": partial 128x128 scale
    # tiles are rejected for swizzled output (e.g. the 1088x1024 tail shape).
    cfg = nv.make_config(swizzled=True)
    assert _q(1088, 1024, row=_out(), col=_out(A2), cfg=cfg) == nv.NVFP4_ERR_SHAPE
    assert _q(1024, 1040, row=_out(), cfg=cfg) == nv.NVFP4_ERR_SHAPE
    assert "128" in nv.nvfp4_last_error()


def test_row_scaled_gates():
    # "Implement row-scaled NVFP4 fprop recipe": compact scales; the per-row
    # and per-column amaxes are two arrays, so one buffer for both is refused;
    # "Fuse NVFP4 scale swizzling ...": no row-scaled RHT.
    rs = nv.make_config(row_scaled=True)
    assert _q(128, 128, row=_out(), col=_out(), cfg=rs) == nv.NVFP4_ERR_UNSUPPORTED
    assert "distinct" in nv.nvfp4_last_error()
    assert _q(120, 128, col=_out(A2), cfg=rs) == nv.NVFP4_ERR_SHAPE  # column-wise: rows % 16
    assert _q(128, 128, row=_out(), cfg=nv.make_config(row_scaled=True, swizzled=True)) == nv.NVFP4_ERR_UNSUPPORTED
    assert _q(128, 128, row=_out(), cfg=nv.make_config(row_scaled=True, rht=True)) == nv.NVFP4_ERR_UNSUPPORTED
    assert _q(128, 128, row=_out(), cfg=nv.make_config(row_scaled=True, block_2d=True)) == nv.NVFP4_ERR_UNSUPPORTED


def test_rht_gates():
    assert _q(128, 128, row=_out(), col=_out(A2), cfg=nv.make_config(rht=True, block_2d=True)) == \
        nv.NVFP4_ERR_UNSUPPORTED
    # "Write both NVFP4 amax buffers", review thread: one float for both RHT
    # amaxes gives wrong data, so a shared buffer is refused.
    assert _q(128, 128, row=_out(), col=_out(), cfg=nv.make_config(rht=True)) == nv.NVFP4_ERR_UNSUPPORTED


def test_unknown_scale_format_is_unsupported():
    # E4M3 (0) and UE5M3 (1) are the formats; every call below fails validation
    cfg = nv.make_config(scale_fmt=2)
    assert _q(128, 128, row=_out(), cfg=cfg) == nv.NVFP4_ERR_UNSUPPORTED
    assert "scale format" in nv.nvfp4_last_error()
    lib = nv.load()
    groups = (ctypes.c_int64 * 1)(128)
    r = _out()
    assert lib.nvfp4_quantize_grouped(X, 0, 1, groups, 128, ctypes.byref(r), None, ctypes.byref(cfg), None) == \
        nv.NVFP4_ERR_UNSUPPORTED


def test_compute_amax_rejections():
    lib = nv.load()
    assert lib.nvfp4_compute_amax(X, 0, 64, 64, None, None, None, None) == nv.NVFP4_ERR_NULL
    assert lib.nvfp4_compute_amax(X, 0, 64, 64, A + 2, None, None, None) == nv.NVFP4_ERR_ALIGN
    rs = nv.make_config(row_scaled=True)
    assert lib.nvfp4_compute_amax(X, 0, 64, 64, A, A, ctypes.byref(rs), None) == nv.NVFP4_ERR_UNSUPPORTED
    rht = nv.make_config(rht=True)
    assert lib.nvfp4_compute_amax(X, 0, 40, 64, A, A2, ctypes.byref(rht), None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_compute_amax(X, 0, 64, 64, A, A, ctypes.byref(rht), None) == nv.NVFP4_ERR_UNSUPPORTED


def test_dequantize_rejections():
    lib = nv.load()
    q = _out()
    assert lib.nvfp4_dequantize(None, 64, 64, 0, 0, 0, D, None) == nv.NVFP4_ERR_NULL
    assert lib.nvfp4_dequantize(ctypes.byref(q), 64, 40, 0, 0, 0, D, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_dequantize(ctypes.byref(q), 64, 64, 1, 0, 0, D, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_dequantize(ctypes.byref(q), 64, 64, 0, 0, 0, D + 4, None) == nv.NVFP4_ERR_ALIGN
    assert lib.nvfp4_dequantize(ctypes.byref(q), 128, 128, 1, 0, 1, D, None) == nv.NVFP4_ERR_UNSUPPORTED
    assert lib.nvfp4_dequantize(ctypes.byref(q), 64, 64, 0, 2, 0, D, None) == nv.NVFP4_ERR_UNSUPPORTED
    assert "scale format" in nv.nvfp4_last_error()


def test_debug_rht_rejections():
    lib = nv.load()
    assert lib.nvfp4_debug_rht_colwise(X, 0, 40, 64, 0, D, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_debug_rht_colwise(X, 0, 64, 64, 0, None, None) == nv.NVFP4_ERR_NULL


def test_config_struct_matches_header_layout(tmp_path):
    # compile the header with the host C compiler and compare sizes and every field's offset
    C = nv.nvfp4_config_t
    names = [f[0] for f in C._fields_]
    offs = ", ".join(f"offsetof(nvfp4_config_t, {n})" for n in names)
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "nvfp4.h"\n'
                   'int main(void) { printf("%zu %zu %u' + " %zu" * len(names) + '\\n", sizeof(nvfp4_config_t), '
                   'sizeof(nvfp4_out_t), NVFP4_WORKSPACE_BYTES, ' + offs + '); return 0; }\n')
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)])
    size, out_size, ws_bytes, *field_offsets = map(int, subprocess.check_output([str(exe)]).split())
    assert ctypes.sizeof(C) == size
    assert [getattr(C, n).offset for n in names] == field_offsets
    assert ctypes.sizeof(nv.nvfp4_out_t) == out_size
    assert nv.nvfp4_workspace_bytes() == ws_bytes


def test_rht_bf16_needs_rht():
    # every call below fails validation, so nothing is launched
    lib = nv.load()
    cfg = nv.make_config(rht_bf16=True)
    assert lib.nvfp4_compute_amax(X, 0, 64, 64, A, A2, ctypes.byref(cfg), None) == nv.NVFP4_ERR_UNSUPPORTED
    assert "rht_bf16" in nv.nvfp4_last_error()
    r = nv.nvfp4_out_t(D, S, A)
    c = nv.nvfp4_out_t(D + 0x10000, S + 0x10000, A2)
    assert lib.nvfp4_quantize(X, 0, 64, 64, ctypes.byref(r), ctypes.byref(c), ctypes.byref(cfg), None) == \
        nv.NVFP4_ERR_UNSUPPORTED
    assert "rht_bf16" in nv.nvfp4_last_error()
    groups = (ctypes.c_int64 * 2)(32, 32)
    assert lib.nvfp4_quantize_grouped(X, 0, 2, groups, 64, ctypes.byref(r), ctypes.byref(c), ctypes.byref(cfg),
                                      None) == nv.NVFP4_ERR_UNSUPPORTED
    assert "rht_bf16" in nv.nvfp4_last_error()


def test_workspace_must_be_aligned():
    lib = nv.load()
    r = nv.nvfp4_out_t(D, S, A)
    c = nv.nvfp4_out_t(D + 0x10000, S + 0x10000, A2)
    cfg = nv.make_config()
    cfg.workspace = 0x600008
    assert lib.nvfp4_quantize(X, 0, 64, 64, ctypes.byref(r), ctypes.byref(c), ctypes.byref(cfg), None) == \
        nv.NVFP4_ERR_ALIGN
    assert "workspace" in nv.nvfp4_last_error()


def test_debug_e2m1_rejections():
    lib = nv.load()
    assert lib.nvfp4_debug_e2m1_pack(D, S, A, -1, 0, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_debug_e2m1_pack(D, S, A, 8, 4, None) == nv.NVFP4_ERR_UNSUPPORTED
    assert lib.nvfp4_debug_e2m1_pack(D, None, A, 8, nv.NVFP4_DEBUG_SR, None) == nv.NVFP4_ERR_NULL
    assert lib.nvfp4_debug_e2m1_pack(D + 2, S, A, 8, 0, None) == nv.NVFP4_ERR_ALIGN


def test_cast_events_must_not_hold_null():
    lib = nv.load()
    r = nv.nvfp4_out_t(D, S, A)
    cfg = nv.make_config()
    ev = (ctypes.c_void_p * 2)(0x1000, None)
    cfg.cast_events = ctypes.cast(ev, ctypes.c_void_p)
    assert lib.nvfp4_quantize(X, 0, 64, 64, ctypes.byref(r), None, ctypes.byref(cfg), None) == nv.NVFP4_ERR_NULL


def test_swizzled_scales_size_and_rejections():
    lib = nv.load()
    assert nv.nvfp4_swizzled_scales_bytes(1088, 64) == 1152 * 64
    assert nv.nvfp4_swizzled_scales_bytes(100, 7) == 128 * 8
    assert nv.nvfp4_swizzled_scales_bytes(8192, 320) == 8192 * 320
    assert nv.nvfp4_swizzled_scales_bytes(0, 8) == 0 and nv.nvfp4_swizzled_scales_bytes(-1, 8) == 0
    assert lib.nvfp4_swizzle_scales(S, -1, 4, D, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_swizzle_scales(None, 128, 4, D, None) == nv.NVFP4_ERR_NULL
    assert lib.nvfp4_swizzle_scales(S + 2, 128, 4, D, None) == nv.NVFP4_ERR_ALIGN
    assert lib.nvfp4_swizzle_scales(S, 1 << 30, 1 << 10, D, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_swizzle_scales(None, 0, 4, None, None) == nv.NVFP4_OK  # empty: nothing to do


def test_grouped_rejections():
    lib = nv.load()
    r = nv.nvfp4_out_t(D, S, A)
    c = nv.nvfp4_out_t(D + 0x100000, S + 0x100000, A2)
    G = ctypes.c_int64 * 3

    def call(groups, cols=64, cfg=None, row=r, col=c):
        arr = G(*groups) if len(groups) == 3 else (ctypes.c_int64 * len(groups))(*groups)
        return lib.nvfp4_quantize_grouped(X, 0, len(groups), arr, cols, ctypes.byref(row) if row else None,
                                          ctypes.byref(col) if col else None,
                                          None if cfg is None else ctypes.byref(cfg), None)

    assert lib.nvfp4_quantize_grouped(X, 0, 0, None, 64, ctypes.byref(r), None, None, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_quantize_grouped(X, 0, 257, None, 64, ctypes.byref(r), None, None, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_quantize_grouped(X, 0, 2, None, 64, ctypes.byref(r), None, None, None) == nv.NVFP4_ERR_NULL
    assert call([16, -16, 16]) == nv.NVFP4_ERR_SHAPE
    assert call([16, 8, 16]) == nv.NVFP4_ERR_SHAPE              # column-wise output needs multiples of 16
    assert call([128, 64, 128], cols=128, cfg=nv.make_config(swizzled=True)) == nv.NVFP4_ERR_SHAPE
    # row-scaled groups: row-wise only, 1x16, compact, no RHT (valid row-scaled calls are not made here)
    assert call([16, 16, 16], cfg=nv.make_config(row_scaled=True)) == nv.NVFP4_ERR_UNSUPPORTED
    assert call([128, 0, 128], cols=128, cfg=nv.make_config(row_scaled=True, swizzled=True), col=None) == \
        nv.NVFP4_ERR_UNSUPPORTED
    assert call([16, 16, 16], cfg=nv.make_config(row_scaled=True, block_2d=True), col=None) == \
        nv.NVFP4_ERR_UNSUPPORTED
    assert call([16, 16, 16], cfg=nv.make_config(row_scaled=True, rht=True), col=None) == nv.NVFP4_ERR_UNSUPPORTED
    assert call([16, 16, 16], cfg=nv.make_config(rht=True, block_2d=True)) == nv.NVFP4_ERR_UNSUPPORTED
    assert call([16, 16, 16], cols=40) == nv.NVFP4_ERR_SHAPE


def test_size_limits_are_checked_without_overflow():
    # products that overflow 64 bits, and the exact 2^32 limit, are refused
    # before anything is queued (nothing here launches)
    lib = nv.load()
    r = _out()
    for rows, cols in ((1 << 40, 1 << 40), (1 << 62, 16), (65536, 65536), (1 << 32, 16)):
        assert _q(rows, cols, row=r) == nv.NVFP4_ERR_SHAPE, (rows, cols)
        assert lib.nvfp4_compute_amax(X, 0, rows, cols, A, None, None, None) == nv.NVFP4_ERR_SHAPE
        assert lib.nvfp4_dequantize(ctypes.byref(r), rows, cols, 0, 0, 0, D, None) == nv.NVFP4_ERR_SHAPE
    groups = (ctypes.c_int64 * 2)(16, 1 << 62)
    assert lib.nvfp4_quantize_grouped(X, 0, 2, groups, 64, ctypes.byref(r), None, None, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_swizzle_scales(S, 1 << 40, 1 << 40, S, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_swizzle_scales(S, 1 << 17, 1 << 17, S, None) == nv.NVFP4_ERR_SHAPE
    assert nv.nvfp4_swizzled_scales_bytes(1 << 40, 4) == 0
    assert nv.nvfp4_swizzled_scales_bytes(4, 1 << 33) == 0


def test_binding_refuses_host_tensors_and_short_buffers():
    # the binding checks every tensor before calling the library; host
    # tensors stand in for mistakes here (nothing reaches a GPU)
    x = torch.zeros((32, 64), dtype=torch.bfloat16)
    o = nv.Orientation(torch.zeros(32 * 32, dtype=torch.uint8), torch.zeros(32 * 4, dtype=torch.uint8),
                       torch.zeros(1, dtype=torch.float32))
    with pytest.raises(ValueError, match="CUDA"):
        nv.nvfp4_quantize(x, o, None)
    with pytest.raises(ValueError, match="CUDA"):
        nv.quantize(x)
    with pytest.raises(ValueError, match="CUDA"):
        nv.quantize_grouped(x, [16, 16])
    with pytest.raises(ValueError, match="noop"):
        nv.make_config(noop=torch.ones(1))
    with pytest.raises(ValueError, match="workspace"):
        nv.make_config(workspace=torch.zeros(16384, dtype=torch.uint8))
    with pytest.raises(ValueError, match="quantized tensor data"):
        nv.nvfp4_dequantize(o, 32, 64, 0, False, torch.zeros(32 * 64))
    with pytest.raises(ValueError, match="compact"):
        nv.nvfp4_swizzle_scales(torch.zeros(128 * 4, dtype=torch.uint8), 128, 4, torch.zeros(512, dtype=torch.uint8))
