"""Python binding of the MI355X NVFP4 quantize library (``libnvfp4.so``).

Thin ctypes marshalling over the C ABI declared in ``include/nvfp4.h``; the
functions keep the C names. Every step of the quantize path runs in the
library's HIP kernels; torch only supplies device memory and the current
stream. If the library is missing or cannot be loaded, every call raises:
there is no fallback.

Tensors passed in are torch CUDA tensors (on ROCm, HIP devices):
  x         bfloat16 or float32, 2-D, contiguous
  data      uint8 [n][k/2]      scales  uint8 (compact [n][k/16] or swizzled, flat)
  amax      float32 [1] or [n]
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

from . import build as _build

_LIB_PATH = _build.LIB

NVFP4_OK = 0
NVFP4_ERR_NULL = 1
NVFP4_ERR_SHAPE = 2
NVFP4_ERR_ALIGN = 3
NVFP4_ERR_UNSUPPORTED = 4
NVFP4_ERR_HIP = 5

NVFP4_IN_BF16 = 0
NVFP4_IN_FP32 = 1

NVFP4_SCALES_COMPACT = 0
NVFP4_SCALES_GEMM_SWIZZLED = 1

NVFP4_SCALE_E4M3 = 0
NVFP4_SCALE_UE5M3 = 1

NVFP4_AMAX_PATH_AUTO = 0
NVFP4_AMAX_PATH_TWO_PASS = 1
NVFP4_AMAX_PATH_SINGLE_PASS = 2

NVFP4_DEBUG_SR = 1
NVFP4_DEBUG_PAIRWISE = 2

NVFP4_MAX_GROUPS = 256

EXPORTED = ("nvfp4_compute_amax", "nvfp4_quantize", "nvfp4_dequantize", "nvfp4_last_error",
            "nvfp4_workspace_bytes", "nvfp4_swizzle_scales", "nvfp4_swizzled_scales_bytes", "nvfp4_quantize_grouped",
            "nvfp4_debug_rht_colwise", "nvfp4_debug_e2m1_pack", "nvfp4_debug_set_wait_ticks",
            "nvfp4_quantize_noalloc", "nvfp4_debug_set_rht_unit", "nvfp4_debug_set_resident_variant")


class nvfp4_out_t(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("amax", ctypes.c_void_p)]


class nvfp4_config_t(ctypes.Structure):
    _fields_ = [
        ("block_2d", ctypes.c_uint32),
        ("scale_layout", ctypes.c_uint32),
        ("scale_fmt", ctypes.c_uint32),
        ("stochastic", ctypes.c_uint32),
        ("sr_seed", ctypes.c_uint32),
        ("row_scaled", ctypes.c_uint32),
        ("rht", ctypes.c_uint32),
        ("rht_sign_mask", ctypes.c_uint32),
        ("rht_bf16", ctypes.c_uint32),
        ("compute_amax", ctypes.c_uint32),
        ("noop", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("cast_events", ctypes.c_void_p),
        ("amax_path", ctypes.c_uint32),
    ]


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"nvfp4 status {status}: {message}")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load(build_if_missing: bool = True) -> ctypes.CDLL:
    """Load libnvfp4.so (building it first only when it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        if not build_if_missing:
            raise RuntimeError(f"{_LIB_PATH} is not built")
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    U32 = ctypes.c_uint32
    I = ctypes.c_int
    lib.nvfp4_compute_amax.restype = I
    lib.nvfp4_compute_amax.argtypes = [P, I, I64, I64, P, P, ctypes.POINTER(nvfp4_config_t), P]
    lib.nvfp4_quantize.restype = I
    lib.nvfp4_quantize.argtypes = [P, I, I64, I64, ctypes.POINTER(nvfp4_out_t), ctypes.POINTER(nvfp4_out_t),
                                   ctypes.POINTER(nvfp4_config_t), P]
    lib.nvfp4_quantize_noalloc.restype = I
    lib.nvfp4_quantize_noalloc.argtypes = lib.nvfp4_quantize.argtypes
    lib.nvfp4_dequantize.restype = I
    lib.nvfp4_dequantize.argtypes = [ctypes.POINTER(nvfp4_out_t), I64, I64, U32, U32, U32, P, P]
    lib.nvfp4_last_error.restype = ctypes.c_char_p
    lib.nvfp4_last_error.argtypes = []
    lib.nvfp4_workspace_bytes.restype = ctypes.c_uint64
    lib.nvfp4_workspace_bytes.argtypes = []
    lib.nvfp4_quantize_grouped.restype = I
    lib.nvfp4_quantize_grouped.argtypes = [P, I, I64, ctypes.POINTER(ctypes.c_int64), I64,
                                           ctypes.POINTER(nvfp4_out_t), ctypes.POINTER(nvfp4_out_t),
                                           ctypes.POINTER(nvfp4_config_t), P]
    lib.nvfp4_swizzle_scales.restype = I
    lib.nvfp4_swizzle_scales.argtypes = [P, I64, I64, P, P]
    lib.nvfp4_swizzled_scales_bytes.restype = ctypes.c_uint64
    lib.nvfp4_swizzled_scales_bytes.argtypes = [I64, I64]
    lib.nvfp4_debug_rht_colwise.restype = I
    lib.nvfp4_debug_rht_colwise.argtypes = [P, I, I64, I64, U32, P, P]
    lib.nvfp4_debug_e2m1_pack.restype = I
    lib.nvfp4_debug_e2m1_pack.argtypes = [P, P, P, I64, U32, P]
    lib.nvfp4_debug_set_wait_ticks.restype = I
    lib.nvfp4_debug_set_wait_ticks.argtypes = [U32]
    lib.nvfp4_debug_set_rht_unit.restype = I
    lib.nvfp4_debug_set_rht_unit.argtypes = [U32]
    lib.nvfp4_debug_set_resident_variant.restype = I
    lib.nvfp4_debug_set_resident_variant.argtypes = [U32]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != NVFP4_OK:
        raise NVFP4Error(status, nvfp4_last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return NVFP4_IN_BF16
    if x.dtype == torch.float32:
        return NVFP4_IN_FP32
    raise TypeError(f"input must be bfloat16 or float32, got {x.dtype}")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _shape2d(x: torch.Tensor):
    if x.dim() != 2 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("x must be a contiguous 2-D CUDA tensor")
    return x.shape[0], x.shape[1]


# The C ABI takes plain pointers and cannot see buffer sizes; the binding
# checks every tensor it passes against what the call will touch.
def _need(t: Optional[torch.Tensor], n: int, dtypes, what: str) -> None:
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t is None or not t.is_cuda or not t.is_contiguous() or t.dtype not in dtypes or t.numel() < n:
        raise ValueError(f"{what} must be a contiguous CUDA tensor of {'/'.join(str(d) for d in dtypes)} "
                         f"with at least {n} elements")


def _need_orientation(o, n: int, k: int, amax_len: int, what: str) -> None:
    if o is None:
        return
    _need(o.data, n * k // 2, torch.uint8, f"{what} data")
    _need(o.scales, n * k // 16, torch.uint8, f"{what} scales")
    _need(o.amax, amax_len, torch.float32, f"{what} amax")


def make_config(*, block_2d=False, swizzled=False, scale_fmt=NVFP4_SCALE_E4M3, stochastic=False, sr_seed=0,
                row_scaled=False, rht=False, rht_sign_mask=0, compute_amax=True,
                noop: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                rht_bf16=False, amax_path=0) -> nvfp4_config_t:
    """The config struct. It holds references to the noop and workspace
    tensors (a copy made with from_buffer_copy does not: keep them alive
    while such a copy is used)."""
    if noop is not None:
        _need(noop, 1, torch.float32, "noop")
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()
                                  or workspace.numel() * workspace.element_size() < nvfp4_workspace_bytes()):
        raise ValueError(f"workspace must be contiguous CUDA memory of at least {nvfp4_workspace_bytes()} bytes")
    cfg = nvfp4_config_t(int(block_2d), NVFP4_SCALES_GEMM_SWIZZLED if swizzled else NVFP4_SCALES_COMPACT,
                         int(scale_fmt), int(stochastic), int(sr_seed) & 0xFFFFFFFF, int(row_scaled), int(rht),
                         int(rht_sign_mask) & 0xFFFFFFFF, int(rht_bf16), int(compute_amax),
                         None if noop is None else noop.data_ptr(),
                         None if workspace is None else workspace.data_ptr())
    cfg.amax_path = int(amax_path)
    cfg._tensors = (noop, workspace)
    return cfg


@dataclasses.dataclass
class Orientation:
    """One orientation of an NVFP4 tensor: data [n][k/2], scales, amax."""
    data: torch.Tensor
    scales: torch.Tensor
    amax: torch.Tensor

    def as_c(self) -> nvfp4_out_t:
        return nvfp4_out_t(self.data.data_ptr(), self.scales.data_ptr(), self.amax.data_ptr())


def nvfp4_last_error() -> str:
    return load().nvfp4_last_error().decode()


def nvfp4_workspace_bytes() -> int:
    return int(load().nvfp4_workspace_bytes())


def nvfp4_compute_amax(x: torch.Tensor, row_amax: Optional[torch.Tensor], col_amax: Optional[torch.Tensor],
                       cfg: Optional[nvfp4_config_t] = None, stream=None) -> None:
    rows, cols = _shape2d(x)
    if row_amax is not None:
        _need(row_amax, rows if (cfg is not None and cfg.row_scaled) else 1, torch.float32, "row_amax")
    if col_amax is not None:
        _need(col_amax, cols if (cfg is not None and cfg.row_scaled) else 1, torch.float32, "col_amax")
    _check(load().nvfp4_compute_amax(_ptr(x), _dtype_code(x), rows, cols, _ptr(row_amax), _ptr(col_amax),
                                     None if cfg is None else ctypes.byref(cfg), _stream(stream)))


def nvfp4_quantize(x: torch.Tensor, row: Optional[Orientation], col: Optional[Orientation],
                   cfg: Optional[nvfp4_config_t] = None, stream=None) -> None:
    rows, cols = _shape2d(x)
    _need_orientation(row, rows, cols, rows if (cfg is not None and cfg.row_scaled) else 1, "row-wise")
    _need_orientation(col, cols, rows, cols if (cfg is not None and cfg.row_scaled) else 1, "column-wise")
    r = row.as_c() if row is not None else None
    c = col.as_c() if col is not None else None
    _check(load().nvfp4_quantize(_ptr(x), _dtype_code(x), rows, cols, None if r is None else ctypes.byref(r),
                                 None if c is None else ctypes.byref(c), None if cfg is None else ctypes.byref(cfg),
                                 _stream(stream)))


def nvfp4_quantize_noalloc(x: torch.Tensor, row: Optional[Orientation], col: Optional[Orientation],
                           cfg: Optional[nvfp4_config_t] = None, stream=None) -> None:
    """nvfp4_quantize with the library's own per-device scratch in place of a
    workspace (cfg.workspace must be unset); allocates nothing."""
    rows, cols = _shape2d(x)
    _need_orientation(row, rows, cols, rows if (cfg is not None and cfg.row_scaled) else 1, "row-wise")
    _need_orientation(col, cols, rows, cols if (cfg is not None and cfg.row_scaled) else 1, "column-wise")
    r = row.as_c() if row is not None else None
    c = col.as_c() if col is not None else None
    _check(load().nvfp4_quantize_noalloc(_ptr(x), _dtype_code(x), rows, cols, None if r is None else ctypes.byref(r),
                                         None if c is None else ctypes.byref(c),
                                         None if cfg is None else ctypes.byref(cfg), _stream(stream)))


def nvfp4_dequantize(q: Orientation, rows: int, cols: int, scale_layout: int, row_scaled: bool, y: torch.Tensor,
                     stream=None, scale_fmt: int = 0) -> None:
    _need_orientation(q, rows, cols, rows if row_scaled else 1, "quantized tensor")
    _need(y, rows * cols, torch.float32, "y")
    qc = q.as_c()
    _check(load().nvfp4_dequantize(ctypes.byref(qc), rows, cols, scale_layout, scale_fmt, int(row_scaled), _ptr(y),
                                   _stream(stream)))


def nvfp4_quantize_grouped(x: torch.Tensor, group_rows, row: Optional[Orientation], col: Optional[Orientation],
                           cfg: Optional[nvfp4_config_t] = None, stream=None) -> None:
    """x [sum(group_rows)][C]; row/col hold the concatenated per-group outputs
    (data and scales flat or shaped, amax [G])."""
    rows, cols = _shape2d(x)
    _need_orientation(row, rows, cols, rows if (cfg is not None and cfg.row_scaled) else len(group_rows), "row-wise")
    _need_orientation(col, cols, rows, len(group_rows), "column-wise")
    g = (ctypes.c_int64 * len(group_rows))(*[int(m) for m in group_rows])
    r = row.as_c() if row is not None else None
    c = col.as_c() if col is not None else None
    _check(load().nvfp4_quantize_grouped(_ptr(x), _dtype_code(x), len(group_rows), g, cols,
                                         None if r is None else ctypes.byref(r), None if c is None else ctypes.byref(c),
                                         None if cfg is None else ctypes.byref(cfg), _stream(stream)))


def quantize_grouped(x: torch.Tensor, group_rows, *, rowwise=True, columnwise=True,
                     cfg: Optional[nvfp4_config_t] = None, stream=None, use_workspace: bool = True):
    """Allocate the concatenated per-group outputs and run nvfp4_quantize_grouped.
    Returns (row, col) with flat data and scales and amax [G] ([R] for a
    row-scaled config). A workspace is allocated for the call as in
    quantize()."""
    rows, cols = _shape2d(x)
    G = len(group_rows)
    dev = x.device
    cfg = cfg if cfg is not None else make_config()

    def orient(amax_len):
        return Orientation(torch.empty((rows * cols // 2,), dtype=torch.uint8, device=dev),
                           torch.empty((rows * cols // 16,), dtype=torch.uint8, device=dev),
                           torch.empty((amax_len,), dtype=torch.float32, device=dev))

    row = orient(rows if cfg.row_scaled else G) if rowwise else None
    col = orient(G) if columnwise else None
    ws = None
    if use_workspace and not cfg.workspace and cfg.compute_amax and not cfg.row_scaled:
        ws = empty_workspace(dev)
        cfg = nvfp4_config_t.from_buffer_copy(cfg)
        cfg.workspace = ws.data_ptr()
        if stream is not None:
            ws.record_stream(stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream)))
    nvfp4_quantize_grouped(x, group_rows, row, col, cfg, stream)
    del ws
    return row, col


def nvfp4_swizzled_scales_bytes(rows: int, scale_cols: int) -> int:
    return int(load().nvfp4_swizzled_scales_bytes(rows, scale_cols))


def nvfp4_swizzle_scales(compact: torch.Tensor, rows: int, scale_cols: int, swizzled: torch.Tensor,
                         stream=None) -> None:
    """compact: uint8 with rows * scale_cols bytes; swizzled: uint8 with
    nvfp4_swizzled_scales_bytes(rows, scale_cols) bytes."""
    _need(compact, rows * scale_cols, torch.uint8, "compact")
    _need(swizzled, nvfp4_swizzled_scales_bytes(rows, scale_cols), torch.uint8, "swizzled")
    _check(load().nvfp4_swizzle_scales(_ptr(compact), rows, scale_cols, _ptr(swizzled), _stream(stream)))


def nvfp4_debug_rht_colwise(x: torch.Tensor, sign_mask: int, t: torch.Tensor, stream=None) -> None:
    rows, cols = _shape2d(x)
    _need(t, rows * cols, torch.float32, "t")
    _check(load().nvfp4_debug_rht_colwise(_ptr(x), _dtype_code(x), rows, cols, sign_mask & 0xFFFFFFFF, _ptr(t),
                                          _stream(stream)))


def nvfp4_debug_e2m1_pack(v: torch.Tensor, r: Optional[torch.Tensor], out: torch.Tensor, flags: int,
                          stream=None) -> None:
    """v: float32 [2n]; r: int32/uint32 [n] or None; out: uint8 [n]."""
    n = out.numel()
    _need(out, n, torch.uint8, "out")
    _need(v, 2 * n, torch.float32, "v")
    if r is not None:
        _need(r, n, (torch.int32, torch.uint32), "r")
    _check(load().nvfp4_debug_e2m1_pack(_ptr(v), _ptr(r), _ptr(out), n, flags, _stream(stream)))


# ---- allocation helpers (device memory only; no arithmetic) -----------------

def empty_orientation(n: int, k: int, device, amax_len: int = 1) -> Orientation:
    """Uninitialized buffers for one orientation with n rows of k elements."""
    return Orientation(torch.empty((n, k // 2), dtype=torch.uint8, device=device),
                       torch.empty((n * (k // 16),), dtype=torch.uint8, device=device),
                       torch.empty((amax_len,), dtype=torch.float32, device=device))


def empty_workspace(device) -> torch.Tensor:
    """A zero-filled quantize workspace, as its first use needs (torch's
    allocator aligns it to 512 bytes). Reuse it for later calls on one stream:
    the library keeps its arrival counters valid from call to call."""
    return torch.zeros((nvfp4_workspace_bytes(),), dtype=torch.uint8, device=device)


_workspaces = {}


def stream_workspace(device, stream=None) -> torch.Tensor:
    """The workspace that quantize() uses for calls on (device, stream): made
    once, zero-filled, then reused, so that a call costs no extra launch.
    Calls on one stream run in order, so they never share it concurrently."""
    dev = torch.device(device)
    if dev.index is None:
        dev = torch.device(dev.type, torch.cuda.current_device())
    if stream is None:
        handle = torch.cuda.current_stream(dev).cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        handle = stream.cuda_stream
    else:
        handle = int(stream)
    key = (dev.index, handle)
    ws = _workspaces.get(key)
    if ws is None:
        ws = empty_workspace(dev)
        _workspaces[key] = ws
    return ws


def nvfp4_debug_set_wait_ticks(ticks: int) -> None:
    _check(load().nvfp4_debug_set_wait_ticks(int(ticks) & 0xFFFFFFFF))


def nvfp4_debug_set_resident_variant(tiles_per_workgroup: int) -> None:
    _check(load().nvfp4_debug_set_resident_variant(int(tiles_per_workgroup) & 0xFFFFFFFF))


RHT_UNIT_DEFAULT = 0
RHT_UNIT_VALU = 1
RHT_UNIT_MATRIX = 2


def nvfp4_debug_set_rht_unit(unit: int) -> None:
    _check(load().nvfp4_debug_set_rht_unit(int(unit) & 0xFFFFFFFF))


def quantize(x: torch.Tensor, *, rowwise=True, columnwise=True, cfg: Optional[nvfp4_config_t] = None,
             stream=None, use_workspace: bool = True):
    """Allocate outputs for x [R][C] and run nvfp4_quantize. Returns (row, col).

    With use_workspace (and no workspace in cfg) the stream's cached
    workspace is passed, so a computed per-tensor amax takes one launch
    (single pass) or two instead of three."""
    rows, cols = _shape2d(x)
    cfg = cfg if cfg is not None else make_config()
    row = empty_orientation(rows, cols, x.device, rows if cfg.row_scaled else 1) if rowwise else None
    col = empty_orientation(cols, rows, x.device, cols if cfg.row_scaled else 1) if columnwise else None
    ws = None
    if use_workspace and not cfg.workspace and cfg.compute_amax and not cfg.row_scaled:
        ws = stream_workspace(x.device, stream)
        cfg = nvfp4_config_t.from_buffer_copy(cfg)
        cfg.workspace = ws.data_ptr()
    nvfp4_quantize(x, row, col, cfg, stream)
    return row, col
