"""NVFP4 quantization oracle -- TEST INFRASTRUCTURE ONLY.

Python access (ctypes + numpy) to the plain C definition in
``oracle/nvfp4_oracle.c``. Only the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package; the GPU
library never does, and this package never imports the GPU library.

Every array argument is a host numpy array; outputs are returned as new
numpy arrays in the layouts the C functions document:

* row-wise data ``[rows][cols/2]`` (uint8), scales ``[rows][cols/16]``;
* column-wise data ``[cols][rows/2]``, scales ``[cols][rows/16]``;
* scales are compact; ``swizzle_scales`` gives the GEMM-swizzled layout.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# the same source built with OpenMP: only the CPU-baseline timing uses it
_LIB_PARALLEL = os.path.join(_HERE, "liboracle_omp.so")

BF16 = 0
FP32 = 1

_lib = None


def compile_library(src: str, out: str, openmp: bool = False) -> str:
    """Compile an oracle source into a shared library with gcc: binary32
    arithmetic, no contraction, no fast-math; with openmp, its outer loops
    run on all cores (same per-element arithmetic)."""
    tmp = out + ".tmp"
    subprocess.check_call([
        "gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall", "-Wextra",
        "-fPIC", "-shared", *(["-fopenmp"] if openmp else []), src, "-o", tmp, "-lm",
    ])
    os.replace(tmp, out)
    return out


def _stale(lib: str) -> bool:
    return not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC)


def build(force: bool = True) -> str:
    """Compile the oracle, single-threaded (the checker) and with OpenMP
    (the CPU-baseline timing); returns the checker's path."""
    if force or _stale(_LIB):
        compile_library(_SRC, _LIB)
    if force or _stale(_LIB_PARALLEL):
        compile_library(_SRC, _LIB_PARALLEL, openmp=True)
    return _LIB


_lib_parallel = None


@contextlib.contextmanager
def all_cores():
    """Inside the block, the oracle functions run on the OpenMP build (its
    outer loops over rows, columns and blocks spread over OMP_NUM_THREADS
    threads, or all cores). Yields the thread count. Only for timing: the
    results are the single-threaded checker's, bit for bit."""
    global _lib, _lib_parallel
    checker = _load()
    if _lib_parallel is None:
        build(force=False)
        _lib_parallel = bind(ctypes.CDLL(_LIB_PARALLEL))
    _lib = _lib_parallel
    try:
        yield int(_lib_parallel.oracle_num_threads())
    finally:
        _lib = checker


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    _lib = bind(ctypes.CDLL(_LIB))
    return _lib


def bind(lib):
    """Set the C signatures on a loaded oracle library (this package's, or a
    test's deliberately altered copy) and return it."""
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    U32 = ctypes.c_uint32
    U8 = ctypes.c_uint8
    F = ctypes.c_float
    sig = {
        "oracle_load": (F, [P, I, I64]),
        "oracle_e2m1_value": (ctypes.c_double, [U8]),
        "oracle_e2m1_rne": (U8, [F]),
        "oracle_e2m1_sr": (U8, [F, ctypes.c_uint16]),
        "oracle_e4m3_value": (ctypes.c_double, [U8]),
        "oracle_e4m3_rne_satfinite": (U8, [F]),
        "oracle_global_encode_scale": (F, [F]),
        "oracle_block_scale": (U8, [F, F]),
        "oracle_block_encode_multiplier": (F, [U8, F]),
        "oracle_fmix32": (U32, [U32]),
        "oracle_sr_word": (U32, [U32, I, U32]),
        "oracle_rht16": (None, [P, U32, P]),
        "oracle_rht_colwise": (None, [P, I, I64, I64, U32, P]),
        "oracle_rht_colwise_ex": (None, [P, I, I64, I64, U32, I, P]),
        "oracle_round_bf16": (F, [F]),
        "oracle_compute_amax": (None, [P, I, I64, I64, I, U32, P, P]),
        "oracle_quantize": (I, [P, I, I64, I64, I, I, I, U32, I, U32, P, P, P, P, P, P]),
        "oracle_quantize_fmt": (I, [P, I, I64, I64, I, I, I, U32, I, U32, P, P, P, P, P, P, I]),
        "oracle_ue5m3_value": (ctypes.c_double, [U8]),
        "oracle_ue5m3_rne_satfinite": (U8, [F]),
        "oracle_ue5m3_array": (None, [P, I64, P]),
        "oracle_global_encode_scale_fmt": (F, [F, I]),
        "oracle_block_scale_fmt": (U8, [F, F, I]),
        "oracle_block_encode_multiplier_fmt": (F, [U8, F, I]),
        "oracle_dequantize_fmt": (None, [P, P, P, I, I64, I64, P, I]),
        "oracle_swizzle_offset": (I64, [I64, I64, I64]),
        "oracle_swizzle_scales": (I, [P, I64, I64, P]),
        "oracle_swizzle_scales_padded": (None, [P, I64, I64, P]),
        "oracle_dequantize": (None, [P, P, P, I, I64, I64, P]),
        "oracle_e2m1_rne_array": (None, [P, I64, P]),
        "oracle_e2m1_sr_array": (None, [P, P, I64, P]),
        "oracle_e4m3_array": (None, [P, I64, P]),
        "oracle_fmix32_array": (None, [P, I64, P]),
        "oracle_num_threads": (I, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _input(x):
    """(contiguous array, dtype code) for a BF16 (uint16 bits) or FP32 host array."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, BF16
    if x.dtype == np.float32:
        return x, FP32
    raise TypeError("oracle input must be uint16 (BF16 bits) or float32")


# ---- scalar steps -------------------------------------------------------

def e2m1_rne(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_e2m1_rne_array(_ptr(v), v.size, _ptr(out))
    return out


def e2m1_sr(v, r16) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    r16 = np.ascontiguousarray(np.broadcast_to(r16, v.shape), dtype=np.uint16)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_e2m1_sr_array(_ptr(v), _ptr(r16), v.size, _ptr(out))
    return out


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(code)


def e4m3(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_e4m3_array(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(code)


def ue5m3(v) -> np.ndarray:
    """UE5M3 codes (nearest even, saturating to 61440) of non-negative values."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_ue5m3_array(_ptr(v), v.size, _ptr(out))
    return out


def ue5m3_value(code: int) -> float:
    return _load().oracle_ue5m3_value(code)


SCALE_E4M3 = 0
SCALE_UE5M3 = 1


def global_encode_scale(amax: float, scale_fmt: int = SCALE_E4M3) -> float:
    return _load().oracle_global_encode_scale_fmt(amax, scale_fmt)


def block_scale(block_amax: float, S: float, scale_fmt: int = SCALE_E4M3) -> int:
    return _load().oracle_block_scale_fmt(block_amax, S, scale_fmt)


def block_encode_multiplier(s: int, S: float, scale_fmt: int = SCALE_E4M3) -> float:
    return _load().oracle_block_encode_multiplier_fmt(s, S, scale_fmt)


def fmix32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint32)
    out = np.empty(h.shape, np.uint32)
    _load().oracle_fmix32_array(_ptr(h), h.size, _ptr(out))
    return out


def sr_word(seed: int, direction: int, byte_index: int) -> int:
    return _load().oracle_sr_word(seed, direction, byte_index)


def rht16(w, sign_mask: int) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.float32)
    assert w.shape == (16,)
    t = np.empty(16, np.float32)
    _load().oracle_rht16(_ptr(w), sign_mask, _ptr(t))
    return t


def swizzle_offset(r: int, c: int, scale_cols: int) -> int:
    return _load().oracle_swizzle_offset(r, c, scale_cols)


# ---- whole-tensor steps -------------------------------------------------

def round_bf16(v) -> np.ndarray:
    """Each binary32 value rounded to BF16 (nearest, ties to even), as binary32."""
    v = np.asarray(v, np.float32)
    f = _load().oracle_round_bf16
    return np.array([f(float(a)) for a in v.ravel()], np.float32).reshape(v.shape)


def rht_colwise(x, sign_mask: int, bf16: bool = False) -> np.ndarray:
    """Column-wise RHT image t[cols][rows] of x[rows][cols] (rows % 16 == 0);
    bf16 rounds every transformed value to BF16."""
    x, dt = _input(x)
    rows, cols = x.shape
    t = np.empty((cols, rows), np.float32)
    _load().oracle_rht_colwise_ex(_ptr(x), dt, rows, cols, sign_mask, int(bf16), _ptr(t))
    return t


AMAX_PER_TENSOR = 0
AMAX_PER_ROW = 1
AMAX_RHT = 2
AMAX_RHT_BF16 = 3


def compute_amax(x, mode: int = AMAX_PER_TENSOR, sign_mask: int = 0):
    """Returns (amax_row, amax_col): [1] and [1], or, per row, [rows] and
    [cols] (the column-wise tensor of a row-scaled quantize is scaled along
    its own rows, which are the input's columns)."""
    x, dt = _input(x)
    rows, cols = x.shape
    if mode == AMAX_PER_ROW:
        a = np.empty(rows, np.float32)
        b = np.empty(cols, np.float32)
        _load().oracle_compute_amax(_ptr(x), dt, rows, cols, mode, sign_mask, _ptr(a), _ptr(b))
        return a, b
    a = np.empty(1, np.float32)
    b = np.empty(1, np.float32)
    _load().oracle_compute_amax(_ptr(x), dt, rows, cols, mode, sign_mask, _ptr(a), _ptr(b))
    return a, b


def quantize(x, *, rowwise=True, columnwise=True, block_2d=False, row_scaled=False, rht=False,
             sign_mask=0, stochastic=False, sr_seed=0, amax_row=None, amax_col=None, rht_bf16=False,
             scale_fmt=SCALE_E4M3):
    """Quantize with the given amaxes (computed here when None). rht_bf16
    (with rht): the transformed values are rounded to BF16 before the
    column-wise amax, block scales and codes.

    Returns a dict with ``row_data``, ``row_scales``, ``col_data``,
    ``col_scales`` (compact; absent directions are None), ``amax_row``,
    ``amax_col``.
    """
    x, dt = _input(x)
    rows, cols = x.shape
    if amax_row is None and amax_col is None:
        mode = AMAX_PER_ROW if row_scaled else ((AMAX_RHT_BF16 if rht_bf16 else AMAX_RHT) if rht else AMAX_PER_TENSOR)
        amax_row, amax_col = compute_amax(x, mode, sign_mask)
    amax_row = None if amax_row is None else np.ascontiguousarray(amax_row, np.float32)
    amax_col = None if amax_col is None else np.ascontiguousarray(amax_col, np.float32)
    rd = np.empty((rows, cols // 2), np.uint8) if rowwise else None
    rs = np.empty((rows, cols // 16), np.uint8) if rowwise else None
    cd = np.empty((cols, rows // 2), np.uint8) if columnwise else None
    cs = np.empty((cols, rows // 16), np.uint8) if columnwise else None
    rc = _load().oracle_quantize_fmt(
        _ptr(x), dt, rows, cols, int(block_2d), int(row_scaled), (2 if rht_bf16 else 1) if rht else 0, sign_mask,
        int(stochastic), sr_seed, _ptr(amax_row) if rowwise else None,
        _ptr(amax_col) if columnwise else None, _ptr(rd), _ptr(rs), _ptr(cd), _ptr(cs), int(scale_fmt))
    if rc != 0:
        raise ValueError("unsupported oracle configuration")
    return {"row_data": rd, "row_scales": rs, "col_data": cd, "col_scales": cs,
            "amax_row": amax_row if rowwise else None, "amax_col": amax_col if columnwise else None}


def quantize_grouped(x, group_rows, *, rowwise=True, columnwise=True, block_2d=False, rht=False, sign_mask=0,
                     stochastic=False, sr_seed=0, amax_row=None, amax_col=None, rht_bf16=False,
                     scale_fmt=SCALE_E4M3, row_scaled=False):
    """Grouped quantize. The row-scaled page's changed files keep a grouped
    tensor as one tensor per group with per-group amax offsets; reading: the
    consecutive row slices x[s_g : s_g + m_g] (m_g = group_rows[g]) are each
    quantized as a tensor of their own, with the same options (the same SR
    seed, byte indices counted within the group's own arrays).

    Returns flat arrays in group order: row_data (= [R][C/2]), row_scales
    (= [R][C/16], compact), col_data (group g's [C][m_g/2] blocks one after
    another), col_scales (group g's [C][m_g/16] blocks), amax_row [G],
    amax_col [G]. amax_row / amax_col, when given, are per-group arrays.
    row_scaled (row-wise only): each group's amax has one entry per row, so
    amax_row is [R] (the same page's grouped storage sizes it as the sum of
    the groups' rows); a given amax_row is then [R] too.
    """
    if row_scaled:
        columnwise = False
    x, _ = _input(x)
    rows, cols = x.shape
    group_rows = [int(m) for m in group_rows]
    if sum(group_rows) != rows or min(group_rows) < 0:
        raise ValueError("group rows must be non-negative and add up to the input's rows")
    parts = {k: [] for k in ("row_data", "row_scales", "col_data", "col_scales", "amax_row", "amax_col")}
    start = 0
    for g, m in enumerate(group_rows):
        xs = x[start:start + m]
        start += m
        if m == 0:
            if not row_scaled:
                parts["amax_row"].append(np.zeros(1, np.float32))
            parts["amax_col"].append(np.zeros(1, np.float32))
            continue
        given = {}
        if row_scaled and amax_row is not None:
            given = dict(amax_row=np.asarray(amax_row, np.float32)[start - m:start])
        elif amax_row is not None or amax_col is not None:
            given = dict(amax_row=None if amax_row is None else np.asarray(amax_row, np.float32)[g:g + 1],
                         amax_col=None if amax_col is None else np.asarray(amax_col, np.float32)[g:g + 1])
        q = quantize(xs, rowwise=rowwise, columnwise=columnwise, block_2d=block_2d, rht=rht, sign_mask=sign_mask,
                     stochastic=stochastic, sr_seed=sr_seed, rht_bf16=rht_bf16, scale_fmt=scale_fmt,
                     row_scaled=row_scaled, **given)
        for k in ("row_data", "row_scales", "col_data", "col_scales"):
            if q[k] is not None:
                parts[k].append(q[k].reshape(-1))
        parts["amax_row"].append(q["amax_row"] if rowwise else np.zeros(1, np.float32))
        parts["amax_col"].append(q["amax_col"] if columnwise else np.zeros(1, np.float32))
    out = {}
    for k in ("row_data", "row_scales", "col_data", "col_scales"):
        on = rowwise if k.startswith("row") else columnwise
        out[k] = (np.concatenate(parts[k]) if parts[k] else np.zeros(0, np.uint8)) if on else None
    out["amax_row"] = (np.concatenate(parts["amax_row"]).astype(np.float32) if parts["amax_row"]
                       else np.zeros(0, np.float32)) if rowwise else None
    out["amax_col"] = np.concatenate(parts["amax_col"]).astype(np.float32) if columnwise else None
    return out


def swizzle_scales(compact) -> np.ndarray:
    """Compact [rows][scale_cols] -> GEMM-swizzled flat array (rows % 128, scale_cols % 4)."""
    compact = np.ascontiguousarray(compact, np.uint8)
    rows, sc = compact.shape
    out = np.empty(rows * sc, np.uint8)
    if _load().oracle_swizzle_scales(_ptr(compact), rows, sc, _ptr(out)) != 0:
        raise ValueError("swizzled layout needs rows % 128 == 0 and scale_cols % 4 == 0")
    return out


def swizzled_size(rows: int, scale_cols: int) -> int:
    """Bytes of the zero-padded GEMM layout of a [rows][scale_cols] scale matrix."""
    return (rows + 127) // 128 * 128 * ((scale_cols + 3) // 4 * 4)


def swizzle_scales_padded(compact) -> np.ndarray:
    """Compact [rows][scale_cols], any shape -> zero-padded GEMM-swizzled flat array."""
    compact = np.ascontiguousarray(compact, np.uint8)
    rows, sc = compact.shape
    out = np.empty(swizzled_size(rows, sc), np.uint8)
    _load().oracle_swizzle_scales_padded(_ptr(compact), rows, sc, _ptr(out))
    return out


def dequantize(data, scales, amax, rows: int, cols: int, row_scaled: bool = False,
               scale_fmt: int = SCALE_E4M3) -> np.ndarray:
    """One direction, its own orientation [rows][cols], compact scales."""
    data = np.ascontiguousarray(data, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    amax = np.ascontiguousarray(amax, np.float32)
    y = np.empty((rows, cols), np.float32)
    _load().oracle_dequantize_fmt(_ptr(data), _ptr(scales), _ptr(amax), int(row_scaled), rows, cols, _ptr(y),
                                  int(scale_fmt))
    return y
