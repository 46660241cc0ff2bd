"""The kernels' E4M3 (and UE5M3) block-scale encoders are branch-free bit arithmetic:
at and above 2^-6 the binary32 pattern rounded to 3 mantissa bits by an
integer add (0x7FFFF plus the kept low bit, ties to even, a carry bumps
the exponent) and rebiased from 127 to 7; below 2^-6 the nearest-even
multiple of 2^-9; codes past 0x7E saturate. This pins that rule against
the oracle's E4M3 encoder (nearest even over the decoded values,
saturating) on every positive BF16 value, around every rounding midpoint
of the format, over the subnormal range and on random binary32 values."""

from __future__ import annotations

import numpy as np
import pytest

import oracle as O


def formula(sd: np.ndarray, ue5m3: bool = False) -> np.ndarray:
    rebias, quantum, tiny, top = (112, 131072.0, 6.103515625e-05, 0xF7) if ue5m3 else (120, 512.0, 0.015625, 0x7E)
    u = sd.view(np.uint32).astype(np.uint64)
    normal = ((u + 0x7FFFF + ((u >> 20) & 1)) >> 20) - (rebias << 3)
    with np.errstate(over="ignore", invalid="ignore"):  # large sd overflow here but take `normal`
        sub = np.rint(sd * np.float32(quantum)).astype(np.uint64)
    code = np.where(sd < np.float32(tiny), sub, normal & 0xFFFFFFFF)
    return np.minimum(code, top).astype(np.uint8)


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3"])
def test_scale_formula_matches_the_oracle(fmt):
    ue = fmt == "ue5m3"
    rng = np.random.default_rng(12)
    parts = [np.arange(0, 0x7F80, dtype=np.uint32) << 16]  # every positive BF16 value, 0 .. just below inf
    top = 0xF8 if ue else 0x7F
    values = np.array([(O.ue5m3_value if ue else O.e4m3_value)(c) for c in range(top)], dtype=np.float64)
    mids = ((values[:-1] + values[1:]) / 2).astype(np.float32)
    around = np.arange(-2000, 2001, dtype=np.int64)
    for m in mids:
        parts.append((np.int64(m.view(np.uint32)) + around).clip(0, 0x7F7FFFFF).astype(np.uint32))
    parts.append(np.arange(0, 0x38800000 if ue else 0x3C800000, 997, dtype=np.uint32))  # subnormal codes, strided
    parts.append(rng.integers(0, 0x7F800000, 4_000_000, dtype=np.uint32))
    parts.append(np.array([0x7F800000, 0x7F7FFFFF, 0x43E00000, 0x43E40000, 0x43E80000, 0x3C800000, 0x3C7FFFFF,
                           0x47700000, 0x47780000, 0x47800000, 0x38800000, 0x387FFFFF, 0, 1], dtype=np.uint32))
    # +inf, FLT_MAX, 448, 456, 464, 2^-6 and below, 61440, 63488, 65536, 2^-14 and below, 0, smallest denormal
    sd = np.concatenate(parts).view(np.float32)
    want = O.ue5m3(sd) if ue else O.e4m3(sd)
    got = formula(sd, ue)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} differ, first {sd[bad[:4]]} got {got[bad[:4]]} want {want[bad[:4]]}"
