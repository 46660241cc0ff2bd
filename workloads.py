"""Seeded synthetic inputs for the NVFP4 quantize path.

This module is shared by the tests, the benchmark and the smoke check, and
feeds the same bytes to the GPU library and to the CPU oracle. It holds no
arithmetic of the quantization method: only random draws (torch's CPU
generator), the elementwise shaping that gives each workload its value
distribution, and the BF16 cast (torch's round-to-nearest-even).

The pages measure on ``torch.randn`` BF16 matrices at shapes from 1024x1024
to 8192x5120 ("Time per quantize call" on the pages "Write both NVFP4 amax
buffers" and "Fuse NVFP4 scale swizzling on SM120 and SM121"); no public
dataset is involved. The five workloads below keep those shapes and add the
structure each part of the path needs:

* ``c1``  1024x1024 BF16, N(0,1), seed 0: 1D, both directions, compact scales.
* ``c2``  8192x5120 BF16, N(0,1) times a per-column factor 10^(-3+5u),
  u ~ U[0,1), seed 1: 2D blocks, both directions, GEMM-swizzled scales.
* ``c3``  five 1088x1024 FP32 inputs, seed 2, with max|x| exactly
  8, 2, 0.5, 0 (all zero), 32, in that order, for one reused output.
* ``c4``  4096x8192 BF16, N(0,1) times a per-row factor exp(2 n), n ~ N(0,1),
  seed 3: per-row (row-scaled) amax, row-wise output only.
* ``c5``  8192x8192 BF16 N(0,1), seed 4, with 0.1% of the elements set to
  +-200; RHT sign mask and stochastic-rounding seed from seed 5.

BF16 arrays are returned as numpy ``uint16`` holding the bit patterns;
FP32 arrays as ``float32``.
"""

from __future__ import annotations

import hashlib

import numpy as np
import torch


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """FP32 tensor -> BF16 (round to nearest even) -> uint16 bit patterns."""
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float32 values (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def randn_bf16(rows: int, cols: int, seed: int) -> np.ndarray:
    g = torch.Generator().manual_seed(seed)
    return bf16_bits(torch.randn(rows, cols, generator=g))


def c1(rows: int = 1024, cols: int = 1024) -> np.ndarray:
    return randn_bf16(rows, cols, 0)


def c2(rows: int = 8192, cols: int = 5120, seed: int = 1) -> np.ndarray:
    g = torch.Generator().manual_seed(seed)
    z = torch.randn(rows, cols, generator=g)
    u = torch.rand(cols, generator=g)
    f = torch.pow(10.0, -3.0 + 5.0 * u)
    return bf16_bits(z * f[None, :])


C3_MAXIMA = (8.0, 2.0, 0.5, 0.0, 32.0)


def c3(rows: int = 1088, cols: int = 1024, seed: int = 2) -> list:
    """Five FP32 inputs whose max|x| is exactly 8, 2, 0.5, 0, 32."""
    g = torch.Generator().manual_seed(seed)
    out = []
    for m in C3_MAXIMA:
        if m == 0.0:
            out.append(np.zeros((rows, cols), np.float32))
            continue
        z = torch.randn(rows, cols, generator=g)
        x = (z / z.abs().max()) * m  # the largest element becomes exactly +-m
        out.append(x.numpy().astype(np.float32))
    return out


def c4(rows: int = 4096, cols: int = 8192, seed: int = 3) -> np.ndarray:
    g = torch.Generator().manual_seed(seed)
    z = torch.randn(rows, cols, generator=g)
    rho = torch.exp(2.0 * torch.randn(rows, generator=g))
    return bf16_bits(z * rho[:, None])


def c5(rows: int = 8192, cols: int = 8192, seed: int = 4, outlier_fraction: float = 1e-3):
    """Returns (x bf16 bits, rht sign mask, stochastic-rounding seed)."""
    g = torch.Generator().manual_seed(seed)
    z = torch.randn(rows, cols, generator=g).to(torch.bfloat16)
    n = rows * cols
    k = int(round(n * outlier_fraction))
    pos = torch.randperm(n, generator=g)[:k]
    sgn = 2.0 * torch.randint(0, 2, (k,), generator=g).to(torch.float32) - 1.0
    flat = z.view(-1)
    flat[pos] = (200.0 * sgn).to(torch.bfloat16)
    x = flat.view(rows, cols).view(torch.int16).numpy().view(np.uint16).copy()
    return x, rht_sign_mask(5), 5


def rht_sign_mask(seed: int = 5) -> int:
    g = torch.Generator().manual_seed(seed)
    return int(torch.randint(0, 65536, (1,), generator=g).item())


def gaussian_fp32(rows: int, cols: int, seed: int, scale: float = 1.0) -> np.ndarray:
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(rows, cols, generator=g) * scale).numpy().astype(np.float32)
