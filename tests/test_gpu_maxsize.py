"""GPU: the largest accepted input (R * C just below 2^32): 65536 x 65520
BF16, both orientations, 1x16 blocks, checked on sampled blocks across the
whole tensor (first, middle and last tiles) against the oracle computing
those blocks one by one with the tensor's amax; and the row-scaled
column-wise side (one amax per input column) on the same samples. Byte
offsets and the stochastic-rounding byte indices reach 2^31 here."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_05_amd as nv
import oracle as O
from gpu_helpers import DEV, host

pytestmark = pytest.mark.gpu

R, C = 65536, 65520  # R * C = 4,293,918,720 < 2^32
SEED = 11
# (row, column) corners of sampled 16 x 128 regions: first tile, ragged last
# tile column, last rows, and a few in between
SAMPLES = [(0, 0), (0, C - 128), (R - 16, C - 128), (R - 16, 0), (32768, 32768), (12304, 50000 // 16 * 16),
           (65520, 65392 - 128)]


@pytest.fixture(scope="module")
def big():
    if torch.cuda.get_device_properties(0).total_memory < 40 * 2 ** 30:
        pytest.skip("needs about 30 GiB of device memory")
    g = torch.Generator(device=DEV).manual_seed(SEED)
    x = torch.empty((R, C), dtype=torch.bfloat16, device=DEV)
    for r0 in range(0, R, 8192):  # generate in slabs to bound the FP32 temporary
        x[r0:r0 + 8192] = torch.randn((8192, C), generator=g, device=DEV).to(torch.bfloat16)
    x[R - 1, C - 1] = -768.0  # the amax (a BF16 value), in the very last element
    yield x
    del x
    torch.cuda.empty_cache()


def _host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _check_samples(x, row, col, stochastic):
    amax = np.float32(768.0)
    assert host(row.amax)[0] == amax and host(col.amax)[0] == amax
    rd, rs = row.data, row.scales.view(R, C // 16)
    cd, cs = col.data, col.scales.view(C, R // 16)
    for (i, j) in SAMPLES:
        xs = _host_bf16(x[i:i + 16, j:j + 128])
        if not stochastic:
            ref = O.quantize(xs, amax_row=np.float32([amax]), amax_col=np.float32([amax]))
            assert np.array_equal(host(rd[i:i + 16, j // 2:j // 2 + 64]), ref["row_data"]), (i, j)
            assert np.array_equal(host(rs[i:i + 16, j // 16:j // 16 + 8]), ref["row_scales"]), (i, j)
            assert np.array_equal(host(cd[j:j + 128, i // 2:i // 2 + 8]), ref["col_data"]), (i, j)
            assert np.array_equal(host(cs[j:j + 128, i // 16:i // 16 + 1]), ref["col_scales"]), (i, j)
        else:
            # the codes depend on each byte's index in the whole array: rebuild
            # the sampled bytes from the oracle's steps with those indices
            xf = (xs.astype(np.uint32) << 16).view(np.float32)
            S = O.global_encode_scale(float(amax))
            for direction, vals, base_rows, half in ((0, xf, i, C // 2), (1, xf.T, j, R // 2)):
                got = host(rd[i:i + 16, j // 2:j // 2 + 64]) if direction == 0 else host(cd[j:j + 128, i // 2:i // 2 + 8])
                first = (j if direction == 0 else i) // 2
                for r in range(vals.shape[0]):
                    line = vals[r]
                    want = np.empty(line.size // 2, np.uint8)
                    for b in range(line.size // 16):
                        blk = line[16 * b:16 * b + 16]
                        s = O.block_scale(float(np.abs(blk).max()), S)
                        e = np.float32(O.block_encode_multiplier(s, S))
                        v = (blk * e).astype(np.float32)
                        for k in range(8):
                            byte_index = (base_rows + r) * half + first + 8 * b + k
                            w = O.sr_word(9, direction, byte_index)
                            lo = O.e2m1_sr(v[2 * k:2 * k + 1], np.uint16([w & 0xFFFF]))[0]
                            hi = O.e2m1_sr(v[2 * k + 1:2 * k + 2], np.uint16([w >> 16]))[0]
                            want[8 * b + k] = lo | (hi << 4)
                    assert np.array_equal(got[r], want), (direction, i, j, r)


@pytest.mark.parametrize("stochastic", [False, True], ids=["rne", "sr"])
def test_largest_input(big, stochastic):
    cfg = nv.make_config(stochastic=stochastic, sr_seed=9)
    row, col = nv.quantize(big, cfg=cfg)
    torch.cuda.synchronize()
    _check_samples(big, row, col, stochastic)
    del row, col


def test_largest_input_row_scaled_columnwise(big):
    # one amax per input column; sampled columns checked against a plain
    # torch reduction of that column, sampled blocks against the oracle with
    # those amaxes
    _, col = nv.quantize(big, rowwise=False, cfg=nv.make_config(row_scaled=True))
    torch.cuda.synchronize()
    amax = host(col.amax)
    cd, cs = col.data, col.scales.view(C, R // 16)
    for (i, j) in SAMPLES:
        ref_amax = big[:, j:j + 128].abs().amax(dim=0).float().cpu().numpy()
        np.testing.assert_array_equal(amax[j:j + 128], ref_amax, err_msg=f"column amax at {j}")
        xs = _host_bf16(big[i:i + 16, j:j + 128])
        ref = O.quantize(xs, rowwise=False, row_scaled=True, amax_col=ref_amax)
        assert np.array_equal(host(cd[j:j + 128, i // 2:i // 2 + 8]), ref["col_data"]), (i, j)
        assert np.array_equal(host(cs[j:j + 128, i // 16:i // 16 + 1]), ref["col_scales"]), (i, j)
    del col
