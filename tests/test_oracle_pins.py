"""Pins of the CPU oracle to things other than itself.

Each test checks one oracle step against a library routine, a closed form,
a hand-worked block, an invariant of the mathematics, brute force on small
inputs, or a value printed on the pages. None of these recomputes the
oracle's own formula the oracle's way. No GPU is needed.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FLT_MAX = float(np.finfo(np.float32).max)


def f32(v):
    return np.array(v, dtype=np.float32)


def bits(v):
    return f32(v).view(np.uint32)


def from_bits(u):
    return np.array(u, dtype=np.uint32).view(np.float32)


def bf16(vals):
    return W.bf16_bits(torch.tensor(vals, dtype=torch.float32))


# ----------------------------------------------------------------------------
# E4M3 block-scale encoding: pinned to torch's float8_e4m3fn cast (RNE).
# ----------------------------------------------------------------------------

def test_e4m3_decode_matches_torch_for_every_code():
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([O.e4m3_value(int(c)) for c in range(0x7F)], dtype=np.float64)
    np.testing.assert_array_equal(got, ref.astype(np.float64))


def _e4m3_probe_values():
    lim = int(bits(464.0))
    sweep = np.arange(0, lim + 1, 997, dtype=np.uint32)
    # every representable value and every midpoint, +-40 ulps around each
    vals = np.array([O.e4m3_value(c) for c in range(0x7F)])
    mids = 0.5 * (vals[:-1] + vals[1:])
    centers = bits(np.concatenate([vals, mids]).astype(np.float32)).astype(np.int64)
    near = (centers[:, None] + np.arange(-40, 41)[None, :]).ravel()
    near = near[(near >= 0) & (near <= lim)].astype(np.uint32)
    return from_bits(np.unique(np.concatenate([sweep, near])))


def test_e4m3_rne_matches_torch_on_0_to_464():
    v = _e4m3_probe_values()
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3(v)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]


def test_e4m3_saturates_above_464_instead_of_nan():
    # torch's cast is non-saturating above 464; the block scale saturates to 448.
    v = f32([464.00003, 470.0, 1000.0, 1e30, FLT_MAX, np.inf])
    assert list(O.e4m3(v)) == [0x7E] * 6


def test_e4m3_hand_worked_boundaries():
    # 2^-10 is the midpoint of 0 and the smallest subnormal 2^-9 -> even code 0;
    # 3*2^-11 is above it -> code 1; 2^-6 is the smallest normal (e=1, m=0).
    assert list(O.e4m3(f32([0.0, 2.0**-10, 3 * 2.0**-11, 2.0**-6, 448.0]))) == [0, 0, 1, 8, 0x7E]


# ----------------------------------------------------------------------------
# E2M1 round to nearest even: brute force on small inputs with exact rationals.
# ----------------------------------------------------------------------------

def _e2m1_magnitude_from_bits(code):
    # E2M1: 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal.
    e, m = (code >> 1) & 3, code & 1
    return Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))


def _e2m1_nearest_even(v: float) -> int:
    a = abs(Fraction(v))
    best = min(range(8), key=lambda c: (abs(a - _e2m1_magnitude_from_bits(c)), c & 1))
    return best | (8 if math.copysign(1.0, v) < 0 else 0)


def test_e2m1_grid_magnitudes_from_format():
    for c in range(16):
        mag = _e2m1_magnitude_from_bits(c & 7)
        assert O.e2m1_value(c) == (-float(mag) if c & 8 else float(mag))


def test_e2m1_brute_force_all_bf16_values():
    allbits = np.arange(65536, dtype=np.uint32)
    v = (allbits << 16).view(np.float32)
    v = v[np.isfinite(v)]
    got = O.e2m1_rne(v)
    ref = np.array([_e2m1_nearest_even(float(x)) for x in v], np.uint8)
    assert np.array_equal(got, ref)


def test_e2m1_brute_force_fp32_near_every_decision_point():
    pts = [0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, 7.0]
    centers = bits(pts).astype(np.int64)
    u = (centers[:, None] + np.arange(-300, 301)[None, :]).ravel()
    u = u[u >= 0].astype(np.uint32)
    v = from_bits(u)
    v = np.concatenate([v, -v])
    got = O.e2m1_rne(v)
    ref = np.array([_e2m1_nearest_even(float(x)) for x in v], np.uint8)
    assert np.array_equal(got, ref)


def test_e2m1_ties_table():
    # midpoints go to the neighbour with the even (zero) mantissa bit
    ties = {0.25: 0x0, 0.75: 0x2, 1.25: 0x2, 1.75: 0x4, 2.5: 0x4, 3.5: 0x6, 5.0: 0x6}
    for v, c in ties.items():
        assert O.e2m1_rne(f32([v]))[0] == c
        assert O.e2m1_rne(f32([-v]))[0] == c | 8
    assert list(O.e2m1_rne(f32([-0.0, 6.5, 1e30, -1e30, 1e-40, -1e-40]))) == [8, 7, 7, 15, 0, 8]


# ----------------------------------------------------------------------------
# Stochastic rounding: closed forms and statistics.
# ----------------------------------------------------------------------------

def test_sr_up_count_over_all_random_words_is_ceil_frac():
    r = np.arange(65536, dtype=np.uint16)
    for v in [0.1, 0.3, 0.6, 1.1, 1.2345, 1.9, 2.25, 2.9, 3.7, 4.5, 5.999]:
        a = Fraction(float(np.float32(v)))
        mags = [_e2m1_magnitude_from_bits(c) for c in range(8)]
        k = max(i for i in range(8) if mags[i] <= a)
        frac = (a - mags[k]) / (mags[k + 1] - mags[k])
        codes = O.e2m1_sr(np.full(65536, v, np.float32), r)
        up = int(np.sum(codes == k + 1))
        assert up == math.ceil(frac * 65536), v
        assert set(np.unique(codes)) <= {k, k + 1}


def test_sr_grid_values_are_fixed_points_and_saturation():
    r = np.arange(65536, dtype=np.uint16)
    for c in range(8):
        v = float(_e2m1_magnitude_from_bits(c))
        assert np.all(O.e2m1_sr(np.full(65536, v, np.float32), r) == c)
        assert np.all(O.e2m1_sr(np.full(65536, -v, np.float32), r) == c | 8)
    assert np.all(O.e2m1_sr(np.full(65536, 6.7, np.float32), r) == 7)


def test_fmix32_published_vectors():
    # MurmurHash3_x86_32 of the empty key equals fmix32(seed); the published
    # test vectors for seeds 0, 1 and 0xffffffff are 0, 0x514E28B7, 0x81F16F39.
    got = O.fmix32(np.array([0, 1, 0xFFFFFFFF], np.uint32))
    assert [int(x) for x in got] == [0, 0x514E28B7, 0x81F16F39]


def test_sr_words_are_uniform_and_direction_keyed():
    w0 = np.array([O.sr_word(5, 0, b) for b in range(20000)], np.uint64)
    w1 = np.array([O.sr_word(5, 1, b) for b in range(20000)], np.uint64)
    assert not np.any(w0 == w1)
    lo = (w0 & 0xFFFF).astype(np.float64) / 65536
    hi = (w0 >> 16).astype(np.float64) / 65536
    for s in (lo, hi):
        assert abs(s.mean() - 0.5) < 4 * math.sqrt(1 / 12 / s.size)


def test_sr_quantize_is_unbiased_on_a_whole_tensor():
    # every row block and every column block holds a 6 (so S = 448, s = 448,
    # e = 1); the other values are 1.25, half way between 1.0 and 1.5, so
    # about half of them must round up.
    rows, cols = 256, 1024
    x = np.full((rows, cols), 1.25, np.float32)
    x[:, ::16] = 6.0
    x[::16, :] = 6.0
    q = O.quantize(x, rowwise=True, columnwise=True, stochastic=True, sr_seed=5)
    for data in (q["row_data"], q["col_data"]):
        codes = np.stack([data & 0xF, data >> 4], -1).ravel()
        codes = codes[codes != 7]
        frac_up = np.mean(codes == 3)
        assert set(np.unique(codes)) <= {2, 3}
        assert abs(frac_up - 0.5) < 4 * math.sqrt(0.25 / codes.size)


# ----------------------------------------------------------------------------
# 16-point RHT: scipy's Sylvester Hadamard matrix, closed forms, the pages' table.
# ----------------------------------------------------------------------------

def test_rht16_matches_scipy_hadamard_on_bf16_groups():
    H = scipy.linalg.hadamard(16).astype(np.float64)
    rng = np.random.default_rng(0)
    for trial in range(200):
        w = W.bf16_to_float(W.bf16_bits(torch.from_numpy(rng.standard_normal(16).astype(np.float32) * 3)))
        mask = int(rng.integers(0, 65536))
        sigma = np.array([-1.0 if (mask >> k) & 1 else 1.0 for k in range(16)])
        ref = (0.25 * (H @ (sigma * w.astype(np.float64)))).astype(np.float32)
        np.testing.assert_array_equal(O.rht16(w, mask), ref)


def test_rht16_closed_forms():
    e0 = np.zeros(16, np.float32)
    e0[0] = 64.0
    np.testing.assert_array_equal(O.rht16(e0, 0), np.full(16, 16.0, np.float32))
    np.testing.assert_array_equal(O.rht16(e0, 1), np.full(16, -16.0, np.float32))
    for m in range(16):
        em = np.zeros(16, np.float32)
        em[m] = 64.0
        ref = np.array([16.0 * (-1) ** bin(r & m).count("1") for r in range(16)], np.float32)
        np.testing.assert_array_equal(O.rht16(em, 0), ref)
    c = np.full(16, 3.0, np.float32)
    t = O.rht16(c, 0)
    assert t[0] == 12.0 and np.all(t[1:] == 0.0)


def test_rht16_is_an_involution_and_preserves_energy():
    rng = np.random.default_rng(1)
    for _ in range(100):
        w = rng.standard_normal(16).astype(np.float32)
        t = O.rht16(w, 0)
        np.testing.assert_allclose(O.rht16(t, 0), w, rtol=0, atol=1e-6)
        assert abs(np.sum(t.astype(np.float64) ** 2) - np.sum(w.astype(np.float64) ** 2)) < 1e-5 * np.sum(w**2)


def test_rht_colwise_groups_are_columns():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 24)).astype(np.float32)
    mask = 0xA5C3
    t = O.rht_colwise(x, mask)
    for j in (0, 7, 23):
        for g in range(4):
            np.testing.assert_array_equal(t[j, 16 * g:16 * g + 16], O.rht16(x[16 * g:16 * g + 16, j], mask))


def test_rht_amax_magnitudes_printed_on_the_pages():
    fx = json.load(open(os.path.join(GOLDEN, "rht_review_amax.json")))
    rows, cols = fx["shape"]
    x = W.randn_bf16(rows, cols, 11)
    xs = x.copy()
    xs[100, 200] = bf16([64.0])[0]
    mask = W.rht_sign_mask(5)
    plain, spike = fx["cases"]
    a_row, a_col = O.compute_amax(x, O.AMAX_RHT, mask)
    # Gaussian tails: the pages print 4.375 / 5.03125; any seed lands near them.
    assert 3.5 <= a_row[0] <= 5.5 and 3.5 <= a_col[0] <= 6.5
    a_row, a_col = O.compute_amax(xs, O.AMAX_RHT, mask)
    assert a_row[0] == spike["amax_rowwise"]
    # A lone 64 spreads to 64/4 = 16 in each of its group's outputs, plus the
    # neighbours' O(1) share: the printed 16.875. Size 8 would give ~22.6,
    # size 32 ~11.3, an unnormalized transform 64.
    assert 16.0 <= a_col[0] <= 18.5
    assert abs(a_col[0] - spike["amax_columnwise"]) < 1.5


# ----------------------------------------------------------------------------
# Amax: numpy's reduction on the same data; the exact maxima of the sequence.
# ----------------------------------------------------------------------------

def test_amax_per_tensor_and_per_row_match_numpy():
    x = W.randn_bf16(64, 96, 3)
    xf = W.bf16_to_float(x)
    a, b = O.compute_amax(x)
    assert a[0] == np.abs(xf).max() and b[0] == a[0]
    r, c = O.compute_amax(x, O.AMAX_PER_ROW)
    np.testing.assert_array_equal(r, np.abs(xf).max(axis=1))
    np.testing.assert_array_equal(c, np.abs(xf).max(axis=0))


def test_amax_sequence_exact_maxima():
    for m, x in zip(W.C3_MAXIMA, W.c3(rows=64, cols=64)):
        a, b = O.compute_amax(x)
        assert a[0] == m and b[0] == m


# ----------------------------------------------------------------------------
# Scale chain and whole-tensor quantize: hand-worked blocks and invariants.
# ----------------------------------------------------------------------------

def test_global_encode_scale_closed_forms():
    assert O.global_encode_scale(0.0) == 1.0
    assert O.global_encode_scale(6.0) == 448.0
    assert O.global_encode_scale(1.0) == 2688.0
    assert O.global_encode_scale(2688.0) == 1.0
    assert O.global_encode_scale(1e-44) == FLT_MAX


def test_worked_block_exact_grid():
    # amax 6 -> S = 2688/6 = 448, block max 6 -> sd = 1*448 = 448 -> 0x7E, e = 1:
    # every value is already on the grid and encodes to its own code.
    x = bf16([[0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6]])
    q = O.quantize(x, columnwise=False)
    assert q["row_data"].tobytes() == bytes.fromhex("1032547698badcfe")
    assert q["row_scales"].tobytes() == b"\x7e"
    y = O.dequantize(q["row_data"], q["row_scales"], q["amax_row"], 1, 16)
    np.testing.assert_array_equal(y, W.bf16_to_float(x))


def test_worked_block_ties():
    # e = 1 again; the ties go to even codes; bf16(0.1) = 0.10009765625 -> 0.
    x = bf16([[.25, .75, 1.25, 1.75, 2.5, 3.5, 5, 6, -.25, -.75, -1.25, -1.75, -2.5, -3.5, -5, 0.1]])
    q = O.quantize(x, columnwise=False)
    assert q["row_data"].tobytes() == bytes.fromhex("204264 76a8caec0e".replace(" ", ""))


def test_worked_block_scale_rounding():
    # Block 1 has max 1: sd = fl(fl(1/6) * 448) = 74.66667 -> nearest E4M3 is 72
    # (0x69: exponent 13-7 = 6, mantissa 1/8 -> 64 * 1.125); e = fl(448/72) =
    # 6.2222223; 1*e saturates to 6 (code 7), .5e = 3.11 -> 3 (5), .25e = 1.56
    # -> 1.5 (3), .125e = 0.78 -> 1.0 (2); negatives mirror with bit 3.
    x = bf16([[6] + [0] * 15 + [1, .5, .25, .125, -1, -.5, -.25, -.125] + [0] * 8])
    q = O.quantize(x, columnwise=False)
    assert q["row_scales"].tobytes() == b"\x7e\x69"
    assert q["row_data"].tobytes() == bytes.fromhex("0700000000000000" "5723dfab00000000")
    y = O.dequantize(q["row_data"], q["row_scales"], q["amax_row"], 1, 32)
    assert y[0, 16] == np.float32(432.0 / 448.0)  # 6 * 72 / 448 rounded once


def test_worked_block_amax_one():
    # amax 1 -> S = 2688; sd = fl(1/6)*2688 = 448.00000 -> 0x7E; e = 2688/448 = 6;
    # 1*6 = 6 -> code 7; bf16(0.3) = 0.30078125, *6 = 1.8046875 -> 2.0 (code 4).
    q = O.quantize(bf16([[1, 0.3] + [0] * 14]), columnwise=False)
    assert q["row_data"].tobytes() == bytes.fromhex("4700000000000000")
    assert q["row_scales"].tobytes() == b"\x7e"


def test_all_zero_tensor_encodes_zero_with_zero_scales():
    x = np.zeros((32, 32), np.float32)
    q = O.quantize(x)
    for k in ("row_data", "row_scales", "col_data", "col_scales"):
        assert not q[k].any()
    assert q["amax_row"][0] == 0.0 and q["amax_col"][0] == 0.0


def _codes(data):
    return np.stack([data & 0xF, data >> 4], -1).reshape(data.shape[0], -1)


@pytest.mark.parametrize("block_2d", [False, True])
def test_power_of_two_invariance(block_2d):
    # Scaling the tensor by 2^k scales amax, S^-1 and every sd by 2^k exactly,
    # so scale bytes and codes are unchanged.
    x = W.gaussian_fp32(64, 128, 7)
    q0 = O.quantize(x, block_2d=block_2d)
    for k in (-20, -3, 5, 30):
        qk = O.quantize((x * np.float32(2.0**k)).astype(np.float32), block_2d=block_2d)
        assert qk["amax_row"][0] == q0["amax_row"][0] * 2.0**k
        for key in ("row_data", "row_scales", "col_data", "col_scales"):
            assert np.array_equal(qk[key], q0[key]), (k, key)


def test_row_scaled_power_of_two_per_row():
    x = W.gaussian_fp32(16, 64, 8)
    q0 = O.quantize(x, columnwise=False, row_scaled=True)
    f = (2.0 ** np.arange(-8, 8)).astype(np.float32)
    q1 = O.quantize((x * f[:, None]).astype(np.float32), columnwise=False, row_scaled=True)
    assert np.array_equal(q0["row_data"], q1["row_data"])
    assert np.array_equal(q0["row_scales"], q1["row_scales"])
    np.testing.assert_array_equal(q1["amax_row"], q0["amax_row"] * f)


def test_row_scaled_row_equals_per_tensor_single_row():
    x = W.c4(rows=8, cols=256)
    q = O.quantize(x, columnwise=False, row_scaled=True)
    for r in range(8):
        qr = O.quantize(x[r:r + 1], columnwise=False)
        assert np.array_equal(q["row_data"][r], qr["row_data"][0])
        assert np.array_equal(q["row_scales"][r], qr["row_scales"][0])
        assert q["amax_row"][r] == qr["amax_row"][0]


# Row-scaled column-wise side (reading: the column-wise tensor, whose rows
# are the input's columns, is row-scaled along its own rows, so its amax
# buffer has one float per input column, as the quantizer prototype in the
# review thread of "Write both NVFP4 amax buffers" sizes it).

def test_row_scaled_columnwise_column_equals_per_tensor_single_row():
    x = W.c4(rows=64, cols=48, seed=5)
    q = O.quantize(x, rowwise=False, row_scaled=True)
    assert q["amax_col"].shape == (48,)
    for j in range(48):
        qj = O.quantize(np.ascontiguousarray(x[:, j:j + 1].T), columnwise=False)
        assert np.array_equal(q["col_data"][j], qj["row_data"][0]), j
        assert np.array_equal(q["col_scales"][j], qj["row_scales"][0]), j
        assert q["amax_col"][j] == qj["amax_row"][0], j


def test_row_scaled_columnwise_is_row_scaled_rowwise_of_transpose():
    x = W.gaussian_fp32(32, 80, 12)
    x *= (2.0 ** np.linspace(-6, 6, 80)).astype(np.float32)[None, :]
    q = O.quantize(x, row_scaled=True)
    qt = O.quantize(np.ascontiguousarray(x.T), columnwise=False, row_scaled=True)
    assert np.array_equal(q["col_data"], qt["row_data"])
    assert np.array_equal(q["col_scales"], qt["row_scales"])
    np.testing.assert_array_equal(q["amax_col"], qt["amax_row"])
    # and the row-wise side is unchanged by asking for both
    qr = O.quantize(x, columnwise=False, row_scaled=True)
    assert np.array_equal(q["row_data"], qr["row_data"]) and np.array_equal(q["row_scales"], qr["row_scales"])


def test_row_scaled_columnwise_power_of_two_per_column():
    x = W.gaussian_fp32(32, 16, 13)
    q0 = O.quantize(x, rowwise=False, row_scaled=True)
    f = (2.0 ** np.arange(-8, 8)).astype(np.float32)
    q1 = O.quantize((x * f[None, :]).astype(np.float32), rowwise=False, row_scaled=True)
    assert np.array_equal(q0["col_data"], q1["col_data"])
    assert np.array_equal(q0["col_scales"], q1["col_scales"])
    np.testing.assert_array_equal(q1["amax_col"], q0["amax_col"] * f)


def test_row_scaled_columnwise_equal_column_maxima_is_per_tensor_sr():
    # every column holds the tensor's maximum, so every per-column global
    # scale is the per-tensor one, stochastic rounding included
    x = W.gaussian_fp32(48, 32, 14)
    x[5, :] = 9.5
    q = O.quantize(x, rowwise=False, row_scaled=True, stochastic=True, sr_seed=21)
    qt = O.quantize(x, rowwise=False, stochastic=True, sr_seed=21)
    assert np.all(q["amax_col"] == 9.5)
    assert np.array_equal(q["col_data"], qt["col_data"])
    assert np.array_equal(q["col_scales"], qt["col_scales"])


def test_columnwise_is_rowwise_of_transpose():
    x = W.gaussian_fp32(48, 80, 9)
    q = O.quantize(x)
    qt = O.quantize(np.ascontiguousarray(x.T), columnwise=False)
    assert np.array_equal(q["col_data"], qt["row_data"])
    assert np.array_equal(q["col_scales"], qt["row_scales"])


def test_2d_columnwise_is_transpose_of_rowwise():
    x = W.c2(rows=64, cols=96)
    q = O.quantize(x, block_2d=True)
    assert np.array_equal(_codes(q["col_data"]), _codes(q["row_data"]).T)
    # every 16x16 block has one scale: rows of a block agree, and col scales
    # are the same per-block scales seen from the other side
    rs = q["row_scales"].reshape(4, 16, 6)
    assert np.all(rs == rs[:, :1, :])
    cs = q["col_scales"].reshape(6, 16, 4)
    assert np.all(cs == cs[:, :1, :])
    assert np.array_equal(rs[:, 0, :], cs[:, 0, :].T)


def test_block_max_encodes_to_six():
    # With a normal-range block scale, sd/sf is within 1/16 of 1, so the block
    # maximum lands in [5.6, 6.4] and rounds to +-6 (code 7 or 15).
    x = W.gaussian_fp32(64, 256, 10)
    q = O.quantize(x, columnwise=False)
    codes = _codes(q["row_data"]).reshape(64, 16, 16)
    xb = x.reshape(64, 16, 16)
    arg = np.abs(xb).argmax(-1)
    top = np.take_along_axis(codes, arg[..., None], -1)[..., 0]
    assert np.all((top & 7) == 7)


def test_dequantize_error_bound():
    # |x - y| <= half a grid step of v' = x*e, mapped back by sf/S, plus the
    # binary32 rounding of the product and quotient.
    x = W.gaussian_fp32(128, 256, 12, scale=3.0)
    q = O.quantize(x)
    y = O.dequantize(q["row_data"], q["row_scales"], q["amax_row"], 128, 256)
    S = O.global_encode_scale(float(q["amax_row"][0]))
    sf = np.array([O.e4m3_value(int(s)) for s in q["row_scales"].ravel()]).reshape(128, 16)
    sf = np.repeat(sf, 16, axis=1)
    v = np.abs(x) * S / sf
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    bound = 0.5 * step * sf / S * (1 + 1e-6) + 1e-6 * np.abs(x)
    assert np.all(np.abs(x - y) <= bound)
    # column-wise direction round-trips to the transpose
    yc = O.dequantize(q["col_data"], q["col_scales"], q["amax_col"], 256, 128)
    assert np.max(np.abs(yc.T - x)) <= np.max(bound) * 1.01


def test_rowwise_only_and_columnwise_only_match_both():
    x = W.c1(rows=64, cols=64)
    both = O.quantize(x)
    ro = O.quantize(x, columnwise=False)
    co = O.quantize(x, rowwise=False)
    assert ro["col_data"] is None and co["row_data"] is None
    assert np.array_equal(ro["row_data"], both["row_data"])
    assert np.array_equal(co["col_data"], both["col_data"])


# ----------------------------------------------------------------------------
# GEMM-swizzled scale layout: hand-worked offsets and an independent reshape.
# ----------------------------------------------------------------------------

def test_swizzle_offsets_hand_worked():
    assert [O.swizzle_offset(r, c, 4) for r, c in [(0, 0), (0, 3), (1, 0), (32, 0), (33, 2), (127, 3)]] == \
        [0, 3, 16, 4, 22, 511]
    # 256 x 8 scale matrix: (130, 5) sits in tile (1, 1) = 3rd tile -> 1536 + 2*16 + 0*4 + 1
    assert O.swizzle_offset(130, 5, 8) == 1569


def test_swizzle_matches_reshape_transpose_formulation():
    rng = np.random.default_rng(3)
    compact = rng.integers(0, 256, size=(256, 24), dtype=np.uint8)
    # 128x4 tiles in row-major tile order; inside a tile (4, 32, 4) -> (32, 4, 4)
    t = compact.reshape(2, 128, 6, 4).transpose(0, 2, 1, 3)          # [tr][tc][128][4]
    t = t.reshape(2, 6, 4, 32, 4).transpose(0, 1, 3, 2, 4)           # [tr][tc][32][4][4]
    assert np.array_equal(O.swizzle_scales(compact), t.reshape(-1))


def test_swizzle_groups_of_four_are_aligned_words():
    compact = np.arange(128 * 8, dtype=np.int64).reshape(128, 8)
    for r in range(128):
        for c0 in (0, 4):
            offs = [O.swizzle_offset(r, c0 + k, 8) for k in range(4)]
            assert offs[0] % 4 == 0 and offs == list(range(offs[0], offs[0] + 4))
    allo = sorted(O.swizzle_offset(r, c, 8) for r in range(128) for c in range(8))
    assert allo == list(range(128 * 8))
    with pytest.raises(ValueError):
        O.swizzle_scales(np.zeros((64, 8), np.uint8))


def _reshape_swizzle(padded):
    """The GEMM layout as an array reshape: 128x4 tiles in row-major tile
    order, inside a tile [4 row groups of 32][32][4] -> [32][4][4]."""
    pr, pc = padded.shape
    t = padded.reshape(pr // 128, 128, pc // 4, 4).transpose(0, 2, 1, 3)
    t = t.reshape(pr // 128, pc // 4, 4, 32, 4).transpose(0, 1, 3, 2, 4)
    return t.reshape(-1)


@pytest.mark.parametrize("shape", [(1088, 64), (100, 7), (128, 4), (1, 1), (257, 130), (0, 5), (5, 0)])
def test_padded_swizzle_is_the_layout_of_the_zero_padded_matrix(shape):
    rows, sc = shape
    rng = np.random.default_rng(rows * 1000 + sc)
    compact = rng.integers(1, 256, size=shape, dtype=np.uint8)  # no zeros: padding stays visible
    pr, pc = -(-rows // 128) * 128, -(-sc // 4) * 4
    padded = np.zeros((pr, pc), np.uint8)
    padded[:rows, :sc] = compact
    got = O.swizzle_scales_padded(compact)
    assert got.size == O.swizzled_size(rows, sc) == pr * pc
    assert np.array_equal(got, _reshape_swizzle(padded))
    assert np.count_nonzero(got) == rows * sc  # every value once; everything else is padding
    if rows % 128 == 0 and sc % 4 == 0 and rows * sc > 0:
        assert np.array_equal(got, O.swizzle_scales(compact))


def test_rht_columnwise_is_plain_rowwise_of_the_transform():
    # The RHT path's column-wise output is the ordinary row-wise quantization
    # of the transformed tensor t[cols][rows], scaled by max|t|.
    x = W.randn_bf16(64, 48, 13)
    mask = 0x3C5A
    q = O.quantize(x, rht=True, sign_mask=mask)
    t = O.rht_colwise(x, mask)
    assert q["amax_col"][0] == np.abs(t).max()
    assert q["amax_row"][0] == np.abs(W.bf16_to_float(x)).max()
    qt = O.quantize(t, columnwise=False)
    assert np.array_equal(q["col_data"], qt["row_data"])
    assert np.array_equal(q["col_scales"], qt["row_scales"])
    # the row-wise side is untouched by the transform
    qp = O.quantize(x, columnwise=False)
    assert np.array_equal(q["row_data"], qp["row_data"])


def test_explicit_amax_is_used_as_given():
    # A caller-provided amax (e.g. after a cross-device MAX) replaces the local
    # one. Quantizing x against 2a encodes exactly like quantizing x/2 against
    # a: every scale and product only moves by a power of two.
    x = W.gaussian_fp32(32, 64, 14)
    a = np.abs(x).max()
    q2 = O.quantize(x, amax_row=np.float32([2 * a]), amax_col=np.float32([2 * a]))
    qh = O.quantize((x * np.float32(0.5)).astype(np.float32), amax_row=np.float32([a]),
                    amax_col=np.float32([a]))
    assert not np.array_equal(q2["row_scales"], O.quantize(x)["row_scales"])
    for key in ("row_data", "row_scales", "col_data", "col_scales"):
        assert np.array_equal(q2[key], qh[key])


# ----------------------------------------------------------------------------
# Grouped quantize: each row slice is a tensor of its own.
# ----------------------------------------------------------------------------

def test_grouped_single_group_is_plain_quantize():
    x = W.randn_bf16(64, 96, 41)
    g = O.quantize_grouped(x, [64], stochastic=True, sr_seed=3)
    q = O.quantize(x, stochastic=True, sr_seed=3)
    for k in ("row_data", "row_scales", "col_data", "col_scales", "amax_row", "amax_col"):
        assert np.array_equal(g[k], q[k].reshape(-1)), k


def test_grouped_scaling_one_group_changes_only_its_amax():
    # power-of-two invariance per group: codes and scales stay, that group's
    # amax scales by exactly 2^k, the other groups do not move at all
    x = W.gaussian_fp32(96, 64, 42)
    sizes = [32, 48, 16]
    base = O.quantize_grouped(x, sizes, block_2d=True)
    y = x.copy()
    y[32:80] *= np.float32(2.0 ** 7)
    moved = O.quantize_grouped(y, sizes, block_2d=True)
    for k in ("row_data", "row_scales", "col_data", "col_scales"):
        assert np.array_equal(base[k], moved[k]), k
    assert np.array_equal(moved["amax_row"], base["amax_row"] * np.float32([1, 128, 1]))
    assert np.array_equal(moved["amax_col"], base["amax_col"] * np.float32([1, 128, 1]))


def test_grouped_blocks_follow_group_order():
    # swapping two groups swaps their blocks in every output array
    x = W.randn_bf16(64, 48, 43)
    a = O.quantize_grouped(x, [16, 48])
    xs = np.concatenate([x[16:], x[:16]])
    b = O.quantize_grouped(xs, [48, 16])
    assert np.array_equal(b["row_data"], np.concatenate([a["row_data"][16 * 24:], a["row_data"][:16 * 24]]))
    assert np.array_equal(b["col_data"], np.concatenate([a["col_data"][48 * 8:], a["col_data"][:48 * 8]]))
    assert np.array_equal(b["col_scales"], np.concatenate([a["col_scales"][48 * 1:], a["col_scales"][:48 * 1]]))
    assert np.array_equal(b["amax_row"], a["amax_row"][::-1])


def test_grouped_empty_group_has_zero_amax_and_no_bytes():
    x = W.randn_bf16(32, 32, 44)
    g = O.quantize_grouped(x, [16, 0, 16])
    assert g["amax_row"][1] == 0 and g["amax_col"][1] == 0
    assert g["row_data"].size == 32 * 16 and g["col_data"].size == 2 * 32 * 8


# ----------------------------------------------------------------------------
# BF16 transformed values (opt-in RHT variant): the rounding itself against
# torch's BF16 cast, closed forms, and the order of rounding and maximum.
# ----------------------------------------------------------------------------

def _torch_bf16(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(71)
    bits = rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]  # finite values only
    # every tie and its neighbours, in both parities of the kept bit
    hi = rng.integers(0, 2 ** 16, 4096, dtype=np.uint64).astype(np.uint32) << 16
    hi = hi[(hi & 0x7F800000) != 0x7F800000]
    ties = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001, hi, hi | 0xFFFF])
    ties = ties[((ties & 0x7F800000) != 0x7F800000)]
    v = np.concatenate([bits, ties, np.uint32([0, 0x80000000, 1, 0x8000, 0x18000, 0x7F7F7FFF])]).view(np.float32)
    got = O.round_bf16(v)
    ref = _torch_bf16(v)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_rht_bf16_closed_form():
    # one group [1, 2^-9, 0 x 14], mask 0: t_r = (1 +- 2^-9) / 4, the sign
    # from (-1)^popcount(r & 1). 1 + 2^-9 is below the BF16 midpoint above 1,
    # and 1 - 2^-9 is the tie between 1 - 2^-8 and 1 (even: 1), so every
    # BF16 value is exactly 1/4.
    x = np.zeros((16, 16), np.float32)
    x[0, 3], x[1, 3] = 1.0, 2.0 ** -9
    t32 = O.rht_colwise(x, 0)[3]
    t16 = O.rht_colwise(x, 0, bf16=True)[3]
    r = np.arange(16)
    expect32 = np.float32(0.25) * np.where(r % 2 == 0, np.float32(1 + 2 ** -9), np.float32(1 - 2 ** -9))
    assert np.array_equal(t32, expect32)
    assert np.all(t16 == np.float32(0.25))
    a32 = O.compute_amax(x, O.AMAX_RHT, 0)[1][0]
    a16 = O.compute_amax(x, O.AMAX_RHT_BF16, 0)[1][0]
    assert a32 == np.float32(0.25 * (1 + 2 ** -9)) and a16 == np.float32(0.25)
    # the BF16 column: 16 equal values at the amax -> s = 448 (0x7E), e = 24, v' = 6
    q = O.quantize(x, rht=True, rht_bf16=True, rowwise=False)
    assert q["amax_col"][0] == 0.25
    assert q["col_scales"][3, 0] == 0x7E and np.all(q["col_data"][3] == 0x77)
    assert np.all(q["col_data"][:3] == 0) and np.all(q["col_scales"][:3] == 0)


def test_rht_bf16_amax_is_the_rounded_fp32_amax():
    # rounding is monotonic, so max|bf16(t)| == bf16(max|t|), and it is a BF16 value
    for seed in range(5):
        x = W.randn_bf16(64, 96, 72 + seed)
        mask = W.rht_sign_mask(seed)
        a32 = O.compute_amax(x, O.AMAX_RHT, mask)[1][0]
        a16 = O.compute_amax(x, O.AMAX_RHT_BF16, mask)[1][0]
        assert a16 == _torch_bf16([a32])[0]
        assert np.float32(a16).view(np.uint32) & 0xFFFF == 0


def test_rht_bf16_columnwise_is_plain_rowwise_of_the_rounded_transform():
    x = W.randn_bf16(64, 48, 76)
    mask = 0x2D3B
    q = O.quantize(x, rht=True, rht_bf16=True, sign_mask=mask, stochastic=True, sr_seed=4)
    t = _torch_bf16(O.rht_colwise(x, mask))
    qt = O.quantize(t, columnwise=False, stochastic=True, sr_seed=4)
    # the SR byte indices of the column side use direction 1, so compare RNE codes
    qr = O.quantize(x, rht=True, rht_bf16=True, sign_mask=mask)
    qtr = O.quantize(t, columnwise=False)
    assert q["amax_col"][0] == np.abs(t).max()
    assert np.array_equal(qr["col_data"], qtr["row_data"])
    assert np.array_equal(q["col_scales"], qt["row_scales"])
    # the row-wise side does not see the rounding
    assert np.array_equal(q["row_data"], O.quantize(x, rht=True, sign_mask=mask, stochastic=True, sr_seed=4)["row_data"])


# ----------------------------------------------------------------------------
# UE5M3 block scales (opt-in reading; the pages name the format without
# defining it, so these pin the oracle to the stated definition only).
# ----------------------------------------------------------------------------

def test_ue5m3_values_are_the_fp16_values_with_three_mantissa_bits():
    # unsigned, 5 exponent bits (bias 15), 3 mantissa bits: code c is the
    # binary16 number with bits c << 7 (sign 0, low 7 mantissa bits zero)
    codes = np.arange(0xF8, dtype=np.uint16)
    f16 = (codes << 7).view(np.float16).astype(np.float64)
    got = np.array([O.ue5m3_value(int(c)) for c in codes])
    assert np.array_equal(got, f16)
    assert O.ue5m3_value(0xF7) == 61440.0 and O.ue5m3_value(1) == 2.0 ** -17 and O.ue5m3_value(8) == 2.0 ** -14


def _nearest_even_code(x: float, values) -> int:
    """Exact rational nearest-value search over a sorted grid, ties to the even code."""
    fx = Fraction(x)
    best, best_d = None, None
    for k, v in enumerate(values):
        d = abs(fx - Fraction(v))
        if best is None or d < best_d or (d == best_d and k % 2 == 0):
            best, best_d = k, d
    return best


def test_ue5m3_encoding_nearest_even_saturating():
    values = [O.ue5m3_value(c) for c in range(0xF8)]
    probes = []
    for k in range(0xF7):
        mid = np.float32((values[k] + values[k + 1]) / 2)
        probes += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf)), np.float32(values[k])]
    rng = np.random.default_rng(91)
    probes += list((2.0 ** rng.uniform(-20, 16, 3000)).astype(np.float32))
    probes = np.array(probes, np.float32)
    got = O.ue5m3(probes)
    want = np.array([_nearest_even_code(float(p), values) for p in probes])
    assert np.array_equal(got, want)
    # beyond the largest value, and +inf, saturate to 61440
    assert np.all(O.ue5m3(np.float32([61440, 63488, 65536, 1e30, np.inf])) == 0xF7)
    assert O.ue5m3(np.float32([0.0]))[0] == 0


def test_ue5m3_hand_worked_block():
    # 1x32, E4M3's hand-worked blocks with UE5M3 scales: amax 6, S = 368640 / 6 = 61440.
    # Block 0 = [6, 0 x 15]: sd = 61440 -> 0xF7, e = 1, codes 7, 0, ...
    # Block 1 = [1, .5, .25, .125, -1, -.5, -.25, -.125, 0 x 8]: sd = fl(fl(1/6) * 61440)
    # = 10240 = 1.25 * 2^13 -> code (28 << 3) | 2 = 0xE2, e = 6; v' = 6, 3, 1.5, .75
    # -> codes 7, 5, 3, 2 (0.75 is the tie between 0.5 and 1: even code 2).
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 6.0
    x[0, 16:24] = [1, .5, .25, .125, -1, -.5, -.25, -.125]
    q = O.quantize(x, columnwise=False, scale_fmt=O.SCALE_UE5M3)
    assert O.global_encode_scale(6.0, O.SCALE_UE5M3) == 61440.0
    assert list(q["row_scales"][0]) == [0xF7, 0xE2]
    assert bytes(q["row_data"][0]).hex() == "0700000000000000" + "5723dfab00000000"
    y = O.dequantize(q["row_data"], q["row_scales"], q["amax_row"], 1, 32, scale_fmt=O.SCALE_UE5M3)
    assert y[0, 16] == 1.0 and y[0, 0] == 6.0  # 6 * 10240 / 61440 and 6 * 61440 / 61440


def test_ue5m3_keeps_blocks_that_e4m3_flushes():
    # a block 2^-20 below the tensor amax: E4M3's sd = 448 * 2^-20 is under
    # half its smallest subnormal (2^-10), so its codes are all zero; UE5M3's
    # sd = 61440 * 2^-20 is a normal value and the block keeps its codes
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    x[0, 16:20] = np.float32([2.0 ** -20, 2.0 ** -21, -(2.0 ** -20), 2.0 ** -22])
    e4 = O.quantize(x, columnwise=False)
    ue = O.quantize(x, columnwise=False, scale_fmt=O.SCALE_UE5M3)
    assert e4["row_scales"][0, 1] == 0 and not np.any(e4["row_data"][0, 8:] & 0x77)
    assert ue["row_scales"][0, 1] != 0
    assert list(O.dequantize(ue["row_data"], ue["row_scales"], ue["amax_row"], 1, 32,
                             scale_fmt=O.SCALE_UE5M3)[0, 16:20]) == [2.0 ** -20, 2.0 ** -21, -(2.0 ** -20), 2.0 ** -22]


@pytest.mark.parametrize("k", [-9, 5])
def test_ue5m3_power_of_two_invariance(k):
    x = W.gaussian_fp32(32, 64, 92, 3.0)
    a = O.quantize(x, block_2d=True, scale_fmt=O.SCALE_UE5M3)
    b = O.quantize((x * np.float32(2.0 ** k)).astype(np.float32), block_2d=True, scale_fmt=O.SCALE_UE5M3)
    for key in ("row_data", "row_scales", "col_data", "col_scales"):
        assert np.array_equal(a[key], b[key]), key
    assert b["amax_row"][0] == a["amax_row"][0] * np.float32(2.0 ** k)


def test_grouped_rowscaled_with_nearest_even_is_one_rowscaled_call():
    # per-row scaling treats every row on its own, so with nearest-even
    # rounding (no byte-index dependence) the grouping cannot change a byte;
    # with stochastic rounding only the byte indices restart per group
    x = W.c4(rows=80, cols=96, seed=45)
    groups = [16, 0, 48, 16]
    g = O.quantize_grouped(x, groups, row_scaled=True)
    q = O.quantize(x, columnwise=False, row_scaled=True)
    assert g["col_data"] is None and g["amax_row"].shape == (80,)
    for k in ("row_data", "row_scales", "amax_row"):
        assert np.array_equal(g[k], q[k].reshape(-1)), k
    gs = O.quantize_grouped(x, groups, row_scaled=True, stochastic=True, sr_seed=6)
    last = O.quantize(x[64:], columnwise=False, row_scaled=True, stochastic=True, sr_seed=6)
    assert np.array_equal(gs["row_data"][64 * 48:], last["row_data"].reshape(-1))
    assert np.array_equal(gs["row_scales"], q["row_scales"].reshape(-1))  # scales are always nearest even


# ----------------------------------------------------------------------------
# Non-finite inputs: the stated amax policy (NaN wins, else +inf), written out
# in the oracle rather than left to fmaxf (which drops a NaN).
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["tensor", "row", "rht"])
def test_amax_propagates_nan_and_inf(mode):
    for bad, want in ((np.nan, "nan"), (np.inf, "inf"), (-np.inf, "inf")):
        x = np.full((32, 48), 0.5, np.float32)
        x[17, 9] = bad
        x[3, 40] = -7.0  # a finite maximum elsewhere must not hide the NaN or inf
        if mode == "tensor":
            a, b = O.compute_amax(x)
            vals = [a[0], b[0]]
        elif mode == "row":
            a, b = O.compute_amax(x, O.AMAX_PER_ROW)
            vals = [a[17], b[9]]
            assert a[3] == 7.0 and b[40] == 7.0 and a[0] == 0.5 and b[0] == 0.5
        else:
            a, b = O.compute_amax(x, O.AMAX_RHT, 0x9C3A)
            vals = [a[0], b[0]]
        for v in vals:
            assert (np.isnan(v) if want == "nan" else v == np.inf), (mode, bad, vals)
    # NaN beats +inf anywhere
    x = np.zeros((16, 16), np.float32)
    x[0, 0] = np.inf
    x[15, 15] = np.nan
    assert np.isnan(O.compute_amax(x)[0][0])
