"""Pins of the oracle's stochastic-rounding word rule and of how its words
reach the output bytes.

The pages name stochastic rounding as a quantizer option but give no rule
("Fuse NVFP4 scale swizzling on SM120 and SM121", Changes), so the rule is a
reading: K_dir = fmix32(fmix32(seed) ^ (dir + 1)), the word of output byte b
is fmix32(K_dir ^ b) with b counted over the orientation's data array, its
low half drives the byte's even element and its high half the odd one.

What holds the oracle to that reading, from outside the oracle:
  * fmix32 itself: the published MurmurHash3 vectors (test_oracle_pins.py);
  * fixed words and keys for seed 5, worked out from the definition before
    the oracle existed (tests/golden/sr_words_seed5.json);
  * two hand-worked blocks whose bytes depend on every part of the rule;
  * an assembly check: on tensors where every multiplier is 1, each code
    equals the (separately pinned) SR decision applied with the word of its
    own byte index, at byte indices far from 0 in both orientations.
The last test plants plausible mistakes in a copy of the oracle, on the CPU,
and checks that the pins above catch each one.
"""

from __future__ import annotations

import json
import os
import shutil
import tempfile

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sr_words_seed5.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _hex(s):
    return int(s, 16)


# ----------------------------------------------------------------------------
# Checks (each raises AssertionError on a mismatch), shared by the tests below
# and by the planted-mistake test.
# ----------------------------------------------------------------------------

def check_words_seed5():
    g = _golden()
    seed = g["seed"]
    assert int(O.fmix32(np.array([seed], np.uint32))[0]) == _hex(g["fmix32_of_seed"])
    for d, name in enumerate(("rowwise", "columnwise")):
        # the key is the word of byte index 0 before its last mix: fmix32(K ^ 0) = fmix32(K)
        key = _hex(g["key"][name])
        assert O.sr_word(seed, d, 0) == int(O.fmix32(np.array([key], np.uint32))[0]), name
        for b, w in enumerate(g["words"][name]):
            assert O.sr_word(seed, d, b) == _hex(w), (name, b)


def check_words_compose_pinned_fmix32():
    # sr_word(s, d, b) == fmix32(fmix32(fmix32(s) ^ (d + 1)) ^ b), with the
    # oracle's own fmix32 (pinned to MurmurHash3's published vectors)
    rng = np.random.default_rng(11)
    f = lambda v: int(O.fmix32(np.array([v & 0xFFFFFFFF], np.uint32))[0])
    for _ in range(200):
        s, b = (int(v) for v in rng.integers(0, 2**32, 2, dtype=np.uint64))
        d = int(rng.integers(0, 2))
        assert O.sr_word(s, d, b) == f(f(f(s) ^ (d + 1)) ^ b), (s, d, b)


def check_hand_worked_rowwise():
    hw = _golden()["hand_worked"]["rowwise"]
    x = np.array([hw["values"]], np.float32)
    q = O.quantize(x, rowwise=True, columnwise=False, stochastic=True, sr_seed=5)
    assert q["amax_row"][0] == 6.0
    assert q["row_scales"].ravel().tolist() == [0x7E]
    assert q["row_data"].ravel().tolist() == [_hex(b) for b in hw["bytes"]]


def check_hand_worked_columnwise():
    hw = _golden()["hand_worked"]["columnwise"]
    x = np.zeros((16, 16), np.float32)
    x[:, 0] = hw["values"]
    q = O.quantize(x, rowwise=False, columnwise=True, stochastic=True, sr_seed=5)
    assert q["amax_col"][0] == 6.0
    assert q["col_scales"][0].tolist() == [0x7E]
    assert q["col_data"][0].tolist() == [_hex(b) for b in hw["bytes"]]
    assert not q["col_data"][1:].any()


def _unit_multiplier_tensor(rows, cols, seed):
    """Values in (-6, 6) with a 6 in every 1x16 row block and every 16-row
    column block: the amax is 6, every block scale 448 and every multiplier
    1, so each code is the E2M1 rounding of the input value itself."""
    rng = np.random.default_rng(seed)
    x = rng.uniform(-6.0, 6.0, (rows, cols)).astype(np.float32)
    x[:, ::16] = 6.0
    x[::16, :] = 6.0
    return x


def _codes(data):
    """[n][k/2] packed bytes -> [n][k] codes (even element = low nibble)."""
    return np.stack([data & 0xF, data >> 4], -1).reshape(data.shape[0], -1)


def check_assembly_uses_each_bytes_word(rows=48, cols=64, seed=5):
    x = _unit_multiplier_tensor(rows, cols, seed=rows * cols)
    q = O.quantize(x, rowwise=True, columnwise=True, stochastic=True, sr_seed=seed)
    for d, (data, vals) in enumerate(((q["row_data"], x), (q["col_data"], x.T.copy()))):
        n, k = vals.shape
        words = np.array([O.sr_word(seed, d, b) for b in range(n * k // 2)], np.uint32).reshape(n, k // 2)
        r16 = np.stack([words & 0xFFFF, words >> 16], -1).reshape(n, k).astype(np.uint16)
        want = O.e2m1_sr(vals.ravel(), r16.ravel()).reshape(n, k)
        np.testing.assert_array_equal(_codes(data), want, err_msg=f"orientation {d}")


CHECKS = [
    check_words_seed5,
    check_words_compose_pinned_fmix32,
    check_hand_worked_rowwise,
    check_hand_worked_columnwise,
    check_assembly_uses_each_bytes_word,
]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_sr_pin(check):
    check()


# ----------------------------------------------------------------------------
# Planted mistakes: each altered copy of the oracle must fail some check.
# ----------------------------------------------------------------------------

# (description, [(text in the oracle source, replacement)]); every text must
# occur exactly once, so that this test notices when the source moves on.
MUTATIONS = [
    ("inner fmix32 of the seed dropped",
     [("oracle_fmix32(oracle_fmix32(seed) ^ (uint32_t)(dir + 1))", "oracle_fmix32(seed ^ (uint32_t)(dir + 1))")]),
    ("key offset dir instead of dir + 1",
     [("oracle_fmix32(seed) ^ (uint32_t)(dir + 1)", "oracle_fmix32(seed) ^ (uint32_t)(dir)")]),
    ("halves swapped between the even and odd element",
     [("(uint16_t)(r & 0xFFFF));\n    uint8_t hi", "(uint16_t)(r >> 16));\n    uint8_t hi"),
      ("stochastic, (uint16_t)(r >> 16));\n    out[k]", "stochastic, (uint16_t)(r & 0xFFFF));\n    out[k]")]),
    ("element index instead of byte index",
     [("oracle_sr_word(seed, dir, (uint32_t)(byte_base + k))", "oracle_sr_word(seed, dir, (uint32_t)(2 * (byte_base + k)))")]),
    ("byte index counted within the output row",
     [("oracle_sr_word(seed, dir, (uint32_t)(byte_base + k))", "oracle_sr_word(seed, dir, (uint32_t)(k))")]),
    ("one word per element pair shared by both orientations",
     [("oracle_sr_word(seed, dir, (uint32_t)(byte_base + k))", "oracle_sr_word(seed, 0, (uint32_t)(byte_base + k))")]),
]


def _failing_checks():
    failed = []
    for check in CHECKS:
        try:
            check()
        except AssertionError:
            failed.append(check.__name__)
    return failed


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc to build the altered oracle copies")
def test_planted_mistakes_are_caught(monkeypatch):
    import ctypes

    with open(O._SRC) as f:
        src = f.read()
    with tempfile.TemporaryDirectory() as tmp:
        for i, (what, edits) in enumerate(MUTATIONS):
            mutated = src
            for old, new in edits:
                assert mutated.count(old) == 1, (what, old)
                mutated = mutated.replace(old, new)
            path = os.path.join(tmp, f"m{i}.c")
            with open(path, "w") as f:
                f.write(mutated)
            lib = O.bind(ctypes.CDLL(O.compile_library(path, os.path.join(tmp, f"libm{i}.so"))))
            monkeypatch.setattr(O, "_lib", lib)
            assert _failing_checks(), f"no pin catches: {what}"
        monkeypatch.undo()
    # and the real oracle passes them all
    assert _failing_checks() == []
