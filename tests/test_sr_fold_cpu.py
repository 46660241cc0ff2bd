"""The stochastic-rounding kernels hand the SR conversion |v'| rounded up to a
multiple of 2^-23, t = ceil(|fl(v * e)| * 2^23), where v' = fl(v * e) is the
scaled value and e a block's encode multiplier. Where the global encode scale
S lies in a guarded range, they take t = ceil(fl(|v| * fl(e * 2^23 / c)))
instead (c = 4 on the RHT column side, whose 1/4 is folded into the
multiplier; else 1): one multiply fewer per value. Scaling by a power of two
commutes with rounding except where a result underflows or overflows, and
the guard keeps every block multiplier away from both for the smallest
non-zero input of the format. This pins that on the CPU (IEEE binary32, as on
the GPU): for every scale code, every finite BF16 value (and a sample of
FP32 values) and global scales across the guarded range, both give the same
t; just outside the range they do differ, so the guard is needed.
"""

from __future__ import annotations

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CODEC = os.path.join(ROOT, "nvfp4_block_scaled_05_amd", "csrc", "codec.h")

# (scale format, input dtype, c) -> (lo, hi) as powers of two: the fold is
# taken for lo <= S <= hi. lo = 2^-149 * c * (largest scale) / (smallest
# non-zero |value|), rounded up to a power of two; hi keeps e * 2^23 / c at
# most 2^126 for the smallest non-zero scale (2^-9 E4M3, 2^-17 UE5M3).
RANGES = {
    ("e4m3", "bf16", 1): (-7, 94),
    ("e4m3", "bf16", 4): (-5, 94),
    ("e4m3", "fp32", 1): (9, 94),
    ("e4m3", "fp32", 4): (11, 94),
    ("ue5m3", "bf16", 1): (0, 86),
    ("ue5m3", "bf16", 4): (2, 86),
    ("ue5m3", "fp32", 1): (16, 86),
    ("ue5m3", "fp32", 4): (18, 86),
}

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t u(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }
#define FLT_MAX_ 3.40282346638528859812e+38f
/* scale value of a code: E4M3 (bias 7, subnormals m*2^-9) or UE5M3 (bias 15, m*2^-17) */
static float scale_value(int code, int ue) {
  int eb = ue ? 5 : 4, bias = ue ? 15 : 7;
  int e = (code >> 3) & ((1 << eb) - 1), m = code & 7;
  if (e == 0) return ldexpf((float)m, 1 - bias - 3);
  return ldexpf(1.0f + m / 8.0f, e - bias);
}
/* returns the number of (S, code, v) triples where the two forms differ */
static long long check(float S, int ue, int c, const float *vals, long n) {
  const int ncodes = ue ? 0xF8 : 0x7F;
  long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(dynamic)
  for (int code = 0; code < ncodes; ++code) {
    const float sf = scale_value(code, ue);
    float e = code == 0 ? 0.0f : S / sf;
    if (e > FLT_MAX_) e = FLT_MAX_;
    const float e_used = c == 4 ? e * 0.25f : e;            /* the multiplier the values take */
    const float fold = e * (8388608.0f / (float)c);          /* e * 2^23 / c */
    for (long i = 0; i < n; ++i) {
      const float v = vals[i];
      const float ref = ceilf(fabsf(v * e_used) * 8388608.0f);
      const float got = ceilf(fabsf(v) * fold);
      if (u(ref) != u(got)) ++bad;
    }
  }
  return bad;
}
int main(int argc, char **argv) {
  const int ue = atoi(argv[1]), fp32 = atoi(argv[2]), c = atoi(argv[3]);
  const int lo = atoi(argv[4]), hi = atoi(argv[5]);
  /* values: every finite BF16 value, or for FP32 a stride over all finite
     patterns plus every pattern of the lowest 2^16 (the denormal end) */
  long n = 0;
  float *vals = malloc(sizeof(float) * (1u << 18));
  if (!fp32) {
    for (uint32_t h = 0; h < 65536; ++h) {
      float v = f(h << 16);
      if (isfinite(v)) vals[n++] = v;
    }
  } else {
    for (uint32_t b = 0; b < 0x7F800000u; b += 65521u) vals[n++] = f(b);
    for (uint32_t b = 0; b < (1u << 16); ++b) vals[n++] = f(b);
  }
  long long inside = 0, below = 0;
  /* S across [2^lo, 2^hi]: both ends and the two powers next to them, every
     eighth power between, each also with an odd mantissa */
  for (int k = lo; k <= hi; ++k) {
    if (!(k <= lo + 1 || k >= hi - 1 || (k - lo) % 8 == 0)) continue;
    inside += check(ldexpf(1.0f, k), ue, c, vals, n);
    if (k < hi) inside += check(ldexpf(1.7320508f, k), ue, c, vals, n);
  }
  /* just below the range */
  below += check(ldexpf(1.0f, lo - 3), ue, c, vals, n);
  printf("%lld %lld\n", inside, below);
  free(vals);
  return 0;
}
"""


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    d = tmp_path_factory.mktemp("srfold")
    src = d / "fold.c"
    src.write_text(SRC)
    out = d / "fold"
    try:
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", str(src), "-o", str(out), "-lm"])
    except (OSError, subprocess.CalledProcessError):
        pytest.skip("gcc with OpenMP is not available")
    return out


@pytest.mark.parametrize("key", sorted(RANGES), ids=lambda k: f"{k[0]}-{k[1]}-c{k[2]}")
def test_fold_is_exact_inside_the_guard_and_not_below(exe, key):
    fmt, dtype, c = key
    lo, hi = RANGES[key]
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    inside, below = map(int, subprocess.check_output(
        [str(exe), str(int(fmt == "ue5m3")), str(int(dtype == "fp32")), str(c), str(lo), str(hi)], env=env).split())
    assert inside == 0, f"{key}: the folded multiply differs inside the guarded range"
    assert below > 0, f"{key}: no difference just below the range: the guard's lower bound is not tight"


def test_kernel_guard_uses_these_ranges():
    # the ranges here are the ones the kernels test S against
    text = open(CODEC).read()
    for (fmt, dtype, c), (lo, hi) in RANGES.items():
        pat = rf"{{\s*{int(fmt == 'ue5m3')}\s*,\s*{int(dtype == 'fp32')}\s*,\s*{c}\s*,\s*{lo}\s*,\s*{hi}\s*}}"
        assert re.search(pat, text), f"codec.h has no fold range entry for {fmt}/{dtype}/c={c}: {lo}..{hi}"
