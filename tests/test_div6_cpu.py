"""The kernels take fl(m / 6), the first step of every block scale, without
a division: q0 = fl(m * fl(1/6)), corrected once with the exact residual
fma(-q0, 6, m). This pins that identity on the CPU, whose fmaf and binary32
arithmetic are the same IEEE operations as the GPU's: over every
non-negative binary32 value the corrected quotient equals the correctly
rounded one, except below 2^-122 (subnormal quotients) and at +inf, where
the kernels divide instead."""

from __future__ import annotations

import os
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t u(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }
int main(void) {
  const float r = 1.0f / 6.0f;
  const uint32_t lo = u(0x1p-122f), hi = u(3.40282346638528859812e+38f);
  long long bad_inside = 0, bad_outside = 0;
#pragma omp parallel for reduction(+ : bad_inside, bad_outside) schedule(static)
  for (long long i = 0; i <= 0x7F800000LL; ++i) {
    const float m = f((uint32_t)i);
    const float q0 = m * r;
    const float q = fmaf(fmaf(-q0, 6.0f, m), r, q0);
    if (u(q) != u(m / 6.0f)) {
      if ((uint32_t)i >= lo && (uint32_t)i <= hi) ++bad_inside;
      else ++bad_outside;
    }
  }
  printf("%lld %lld\n", bad_inside, bad_outside);
  return 0;
}
"""


def test_div6_is_the_correctly_rounded_quotient(tmp_path):
    src = tmp_path / "div6.c"
    src.write_text(SRC)
    exe = tmp_path / "div6"
    try:
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", str(src), "-o", str(exe), "-lm"])
    except (OSError, subprocess.CalledProcessError):
        pytest.skip("gcc with OpenMP is not available")
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    inside, outside = map(int, subprocess.check_output([str(exe)], env=env).split())
    assert inside == 0, "the corrected quotient differs from m / 6 for a finite m >= 2^-122"
    assert outside > 0  # the guarded range does differ: the guard is needed
