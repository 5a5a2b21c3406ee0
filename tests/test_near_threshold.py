"""The diagnostics' near-max band test, checked for every pair of bf16 magnitudes (CPU).

The statistics count an element in the near-max band of its block when 3|x| > 2 bmax.  The
kernel takes it per block as |x| > t with t = RN32(bmax * RN32(2/3)) and the low 16 bits of
t cleared (|x| and bmax are bf16 values).  This test runs, in binary32 arithmetic with
subnormals and no contraction, the kernel's form against 1.5|x| > bmax (exact for bf16 |x|,
so the band's definition) for every finite bf16 bmax and every bf16 |x| <= bmax: 532,701,120
pairs in about two seconds."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

import pytest

SRC = r"""
#include <stdio.h>
#include <stdint.h>
#include <string.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t u(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }
int main(void) {
  const volatile float c = 0.6666667f;
  long bad = 0, n = 0;
  for (uint32_t bb = 0; bb < 0x7F80; ++bb) {
    const float b = f(bb << 16);
    const volatile float prod = b * c;
    const float t = f(u(prod) & 0xFFFF0000u);
    for (uint32_t ab = 0; ab <= bb; ++ab) {
      const float a = f(ab << 16);
      const volatile float p = 1.5f * a;
      ++n;
      if ((p > b) != (a > t)) ++bad;
    }
  }
  printf("%ld %ld\n", n, bad);
  return 0;
}
"""


def test_near_band_threshold_equals_definition():
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "near.c"), os.path.join(d, "near")
        with open(src, "w") as fh:
            fh.write(SRC)
        # SSE arithmetic: IEEE binary32 with subnormals (no x87 excess precision, no FTZ)
        subprocess.run([cc, "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", exe, src],
                       check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    pairs, bad = int(out[0]), int(out[1])
    assert pairs == 532_701_120
    assert bad == 0
