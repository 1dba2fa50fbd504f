"""The pack kernels form a scale's fp32 quotient range / L (L = 2^b - 1 levels)
without a divide: q0 = range * fl(1/L), r = fma(-q0, L, range) (exact), q = fma(r,
fl(1/L), q0).  The quantizer contract asks for the correctly rounded quotient, so
this pins the identity on the CPU with IEEE fp32 and a true fma (C, fmaf): every
float of eight whole binades across the range scales take, every subnormal, and 2^22
random non-negative finite floats per L, for each L the library uses.  (The identity
was also run over every non-negative finite float for each L: no mismatch.)
"""

import os
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static uint64_t bad = 0;
static void check(uint32_t u, float L, float y) {
  float a; memcpy(&a, &u, 4);
  const float want = a / L;
  const float q0 = a * y;
  const float q = fmaf(fmaf(-q0, L, a), y, q0);
  if (memcmp(&want, &q, 4) != 0) ++bad;
}
int main(void) {
  const float Ls[5] = {1.0f, 3.0f, 7.0f, 15.0f, 255.0f};
  const int exps[4] = {1, 112, 127, 142};  /* biased exponents */
  uint64_t s = 0x9e3779b97f4a7c15ull;
  for (int li = 0; li < 5; ++li) {
    const volatile float Lv = Ls[li];
    const float L = Lv, y = 1.0f / L;
    for (int e = 0; e < 4; ++e)
      for (uint32_t m = 0; m < (1u << 23); ++m) check(((uint32_t)exps[e] << 23) | m, L, y);
    for (uint32_t m = 0; m < (1u << 23); ++m) check(m, L, y);            /* zero and subnormals */
    for (int i = 0; i < (1 << 22); ++i) {
      s ^= s << 13; s ^= s >> 7; s ^= s << 17;
      const uint32_t u = (uint32_t)(s >> 33) % 0x7f800000u;
      check(u, L, y);
    }
  }
  printf("%llu\n", (unsigned long long)bad);
  return 0;
}
"""


def test_quotient_by_levels_is_correctly_rounded(tmp_path):
    cc = shutil.which("gcc")
    if not cc:
        pytest.skip("gcc is missing")
    src = tmp_path / "div.c"
    exe = tmp_path / "div"
    src.write_text(SRC)
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-fno-fast-math", str(src), "-o", str(exe), "-lm"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True, timeout=300).stdout
    assert out.strip() == "0", out
