"""The SwiGLU epilogue divides the block amax by 6 as a product with RN(1/6)
plus one FMA correction (device.hpp, div6_rn) instead of an IEEE division.
The requant's scale byte is bit-exact only if the two agree; this checks them
against each other for every fp32 value the epilogue can divide (6 * 2^-9 up
to the largest finite float), with the CPU's correctly rounded fmaf."""
import os
import shutil
import subprocess
import tempfile

import pytest

C_SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
int main(void) {
#ifndef __FMA__
  return 2;
#endif
  const float c = 1.0f / 6.0f;
  volatile float six = 6.0f;
  uint64_t bad = 0, n = 0;
  for (uint32_t u = u_of(6.0f * 0x1p-9f); u < 0x7F800000u; ++u) {
    const float x = f_of(u);
    const float q0 = x * c;
    const float r = fmaf(-q0, 6.0f, x);
    const float q1 = fmaf(r, c, q0);
    bad += u_of(q1) != u_of(x / six);
    ++n;
  }
  printf("%llu %llu %a\n", (unsigned long long)n, (unsigned long long)bad, c);
  return bad != 0;
}
"""


def test_div6_matches_ieee_division_over_the_epilogue_range():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "d6.c"), os.path.join(d, "d6")
        open(src, "w").write(C_SRC)
        subprocess.run([gcc, "-O2", "-mfma", "-ffp-contract=off", src, "-o", exe, "-lm"], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    if r.returncode == 2:
        pytest.skip("no hardware FMA on this CPU")
    n, bad, c = r.stdout.split()
    assert c == "0x1.555556p-3"          # RN(1/6), the constant div6_rn multiplies by
    assert int(n) > 1_100_000_000 and int(bad) == 0, r.stdout
