"""The division identity the dense kernel's floors rely on, checked on the CPU.

For many weights w over one exact sum S, the kernel takes the binary64
quotient RN64(w / S) as RN64(q0 + e y) with y = RN64(1 / S), q0 = RN64(w y)
and the residual e = w - S q0 taken with one fused multiply-add (exact for a
faithful q0); the floors use it scaled by 2^24 (S 2^-24 and its reciprocal in
place of S and y), which gives RN64(w / S) 2^24 exactly.  For a correctly rounded reciprocal and no underflow this is the
correctly rounded quotient (Markstein's theorem; "Handbook of Floating-Point
Arithmetic", division by fused multiply-add).  The kernel's operands are a
binary32 weight in (0, 1] (subnormals included) and a binary64 sum in
[1, 2^21).  This test compares the identity with IEEE division on random and
binade-edge pairs of that range, in C with the C library's correctly rounded
fma; it is a pin of the arithmetic, not of the GPU code (the GPU parity tests
compare the kernel's counts with the oracle bit for bit).
"""
import os
import shutil
import subprocess
import tempfile

import pytest

C_SOURCE = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static uint64_t st = 0x9e3779b97f4a7c15ull;
static inline uint64_t next(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
int main(void) {
  long bad = 0;
  for (long it = 0; it < 1000000L; ++it) {
    uint32_t wb = (uint32_t)(next() % 0x3f800000u) + 1u;   /* (0, 1): every binary32 pattern, subnormals too */
    if ((it & 255) == 0) wb = 0x3f800000u;                  /* w = 1 */
    float wf; memcpy(&wf, &wb, 4);
    const double w = (double)wf;
    uint64_t sb = 0x3ff0000000000000ull + (next() % (21ull << 52));   /* [1, 2^21) */
    if ((it & 7) == 0) sb = (sb & ~0xfffffull) | ((next() & 1) ? 0 : 0xfffffull);  /* near binade edges */
    double s; memcpy(&s, &sb, 8);
    const double y = 1.0 / s;
    const double q0 = w * y;
    const double e = fma(-q0, s, w);
    const double q = fma(e, y, q0);
    if (q != w / s) {
      if (bad < 5) printf("w=%a s=%a div=%a recip=%a\n", w, s, w / s, q);
      ++bad;
    }
    /* the scaled form the floors use: sm = s 2^-24, ym = RN(1 / sm) */
    const double sm = s * 0x1p-24, ym = 1.0 / sm;
    const double p0 = w * ym;
    const double qs = fma(fma(-p0, sm, w), ym, p0);
    if (qs != (w / s) * 16777216.0) {
      if (bad < 5) printf("scaled: w=%a s=%a div=%a recip=%a\n", w, s, (w / s) * 16777216.0, qs);
      ++bad;
    }
  }
  printf("%ld\n", bad);
  return bad != 0;
}
"""


def test_reciprocal_division_is_correctly_rounded():
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "m.c"), os.path.join(d, "m")
        with open(src, "w") as f:
            f.write(C_SOURCE)
        # -ffp-contract=off: the products and sums are the separate roundings written above
        subprocess.run([cc, "-O2", "-ffp-contract=off", "-o", exe, src, "-lm"], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout
