"""The finalize step's quotient: one correctly rounded reciprocal per row and
one remainder correction per element (Markstein's theorem) must give the
correctly rounded A / L, i.e. the same bits as an IEEE division, for every
normal quotient.  The kernels form O = A / L this way (RL-Kernel page,
section 2: one final rounding after the exact FlashAttention-2 rescale), so the
check runs the same fp32 operation sequence on the host, with the C library's
fmaf as the fused multiply-add, against the host's IEEE fp32 division."""
import os
import shutil
import subprocess
import tempfile

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
int main(int argc, char** argv) {
  const long n = atol(argv[1]);
  long bad = 0, normal = 0;
  for (long i = 0; i < n; ++i) {
    const uint64_t x = next(), y = next();
    /* L as the kernels see it: 1 <= L < 2^21; a quarter of the draws with
       mantissas next to all-ones, a quarter next to zero. */
    uint32_t lm = (uint32_t)(x & 0x7fffff);
    const int mode = (int)((x >> 23) & 3);
    if (mode == 0) lm = 0x7fffff - (uint32_t)((x >> 25) & 7);
    if (mode == 1) lm = (uint32_t)((x >> 25) & 7);
    const float L = f_of((uint32_t)(127 + (x >> 30) % 21) << 23 | lm);
    /* A of either sign from 2^-40 to 2^30; one draw in eight lands within an
       ulp of a multiple of L (quotients next to representable values). */
    float A = f_of((uint32_t)((y >> 40) & 1) << 31 | (uint32_t)(87 + y % 70) << 23 |
                   (uint32_t)((y >> 8) & 0x7fffff));
    if (((y >> 41) & 7) == 0) {
      A = (float)(1 + ((y >> 44) & 0xffff)) * L;
      A = f_of(u_of(A) + (uint32_t)((int)((y >> 60) & 3) - 1));
    }
    const float r = 1.0f / L;
    const float q0 = A * r;
    const float e = fmaf(-q0, L, A);
    const float q = fmaf(e, r, q0);
    const float ref = A / L;
    if (fabsf(ref) < 1.17549435e-38f) continue; /* subnormal quotient: not claimed */
    ++normal;
    if (u_of(q) != u_of(ref)) ++bad;
  }
  printf("%ld %ld\n", normal, bad);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_and_correction_equal_ieee_division():
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "q.c"), os.path.join(d, "q")
        open(c, "w").write(SRC)
        # -ffp-contract=off: only the explicit fmaf calls fuse, as in the kernels.
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, c, "-lm"], check=True)
        out = subprocess.run([exe, "20000000"], check=True, capture_output=True, text=True).stdout
    normal, bad = map(int, out.split())
    assert normal > 19_000_000
    assert bad == 0


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_planted_slip_is_caught():
    """Dropping the correction (q = A * r, the reciprocal product alone) must
    disagree with the division somewhere in the same draws."""
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "q.c"), os.path.join(d, "q")
        open(c, "w").write(SRC.replace("const float q = fmaf(e, r, q0);", "const float q = q0 + 0.0f * e;"))
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, c, "-lm"], check=True)
        out = subprocess.run([exe, "2000000"], check=True, capture_output=True, text=True).stdout
    normal, bad = map(int, out.split())
    assert bad > 0
