"""The kernels' division by 2^b - 1 (b = 2, 3, 4) is correctly rounded.

The step of a b-bit grid is a range divided by D = 2^b - 1.  The kernels divide
by the constant with a product by RN(1/D) and one fma residual correction (the
helper `div_small` in the HIP sources), with the product taken as the quotient
when the correction is NaN (x infinite).  This test runs the same sequence of
IEEE fp32 operations on the CPU and compares it bit for bit with x / D for

* every x whose exponent field is 0..5, of both signs: the subnormals and the
  binades where the product q0 or the result can be subnormal (|x| < 2^-120,
  above 15 * 2^-126);
* every x of the binade [1, 2), of both signs;
* every x whose exponent field is 254 or 255, of both signs: the largest
  finite values, the infinities and every NaN.

Why that suffices: the residual r = q0 D - x is a multiple of ulp(q0) of
magnitude at most a few ulp(q0), so the fma gives it exactly whatever the
binade; the fma never overflows either (q0 D is within an ulp of x).  For
every normal x with q0 and the result normal, each step of the sequence and
the division itself therefore commute with scaling x by a power of two, and
the outcome depends only on the significand.
"""
import os
import subprocess

import pytest

C_SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <sys/wait.h>
#include <unistd.h>
static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
/* The empty asm statements keep the compiler from merging the negations into
   the fmas (-fma(a, b, -c) -> fma(-a, b, c) is wrong for a zero result). */
static float div_small(float x, float d, float y) {
  float q0 = x * y;
  __asm__("" : "+x"(q0));
  float r = fmaf(q0, d, -x);
  __asm__("" : "+x"(r));
  const float q = fmaf(-r, y, q0);
  return q == q ? q : q0;
}
static unsigned long long check(float d, uint32_t e_lo, uint32_t e_hi) {
  const float y = 1.0f / d;
  unsigned long long bad = 0;
  for (uint32_t s = 0; s < 2; ++s)
    for (uint32_t e = e_lo; e <= e_hi; ++e)
      for (uint32_t m = 0; m < (1u << 23); ++m) {
        const float x = f_of((s << 31) | (e << 23) | m);
        const float q = div_small(x, d, y), ref = x / d;
        if (isnan(ref) ? !isnan(q) : u_of(q) != u_of(ref)) ++bad;
      }
  return bad;
}
int main(void) {
  /* One process per divisor: the subnormal binades run slowly on x86 (every
     operation on them takes a microcode assist). */
  const float ds[3] = {3.0f, 7.0f, 15.0f};
  for (int k = 0; k < 3; ++k) {
    if (fork() == 0) {
      const unsigned long long b = check(ds[k], 0, 5) + check(ds[k], 127, 127) + check(ds[k], 254, 255);
      printf("D=%g mismatches=%llu\n", ds[k], b);
      return b != 0;
    }
  }
  int fails = 0, st;
  for (int k = 0; k < 3; ++k) fails += wait(&st) < 0 || !WIFEXITED(st) || WEXITSTATUS(st) != 0;
  return fails != 0;
}
"""


def test_div_small_is_correctly_rounded(tmp_path):
    src = tmp_path / "div_small.c"
    exe = tmp_path / "div_small"
    src.write_text(C_SRC)
    # -ffp-contract=off: the product q0 must be rounded on its own, as in the kernel.
    # fmaf is IEEE fused multiply-add either way; -mfma only makes it an instruction.
    flags = ["-O2", "-ffp-contract=off", "-fno-fast-math"]
    if os.path.exists("/proc/cpuinfo") and " fma " in open("/proc/cpuinfo").read():
        flags.append("-mfma")
    subprocess.run(["gcc", *flags, str(src), "-o", str(exe), "-lm"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    for d in ("3", "7", "15"):
        assert f"D={d} mismatches=0" in out.stdout
