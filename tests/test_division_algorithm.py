"""CPU check of the quantizer kernel's division step.

The kernel computes fl32(w / c1) as one fused multiply-add correction of
w * RN(1/c1) (Markstein's reciprocal-based division; its fast path, used when
|w| >= 2^-100 and c1 in [2^-100, 2^100]).  The snippet below restates that arithmetic in C (gcc, IEEE fmaf)
and checks it against the correctly rounded quotient on random pairs, on
quotients placed exactly at, and one ulp around, every NF4 threshold, and
on worst-case-looking significands.  It shares nothing with the oracle.
"""

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
static float fast_div(float w, float c, float y) {
  float q0 = w * y;
  float r0 = fmaf(-c, q0, w);
  return fmaf(r0, y, q0);
}
static uint64_t st = 88172645463325252ull;
static uint32_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return (uint32_t)(st >> 16); }
static float bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t fb(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }
int main(int argc, char** argv) {
  const float T[7] = {0.0847181827f, 0.171643645f, 0.263425529f, 0.363861799f, 0.479513973f, 0.624888897f, 0.853784382f};
  long bad = 0, n = 0;
  /* random pairs with |w| <= c */
  for (long i = 0; i < 20000000; ++i) {
    uint32_t ce = 27 + rnd() % 200;           /* c in [2^-100, 2^100] */
    float c = bits((ce << 23) | (rnd() & 0x7FFFFF));
    float w = c * (float)((int32_t)rnd()) * 4.656612873e-10f;
    if (fabsf(w) > c) w = c;
    if (fabsf(w) < 0x1p-100f) continue;
    float y = 1.0f / c;
    if (fast_div(w, c, y) != w / c) ++bad;
    ++n;
  }
  /* quotients at and around each threshold: w = fl(t' * c) for t' = t, t +- k ulp */
  for (long i = 0; i < 2000000; ++i) {
    float c = bits(((100 + rnd() % 50) << 23) | (rnd() & 0x7FFFFF));
    float t = T[rnd() % 7];
    int k = (int)(rnd() % 7) - 3;
    float tk = bits(fb(t) + k);
    if (rnd() & 1) tk = -tk;
    float w = tk * c;
    for (int d = -2; d <= 2; ++d) {
      float wd = bits(fb(w) + d);
      if (fabsf(wd) > c) continue;
      float y = 1.0f / c;
      if (fast_div(wd, c, y) != wd / c) ++bad;
      ++n;
    }
  }
  /* significands of all ones / just above one for c */
  for (uint32_t e = 100; e < 150; ++e)
    for (uint32_t m = 0; m < 4096; ++m) {
      float c = bits((e << 23) | (m < 2048 ? (0x7FFFFF - m) : (m - 2048)));
      float y = 1.0f / c;
      for (int j = 0; j < 64; ++j) {
        float w = bits(fb(c) - (rnd() % (1u << 24)));
        if (fabsf(w) < 0x1p-100f) continue;
        if (fast_div(w, c, y) != w / c) ++bad;
        if (fast_div(-w, c, y) != -w / c) ++bad;
        n += 2;
      }
    }
  printf("%ld %ld\n", n, bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_fast_division_is_correctly_rounded():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "div.c")
        exe = os.path.join(d, "div")
        with open(src, "w") as f:
            f.write(C_SRC)
        # -ffp-contract=off keeps w*y an fp32 product; fmaf is the IEEE fused op
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-mfma", src, "-o", exe, "-lm"], check=True)
        res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        n, bad = map(int, res.stdout.split())
        assert n > 20_000_000
        assert bad == 0, f"{bad} of {n} quotients differ from IEEE division"
