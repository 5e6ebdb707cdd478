"""The flush kernel divides by a group's scale as q0 = x*y, r = fma(-q0, s, x), q = fma(r, y, q0)
with y = 1/s correctly rounded (Markstein's correction step).  The codes are bit-exact only if
that quotient equals the correctly rounded x / s of the quantizer definition.  This CPU test
checks the identity over every finite fp16 x against scales formed the way the quantizer forms
them, s = max((max - min) / 255, 1e-8) for fp16 min and max, plus the clamped scale itself.
The same quotient gives the zero-point rint(-min / s) (-min is an fp16 value too), compared bit
for bit once given the sign of -min, as the division's has.  (It exercises the arithmetic
identity only; the kernels' codes are compared with the oracle's in the GPU parity tests.)"""
import os
import subprocess
import tempfile

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float h2f(uint16_t h) {
  uint32_t s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023, f;
  if (e == 0) { float v = ldexpf((float)m, -24); return s ? -v : v; }
  if (e == 31) f = (s << 31) | 0x7f800000u | (m << 13);
  else f = (s << 31) | ((e - 15 + 127) << 23) | (m << 13);
  float r; memcpy(&r, &f, 4); return r;
}
static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
int main(int argc, char** argv) {
  const long ns = atol(argv[1]);
  static float xs[65536]; int nx = 0;
  for (int h = 0; h < 65536; ++h) { float v = h2f((uint16_t)h); if (isfinite(v)) xs[nx++] = v; }
  long bad = 0, tot = 0;
  for (long i = 0; i < ns; ++i) {
    float mn = xs[rnd() % nx], mx = xs[rnd() % nx];
    if (mn > mx) { float t = mn; mn = mx; mx = t; }
    float s = (mx - mn) / 255.0f;
    if (s < 1e-8f || i == 0) s = 1e-8f;
    volatile float one = 1.0f;
    const float y = one / s;
    for (int j = 0; j < nx; ++j) {
      const float x = xs[j];
      const float q = x / s;
      const float q0 = x * y;
      const float r = fmaf(-q0, s, x);
      const float q1 = fmaf(r, y, q0);
      ++tot;
      if (rintf(q1) != rintf(q)) ++bad;
      /* the zero-point: rint(-mn / s) with the sign of -mn, compared bit for bit */
      const float z = rintf(x / s), z1 = copysignf(rintf(q1), x);
      uint32_t uz, uz1; memcpy(&uz, &z, 4); memcpy(&uz1, &z1, 4);
      if (uz != uz1) ++bad;
    }
  }
  printf("%ld %ld\n", tot, bad);
  return 0;
}
"""


def test_fma_corrected_quotient_equals_division():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "div.c"), os.path.join(d, "div")
        with open(src, "w") as f:
            f.write(SRC)
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", src, "-o", exe,
                               "-lm"])
        out = subprocess.run([exe, "3000"], capture_output=True, text=True, check=True).stdout
    tot, bad = map(int, out.split())
    assert tot > 1.8e8 and bad == 0, (tot, bad)


SRC255 = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float h2f(uint16_t h) {
  uint32_t s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023, f;
  if (e == 0) { float v = ldexpf((float)m, -24); return s ? -v : v; }
  if (e == 31) f = (s << 31) | 0x7f800000u | (m << 13);
  else f = (s << 31) | ((e - 15 + 127) << 23) | (m << 13);
  float r; memcpy(&r, &f, 4); return r;
}
static uint64_t st = 0x2545F4914F6CDD1Dull;
static uint64_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
static float scale_div(float mn, float mx) {      /* the quantizer's definition */
  float s = (mx - mn) / 255.0f;
  return s < 1e-8f ? 1e-8f : s;
}
static float scale_fma(float mn, float mx) {      /* the kernels' evaluation */
  const float d = mx - mn, y = 1.0f / 255.0f;
  const float q0 = d * y;
  float s = fmaf(fmaf(-q0, 255.0f, d), y, q0);
  return s < 1e-8f ? 1e-8f : s;
}
int main(int argc, char** argv) {
  const long ns = atol(argv[1]);
  static float xs[65536]; int nx = 0;
  for (int h = 0; h < 65536; ++h) { float v = h2f((uint16_t)h); if (isfinite(v)) xs[nx++] = v; }
  long bad = 0, tot = 0;
  for (long i = 0; i < ns + (long)nx; ++i) {
    float mn, mx;
    if (i < nx) { mn = xs[i]; mx = xs[(i * 7919) % nx]; }   /* every fp16 value as one end */
    else { mn = xs[rnd() % nx]; mx = xs[rnd() % nx]; }
    if (mn > mx) { float t = mn; mn = mx; mx = t; }
    const float a = scale_div(mn, mx), b = scale_fma(mn, mx);
    uint32_t ua, ub; memcpy(&ua, &a, 4); memcpy(&ub, &b, 4);
    ++tot;
    if (ua != ub) ++bad;
  }
  printf("%ld %ld\n", tot, bad);
  return 0;
}
"""


def test_scale_by_reciprocal_and_correction_equals_division():
    """The quantizer's scale (max - min) / 255 (then clamped to 1e-8) is evaluated as
    q0 = d * y, q = fma(fma(-q0, 255, d), y, q0) with y = 1/255 correctly rounded.  Bit for bit
    the same scale over 3e7 random pairs of finite fp16 values and every fp16 value as one end
    (a one-off sweep of all 2.0e9 ordered pairs found no difference after the clamp; the only
    unclamped one was the sign of a zero difference)."""
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "div255.c"), os.path.join(d, "div255")
        with open(src, "w") as f:
            f.write(SRC255)
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", src, "-o", exe,
                               "-lm"])
        out = subprocess.run([exe, "30000000"], capture_output=True, text=True, check=True).stdout
    tot, bad = map(int, out.split())
    assert tot > 3e7 and bad == 0, (tot, bad)
