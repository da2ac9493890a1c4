/* CPU check of the quotient method of the float8 encode kernels.
 *
 * The kernels compute x / s as q0 = |x| * r, e = |x| - q0 * s (one fused
 * multiply-add), q = min(q0 + e * r, FMAX) (one fused multiply-add) with the
 * sign of x restored, where r = 1 / s is itself an IEEE division; q0 is first
 * clamped to FMAX + 1 so no step overflows.  FMAX is 448 for E4M3 and 57344
 * for E5M2.  Restated here in C (fmaf is the correctly rounded fused
 * multiply-add) and compared with the IEEE quotient clamped to +-FMAX, for
 * every finite bf16 x.  A pair may differ only where both values are at most
 * half the format's smallest subnormal in magnitude (2^-10 for E4M3, 2^-17
 * for E5M2) with the same sign: every such value encodes to a zero code of
 * that sign (a tie at that point rounds to the even code, zero), so the codes
 * agree.
 *
 * With a dynamic scale s = amax / FMAX the kernels drop both clamps (no
 * encoded |x| exceeds amax, so no step can overflow); that form is checked
 * too, for every finite bf16 x with |x| <= amax.  Its quotient may then lie
 * a rounding above FMAX, where the format's largest code still applies: it
 * must stay below FMAX (1 + 2^-10), far under the midpoint to the next
 * binade.
 *
 * usage: quotient_check STRIDE [e5m2]
 *          every STRIDE-th dynamic scale amax/FMAX over the positive finite
 *          bf16 amax, plus fixed edge scales; exit status 1 on a mismatch
 *          that could change a code.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t to_bits(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }

static float FMAX = 448.f, ZERO_BELOW = 0x1p-10f;

static float ieee(float x, float s) { return fminf(fmaxf(x / s, -FMAX), FMAX); }

static float method(float x, float s, float r) {
  const float a = fabsf(x);
  const float q0 = fminf(a * r, FMAX + 1.f);
  const float e = fmaf(-q0, s, a);
  const float q = fminf(fmaf(e, r, q0), FMAX);
  return copysignf(q, x);
}

static float method_dyn(float x, float s, float r) {
  const float a = fabsf(x);
  const float q0 = a * r;
  const float e = fmaf(-q0, s, a);
  return copysignf(fmaf(e, r, q0), x);
}

static long check_dyn(float s, float amax) {
  const float r = 1.0f / s;
  long bad = 0;
  for (uint32_t b = 0; b < 65536; ++b) {
    const float x = from_bits(b << 16);
    if (!isfinite(x) || fabsf(x) > amax) continue;
    const float w = ieee(x, s), g = method_dyn(x, s, r);
    if (to_bits(w) == to_bits(g)) continue;
    if (fabsf(w) <= ZERO_BELOW && fabsf(g) <= ZERO_BELOW && signbit(w) == signbit(g)) continue;
    if (fabsf(w) == FMAX && fabsf(g) > FMAX && fabsf(g) <= FMAX * (1.0f + 0x1p-10f) && signbit(w) == signbit(g))
      continue;
    if (bad < 3) printf("mismatch (dynamic): s=%a x=%a ieee=%a method=%a\n", s, x, w, g);
    ++bad;
  }
  return bad;
}

static long check(float s) {
  const float r = 1.0f / s;
  long bad = 0;
  for (uint32_t b = 0; b < 65536; ++b) {
    const float x = from_bits(b << 16);
    if (!isfinite(x)) continue;
    const float w = ieee(x, s), g = method(x, s, r);
    if (to_bits(w) == to_bits(g)) continue;
    if (fabsf(w) <= ZERO_BELOW && fabsf(g) <= ZERO_BELOW && signbit(w) == signbit(g)) continue;
    if (bad < 3) printf("mismatch: s=%a x=%a ieee=%a method=%a\n", s, x, w, g);
    ++bad;
  }
  return bad;
}

int main(int argc, char **argv) {
  const int stride = argc > 1 ? atoi(argv[1]) : 1;
  if (argc > 2 && strcmp(argv[2], "e5m2") == 0) {
    FMAX = 57344.f;
    ZERO_BELOW = 0x1p-17f;
  }
  long bad = 0, n = 0;
  for (uint32_t b = 1; b < 0x7f80; b += (uint32_t)stride) {   /* dynamic scales */
    const float amax = from_bits(b << 16), s = amax / FMAX;
    if (!(s >= 0x1p-80f && s <= 0x1p80f)) continue;
    bad += check(s);
    bad += check_dyn(s, amax);
    ++n;
  }
  const float edge[] = {0x1p-80f, 0x1p80f, 0x1.fffffep79f, 0x1.000002p-80f, 1.0f, 0.125f,
                        1.0f / 448, 4.25f / 448, 93.0f / 448, 1.0f / 57344, 93.0f / 57344,
                        0x1.555556p-22f, 0x1.fffffep-1f, 0x1.000002p0f, 3.0f, 0x1.7ffffep5f};
  for (size_t i = 0; i < sizeof edge / sizeof edge[0]; ++i) {
    bad += check(edge[i]);
    ++n;
  }
  printf("%ld scales, %ld mismatches\n", n, bad);
  return bad != 0;
}
