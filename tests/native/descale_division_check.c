/* Host check of the FMA-corrected division the fp8 KV append uses: for
 * descales d in [2^-60, 2^60], x any bf16 value (NaN excepted) clamped to
 * +-449 d, q0 = x (1/d), r = fma(-q0, d, x), q = fma(r, 1/d, q0) with the
 * sign of q0 must give the same OCP E4M3 code (round to nearest even,
 * saturating at 448) as the IEEE quotient x / d, and the same binary32
 * quotient wherever 2^-10 <= |x / d| <= 448.  Written from the definitions;
 * compiled with FP contraction off so that every operation rounds once.
 * usage: descale_division_check [number of random descales]  (exit 0: clean) */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t to_bits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

/* OCP E4M3 code of a finite value: 3 mantissa bits, bias 7, subnormal step
 * 2^-9, largest finite 448, round to nearest even, saturating */
static int e4m3(float f) {
  const int s = signbit(f) ? 0x80 : 0;
  const double a = fabs((double)f);
  if (a >= 448.0) return s | 0x7E;
  if (a < ldexp(1.0, -6)) return s | (int)nearbyint(a * 512.0);   /* 8 is the smallest normal */
  int e;
  const double m = 2.0 * frexp(a, &e);                              /* a = m 2^(e-1), m in [1, 2) */
  e -= 1;
  int mant = (int)nearbyint((m - 1.0) * 8.0);
  if (mant == 8) { mant = 0; e += 1; }
  const int code = ((e + 7) << 3) | mant;
  return s | (code > 0x7E ? 0x7E : code);
}

static long checked = 0, bad = 0;

static void check_descale(float d) {
  const float y = 1.0f / d, m = 449.0f * d;
  for (uint32_t h = 0; h < 65536; ++h) {
    const float x = from_bits(h << 16);
    if (isnan(x)) continue;
    const float xc = fminf(fmaxf(x, -m), m);
    const float q0 = xc * y;
    const float r = fmaf(-q0, d, xc);
    const float q = copysignf(fmaf(r, y, q0), q0);
    const float ref = x / d;
    const float qs = fminf(fmaxf(q, -448.0f), 448.0f), refs = fminf(fmaxf(ref, -448.0f), 448.0f);
    ++checked;
    const int code_bad = e4m3(qs) != e4m3(refs);
    const int quot_bad = fabsf(ref) <= 448.0f && fabsf(ref) >= 0x1p-10f && to_bits(q) != to_bits(ref);
    if (code_bad || quot_bad) {
      if (bad < 8) printf("mismatch d=%a x=%a ref=%a q=%a\n", d, x, ref, q);
      ++bad;
    }
  }
}

int main(int argc, char** argv) {
  const int n = argc > 1 ? atoi(argv[1]) : 200;
  for (int e = -60; e <= 60; ++e) {
    check_descale(ldexpf(1.0f, e));
    check_descale(nextafterf(ldexpf(1.0f, e), INFINITY));
    check_descale(nextafterf(ldexpf(2.0f, e), 0.0f));
  }
  const float special[] = {1.0f / 448, 3.0f / 448, 1.0f / 3, 0.1f, 0.7f, 1.5f, 3.0f, 7.0f, 1e-3f, 1e3f, 448.0f, 1.0f / 449};
  for (unsigned i = 0; i < sizeof special / sizeof *special; ++i) check_descale(special[i]);
  uint64_t s = 88172645463325252ull;                 /* xorshift64 */
  for (int i = 0; i < n; ++i) {
    uint32_t b;
    do {
      s ^= s << 13; s ^= s >> 7; s ^= s << 17;
      b = (uint32_t)(s & 0x7FFFFFFFu);
    } while ((int)(b >> 23) - 127 < -60 || (int)(b >> 23) - 127 > 60);
    check_descale(from_bits(b));
  }
  printf("checked %ld quotients, %ld mismatches\n", checked, bad);
  return bad != 0;
}
