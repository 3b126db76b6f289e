/* Host check of the quotient used by the GPU epilogues that quantise h:
 *   y = RN(1 / b), q0 = RN(a * y), r = fma(-q0, b, a), q = (r == 0 ? q0 : fma(r, y, q0))
 * with b = RN(amax / 448) and |a| <= amax.  The E4M3 code (round to nearest
 * even, 3 mantissa bits, exponent bias 7, subnormals in units of 2^-9) of q
 * must equal that of the IEEE quotient RN(a / b) for amax >= 2^-80.
 * Usage: row_div_check STRIDE N_RANDOM  (every STRIDE-th float pattern a,
 * for fixed and N_RANDOM random amax); exit status 1 on any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bits_to_f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

static int e4m3_code(float v) {
  const int s = signbit(v) ? 0x80 : 0;
  double x = fabs((double)v);
  if (x == 0) return s;
  int e;
  frexp(x, &e);
  e -= 1; /* x in [2^e, 2^(e+1)) */
  if (e < -6) return s | (int)nearbyint(x * 512.0); /* subnormal (8 -> smallest normal) */
  double m = nearbyint(ldexp(x, 3 - e));            /* 8 .. 16 */
  if (m == 16) { m = 8; e += 1; }
  return s | ((e + 7) << 3) | ((int)m - 8);
}

int main(int argc, char** argv) {
  const uint32_t stride = argc > 1 ? (uint32_t)atoi(argv[1]) : 1009;
  const int n_random = argc > 2 ? atoi(argv[2]) : 8;
  const float fixed[] = {0x1p-80f, 0x1.b33334p-80f, 448.0f, 1.0f, 3.0f, 0x1.fffffep-1f, 0x1.000002p0f, 0x1.fffffep+127f};
  const int n_fixed = (int)(sizeof(fixed) / sizeof(fixed[0]));
  uint64_t state = 0x9E3779B97F4A7C15ull;
  long checked = 0, bad = 0;
  for (int i = 0; i < n_fixed + n_random; ++i) {
    float amax;
    if (i < n_fixed) {
      amax = fixed[i];
    } else {
      do { /* xorshift64 draw of a finite positive float >= 2^-80 */
        state ^= state << 13; state ^= state >> 7; state ^= state << 17;
        amax = bits_to_f((uint32_t)state & 0x7FFFFFFFu);
      } while (!isfinite(amax) || amax < 0x1p-80f);
    }
    const float b = amax / 448.0f, y = 1.0f / b;
    for (uint64_t au = i % stride; au < 0x100000000ull; au += stride) {
      const float a = bits_to_f((uint32_t)au);
      if (!isfinite(a) || fabsf(a) > amax) continue;
      const float q0 = a * y;
      const float r = fmaf(-q0, b, a);
      const float q = r == 0.0f ? q0 : fmaf(r, y, q0);
      ++checked;
      if (e4m3_code(q) != e4m3_code(a / b)) {
        if (bad < 5) printf("mismatch amax=%a a=%a q=%a exact=%a\n", amax, a, q, a / b);
        ++bad;
      }
    }
    /* the values the kernels meet most: a near +-amax and tiny, every one */
    uint32_t amax_bits;
    memcpy(&amax_bits, &amax, 4);
    for (int k = -4096; k <= 4096; ++k) {
      const float a = bits_to_f((uint32_t)((int64_t)amax_bits + k));
      const float as[2] = {a, -a};
      for (int j = 0; j < 2; ++j) {
        if (!isfinite(as[j]) || fabsf(as[j]) > amax) continue;
        const float q0 = as[j] * y, r = fmaf(-q0, b, as[j]);
        const float q = r == 0.0f ? q0 : fmaf(r, y, q0);
        ++checked;
        if (e4m3_code(q) != e4m3_code(as[j] / b)) ++bad;
      }
    }
  }
  printf("checked %ld quotients, %ld code mismatches\n", checked, bad);
  return bad != 0;
}
