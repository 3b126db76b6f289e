/* Exhaustive check of the oracle's FP32 -> E4M3 encoder over all 2^32 FP32
 * bit patterns against a nearest-code search.
 *
 * The search knows only the E4M3 values (OCP E4M3FN: a code with exponent
 * field e and mantissa m is m * 2^-9 when e = 0, else (8 + m) * 2^(e - 10);
 * "ktransformers #2245", Semantics and scope) and the rounding rule of the
 * readings: the nearest of the 127 non-negative finite values, ties to the
 * even code, magnitudes at or above 448 saturate to 448, the sign of the
 * input is kept (so -0 and negative values that round to zero give 0x80), a
 * NaN gives +0.  It shares nothing with the oracle's bit manipulation: the
 * table is built from the closed form in double, and the decision is a binary
 * search plus an exact comparison with the midpoint of the two neighbours.
 *
 * Usage: encode_walk /path/to/liboracle.so   (exit status 0 iff no mismatch)
 */
#include <dlfcn.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

typedef uint32_t (*encode_fn)(float);

static double mags[127]; /* code c (0..126) -> its value, ascending */

static uint32_t nearest_code(float v) {
  if (isnan(v)) return 0u;
  const uint32_t sign = signbit(v) ? 0x80u : 0u;
  const double a = fabs((double)v);
  if (a >= mags[126]) return sign | 126u;
  int lo = 0, hi = 126; /* mags[lo] <= a < mags[hi] */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (mags[mid] <= a) lo = mid; else hi = mid;
  }
  const double m = 0.5 * (mags[lo] + mags[hi]); /* exact: short mantissas */
  int c;
  if (a < m) c = lo;
  else if (a > m) c = hi;
  else c = (lo % 2 == 0) ? lo : hi;
  return sign | (uint32_t)c;
}

int main(int argc, char** argv) {
  if (argc < 2) {
    fprintf(stderr, "usage: %s liboracle.so\n", argv[0]);
    return 2;
  }
  void* lib = dlopen(argv[1], RTLD_NOW);
  if (!lib) {
    fprintf(stderr, "dlopen: %s\n", dlerror());
    return 2;
  }
  encode_fn enc = (encode_fn)dlsym(lib, "orc_e4m3_encode");
  if (!enc) {
    fprintf(stderr, "dlsym: %s\n", dlerror());
    return 2;
  }
  for (int c = 0; c < 127; ++c) {
    const int e = c >> 3, m = c & 7;
    mags[c] = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
  }
  long long bad = 0;
  int64_t first_bad = -1;
#pragma omp parallel for schedule(static) reduction(+ : bad)
  for (int64_t i = 0; i < (int64_t)1 << 32; ++i) {
    const uint32_t u = (uint32_t)i;
    float v;
    memcpy(&v, &u, 4);
    if (enc(v) != nearest_code(v)) {
      ++bad;
#pragma omp critical
      if (first_bad < 0) first_bad = (int64_t)u;
    }
  }
  printf("%lld mismatches over 4294967296 patterns", bad);
  if (bad) printf(" (e.g. 0x%08x)", (uint32_t)first_bad);
  printf("\n");
  return bad == 0 ? 0 : 1;
}
