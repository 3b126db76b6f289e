/* Driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of the
 * CPU oracle (oracle/oracle.c) and the input generator (gen/gen.c), compiled
 * into this program with -fsanitize=address,undefined (no OpenMP).  It runs
 * every exported routine of both on small layers, including the edges they
 * handle: a non-128-multiple intermediate size, skip and out-of-range expert
 * ids, a shared-expert slot, a clamped SiLU, NaN / Inf rows, an unaligned
 * share requant and the router's special rows.  Exit status 0 means no
 * sanitizer report (reports abort the program) and every call returned its
 * expected status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t E, H, I;
  const uint8_t *gate, *up, *down;
  const float *gate_scale, *up_scale, *down_scale;
} orc_layer;

typedef struct {
  uint8_t* xq;
  float* sx;
  float* gu;
  uint8_t* hq;
  float* sh;
  float* y;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv;
  uint16_t* hb;
} orc_debug;

void gen_layer(uint64_t, int32_t, int32_t, int32_t, int32_t, int32_t, float, uint8_t*, uint8_t*, uint8_t*,
               float*, float*, float*);
void gen_tokens(uint64_t, int64_t, int32_t, double, float, uint16_t*, uint8_t*);
void gen_logits(uint64_t, int64_t, int32_t, int32_t, int32_t, double, float*);
void gen_routing(uint64_t, int64_t, int32_t, int32_t, int32_t, int32_t, double, int32_t*, float*);

void orc_set_fault(int32_t);
void orc_set_activation_limit(float);
float orc_e4m3_decode(uint32_t);
uint32_t orc_e4m3_encode(float);
void orc_decode_array(const uint8_t*, int64_t, float*);
void orc_encode_array(const float*, int64_t, uint8_t*);
void orc_bf16_to_f32_array(const uint16_t*, int64_t, float*);
void orc_f32_to_bf16_array(const float*, int64_t, uint16_t*);
void orc_quantize_rows(const float*, int64_t, int64_t, uint8_t*, float*);
int64_t orc_plan(const int32_t*, int64_t, int32_t, int32_t, int32_t*, int32_t*, int32_t*, int32_t*);
void orc_silu_mul_array(const float*, const float*, int64_t, float*);
int64_t orc_forward(const orc_layer*, int32_t, const uint16_t*, const int32_t*, const float*, int64_t, float,
                    int32_t, void*, const orc_debug*, int32_t);
int64_t orc_forward_a16(const orc_layer*, int32_t, const uint16_t*, const int32_t*, const float*, int64_t,
                        float, int32_t, void*, const orc_debug*, int32_t);
int32_t orc_bruteforce_fp64(const orc_layer*, int32_t, const uint16_t*, const int32_t*, const float*, int64_t,
                            double, int32_t, double*, int32_t);
int64_t orc_down_combine(const orc_layer*, int32_t, const uint8_t*, const float*, const int32_t*, const float*,
                         int64_t, float, int32_t, void*, float*, int32_t);
int32_t orc_route(const float*, int64_t, int32_t, int32_t, int32_t, int32_t*, double*);
int32_t orc_slice_matrix(const uint8_t*, const float*, int64_t, int64_t, int32_t, int64_t, int64_t, uint8_t*,
                         float*);

static int failures = 0;
#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++failures;                                             \
    }                                                         \
  } while (0)

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

/* One layer: E experts (the last shared when n_shared), all routines. */
static void run_layer(int32_t E, int32_t k, int32_t H, int32_t I, int64_t T, int32_t n_shared, float limit) {
  const int64_t nI = (I + 127) / 128, nH = H / 128, Ip = 128 * nI;
  uint8_t* gate = xmalloc((size_t)E * I * H);
  uint8_t* up = xmalloc((size_t)E * I * H);
  uint8_t* down = xmalloc((size_t)E * H * I);
  float* gs = xmalloc(sizeof(float) * (size_t)(E * nI * nH));
  float* us = xmalloc(sizeof(float) * (size_t)(E * nI * nH));
  float* ds = xmalloc(sizeof(float) * (size_t)(E * nH * nI));
  gen_layer(7, E, H, I, 0, E, 0.02f, gate, up, down, gs, us, ds);
  gate[0] = 0x7F; /* a NaN code decodes to a signed zero */
  down[E * H * I - 1] = 0xFF;
  uint16_t* x = xmalloc(sizeof(uint16_t) * (size_t)(T * H));
  uint8_t* outl = xmalloc((size_t)T);
  gen_tokens(7, T, H, 0.1, 100.0f, x, outl);
  x[1 * H + 3] = 0x7FC0; /* a NaN in row 1 */
  x[2 * H + 5] = 0x7F80; /* +Inf in row 2 */
  const int32_t kr = k - n_shared, Er = E - n_shared;
  int32_t* ids_r = xmalloc(sizeof(int32_t) * (size_t)(T * kr));
  float* w_r = xmalloc(sizeof(float) * (size_t)(T * kr));
  gen_routing(7, T, Er, kr, 1, 0, 1.2, ids_r, w_r);
  float* logits = xmalloc(sizeof(float) * (size_t)(T * Er));
  gen_logits(7, T, Er, 3, Er > 2 ? 1 : 0, 1.2, logits);
  int32_t* ids = xmalloc(sizeof(int32_t) * (size_t)(T * k));
  float* w = xmalloc(sizeof(float) * (size_t)(T * k));
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t j = 0; j < k; ++j) {
      ids[t * k + j] = j < kr ? ids_r[t * kr + j] : Er;
      w[t * k + j] = j < kr ? w_r[t * kr + j] : 1.0f;
    }
  }
  ids[0] = -1;          /* skip slot */
  if (kr > 1) ids[1] = Er + 5; /* out of range: skipped and counted (a shared layer's routed id Er too) */

  orc_layer L = {E, H, I, gate, up, down, gs, us, ds};
  const int64_t S = T * k;
  orc_debug d;
  d.xq = xmalloc((size_t)(T * H));
  d.sx = xmalloc(sizeof(float) * (size_t)(T * nH));
  d.gu = xmalloc(sizeof(float) * (size_t)(S * 2 * Ip));
  d.hq = xmalloc((size_t)(S * Ip));
  d.sh = xmalloc(sizeof(float) * (size_t)(S * nI));
  d.y = xmalloc(sizeof(float) * (size_t)(S * H));
  d.counts = xmalloc(sizeof(int32_t) * (size_t)E);
  d.offsets = xmalloc(sizeof(int32_t) * (size_t)(E + 1));
  d.perm = xmalloc(sizeof(int32_t) * (size_t)S);
  d.inv = xmalloc(sizeof(int32_t) * (size_t)S);
  d.hb = xmalloc(sizeof(uint16_t) * (size_t)(S * Ip));
  uint16_t* out16 = xmalloc(sizeof(uint16_t) * (size_t)(T * H));
  float* out32 = xmalloc(sizeof(float) * (size_t)(T * H));
  double* out64 = xmalloc(sizeof(double) * (size_t)(T * H));

  orc_set_activation_limit(limit);
  const int64_t bad = orc_forward(&L, k, x, ids, w, T, 2.5f, 0, out16, &d, n_shared);
  CHECK(bad == (kr > 1 ? 1 : 0));
  CHECK(orc_forward(&L, k, x, ids, w, T, 2.5f, 1, out32, NULL, n_shared) == bad);
  const int64_t P = d.offsets[E];
  float* y2 = xmalloc(sizeof(float) * (size_t)(P * H));
  CHECK(orc_down_combine(&L, k, d.hq, d.sh, ids, w, T, 2.5f, 1, out32, y2, n_shared) == P);
  CHECK(orc_forward_a16(&L, k, x, ids, w, T, 2.5f, 0, out16, &d, n_shared) == bad);
  CHECK(orc_bruteforce_fp64(&L, k, x, ids, w, T, 2.5, 1, out64, n_shared) == 0);
  CHECK(orc_bruteforce_fp64(&L, k, x, ids, w, T, 2.5, 0, out64, n_shared) == 0);
  orc_set_activation_limit(0.0f);
  /* invalid arguments are refused */
  CHECK(orc_forward(&L, 0, x, ids, w, T, 1.0f, 0, out16, NULL, 0) < 0);
  CHECK(orc_forward(&L, k, x, ids, w, T, 1.0f, 0, out16, NULL, k) < 0);

  /* plan, router, slice */
  int32_t* c2 = xmalloc(sizeof(int32_t) * (size_t)E);
  int32_t* o2 = xmalloc(sizeof(int32_t) * (size_t)(E + 1));
  CHECK(orc_plan(ids, T, k, E, c2, o2, d.perm, d.inv) == bad);
  int32_t* rid = xmalloc(sizeof(int32_t) * (size_t)(T * kr));
  double* rw = xmalloc(sizeof(double) * (size_t)(T * kr));
  logits[0] = NAN;
  logits[Er] = -INFINITY;
  CHECK(orc_route(logits, T, Er, kr, 0, rid, rw) == 0);
  CHECK(orc_route(logits, T, Er, kr, 1, rid, rw) == 0);
  CHECK(orc_route(logits, T, Er, Er + 1, 1, rid, rw) < 0);
  const int64_t len = I > 64 ? I - 50 : I;
  const int64_t off = I - len;
  uint8_t* sc = xmalloc((size_t)(len * H));
  float* ss = xmalloc(sizeof(float) * (size_t)(((len + 127) / 128) * nH));
  CHECK(orc_slice_matrix(gate, gs, I, H, 0, off, len, sc, ss) == 0);
  uint8_t* sc2 = xmalloc((size_t)(H * len));
  float* ss2 = xmalloc(sizeof(float) * (size_t)(nH * ((len + 127) / 128)));
  CHECK(orc_slice_matrix(down, ds, H, I, 1, off, len, sc2, ss2) == 0);
  CHECK(orc_slice_matrix(gate, gs, I, H, 0, off, I + 1, sc, ss) < 0);

  free(gate), free(up), free(down), free(gs), free(us), free(ds), free(x), free(outl), free(ids_r);
  free(w_r), free(logits), free(ids), free(w), free(d.xq), free(d.sx), free(d.gu), free(d.hq), free(d.sh);
  free(d.y), free(d.counts), free(d.offsets), free(d.perm), free(d.inv), free(d.hb), free(out16);
  free(out32), free(out64), free(y2), free(c2), free(o2), free(rid), free(rw), free(sc), free(ss), free(sc2);
  free(ss2);
}

int main(void) {
  /* codecs over every code / many patterns */
  uint8_t codes[256];
  float vals[256];
  for (int i = 0; i < 256; ++i) codes[i] = (uint8_t)i;
  orc_decode_array(codes, 256, vals);
  for (int i = 0; i < 256; ++i) CHECK((i & 0x7F) == 0x7F ? vals[i] == 0.0f : isfinite(vals[i]));
  float f[1024];
  uint8_t q[1024];
  uint16_t b[1024];
  for (int i = 0; i < 1024; ++i) f[i] = (float)(i - 512) * 0.913f;
  f[0] = NAN, f[1] = INFINITY, f[2] = -INFINITY, f[3] = -0.0f, f[4] = 1e-40f;
  orc_encode_array(f, 1024, q);
  orc_f32_to_bf16_array(f, 1024, b);
  orc_bf16_to_f32_array(b, 1024, f);
  float s[8];
  orc_quantize_rows(f + 8, 2, 384, q, s);
  float g[64], u[64], h[64];
  for (int i = 0; i < 64; ++i) g[i] = (float)(i - 32) * 3.1f, u[i] = 1.0f - (float)i / 16.0f;
  g[0] = -1000.0f, g[1] = 1000.0f;
  orc_silu_mul_array(g, u, 64, h);

  run_layer(8, 2, 256, 128, 24, 0, 0.0f);  /* one h group, the tiny layer's shape */
  run_layer(5, 3, 384, 192, 17, 0, 0.0f);  /* I padded to 256 */
  run_layer(6, 3, 256, 64, 9, 1, 0.0f);    /* a shared expert */
  run_layer(4, 2, 256, 320, 11, 0, 1.5f);  /* clamped SiLU, odd block counts */
  run_layer(3, 1, 128, 200, 5, 0, 0.0f);   /* top-1, one K block */
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("sanitized oracle and generator: ok\n");
  return 0;
}
