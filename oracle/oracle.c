/*
 * CPU oracle for the routed-expert FP8 MoE prefill layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant generator with the GPU path.
 *
 * Plain, slow, obviously ordered: FP32 arithmetic in the order the steps are
 * stated, no blocking or fusion beyond that.  Built without fast-math and with
 * floating-point contraction off, so every a*b+c below is a rounded multiply
 * followed by a rounded add.
 *
 * What it computes, for token t with routed scale rho (sources: the pages
 * "ktransformers #2244" (Design: W8A8 GPU prefill, unclamped SiLU, routed
 * scaling kept), "hpc-ops #80" (gap table row 6: blockwise FP8 MoE, 192->256
 * zero padding), "ktransformers #2245" (Semantics and scope: E4M3 decode) and
 * "TensorFold #2852" (description: plan / grouped gate+up / epilogue / grouped
 * down / combine; exactness paragraph: whole K per pass, deterministic member
 * order)):
 *
 *   out_t = cast( rho * sum_{j<k} w[t,j] * y[t,j] ),
 *   y[t,j] = D_e . Q( silu(G_e . Q(x_t)) * (U_e . Q(x_t)) ),  e = ids[t,j]
 *
 * where Q is dynamic E4M3 quantisation per row and per 128-column group and
 * every matrix product is a sum over 128-wide K blocks of an FP32 dot of
 * decoded codes times (activation scale * weight block scale).
 * orc_forward_a16 is the W8A16 form of the same layer (see forward_impl).
 *
 * parity pins: see tests/test_oracle_*.py.  Every function below is pinned
 * there against something other than itself.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- planted faults (tests of the pins only; 0 in normal use) ---------- */
enum {
  FAULT_NONE = 0,
  FAULT_WEIGHT_SCALE_INDEX = 1, /* use the next K block's weight scale       */
  FAULT_DROP_LAST_KBLOCK = 2,   /* skip the last 128-wide K block            */
  FAULT_UNSTABLE_PLAN = 3,      /* rows within an expert in descending order */
  FAULT_SILU_CLAMP = 4,         /* clamp the gate at 10 before SiLU          */
  FAULT_PAD_GARBAGE = 5,        /* padded rows of gate/up hold code 0x38     */
  FAULT_NAN_CODE_IS_NAN = 6,    /* decode 0x7F/0xFF as NaN                   */
  FAULT_GROUP_64 = 7,           /* activation amax over 64 columns           */
  FAULT_DOWN_SCALE_TRANSPOSED = 8,
  FAULT_ENCODE_TRUNCATE = 9,    /* encode by truncation instead of RNE       */
  FAULT_DROP_RHO = 10,
  FAULT_SILU_SIGN = 11,         /* silu(-g)                                  */
  FAULT_GATE_UP_SWAP = 12,      /* silu(u) * g                               */
  FAULT_ROUTE_TIE_HIGH = 13,    /* router ties go to the higher expert id    */
  FAULT_ROUTE_ALL_EXPERTS = 14, /* softmax weights normalised over all E     */
  FAULT_SHARED_INSIDE_RHO = 15, /* shared slots scaled by rho too            */
  FAULT_SLICE_SCALE_BLOCK = 16, /* requant reads the next checkpoint block's scale */
  FAULT_A16_H_TRUNCATE = 17,    /* W8A16: h to BF16 by truncation, not RNE   */
};
static int g_fault = FAULT_NONE;
void orc_set_fault(int32_t f) { g_fault = f; }

/* Clamped SwiGLU variant ("ktransformers #2244", Design: GLM-5.3-Flash clamps
 * at ten, full GLM does not; the formula is not given, so the limit is an
 * explicit parameter).  L > 0: the gate is capped at L and the up value
 * clipped to [-L, L] before h = silu(gate) * up; NaN passes through.  0: the
 * unclamped SiLU.  Applies to orc_forward and orc_bruteforce_fp64 until
 * changed. */
static float g_act_limit = 0.0f;
void orc_set_activation_limit(float limit) { g_act_limit = limit; }

int32_t orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- codecs ----------------------------------------------------------- */

/* E4M3 (OCP E4M3FN: bias 7, no infinities, S.1111.111 is NaN) to FP32, by
 * closed form ("ktransformers #2245", Semantics and scope): normals are
 * (1 + m/8) * 2^(e-7); subnormals are m * 2^-9; signed zeros are kept; the NaN
 * codes decode to a zero of their sign. */
float orc_e4m3_decode(uint32_t code) {
  uint32_t s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
  float mag;
  if (e == 15u && m == 7u)
    mag = (g_fault == FAULT_NAN_CODE_IS_NAN) ? NAN : 0.0f;
  else if (e == 0u)
    mag = ldexpf((float)m, -9);
  else
    mag = ldexpf(1.0f + (float)m / 8.0f, (int)e - 7);
  return s ? -mag : mag;
}

/* FP32 to E4M3: round to nearest, ties to the even code; |v| >= 448 saturates
 * to +-448; a zero result keeps the sign of v; NaN gives +0 (the row it came
 * from is poisoned through its NaN scale anyway).  Works on the FP32 bit
 * pattern: the 3-bit mantissa keeps the top 3 of 23 FP32 mantissa bits.  */
uint32_t orc_e4m3_encode(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0u;              /* NaN */
  if (a >= 0x43E00000u) return sign | 0x7Eu;   /* >= 448: saturate */
  if (a < 0x3C800000u) {                       /* < 2^-6: step 2^-9 */
    float f;
    memcpy(&f, &a, 4);
    float q = f * 512.0f; /* exact */
    float m = (g_fault == FAULT_ENCODE_TRUNCATE) ? truncf(q) : nearbyintf(q);
    return sign | (uint32_t)m;
  }
  uint32_t r = (g_fault == FAULT_ENCODE_TRUNCATE) ? a : a + 0x7FFFFu + ((a >> 20) & 1u);
  uint32_t code = (r >> 20) - (120u << 3); /* FP32 exponent bias 127 -> 7 */
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

float orc_bf16_to_f32(uint32_t b) {
  uint32_t u = (b & 0xFFFFu) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* FP32 to BF16, round to nearest even; NaN stays a (quiet) NaN. */
uint32_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
  uint32_t lsb = (u >> 16) & 1u;
  return ((u + 0x7FFFu + lsb) >> 16) & 0xFFFFu;
}

void orc_decode_array(const uint8_t* in, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(in[i]);
}
void orc_encode_array(const float* in, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e4m3_encode(in[i]);
}
void orc_bf16_to_f32_array(const uint16_t* in, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f32(in[i]);
}
void orc_f32_to_bf16_array(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)orc_f32_to_bf16(in[i]);
}

/* ---- dynamic activation quantisation ----------------------------------- */

/* Per row and per group of 128 consecutive columns starting at column 0:
 * a = max|x| (NaN if any element is NaN); s = a / 448 (IEEE FP32 division);
 * a == 0 gives s = 0 and all codes +0; otherwise q = encode(x / s).
 * x: f32[rows][cols], cols % 128 == 0; q: u8[rows][cols]; s: f32[rows][cols/128]. */
void orc_quantize_rows(const float* x, int64_t rows, int64_t cols, uint8_t* q, float* s) {
  const int64_t G = 128;
  const int64_t ng = cols / G;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t g = 0; g < ng; ++g) {
      const float* xv = x + r * cols + g * G;
      uint8_t* qv = q + r * cols + g * G;
      int64_t span = (g_fault == FAULT_GROUP_64) ? 64 : G;
      float amax = 0.0f;
      int has_nan = 0;
      for (int64_t c = 0; c < span; ++c) {
        float a = fabsf(xv[c]);
        if (isnan(a))
          has_nan = 1;
        else if (a > amax)
          amax = a;
      }
      if (has_nan) amax = NAN;
      float sc = amax / 448.0f;
      s[r * ng + g] = sc;
      for (int64_t c = 0; c < G; ++c)
        qv[c] = (amax == 0.0f) ? 0u : (uint8_t)orc_e4m3_encode(xv[c] / sc);
    }
  }
}

/* ---- plan --------------------------------------------------------------- */

/* Stable counting sort of the routing slots f = t*k + j by expert id.
 * Slots with id < 0 are skip slots; ids >= E are skipped and counted as bad.
 * counts: i32[E]; offsets: i32[E+1] (exclusive prefix sums; offsets[E] is
 * the number of routed slots); perm: i32[>= offsets[E]] sorted position -> f,
 * ascending f within an expert; inv: i32[T*k] f -> sorted position, or -1.
 * Returns the number of bad ids.  ("TensorFold #2852": the router plans all
 * slots and skips a designated id; member order is a deterministic rank.) */
int64_t orc_plan(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv) {
  int64_t P = T * (int64_t)k, bad = 0;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < P; ++f) {
    int32_t e = ids[f];
    if (e >= E) ++bad;
    if (e >= 0 && e < E) ++counts[e];
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
  for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t i = 0; i < P; ++i) {
    int64_t f = (g_fault == FAULT_UNSTABLE_PLAN) ? P - 1 - i : i;
    int32_t e = ids[f];
    if (e >= 0 && e < E) {
      perm[cursor[e]] = (int32_t)f;
      inv[f] = cursor[e]++;
    } else {
      inv[f] = -1;
    }
  }
  free(cursor);
  return bad;
}

/* ---- the layer ---------------------------------------------------------- */

typedef struct {
  int32_t E, H, I;
  const uint8_t* gate;      /* u8[E][I][H] */
  const uint8_t* up;        /* u8[E][I][H] */
  const uint8_t* down;      /* u8[E][H][I] */
  const float* gate_scale;  /* f32[E][ceil(I/128)][H/128] */
  const float* up_scale;    /* f32[E][ceil(I/128)][H/128] */
  const float* down_scale;  /* f32[E][H/128][ceil(I/128)] */
} orc_layer;

/* Optional intermediate outputs (any pointer may be NULL).  Rows of the
 * per-slot arrays are in sorted (plan) order; P = number of routed slots.
 * xq u8[T][H], sx f32[T][H/128], gu f32[P][2*Ip] (gate then up),
 * hq u8[P][Ip], sh f32[P][Ip/128], y f32[P][H],
 * counts i32[E], offsets i32[E+1], perm i32[T*k], inv i32[T*k],
 * hb u16[P][Ip] (W8A16 only: h as BF16 bits; xq, sx, hq, sh are not
 * written in that mode). */
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

/* Padded gate/up row n in [0, 2*Ip) of expert e as codes (gate rows first);
 * rows at or beyond I are the zero padding up to Ip = 128*ceil(I/128). */
static void gate_up_row(const orc_layer* L, int64_t e, int64_t n, int64_t Ip, float* out) {
  int64_t H = L->H, I = L->I;
  int64_t r = n < Ip ? n : n - Ip;
  const uint8_t* src = (n < Ip ? L->gate : L->up) + (e * I + r) * H;
  for (int64_t c = 0; c < H; ++c) {
    if (r < I)
      out[c] = orc_e4m3_decode(src[c]);
    else
      out[c] = (g_fault == FAULT_PAD_GARBAGE) ? 1.0f : 0.0f;
  }
}

static float gate_up_scale(const orc_layer* L, int64_t e, int64_t n, int64_t Ip, int64_t kb) {
  int64_t nI = Ip / 128, nH = L->H / 128;
  int64_t r = n < Ip ? n : n - Ip;
  const float* S = (n < Ip ? L->gate_scale : L->up_scale) + e * nI * nH;
  if (g_fault == FAULT_WEIGHT_SCALE_INDEX) kb = (kb + 1) % nH;
  return S[(r / 128) * nH + kb];
}

/* One output element: sum over 128-wide K blocks, in ascending order, of the
 * FP32 dot of decoded operands (ascending column order) times the product of
 * the row's activation scale and the weight block scale. */
static float blocked_dot(const float* a, const float* a_scale, const float* b,
                         const float* b_scale, int64_t K) {
  int64_t nkb = K / 128;
  if (g_fault == FAULT_DROP_LAST_KBLOCK) nkb -= 1;
  float acc = 0.0f;
  for (int64_t kb = 0; kb < nkb; ++kb) {
    float p = 0.0f;
    for (int64_t c = kb * 128; c < kb * 128 + 128; ++c) p = p + a[c] * b[c];
    acc = acc + p * (a_scale[kb] * b_scale[kb]);
  }
  return acc;
}

static float silu_mul(float g, float u) {
  if (g_fault == FAULT_GATE_UP_SWAP) {
    float t = g;
    g = u;
    u = t;
  }
  if (g_fault == FAULT_SILU_CLAMP && g > 10.0f) g = 10.0f;
  if (g_fault == FAULT_SILU_SIGN) g = -g;
  if (g_act_limit > 0.0f) {
    const float L = g_act_limit;
    if (g > L) g = L;
    if (u > L) u = L;
    if (u < -L) u = -L;
  }
  /* e^-g correctly rounded to FP32: evaluated in double and rounded once
   * (the pages fix only "z / (1 + e^-z)" in FP32; a correctly rounded
   * exponential makes that value independent of any libm's last bit). */
  const float e = (float)exp(-(double)g);
  return (g / (1.0f + e)) * u;
}

/* h = silu(g) * u elementwise, as the layer computes it (test access). */
void orc_silu_mul_array(const float* g, const float* u, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = silu_mul(g[i], u[i]);
}

/* Down projection of the decoded h rows (sorted order) and the weighted
 * combine: y[p] = D_e . h[p] blockwise as above; out[t] = cast(rho * sum_j
 * w[t,j] * y[inv[t*k+j]]), FP32, ascending j, one rounding at the end.
 * The last n_shared slots of a token are always-on shared-expert slots
 * ("TensorFold #2852": nine slots planned over E+1 expert ids): they are
 * added after the routed sum is scaled, outside rho,
 *   out[t] = cast(rho * sum_{j < k-n_shared} w y  +  sum_{j >= k-n_shared} w y). */
static void down_and_combine(const orc_layer* L, int64_t k, const float* hd, const float* sh,
                             const int32_t* counts, const int32_t* offsets, const int32_t* inv,
                             const float* w, int64_t T, float rho, int32_t out_dtype, void* out,
                             float* y, int64_t n_shared) {
  const int64_t E = L->E, H = L->H, I = L->I;
  const int64_t Ip = 128 * ((I + 127) / 128), nH = H / 128, nI = Ip / 128;
#pragma omp parallel
  {
    float* wrow = (float*)malloc(sizeof(float) * (size_t)Ip);
    float* wsc = (float*)malloc(sizeof(float) * (size_t)nI);
#pragma omp for collapse(2) schedule(dynamic, 8)
    for (int64_t e = 0; e < E; ++e) {
      for (int64_t n = 0; n < H; ++n) {
        if (counts[e] == 0) continue;
        const uint8_t* src = L->down + (e * H + n) * I;
        for (int64_t c = 0; c < Ip; ++c) wrow[c] = c < I ? orc_e4m3_decode(src[c]) : 0.0f;
        const float* ds = L->down_scale + e * nH * nI;
        for (int64_t kb = 0; kb < nI; ++kb)
          wsc[kb] = (g_fault == FAULT_DOWN_SCALE_TRANSPOSED)
                        ? ds[(kb % nH) * nI + ((n / 128) % nI)]
                        : ds[(n / 128) * nI + kb];
        for (int64_t p = offsets[e]; p < offsets[e + 1]; ++p)
          y[p * H + n] = blocked_dot(hd + p * Ip, sh + p * nI, wrow, wsc, Ip);
      }
    }
    free(wrow);
    free(wsc);
  }

  /* weighted combine: ascending slot order, FP32, rho once, one rounding */
  float r = (g_fault == FAULT_DROP_RHO) ? 1.0f : rho;
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t n = 0; n < H; ++n) {
      float acc = 0.0f;
      for (int64_t j = 0; j < k - n_shared; ++j) {
        int32_t p = inv[t * k + j];
        if (p >= 0) acc = acc + w[t * k + j] * y[(int64_t)p * H + n];
      }
      float v = r * acc;
      for (int64_t j = k - n_shared; j < k; ++j) {
        int32_t p = inv[t * k + j];
        if (p >= 0) v = v + (g_fault == FAULT_SHARED_INSIDE_RHO ? r : 1.0f) * w[t * k + j] * y[(int64_t)p * H + n];
      }
      if (out_dtype == 0)
        ((uint16_t*)out)[t * H + n] = (uint16_t)orc_f32_to_bf16(v);
      else
        ((float*)out)[t * H + n] = v;
    }
  }
}

/*
 * The routed-expert layer on T tokens.
 * x: bf16 bits u16[T][H]; ids: i32[T][k]; w: f32[T][k].
 * out_dtype 0: out is bf16 bits u16[T][H]; 1: out is f32[T][H].
 * n_shared: the last n_shared slots of each token are shared-expert slots
 * (see down_and_combine); 0 for the routed layer alone.
 * a16 = 0: W8A8 as stated at the top of this file.  a16 = 1: W8A16, the
 * pages' path for decode and short continuations ("ktransformers #2244",
 * Design: prefill of at least 256 tokens uses W8A8 on the GPU, shorter
 * continuations and decode use W8A16): the activations entering each GEMM
 * stay 16-bit, i.e. x as given (BF16, exact in FP32) and h = silu(g) * u
 * rounded to BF16 (round to nearest even); every block product is then the
 * FP32 dot of the activations and the decoded weight codes times the weight
 * block scale (the activation scale of the W8A8 form is 1).
 * Returns the number of bad expert ids (those slots are skipped), or -1 on a
 * bad argument.
 */
static int64_t forward_impl(const orc_layer* L, int32_t k, const uint16_t* x, const int32_t* ids,
                            const float* w, int64_t T, float rho, int32_t out_dtype, void* out,
                            const orc_debug* dbg, int32_t n_shared, int32_t a16) {
  const int64_t E = L->E, H = L->H, I = L->I;
  if (E < 1 || k < 1 || H % 128 != 0 || I < 1 || T < 0 || n_shared < 0 || n_shared >= k) return -1;
  const int64_t Ip = 128 * ((I + 127) / 128), nH = H / 128, nI = Ip / 128;
  const int64_t S = T * k;

  /* quantise the hidden rows */
  float* xf = (float*)malloc(sizeof(float) * (size_t)(T * H + 1));
  uint8_t* xq = (uint8_t*)malloc((size_t)(T * H + 1));
  float* sx = (float*)malloc(sizeof(float) * (size_t)(T * nH + 1));
  for (int64_t i = 0; i < T * H; ++i) xf[i] = orc_bf16_to_f32(x[i]);
  float* xd = xf; /* the activations of the first GEMM */
  if (a16) {
    for (int64_t i = 0; i < T * nH; ++i) sx[i] = 1.0f;
  } else {
    orc_quantize_rows(xf, T, H, xq, sx);
    for (int64_t i = 0; i < T * H; ++i) xd[i] = orc_e4m3_decode(xq[i]); /* decoded codes of xq */
  }

  /* plan */
  int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S + 1));
  int32_t* inv = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S + 1));
  int64_t bad = orc_plan(ids, T, k, (int32_t)E, counts, offsets, perm, inv);
  const int64_t P = offsets[E];

  /* gate and up for every routed slot, in sorted order */
  float* gu = (float*)malloc(sizeof(float) * (size_t)(P * 2 * Ip + 1));
#pragma omp parallel
  {
    float* wrow = (float*)malloc(sizeof(float) * (size_t)H);
    float* wsc = (float*)malloc(sizeof(float) * (size_t)nH);
#pragma omp for collapse(2) schedule(dynamic, 8)
    for (int64_t e = 0; e < E; ++e) {
      for (int64_t n = 0; n < 2 * Ip; ++n) {
        if (counts[e] == 0) continue;
        gate_up_row(L, e, n, Ip, wrow);
        for (int64_t kb = 0; kb < nH; ++kb) wsc[kb] = gate_up_scale(L, e, n, Ip, kb);
        for (int64_t p = offsets[e]; p < offsets[e + 1]; ++p) {
          int64_t t = perm[p] / k;
          gu[p * 2 * Ip + n] = blocked_dot(xd + t * H, sx + t * nH, wrow, wsc, H);
        }
      }
    }
    free(wrow);
    free(wsc);
  }

  /* h = silu(gate) * up, then quantised per row and 128-group */
  float* h = (float*)malloc(sizeof(float) * (size_t)(P * Ip + 1));
  for (int64_t p = 0; p < P; ++p)
    for (int64_t i = 0; i < Ip; ++i) h[p * Ip + i] = silu_mul(gu[p * 2 * Ip + i], gu[p * 2 * Ip + Ip + i]);
  uint8_t* hq = (uint8_t*)malloc((size_t)(P * Ip + 1));
  float* sh = (float*)malloc(sizeof(float) * (size_t)(P * nI + 1));
  uint16_t* hb = NULL;
  float* hd = h; /* the activations of the second GEMM */
  if (a16) {
    hb = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(P * Ip + 1));
    for (int64_t i = 0; i < P * Ip; ++i) {
      uint32_t b;
      if (g_fault == FAULT_A16_H_TRUNCATE) {
        uint32_t u;
        memcpy(&u, &h[i], 4);
        b = u >> 16;
      } else {
        b = orc_f32_to_bf16(h[i]);
      }
      hb[i] = (uint16_t)b;
      hd[i] = orc_bf16_to_f32(b);
    }
    for (int64_t i = 0; i < P * nI; ++i) sh[i] = 1.0f;
  } else {
    orc_quantize_rows(h, P, Ip, hq, sh);
    for (int64_t i = 0; i < P * Ip; ++i) hd[i] = orc_e4m3_decode(hq[i]); /* decoded codes of hq */
  }

  float* y = (float*)malloc(sizeof(float) * (size_t)(P * H + 1));
  down_and_combine(L, k, hd, sh, counts, offsets, inv, w, T, rho, out_dtype, out, y, n_shared);

  if (dbg) {
    if (dbg->xq && !a16) memcpy(dbg->xq, xq, (size_t)(T * H));
    if (dbg->sx && !a16) memcpy(dbg->sx, sx, sizeof(float) * (size_t)(T * nH));
    if (dbg->gu) memcpy(dbg->gu, gu, sizeof(float) * (size_t)(P * 2 * Ip));
    if (dbg->hq && !a16) memcpy(dbg->hq, hq, (size_t)(P * Ip));
    if (dbg->sh && !a16) memcpy(dbg->sh, sh, sizeof(float) * (size_t)(P * nI));
    if (dbg->hb && a16) memcpy(dbg->hb, hb, sizeof(uint16_t) * (size_t)(P * Ip));
    if (dbg->y) memcpy(dbg->y, y, sizeof(float) * (size_t)(P * H));
    if (dbg->counts) memcpy(dbg->counts, counts, sizeof(int32_t) * (size_t)E);
    if (dbg->offsets) memcpy(dbg->offsets, offsets, sizeof(int32_t) * (size_t)(E + 1));
    if (dbg->perm) memcpy(dbg->perm, perm, sizeof(int32_t) * (size_t)P);
    if (dbg->inv) memcpy(dbg->inv, inv, sizeof(int32_t) * (size_t)S);
  }
  free(xf);
  free(xq);
  free(sx);
  free(counts);
  free(offsets);
  free(perm);
  free(inv);
  free(gu);
  free(h);
  free(hq);
  free(hb);
  free(sh);
  free(y);
  return bad;
}

int64_t orc_forward(const orc_layer* L, int32_t k, const uint16_t* x, const int32_t* ids,
                    const float* w, int64_t T, float rho, int32_t out_dtype, void* out,
                    const orc_debug* dbg, int32_t n_shared) {
  return forward_impl(L, k, x, ids, w, T, rho, out_dtype, out, dbg, n_shared, 0);
}

int64_t orc_forward_a16(const orc_layer* L, int32_t k, const uint16_t* x, const int32_t* ids,
                        const float* w, int64_t T, float rho, int32_t out_dtype, void* out,
                        const orc_debug* dbg, int32_t n_shared) {
  return forward_impl(L, k, x, ids, w, T, rho, out_dtype, out, dbg, n_shared, 1);
}

/* ---- brute force B (FP64, dense over experts, tiny inputs only) --------- */

/* Nearest E4M3 code to v by exhaustive search over the finite magnitudes
 * (codes 0x00..0x7E, increasing), ties to the even code, sign from v.  A
 * different method from orc_e4m3_encode; shares only the pinned decoder. */
static uint32_t nearest_code_fp64(double v, const double* mag) {
  if (isnan(v)) return 0u;
  uint32_t sign = signbit(v) ? 0x80u : 0u;
  double a = fabs(v);
  uint32_t best = 0;
  double bd = INFINITY;
  for (uint32_t c = 0; c < 0x7Fu; ++c) {
    double d = fabs(a - mag[c]);
    if (d < bd || (d == bd && (c & 1u) == 0u)) {
      bd = d;
      best = c;
    }
  }
  return sign | best;
}

/* Quantise-dequantise a vector in FP64 per 128-group (v has n entries, n a
 * multiple of 128; trailing entries may be zero padding). */
static void qdq_fp64(const double* v, int64_t n, double* out, const double* mag) {
  for (int64_t g = 0; g < n / 128; ++g) {
    double amax = 0.0;
    int nan = 0;
    for (int64_t c = g * 128; c < g * 128 + 128; ++c) {
      if (isnan(v[c])) nan = 1;
      else if (fabs(v[c]) > amax) amax = fabs(v[c]);
    }
    if (nan) amax = NAN;
    double s = amax / 448.0;
    for (int64_t c = g * 128; c < g * 128 + 128; ++c) {
      if (amax == 0.0) {
        out[c] = 0.0;
        continue;
      }
      uint32_t q = nearest_code_fp64(v[c] / s, mag);
      out[c] = (double)orc_e4m3_decode(q) * s;
    }
  }
}

/*
 * Dense per-token evaluation in FP64: for every token, loop over all E
 * experts, weight expert e by coef_e = sum of the routing weights of the
 * slots that chose it, dequantise every operand first (code * scale) and
 * evaluate the expert FFN.  quantize_activations = 1 redoes the per-row
 * 128-group E4M3 quantisation of x and of h in FP64 (W8A8); 0 keeps x and h
 * unquantised (W8A16).  out: f64[T][H].
 */
int32_t orc_bruteforce_fp64(const orc_layer* L, int32_t k, const uint16_t* x,
                            const int32_t* ids, const float* w, int64_t T, double rho,
                            int32_t quantize_activations, double* out, int32_t n_shared) {
  const int64_t E = L->E, H = L->H, I = L->I;
  const int64_t nI = (I + 127) / 128, nH = H / 128, Ip = 128 * nI;
  double mag[127];
  for (int c = 0; c < 127; ++c) mag[c] = (double)orc_e4m3_decode((uint32_t)c);
  double* xv = (double*)malloc(sizeof(double) * (size_t)H);
  double* xa = (double*)malloc(sizeof(double) * (size_t)H);
  double* hv = (double*)malloc(sizeof(double) * (size_t)Ip);
  double* ha = (double*)malloc(sizeof(double) * (size_t)Ip);
  double* os = (double*)malloc(sizeof(double) * (size_t)H);
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t c = 0; c < H; ++c) xv[c] = (double)orc_bf16_to_f32(x[t * H + c]);
    if (quantize_activations)
      qdq_fp64(xv, H, xa, mag);
    else
      memcpy(xa, xv, sizeof(double) * (size_t)H);
    double* o = out + t * H;
    for (int64_t n = 0; n < H; ++n) o[n] = os[n] = 0.0;
    for (int64_t e = 0; e < E; ++e) {
      double coef = 0.0, coef_s = 0.0;  /* routed slots; shared slots (outside rho) */
      int chosen = 0;
      for (int64_t j = 0; j < k; ++j)
        if (ids[t * k + j] == e) {
          if (j < k - n_shared)
            coef += (double)w[t * k + j];
          else
            coef_s += (double)w[t * k + j];
          chosen = 1;
        }
      if (!chosen) continue;
      for (int64_t i = 0; i < Ip; ++i) hv[i] = 0.0;
      for (int64_t i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int64_t c = 0; c < H; ++c) {
          double wg = (double)orc_e4m3_decode(L->gate[(e * I + i) * H + c]) *
                      (double)L->gate_scale[(e * nI + i / 128) * nH + c / 128];
          double wu = (double)orc_e4m3_decode(L->up[(e * I + i) * H + c]) *
                      (double)L->up_scale[(e * nI + i / 128) * nH + c / 128];
          g += xa[c] * wg;
          u += xa[c] * wu;
        }
        if (g_act_limit > 0.0f) {
          const double L = (double)g_act_limit;
          g = g > L ? L : g;
          u = u > L ? L : (u < -L ? -L : u);
        }
        hv[i] = g / (1.0 + exp(-g)) * u;
      }
      if (quantize_activations)
        qdq_fp64(hv, Ip, ha, mag);
      else
        memcpy(ha, hv, sizeof(double) * (size_t)Ip);
      for (int64_t n = 0; n < H; ++n) {
        double yv = 0.0;
        for (int64_t i = 0; i < I; ++i)
          yv += ha[i] * (double)orc_e4m3_decode(L->down[(e * H + n) * I + i]) *
                (double)L->down_scale[(e * nH + n / 128) * nI + i / 128];
        o[n] += coef * yv;
        os[n] += coef_s * yv;
      }
    }
    for (int64_t n = 0; n < H; ++n) o[n] = o[n] * rho + os[n];
  }
  free(os);
  free(xv);
  free(xa);
  free(hv);
  free(ha);
  return 0;
}

/*
 * The second half of the layer from given h codes: hq u8[P][Ip] and
 * sh f32[P][Ip/128] in the sorted order of the plan of ids (P = routed
 * slots).  Used to continue the oracle from another implementation's h
 * codes where an FP32 value decided a code near a rounding boundary.
 * out as in orc_forward; y (optional) f32[P][H].  Returns P, or -1.
 */
int64_t orc_down_combine(const orc_layer* L, int32_t k, const uint8_t* hq, const float* sh,
                         const int32_t* ids, const float* w, int64_t T, float rho,
                         int32_t out_dtype, void* out, float* y_out, int32_t n_shared) {
  const int64_t E = L->E, H = L->H, I = L->I;
  if (E < 1 || k < 1 || H % 128 != 0 || I < 1 || T < 0 || n_shared < 0 || n_shared >= k) return -1;
  const int64_t Ip = 128 * ((I + 127) / 128), S = T * k;
  int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S + 1));
  int32_t* inv = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S + 1));
  orc_plan(ids, T, k, (int32_t)E, counts, offsets, perm, inv);
  const int64_t P = offsets[E];
  float* hd = (float*)malloc(sizeof(float) * (size_t)(P * Ip + 1));
  for (int64_t i = 0; i < P * Ip; ++i) hd[i] = orc_e4m3_decode(hq[i]);
  float* y = (float*)malloc(sizeof(float) * (size_t)(P * H + 1));
  down_and_combine(L, k, hd, sh, counts, offsets, inv, w, T, rho, out_dtype, out, y, n_shared);
  if (y_out) memcpy(y_out, y, sizeof(float) * (size_t)(P * H));
  free(counts);
  free(offsets);
  free(perm);
  free(inv);
  free(hd);
  free(y);
  return P;
}

/* ---- the router (upstream of the layer, fused on the device) ------------ */

/* Orders two experts for top-k: larger logit first; a NaN logit ranks below
 * every number; equal logits go to the lower expert id. */
static int route_before(float la, int32_t a, float lb, int32_t b) {
  int na = la != la, nb = lb != lb;
  if (na != nb) return nb;           /* the non-NaN one first */
  if (!na && la != lb) return la > lb;
  if (g_fault == FAULT_ROUTE_TIE_HIGH) return a > b;
  return a < b;
}

/*
 * Top-k routing of one token's router logits ("hpc-ops #80", gap table: the
 * router's top-k is part of the fused MoE step; "TensorFold #2852": top-k
 * slots in descending score).  The k experts with the largest logits, in
 * descending order, ties to the lower id (sigmoid and exp are increasing, so
 * this is also the order of the scores).  Weights, in FP64:
 *   kind 0 (softmax): s_j = exp(l_j - l_0), w_j = s_j / sum of the chosen s
 *                     (softmax over all experts, renormalised over the chosen);
 *   kind 1 (sigmoid): s_j = 1 / (1 + exp(-l_j)), w_j = s_j / sum of chosen s.
 * A chosen set with no mass (sum 0, or a softmax whose largest chosen logit
 * is -inf) gets all-zero weights.
 * logits f32[T][E]; ids i32[T][k]; w f64[T][k].  Returns 0, or -1.
 */
int32_t orc_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t kind,
                  int32_t* ids, double* w) {
  if (T < 0 || E < 1 || k < 1 || k > E || (kind != 0 && kind != 1)) return -1;
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    memset(taken, 0, (size_t)E);
    for (int32_t j = 0; j < k; ++j) {      /* selection, one slot at a time */
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || route_before(l[e], e, l[best], best))) best = e;
      taken[best] = 1;
      ids[t * k + j] = best;
    }
    double sum = 0.0;
    const double l0 = (double)l[ids[t * k]];
    double* wt = w + t * k;
    if (kind == 0 && g_fault == FAULT_ROUTE_ALL_EXPERTS) {
      double all = 0.0;
      for (int32_t e = 0; e < E; ++e) all += exp((double)l[e] - l0);
      for (int32_t j = 0; j < k; ++j) wt[j] = exp((double)l[ids[t * k + j]] - l0) / all;
      continue;
    }
    for (int32_t j = 0; j < k; ++j) {
      const double lj = (double)l[ids[t * k + j]];
      wt[j] = kind == 0 ? exp(lj - l0) : 1.0 / (1.0 + exp(-lj));
    }
    const int no_mass = kind == 0 && l0 == -INFINITY;
    for (int32_t j = 0; j < k; ++j) sum += wt[j];
    for (int32_t j = 0; j < k; ++j) wt[j] = (no_mass || sum == 0.0) ? 0.0 : wt[j] / sum;
  }
  free(taken);
  return 0;
}

/* ---- load-time slice of the intermediate dimension ---------------------- */

/*
 * One matrix M [R][C] (E4M3 codes) with FP32 block scales [ceil(R/128)]
 * [ceil(C/128)], sliced along the intermediate dimension: rows (axis 0, the
 * gate / up matrices) or columns (axis 1, the down matrix), keeping
 * [off, off + len).  ("hpc-ops #80", gap table row 6: a tensor-parallel
 * rank's non-128-multiple share gets zero padding and a load-time weight
 * requant.)  If off is a multiple of 128 the slice's blocks are the
 * checkpoint's: codes and the covering blocks' scales are copied.  Otherwise
 * every block of the slice is requantised: v = dec(code) * S_ckpt in FP32
 * (S of the checkpoint block that held the element), s = max|v| / 448 over
 * the slice's 128x128 block (IEEE division; 0 if the block is all zero),
 * code = enc(v / s) (IEEE division, RNE to E4M3).
 * out_codes: [len][C] or [R][len]; out_scales: [ceil(len/128)][ceil(C/128)]
 * or [ceil(R/128)][ceil(len/128)].  Returns 0, or -1 on bad arguments.
 */
int32_t orc_slice_matrix(const uint8_t* codes, const float* scales, int64_t R, int64_t C,
                         int32_t axis, int64_t off, int64_t len, uint8_t* out_codes,
                         float* out_scales) {
  const int64_t full = axis == 0 ? R : C;
  if (R < 1 || C < 1 || (axis != 0 && axis != 1) || off < 0 || len < 1 || off + len > full) return -1;
  const int64_t rb = (R + 127) / 128, cb = (C + 127) / 128;
  const int64_t oR = axis == 0 ? len : R, oC = axis == 0 ? C : len;
  const int64_t orb = (oR + 127) / 128, ocb = (oC + 127) / 128;
  for (int64_t bi = 0; bi < orb; ++bi) {
    for (int64_t bj = 0; bj < ocb; ++bj) {
      const int64_t r0 = bi * 128, r1 = r0 + 128 < oR ? r0 + 128 : oR;
      const int64_t c0 = bj * 128, c1 = c0 + 128 < oC ? c0 + 128 : oC;
      if (off % 128 == 0) {
        /* the block coincides with a checkpoint block (or its start) */
        const int64_t sr = axis == 0 ? (r0 + off) / 128 : bi, sc = axis == 0 ? bj : (c0 + off) / 128;
        out_scales[bi * ocb + bj] = scales[sr * cb + sc];
        for (int64_t r = r0; r < r1; ++r)
          for (int64_t c = c0; c < c1; ++c) {
            const int64_t gr = axis == 0 ? r + off : r, gc = axis == 0 ? c : c + off;
            out_codes[r * oC + c] = codes[gr * C + gc];
          }
        continue;
      }
      float amax = 0.0f;
      for (int64_t pass = 0; pass < 2; ++pass) {
        const float s = amax / 448.0f;
        for (int64_t r = r0; r < r1; ++r)
          for (int64_t c = c0; c < c1; ++c) {
            const int64_t gr = axis == 0 ? r + off : r, gc = axis == 0 ? c : c + off;
            int64_t sbr = gr / 128, sbc = gc / 128;
            if (g_fault == FAULT_SLICE_SCALE_BLOCK) {
              if (axis == 0) sbr = (sbr + 1) % rb; else sbc = (sbc + 1) % cb;
            }
            const float v = orc_e4m3_decode(codes[gr * C + gc]) * scales[sbr * cb + sbc];
            if (pass == 0) {
              const float a = fabsf(v);
              if (a > amax) amax = a;
            } else {
              out_codes[r * oC + c] = (uint8_t)(amax == 0.0f ? 0u : orc_e4m3_encode(v / s));
            }
          }
        if (pass == 0) out_scales[bi * ocb + bj] = amax / 448.0f;
      }
    }
  }
  return 0;
}
