/*
 * Seeded synthetic inputs for the routed-expert FP8 MoE prefill layer.
 *
 * This module produces the *inputs* of the method and nothing else: a
 * block-quantised FP8 expert layer (the checkpoint a serving stack would hand
 * over), BF16 hidden rows with a few outlier rows, and top-k routing
 * decisions with normalised weights.  Both the CPU oracle and the GPU path
 * consume what it writes; it contains none of the arithmetic the method
 * itself performs (no activation quantiser, no GEMM, no SiLU, no combine).
 * The weight rounding below is the checkpoint maker's step: any byte array
 * is a valid FP8 layer, so that routine is not under test.
 *
 * Randomness is counter based: every value is a pure function of
 * (seed, tensor tag, element index), built from the SplitMix64 finaliser
 * (Steele, Lea, Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014), so any slice of a tensor can be produced independently and in
 * parallel with identical results.  Normals use the Box-Muller transform.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum {
  TAG_GATE = 1,
  TAG_UP = 2,
  TAG_DOWN = 3,
  TAG_X = 4,
  TAG_OUTLIER = 5,
  TAG_LOGIT = 6,
  TAG_GUMBEL = 7,
  TAG_EXPERT_PERM = 8,
};

static inline uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tag) {
  return splitmix64(splitmix64(seed) ^ (tag * 0xD1B54A32D192ED03ull));
}

static inline uint64_t draw(uint64_t key, uint64_t idx) {
  return splitmix64(key ^ splitmix64(idx));
}

/* uniform on (0, 1] with 24 random bits */
static inline float unit_open0(uint64_t r) {
  return (float)((r >> 40) + 1) * (1.0f / 16777216.0f);
}
/* uniform on [0, 1) with 24 random bits */
static inline float unit_closed0(uint64_t r) {
  return (float)(r >> 40) * (1.0f / 16777216.0f);
}
/* uniform on (0, 1) in double, 52 random bits */
static inline double unit_open_d(uint64_t r) {
  return ((double)(r >> 12) + 0.5) * (1.0 / 4503599627370496.0);
}

/* Standard normal for element idx of a stream (Box-Muller on the pair
 * idx/2: even idx takes the cosine branch, odd idx the sine branch). */
static inline float normal_at(uint64_t key, uint64_t idx) {
  uint64_t pair = idx >> 1;
  float u1 = unit_open0(draw(key, 2 * pair));
  float u2 = unit_closed0(draw(key, 2 * pair + 1));
  float rad = sqrtf(-2.0f * logf(u1));
  float ang = 6.28318530717958647692f * u2;
  return (idx & 1) ? rad * sinf(ang) : rad * cosf(ang);
}

/* Fill n consecutive normals starting at idx0 (idx0 even is fastest). */
static void normals(uint64_t key, uint64_t idx0, int64_t n, float* out) {
  int64_t i = 0;
  if (idx0 & 1) {
    out[0] = normal_at(key, idx0);
    i = 1;
  }
  for (; i + 1 < n; i += 2) {
    uint64_t pair = (idx0 + (uint64_t)i) >> 1;
    float u1 = unit_open0(draw(key, 2 * pair));
    float u2 = unit_closed0(draw(key, 2 * pair + 1));
    float rad = sqrtf(-2.0f * logf(u1));
    float ang = 6.28318530717958647692f * u2;
    out[i] = rad * cosf(ang);
    out[i + 1] = rad * sinf(ang);
  }
  if (i < n) out[i] = normal_at(key, idx0 + (uint64_t)i);
}

/* Checkpoint-maker rounding of a value already divided by its block scale
 * (|v| <= 448 up to one rounding) to the nearest E4M3 byte, ties to the even
 * code, saturating at 448.  Built from frexp/nearbyint. */
static uint8_t checkpoint_round(float v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  float a = fabsf(v);
  if (!(a < 448.0f)) return (uint8_t)(sign | 0x7E);
  if (a == 0.0f) return sign;
  int ex;
  (void)frexpf(a, &ex);
  int e = ex - 1; /* a in [2^e, 2^(e+1)) */
  if (e < -6) {
    int m = (int)nearbyintf(a * 512.0f);
    return (uint8_t)(sign | m);
  }
  int q = (int)nearbyintf(ldexpf(a, 3 - e)); /* 8..16 */
  if (q == 16) {
    e += 1;
    q = 8;
  }
  int code = ((e + 7) << 3) | (q - 8);
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(sign | code);
}

/*
 * One weight tensor of one expert: rows x cols values 0.02*N(0,1), quantised
 * per 128x128 block (edge blocks may be partial) with scale = amax/448.
 * codes: u8[rows][cols]; scales: f32[ceil(rows/128)][ceil(cols/128)].
 */
static void gen_matrix(uint64_t seed, int tag, int64_t e, int64_t rows, int64_t cols,
                       float stddev, uint8_t* codes, float* scales) {
  uint64_t key = stream_key(seed, (uint64_t)tag);
  int64_t nrb = (rows + 127) / 128, ncb = (cols + 127) / 128;
  float* strip = (float*)malloc(sizeof(float) * 128 * (size_t)cols);
  for (int64_t rb = 0; rb < nrb; ++rb) {
    int64_t r0 = rb * 128, r1 = r0 + 128 < rows ? r0 + 128 : rows;
    for (int64_t r = r0; r < r1; ++r)
      normals(key, (uint64_t)((e * rows + r) * cols), cols, strip + (r - r0) * cols);
    for (int64_t i = 0; i < (r1 - r0) * cols; ++i) strip[i] *= stddev;
    for (int64_t cb = 0; cb < ncb; ++cb) {
      int64_t c0 = cb * 128, c1 = c0 + 128 < cols ? c0 + 128 : cols;
      float amax = 0.0f;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
          float a = fabsf(strip[(r - r0) * cols + c]);
          if (a > amax) amax = a;
        }
      float s = amax / 448.0f;
      scales[rb * ncb + cb] = s;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c)
          codes[r * cols + c] =
              s > 0.0f ? checkpoint_round(strip[(r - r0) * cols + c] / s) : 0;
    }
  }
  free(strip);
}

/*
 * Experts [e_begin, e_end) of a layer with E experts, hidden H, intermediate
 * I.  Output arrays start at expert e_begin:
 *   gate, up: u8[n][I][H]; down: u8[n][H][I]
 *   gate_s, up_s: f32[n][ceil(I/128)][H/128]; down_s: f32[n][H/128][ceil(I/128)]
 */
void gen_layer(uint64_t seed, int32_t E, int32_t H, int32_t I, int32_t e_begin,
               int32_t e_end, float stddev, uint8_t* gate, uint8_t* up, uint8_t* down,
               float* gate_s, float* up_s, float* down_s) {
  (void)E;
  int64_t nI = (I + 127) / 128, nH = (H + 127) / 128;
  int64_t n = e_end - e_begin;
  int64_t wsz = (int64_t)I * H, ssz = nI * nH;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t job = 0; job < 3 * n; ++job) {
    int64_t le = job / 3, which = job % 3, e = e_begin + le;
    if (which == 0)
      gen_matrix(seed, TAG_GATE, e, I, H, stddev, gate + le * wsz, gate_s + le * ssz);
    else if (which == 1)
      gen_matrix(seed, TAG_UP, e, I, H, stddev, up + le * wsz, up_s + le * ssz);
    else
      gen_matrix(seed, TAG_DOWN, e, H, I, stddev, down + le * wsz, down_s + le * ssz);
  }
}

static uint16_t to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef struct {
  uint64_t key;
  int64_t idx;
} keyed;

static int cmp_keyed(const void* a, const void* b) {
  const keyed* x = (const keyed*)a;
  const keyed* y = (const keyed*)b;
  if (x->key != y->key) return x->key < y->key ? -1 : 1;
  return x->idx < y->idx ? -1 : (x->idx > y->idx);
}

/*
 * Hidden rows x: bf16[T][H], values N(0,1).  ceil(outlier_frac*T) distinct
 * rows (the ones with the smallest per-row random key) are multiplied by
 * outlier_mult before the BF16 rounding.  Row t of a workload is the same
 * whatever T is, apart from which rows are outliers.
 */
void gen_tokens(uint64_t seed, int64_t T, int32_t H, double outlier_frac,
                float outlier_mult, uint16_t* x, uint8_t* is_outlier) {
  int64_t n_out = (int64_t)ceil(outlier_frac * (double)T - 1e-9);
  if (n_out < 0) n_out = 0;
  if (n_out > T) n_out = T;
  memset(is_outlier, 0, (size_t)T);
  if (n_out > 0) {
    uint64_t okey = stream_key(seed, TAG_OUTLIER);
    keyed* k = (keyed*)malloc(sizeof(keyed) * (size_t)T);
    for (int64_t t = 0; t < T; ++t) {
      k[t].key = draw(okey, (uint64_t)t);
      k[t].idx = t;
    }
    qsort(k, (size_t)T, sizeof(keyed), cmp_keyed);
    for (int64_t i = 0; i < n_out; ++i) is_outlier[k[i].idx] = 1;
    free(k);
  }
  uint64_t key = stream_key(seed, TAG_X);
#pragma omp parallel
  {
    float* row = (float*)malloc(sizeof(float) * (size_t)H);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      normals(key, (uint64_t)(t * H), H, row);
      float m = is_outlier[t] ? outlier_mult : 1.0f;
      for (int32_t c = 0; c < H; ++c) x[t * H + c] = to_bf16_rne(row[c] * m);
    }
    free(row);
  }
}

enum { ROUTE_SOFTMAX = 0, ROUTE_SIGMOID_NORMAL = 1, ROUTE_SIGMOID_UNIFORM = 2, ROUTE_ZIPF = 3 };

/*
 * Top-k routing decisions (the router runs upstream of the method; its
 * outputs are the method's inputs).
 *   ROUTE_SOFTMAX:          logits N(0,1); top-k by logit; w = softmax over
 *                           the chosen logits (= renormalised softmax probs).
 *   ROUTE_SIGMOID_NORMAL:   logits N(0,1); score = sigmoid; top-k by score;
 *                           w = score / sum of chosen scores.
 *   ROUTE_SIGMOID_UNIFORM:  as above with logits U(0,1).
 *   ROUTE_ZIPF:             popularity p_r ~ r^-zipf_s over a seeded
 *                           permutation of the experts, the n_masked lowest
 *                           ranks get p = 0; logit = log p + Gumbel noise;
 *                           top-k by logit; w = sigmoid(logit) normalised.
 * Slots are ordered by descending score, ties to the lower expert id.
 * ids: i32[T][k]; w: f32[T][k].
 */
/* Zipf log-popularity per expert (n_masked lowest ranks get -inf). */
static double* zipf_logp(uint64_t seed, int32_t E, int32_t n_masked, double zipf_s) {
  double* logp = (double*)malloc(sizeof(double) * (size_t)E);
  keyed* order = (keyed*)malloc(sizeof(keyed) * (size_t)E);
  uint64_t pkey = stream_key(seed, TAG_EXPERT_PERM);
  for (int32_t e = 0; e < E; ++e) {
    order[e].key = draw(pkey, (uint64_t)e);
    order[e].idx = e;
  }
  qsort(order, (size_t)E, sizeof(keyed), cmp_keyed);
  for (int32_t r = 0; r < E; ++r) {
    int64_t e = order[r].idx;
    logp[e] = (r < E - n_masked) ? -zipf_s * log((double)(r + 1)) : -INFINITY;
  }
  free(order);
  return logp;
}

/* The routing logit of (token t, expert e) for a routing kind. */
static double logit_at(int32_t kind, uint64_t lkey, uint64_t gkey, const double* logp,
                       int64_t t, int32_t E, int32_t e) {
  uint64_t idx = (uint64_t)(t * E + e);
  switch (kind) {
    case ROUTE_SOFTMAX:
    case ROUTE_SIGMOID_NORMAL:
      return (double)normal_at(lkey, idx);
    case ROUTE_SIGMOID_UNIFORM:
      return unit_open_d(draw(lkey, idx));
    default: {
      double u = unit_open_d(draw(gkey, idx));
      return logp[e] - log(-log(u));
    }
  }
}

/*
 * Router logits as FP32 [T][E], drawn exactly as gen_routing draws them
 * (the input of an on-device router).
 */
void gen_logits(uint64_t seed, int64_t T, int32_t E, int32_t kind, int32_t n_masked,
                double zipf_s, float* logits) {
  double* logp = kind == ROUTE_ZIPF ? zipf_logp(seed, E, n_masked, zipf_s) : NULL;
  uint64_t lkey = stream_key(seed, TAG_LOGIT);
  uint64_t gkey = stream_key(seed, TAG_GUMBEL);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int32_t e = 0; e < E; ++e)
      logits[t * E + e] = (float)logit_at(kind, lkey, gkey, logp, t, E, e);
  free(logp);
}

void gen_routing(uint64_t seed, int64_t T, int32_t E, int32_t k, int32_t kind,
                 int32_t n_masked, double zipf_s, int32_t* ids, float* w) {
  double* logp = kind == ROUTE_ZIPF ? zipf_logp(seed, E, n_masked, zipf_s) : NULL;
  uint64_t lkey = stream_key(seed, TAG_LOGIT);
  uint64_t gkey = stream_key(seed, TAG_GUMBEL);
#pragma omp parallel
  {
    double* score = (double*)malloc(sizeof(double) * (size_t)E);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      for (int32_t e = 0; e < E; ++e) {
        double l = logit_at(kind, lkey, gkey, logp, t, E, e);
        score[e] = l;
        taken[e] = 0;
      }
      double sum = 0.0, lmax = -INFINITY;
      double sel[64];
      for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e)
          if (!taken[e] && (best < 0 || score[e] > score[best])) best = e;
        taken[best] = 1;
        ids[t * k + j] = best;
        sel[j] = score[best];
        if (j == 0) lmax = score[best];
      }
      for (int32_t j = 0; j < k; ++j) {
        double v;
        if (kind == ROUTE_SOFTMAX)
          v = exp(sel[j] - lmax);
        else
          v = 1.0 / (1.0 + exp(-sel[j]));
        sel[j] = v;
        sum += v;
      }
      for (int32_t j = 0; j < k; ++j) w[t * k + j] = (float)(sel[j] / sum);
    }
    free(score);
    free(taken);
  }
  free(logp);
}
