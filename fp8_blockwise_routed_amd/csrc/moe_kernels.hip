// HIP kernels of the routed-expert FP8 MoE prefill pass, written for gfx950
// (CDNA4: wave64, FP8 MFMA 16x16x128, 160 KiB LDS per CU).
//
// Launch order per pass (after "TensorFold #2852", description: plan, grouped
// gate+up, gate-up epilogue, grouped down, combine):
//   plan      one workgroup: stable counting sort of the (token, slot) pairs by
//             expert, inverse map, and two tile lists (small / big experts)
//   quant     BF16 rows -> E4M3 codes + FP32 scale per 128-column group
//   gate_up   grouped FP8 GEMM against [gate; up] of each expert, FP32
//             accumulation with per-K-block scale promotion, fused epilogue
//             h = silu(g) * u and per-128-group E4M3 quantisation of h
//   down      grouped FP8 GEMM of h against down, FP32 rows y (sorted order)
//   combine   out[t] = rho * sum_j w[t,j] * y[t,j], ascending j, one rounding
//
// Exactness: every GEMM variant issues the same MFMA per 16x16 output tile
// and K block, applies the block scales in the same order and never splits K,
// so an output row depends only on its own input row ("TensorFold #2852",
// exactness paragraph).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "moe_internal.h"

namespace moe {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- helpers --

__device__ __forceinline__ i32x4 ld16(const void* p) {
  return *reinterpret_cast<const i32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, i32x4 v) { *reinterpret_cast<i32x4*>(p) = v; }
__device__ __forceinline__ f32x4 ld16f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

__device__ __forceinline__ i32x8 cat(i32x4 lo, i32x4 hi) {
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// D = A(16x128 E4M3) * B(128x16 E4M3), FP32, zero accumulator in.  Lane l
// holds row/column l%16 and 32 K bytes for lane group l/16 in both operands;
// D lane l, element i is row 4*(l/16)+i, column l%16.
__device__ __forceinline__ f32x4 mfma_e4m3(i32x8 a, i32x8 b) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

// |v| as an ordered integer: NaN > Inf > finite, so an unsigned max over these
// is a NaN-propagating max|v|.
__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Max over the 16 lanes that share l/16 (one DPP row): lane pairs, then
// quads, then the mirrored halves of 8 and of 16 lanes.
__device__ __forceinline__ uint32_t max16(uint32_t v) {
  v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

// FP32 -> OCP E4M3 byte: round to nearest, ties to even; saturate at 448;
// zero results keep the sign; NaN gives +0.
__device__ __forceinline__ uint32_t to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0u;
  if (a >= 0x43E00000u) return sign | 0x7Eu;            // >= 448
  if (a < 0x3C800000u) {                                 // < 2^-6: multiples of 2^-9
    const float q = __uint_as_float(a) * 512.0f;
    return sign | (uint32_t)__builtin_rintf(q);
  }
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);  // keep 3 mantissa bits, RNE
  return sign | ((r >> 20) - (120u << 3));
}

// E4M3 codes of v0 and v1 in bytes 0 and 1 by the packed hardware
// conversion, which rounds exactly as to_e4m3 for every |v| < 464 (checked
// over all such floats on gfx950).  Used for h / s, where the choice of s
// keeps |h / s| <= 448 (1 + 2^-23); NaN gives a NaN code instead of 0.
__device__ __forceinline__ uint32_t e4m3_pair(float v0, float v1) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false) & 0xFFFFu;
}

// v / sc rounded as an IEEE division rounds it, from the correctly rounded
// reciprocal y = 1 / sc shared by a whole row: q0 = v y, then one correction
// with the remainder v - q0 sc, which an FMA gives exactly whenever it is a
// normal float (Markstein, "Computation of elementary functions on the IBM
// RISC System/6000 processor", 1990: a correctly rounded reciprocal and a
// quotient within one ulp give the correctly rounded quotient after one such
// step).  With sc = amax / 448, |v| <= amax and amax >= 2^-80, a remainder
// can only be subnormal where |v / sc| is far below 2^-10, whose E4M3 code is
// +-0 either way, so the codes equal those of the divisions (three operations
// instead of a division's ten).  A zero remainder keeps q0, so -0 stays -0.
constexpr float kRowDivMin = 0x1p-80f;  // smaller nonzero amax: divide
__device__ __forceinline__ float row_div(float v, float sc, float y) {
  const float q0 = v * y;
  const float r = __builtin_fmaf(-q0, sc, v);
  return r == 0.0f ? q0 : __builtin_fmaf(r, y, q0);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
  return ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16) & 0xFFFFu;
}

// silu(g) * u = g / (1 + e^-g) * u with the hardware exp2 and reciprocal
// (each within a few ulp).  g = -inf gives NaN and g = +inf gives inf, as the
// quotient does.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// The clamped variant for L > 0: gate capped at L, up clipped to [-L, L]
// (comparisons, so NaN passes through); L = 0 is the plain silu_mul.
__device__ __forceinline__ float silu_mul_act(float g, float u, float L) {
  if (L > 0.0f) {
    g = g > L ? L : g;
    u = u > L ? L : (u < -L ? -L : u);
  }
  return silu_mul(g, u);
}

// -------------------------------------------------------------------- plan --
// Counting sort of the (token, slot) pairs by expert that keeps slot order
// within an expert, in three passes over chunks of 1024 slots: per-chunk
// histograms, one workgroup for the offsets and tile lists, per-chunk stable
// scatter.

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  // scratch: kPlanWaves ints
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int base = 0, all = 0;
  for (int w = 0; w < kPlanWaves; ++w) {
    int s = scratch[w];
    if (w < wave) base += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return base + x - v;
}

// Expert of slot f = t*k + j: the caller's id for a routed slot (ids >= the
// routed expert count are flagged and skipped), the shared expert for the
// trailing slot.
__device__ __forceinline__ int slot_expert(const PlanArgs& a, int f, bool& bad) {
  const int t = f / a.k, j = f - t * a.k;
  if (j >= a.k_routed) return a.E - 1;
  const int e = a.ids[t * a.k_routed + j];
  if (e >= a.E_routed) {
    bad = true;
    return -1;
  }
  return e;
}

// Pass 1, one workgroup per chunk of kPlanThreads slots: the chunk's count
// per expert, chunk[c][e].
__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(PlanArgs a) {
  __shared__ int cnt[kMaxExperts];
  const int tid = threadIdx.x, E = a.E, P = a.T * a.k;
  for (int e = tid; e < kMaxExperts; e += kPlanThreads) cnt[e] = 0;
  __syncthreads();
  const int f = blockIdx.x * kPlanThreads + tid;
  bool bad = false;
  if (f < P) {
    const int e = slot_expert(a, f, bad);
    if (e >= 0) atomicAdd(&cnt[e], 1);
  }
  if (bad) *a.err = 1;
  __syncthreads();
  for (int e = tid; e < E; e += kPlanThreads) a.chunk[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Pass 2, one workgroup: per-expert totals, offsets and tile lists, and
// chunk[c][e] turned into the position of chunk c's first row of expert e.
__global__ __launch_bounds__(kPlanThreads) void plan_offsets_kernel(PlanArgs a) {
  __shared__ int scan_scratch[kPlanWaves];
  const int tid = threadIdx.x, E = a.E, P = a.T * a.k;
  const int n_chunks = (P + kPlanThreads - 1) / kPlanThreads;
  int n = 0;
  if (tid < E)
    for (int c0 = 0; c0 < n_chunks; c0 += 8) {
      int m[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) m[j] = c0 + j < n_chunks ? a.chunk[(size_t)(c0 + j) * E + tid] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) n += m[j];
    }
  int total;
  const int off = block_exclusive_scan(n, scan_scratch, &total);
  // each expert's rows go to one list: <= kSmallRows rows one streaming tile,
  // <= kNarrowRows one 128-row tile, more rows near-equal tiles of at most
  // kWideRows
  const int is_small = (n >= 1 && n <= kSmallRows) ? 1 : 0;
  const int is_narrow = (n > kSmallRows && n <= kNarrowRows) ? 1 : 0;
  const int n_wide = n > kNarrowRows ? (n + kWideRows - 1) / kWideRows : 0;
  int n_small_all, n_narrow_all, n_wide_all;
  const int small_at = block_exclusive_scan(is_small, scan_scratch, &n_small_all);
  const int narrow_at = block_exclusive_scan(is_narrow, scan_scratch, &n_narrow_all);
  const int wide_at = block_exclusive_scan(n_wide, scan_scratch, &n_wide_all);
  if (tid < E) {
    a.counts[tid] = n;
    a.offsets[tid] = off;
    // eight chunk counts in flight per round (a store to a.chunk would
    // otherwise keep the next load behind it)
    int run = off;
    for (int c0 = 0; c0 < n_chunks; c0 += 8) {
      int m[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) m[j] = c0 + j < n_chunks ? a.chunk[(size_t)(c0 + j) * E + tid] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (c0 + j < n_chunks) {
          a.chunk[(size_t)(c0 + j) * E + tid] = run;
          run += m[j];
        }
    }
    if (is_small) a.small_tiles[small_at] = Tile{tid, off, n, small_at, 1, 0, 0, 0};
    if (is_narrow) a.narrow_tiles[narrow_at] = Tile{tid, off, n, narrow_at, 1, 0, 0, 0};
    if (n_wide) {
      // split n rows into n_wide tiles of near-equal size, multiples of 16 rows
      const int per = ((n + n_wide - 1) / n_wide + 15) & ~15;
      for (int i = 0; i < n_wide; ++i) {
        const int r0 = i * per;
        const int r = (n - r0) < per ? (n - r0) : per;
        a.wide_tiles[wide_at + i] = Tile{tid, off + r0, r, wide_at, n_wide, 0, 0, 0};
      }
    }
  }
  if (tid == 0) {
    a.offsets[E] = total;
    a.n_tiles[0] = n_small_all;
    a.n_tiles[1] = n_narrow_all;
    a.n_tiles[2] = n_wide_all;
  }
}

// Pass 3, one workgroup per chunk: stable scatter.  A slot's position is its
// chunk's first position for its expert, plus the slots of that expert in
// earlier waves of the chunk (per-wave counts), plus its rank among the
// wave's lanes with the same expert (a ballot match on the id bits).
__global__ __launch_bounds__(kPlanThreads) void plan_scatter_kernel(PlanArgs a) {
  __shared__ int cursor[kMaxExperts];
  __shared__ int wcnt[kPlanWaves][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, P = a.T * a.k;
  const int f = blockIdx.x * kPlanThreads + tid;
  bool ignored = false;
  const int e = f < P ? slot_expert(a, f, ignored) : -1;
  const bool valid = e >= 0;
  for (int x = tid; x < E; x += kPlanThreads) cursor[x] = a.chunk[(size_t)blockIdx.x * E + x];
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 10; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t bm = __ballot(bit);
    same &= bit ? bm : ~bm;
  }
  const int rank = __popcll(same & lt_mask);
  const int group = __popcll(same);
  // every wave's count for every expert present in the chunk (0 elsewhere)
  for (int w = 0; w < kPlanWaves; ++w)
    if (valid) wcnt[w][e] = 0;
  __syncthreads();
  if (valid && rank == 0) wcnt[wave][e] = group;
  __syncthreads();
  if (valid) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wcnt[w][e];
    const int pos = cursor[e] + before + rank;
    a.perm[pos] = f;
    a.inv[f] = pos;
  } else if (f < P) {
    a.inv[f] = -1;
  }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  const int P = a.T * a.k;
  const int n_chunks = (P + kPlanThreads - 1) / kPlanThreads;
  if (n_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(plan_count_kernel, dim3(n_chunks), dim3(kPlanThreads), 0, s, a);
  hipLaunchKernelGGL(plan_offsets_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  hipLaunchKernelGGL(plan_scatter_kernel, dim3(n_chunks), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ router --
// One wave per token.  Each lane holds up to kRoutePerLane logits (experts
// lane, lane + 64, ...) as 64-bit keys that order the experts for top-k:
// high word = the logit's bits mapped to an unsigned order (NaN -> 1 and an
// absent expert -> 0, below every number; -0 is folded into +0), low word =
// ~id, so the larger key is the larger logit and, among equal logits, the
// lower id.  k rounds of a wave-wide max pick the slots in descending order;
// lane j then keeps slot j and computes its score and weight.

__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  uint32_t ord;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) ord = 1u;   // NaN
  else ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)~(uint32_t)e;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;  // the whole wave leaves
  const float* l = a.logits + t * a.E;
  uint64_t key[kRoutePerLane];
#pragma unroll
  for (int i = 0; i < kRoutePerLane; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < a.E ? route_key(l[e], e) : 0ull;
  }
  int my_id = 0;
  for (int j = 0; j < a.k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kRoutePerLane; ++i) best = key[i] > best ? key[i] : best;
    const uint64_t win = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < kRoutePerLane; ++i)
      if (key[i] == win) key[i] = 0ull;  // keys are unique (they hold the id)
    if (lane == j) my_id = (int)~(uint32_t)win;
  }
  const bool slot = lane < a.k;
  const float lj = slot ? l[my_id] : 0.0f;
  const float l0 = __shfl(lj, 0);
  float sc = 0.0f;
  if (slot) sc = a.kind == 0 ? expf(lj - l0) : 1.0f / (1.0f + expf(-lj));
  const float sum = wave_sum_f32(sc);
  const bool no_mass = (a.kind == 0 && l0 == -INFINITY) || sum == 0.0f;
  if (slot) {
    a.ids[t * a.k + lane] = my_id;
    a.w[t * a.k + lane] = no_mass ? 0.0f : sc / sum;
  }
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  hipLaunchKernelGGL(route_kernel, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------- quant --
// 16 lanes per 128-column group, 8 BF16 values (16 bytes) per lane.

__global__ __launch_bounds__(256) void quant_kernel(QuantArgs a) {
  // a block takes group kg of 16 consecutive rows, so the K-block-major
  // scales (sxT) leave as one 64-byte run per block
  const int nH = a.H / kBlock;
  const int kg = (int)(blockIdx.x % (unsigned)nH);
  const int64_t t = (int64_t)(blockIdx.x / (unsigned)nH) * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (t >= a.T) return;  // whole 16-lane groups leave together
  const uint16_t* src = a.x + t * a.H + kg * kBlock + sub * 8;
  const i32x4 raw = ld16(src);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32((uint32_t)raw[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32((uint32_t)raw[i] >> 16);
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = umax(m, abs_bits(v[i]));
  m = max16(m);
  const float amax = __uint_as_float(m);
  const float s = __fdiv_rn(amax, 448.0f);
  uint32_t lo = 0, hi = 0;
  if (amax >= kRowDivMin) {  // the group's quotients by one reciprocal (row_div)
    const float y = __fdiv_rn(1.0f, s);
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= to_e4m3(row_div(v[i], s, y)) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= to_e4m3(row_div(v[4 + i], s, y)) << (8 * i);
  } else if (amax != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= to_e4m3(__fdiv_rn(v[i], s)) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= to_e4m3(__fdiv_rn(v[4 + i], s)) << (8 * i);
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(a.xq + t * a.H + kg * kBlock + sub * 8);
  dst[0] = lo;
  dst[1] = hi;
  if (sub == 0) {
    a.sx[t * nH + kg] = s;
    a.sxT[(int64_t)kg * a.T + t] = s;
  }
}

hipError_t launch_quant(const QuantArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)(a.H / kBlock) * ((a.T + 15) / 16);
  hipLaunchKernelGGL(quant_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- GEMM common --
// Buffer resources (SGPR base + VGPR offset + SGPR/immediate offset) keep the
// per-lane address state of the streaming loads at one VGPR each.

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ i32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
// Weight stream loads: read once per pass, cache policy kWeightAux.
__device__ __forceinline__ i32x4 wload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kWeightAux);
}
__device__ __forceinline__ float bloadf(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Activation tile in LDS: BM rows x 128 bytes per K block; logical 16-byte
// chunk c of row r sits in slot c ^ swz(r).  An MFMA fragment read takes one
// chunk of 16 consecutive rows: gfx950's LDS serves 256 bytes (64 banks) per
// pass, so those 16 reads must fill 16 distinct 16-byte bank groups.  Rows
// 128 bytes apart alternate between the two bank halves, and swz gives the 8
// rows of each half 8 distinct slots (bit 3 of the row flips bit 0 of the
// slot), so every 8- or 16-row group is conflict-free.  Only bits 0-3 of the
// row matter, so subtiles of 16 rows share the lane's slot.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// h staging tile of the gate_up epilogues: 128 bytes per row, 16-byte chunk c
// of row r in slot c ^ ((r / 4) & 7).  The byte writes of one instruction
// cover rows 4 apart (one per 16-lane group), which the XOR spreads over
// distinct banks; the copy-out reads whole aligned chunks.
__device__ __forceinline__ int h_off(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 2) & 7)) << 4); }

// ----------------------------------------------------------- tile helpers --

typedef __attribute__((address_space(3))) void lds_void_t;

// One wave instruction: each lane loads `bytes` (4 or 16) from r at
// voff + soff and the wave writes them contiguously at lds_base.
template <int AUX>
__device__ __forceinline__ void dma16(rsrc_t r, uint8_t* lds_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, voff, soff, 0, AUX);
}
__device__ __forceinline__ void dma4(rsrc_t r, void* lds_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 4, voff, soff, 0, 0);
}

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>), in order.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(static_cast<F&&>(f));
  }
}

// Empty asm that takes the four accumulator tiles of a subtile as read-write
// VGPR operands: it emits nothing, but the FMAs that produce them cannot be
// moved past it, so a subtile's promotion stays beside the next subtile's
// MFMAs instead of drifting to the end of the K step.
__device__ __forceinline__ void pin_in_place(f32x4 (&a)[4]) {
  asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}

// K-loop barrier of the LDS-DMA ring.  The compiler lowers __syncthreads()
// after waiting for every LDS-DMA load the wave has in flight, which would
// drain the ring each K step; this barrier leaves them in flight.  Callers
// first wait (vmcnt) for the loads of the stage the other waves read next,
// and for their own LDS reads (lgkmcnt) of the stage the next DMA reuses.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Work-item order of the large-expert GEMMs.  The items (tile, weight block)
// of one expert are visited in blocks of kItemTiles row tiles x kItemBlocks
// weight blocks, and each run of 32 consecutive items goes to the 32 CUs of
// one XCD, so the workgroups running side by side on an XCD share each weight
// chunk ~4 ways and each activation tile ~8 ways in that XCD's L2.
// Item i: the tile at position i / NB in tile-major order has the same
// expert, whose items start at first * NB.
constexpr int kItemTiles = 4, kItemBlocks = 8, kXcds = 8;

struct Item {
  int e, p0, rows, nb;
};

// The tile lists are written by the plan launch and only read afterwards, so
// the GEMMs read them through the scalar cache (constant address space): a
// vector load would count in vmcnt, and waiting for it would also wait for
// every operand load the wave has in flight.
typedef const __attribute__((address_space(4))) Tile* ctile_ptr;

// All fields are workgroup-uniform; readfirstlane keeps them in SGPRs so the
// buffer descriptors built from them stay scalar.
__device__ __forceinline__ Item item_of(int i, int NB, const Tile* tiles_) {
  constexpr int IT = kItemTiles, IB = kItemBlocks;
  const ctile_ptr tiles = (ctile_ptr)tiles_;
  const int tg = i / NB;
  const int first = __builtin_amdgcn_readfirstlane(tiles[tg].first);
  const int me = __builtin_amdgcn_readfirstlane(tiles[tg].count);
  const int li = i - first * NB;
  const int full = NB / IB;
  int nbb = li / (me * IB), rem, nbs;
  if (nbb < full) {
    rem = li - nbb * me * IB;
    nbs = IB;
  } else {
    nbb = full;
    rem = li - full * me * IB;
    nbs = NB - full * IB;
  }
  const int per_mb = IT * nbs;
  const int mb = rem / per_mb;
  const int r2 = rem - mb * per_mb;
  const int m_in = r2 / nbs;
  const ctile_ptr t = tiles + first + mb * IT + m_in;
  Item it;
  it.e = __builtin_amdgcn_readfirstlane(t->e);
  it.p0 = __builtin_amdgcn_readfirstlane(t->p0);
  it.rows = __builtin_amdgcn_readfirstlane(t->rows);
  it.nb = __builtin_amdgcn_readfirstlane(nbb * IB + (r2 - m_in * nbs));
  return it;
}

// r-th item of this workgroup: consecutive 32-item runs per XCD when the grid
// is a multiple of the XCD count (workgroups are dealt to XCDs round-robin)
__device__ __forceinline__ int item_index(int r) {
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  if (G % kXcds) return b + r * G;
  const int slots = G / kXcds;
  return (r * kXcds + b % kXcds) * slots + b / kXcds;
}

// The items of a launch over two tile lists (n1 items of the first, then n2
// of the second), dealt in the XCD runs of item_index, with the two lists'
// runs interleaved in proportion to their counts: in every round some XCDs
// stream the weight-bound items of one list while the others compute the
// MFMA-bound items of the other, instead of one phase after the other.
// next(q) returns the item at or after position q of this workgroup's
// sequence and moves q past it: the first list's item i as i, the second's
// as n1 + i, n1 + n2 past the end.  Positions beyond a list's last, partial
// run are skipped.
struct MixedItems {
  int n1, n2, run, r1, r2, total;
  __device__ __forceinline__ MixedItems(int n1_, int n2_) : n1(n1_), n2(n2_) {
    const int G = (int)gridDim.x;
    run = (G % kXcds) ? G : G / kXcds;
    r1 = (n1 + run - 1) / run;
    r2 = (n2 + run - 1) / run;
    total = (r1 + r2) * run;
  }
  __device__ __forceinline__ int next(int& q) const {
    if (!kMixLists) {  // the first list, then the second
      const int g = item_index(q++);
      return g < n1 + n2 ? g : n1 + n2;
    }
    for (;; ++q) {
      const int g = item_index(q);
      if (g >= total) return n1 + n2;
      const int j = g / run, o = g - j * run;
      const int c2 = (int)((long long)j * r2 / (r1 + r2));
      const bool second = (int)((long long)(j + 1) * r2 / (r1 + r2)) > c2;
      const int i = (second ? c2 : j - c2) * run + o;
      if (i < (second ? n2 : n1)) {
        ++q;
        return second ? n1 + i : i;
      }
    }
  }
};

// Streaming gate_up for experts with at most 16 rows (the HBM-bound regime):
// one 16-row subtile, so every weight byte feeds one MFMA.  No LDS activation
// tile and no barrier inside the K loop: each wave loads its own activation
// fragment (L2 resident) and weight fragments straight into registers, D K
// blocks deep, so the four waves stream independently.  Row scales for all K
// blocks are staged in LDS once per tile.  Same MFMA, promotion order and
// epilogue arithmetic as the tile kernels, so a row's bits do not depend on
// which kernel ran it.
template <int D>
__global__ __launch_bounds__(kThreads, kGateUpWgPerCu) void gate_up_stream_kernel(GateUpArgs a) {
  constexpr int BM = kSmallRows;
  __shared__ float sxt[BM][kMaxKBlocks];
  __shared__ float ws_lds[2 * kMaxKBlocks];
  __shared__ int tok_lds[BM];
  __shared__ uint32_t red_lds[kWaves][BM];
  __shared__ __attribute__((aligned(16))) uint8_t h_lds[BM * 128];
  __shared__ float sh_lds[BM];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int H = a.H, Ip = a.Ip, nH = H / kBlock, NB = Ip / kBlock;
  const int n_items = a.n_tiles[0] * NB;
  const rsrc_t xr = make_rsrc(a.xq, (uint32_t)a.xq_bytes);
  const uint32_t bvoff = (uint32_t)(wave * 8192 + lane * 16);

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int tile = item / NB, nb = item - tile * NB;
    const ctile_ptr td = (ctile_ptr)a.tiles + tile;
    const int e = td->e, p0 = td->p0, rows = td->rows;

    __syncthreads();  // LDS of the previous item is no longer read
    if (tid < BM) tok_lds[tid] = a.perm[p0 + (tid < rows ? tid : 0)] / a.k;
    {
      const float* ws = a.s13 + (size_t)(e * NB + nb) * nH * 2;
      for (int i = tid; i < 2 * nH; i += kThreads) ws_lds[i] = ws[i];
    }
    __syncthreads();
    for (int i = tid; i < BM * nH; i += kThreads) {
      const int r = i / nH, kb = i - r * nH;
      sxt[r][kb] = a.sx[(size_t)tok_lds[r] * nH + kb];
    }
    __syncthreads();

    const rsrc_t wr = make_rsrc(a.w13 + (size_t)(e * NB + nb) * nH * kGateUpChunk, (uint32_t)(nH * kGateUpChunk));
    const uint32_t avo = (uint32_t)(tok_lds[col] * H + grp * 32);
    i32x8 A[D], B[D][4];
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Block kb's operands; kb >= nH reads out of range (zeros, no memory access).
    auto load = [&](int kb, i32x8& af, i32x8(&bf)[4]) {
      const bool in = kb < nH;
      const uint32_t oob = in ? 0u : 0x80000000u;
      const uint32_t so = in ? (uint32_t)(kb * kGateUpChunk) : 0u;
      const uint32_t sa = in ? (uint32_t)(kb * kBlock) : 0u;
      af = cat(bload16(xr, avo + oob, sa), bload16(xr, avo + oob, sa + 16));
#pragma unroll
      for (int t = 0; t < 4; ++t)
        bf[t] = cat(wload16(wr, bvoff + oob, so + t * 2048), wload16(wr, bvoff + oob, so + t * 2048 + 1024));
    };
    auto compute = [&](int kb, const i32x8& af, const i32x8(&bf)[4]) {
      f32x4 p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) p[t] = mfma_e4m3(af, bf[t]);
      const float wsg = ws_lds[2 * kb], wsu = ws_lds[2 * kb + 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float rs = sxt[grp * 4 + i][kb];
        const float sg = rs * wsg, su = rs * wsu;
        acc[0][i] = __builtin_fmaf(p[0][i], sg, acc[0][i]);
        acc[1][i] = __builtin_fmaf(p[1][i], sg, acc[1][i]);
        acc[2][i] = __builtin_fmaf(p[2][i], su, acc[2][i]);
        acc[3][i] = __builtin_fmaf(p[3][i], su, acc[3][i]);
      }
    };

#pragma unroll
    for (int s = 0; s < D - 1; ++s) load(s, A[s], B[s]);
    for (int kb0 = 0; kb0 < nH; kb0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        load(kb0 + s + D - 1, A[(s + D - 1) % D], B[(s + D - 1) % D]);
        if (kb0 + s < nH) compute(kb0 + s, A[s], B[s]);
      }
    }

    // epilogue: h = silu(gate) * up, per-row amax over the 128 columns, E4M3
    if (a.gu_dbg) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = grp * 4 + i;
        if (r < rows) {
          float* g = a.gu_dbg + (size_t)(p0 + r) * 2 * Ip + nb * kBlock + wave * 32 + col;
          g[0] = acc[0][i];
          g[16] = acc[1][i];
          g[Ip] = acc[2][i];
          g[Ip + 16] = acc[3][i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[0][i] = silu_mul_act(acc[0][i], acc[2][i], a.act_limit);
      acc[1][i] = silu_mul_act(acc[1][i], acc[3][i], a.act_limit);
      const uint32_t mb = max16(umax(abs_bits(acc[0][i]), abs_bits(acc[1][i])));
      if (col == 0) red_lds[wave][grp * 4 + i] = mb;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = grp * 4 + i;
      const uint32_t mb = umax(umax(red_lds[0][r], red_lds[1][r]), umax(red_lds[2][r], red_lds[3][r]));
      const float amax = __uint_as_float(mb);
      const float sc = __fdiv_rn(amax, 448.0f);
      const uint32_t c = amax != 0.0f ? e4m3_pair(__fdiv_rn(acc[0][i], sc), __fdiv_rn(acc[1][i], sc)) : 0u;
      h_lds[r * 128 + wave * 32 + col] = (uint8_t)c;
      h_lds[r * 128 + wave * 32 + 16 + col] = (uint8_t)(c >> 8);
      if (wave == 0 && col == 0) sh_lds[r] = sc;
    }
    __syncthreads();
    if ((tid >> 3) < rows)
      st16(a.hq + (size_t)(p0 + (tid >> 3)) * Ip + nb * kBlock + (tid & 7) * 16,
           ld16(&h_lds[(tid >> 3) * 128 + (tid & 7) * 16]));
    if (tid < rows) {
      a.sh[(size_t)(p0 + tid) * NB + nb] = sh_lds[tid];
      a.shT[(size_t)nb * a.P + p0 + tid] = sh_lds[tid];
    }
  }
}

// gate_up for experts with more than kNarrowRows rows: a 512-thread workgroup
// (two waves per SIMD, up to 256 registers each) computes a tile of up to 256
// rows x (128 gate + 128 up) columns of one 128-row block nb, so the epilogue
// sees whole 128-wide groups of h.  Both operands arrive in LDS by
// buffer-load-to-LDS, double-buffered by K block: the activation rows,
// gathered through the plan's permutation (32 KiB per K block; each lane
// fetches the 16-byte chunk that lands in its swizzled slot), and the
// expert's 32 KiB weight chunk, read once per workgroup.  Wave w = 4 mh + wn
// owns rows 128 mh .. +127 and 32-column group wn of gate and up (4 n-tiles):
// each activation fragment it reads feeds four MFMAs.  Same 16x16 tiles,
// MFMAs and promotion order as the streaming kernel.
//
// Per K block the tile moves 64 KiB through the vector memory pipe for
// 256 x 256 x 128 MACs: half the MFMA time at peak, at the ~64 bytes per
// cycle a CU's loads reach from L2 when enough are in flight; a 128-row tile
// would move 48 KiB for half the MACs.  Two 64 KiB stages are all the LDS
// holds, so block kb + 1 is loaded while block kb is multiplied and each K
// step ends with vmcnt(0) and a barrier: the loads drain at every step's end.
// A half with few rows multiplies fewer 16-row subtiles (8, 4 or none) but
// runs the same loads and barriers.
constexpr int kWideThreads = 512;
static_assert(kWideRows == 256, "a tile is two 128-row halves");

// kDbg: also write gate/up before the epilogue to a.gu_dbg (inspection
// launches only; the pass launches the variant without that code).
template <bool kDbg>
__global__ __launch_bounds__(kWideThreads, 1) void gate_up_wide_kernel(GateUpArgs a) {
  constexpr int BM = kWideRows;
  constexpr int NS = 2;  // LDS stages (1 K block ahead)
  // one LDS object per stage, indexed only by compile-time stage numbers, so
  // the compiler can tell a DMA into one stage from reads of another and does
  // not make the MFMA reads wait for the DMAs just issued
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds0[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds1[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t w_lds0[kGateUpChunk];
  __shared__ __attribute__((aligned(1024))) uint8_t w_lds1[kGateUpChunk];
  // Promotion factors of a K block, per stage: row scale x gate weight scale
  // for rows 0-255, then row scale x up weight scale.  Waves 0-3 form them
  // for their rows 64w .. + 63 at the end of the step before, so the matrix
  // waves read two products per row instead of multiplying eight times per
  // subtile.  sx0_lds takes block 0's row scales by DMA (the other half:
  // waves 4-7's out-of-range loads).
  __shared__ __attribute__((aligned(256))) float cs_lds0[2 * BM];
  __shared__ __attribute__((aligned(256))) float cs_lds1[2 * BM];
  __shared__ __attribute__((aligned(256))) float sx0_lds[2 * BM];
  // row list and weight scales of the current item and of the next one
  __shared__ float ws_lds[2][2 * kMaxKBlocks];
  __shared__ int tok_lds[2][BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mh = wave >> 2, wn = wave & 3;
  const int col = lane & 15, grp = lane >> 4;
  const int H = a.H, Ip = a.Ip, nH = H / kBlock, NB = Ip / kBlock;
  const int n_items = a.n_tiles[0] * NB;
  const rsrc_t xr = make_rsrc(a.xq, (uint32_t)a.xq_bytes);
  const rsrc_t sr = make_rsrc(a.sxT, (uint32_t)a.sxT_bytes);
  const rsrc_t pr = make_rsrc(a.perm, (uint32_t)a.P * 4u);
  // B fragments of the wave: n-tiles g0, g1, u0, u1 of 32-column group wn
  const int w_rd = wn * 8192 + lane * 16;
  // A fragments: rows 128 mh + 16 m + lane % 16 (swz(row) = swz(lane))
  const int afr = (mh * 128 + (lane & 15)) * 128;
  const int afc0 = ((2 * grp) ^ swz(lane)) << 4, afc1 = ((2 * grp + 1) ^ swz(lane)) << 4;

  // An item's slot list (tile rows; the token is slot / k) and weight scales,
  // straight into LDS buffer buf: waves 0-3 the slots of rows 64w .. + 63,
  // waves 4-7 weight scales 64 (w - 4) .. + 63 (out of range past 2 nH)
  auto meta_dma = [&](int buf, const Item& it) __attribute__((always_inline)) {
    if (wave < 4) {
      dma4(pr, &tok_lds[buf][wave * 64], (uint32_t)((it.p0 + (tid < it.rows ? tid : 0)) * 4), 0u);
    } else {
      const int i = tid - BM;
      const rsrc_t wsr = make_rsrc(a.s13 + (size_t)(it.e * NB + it.nb) * nH * 2, (uint32_t)(2 * nH * 4));
      dma4(wsr, &ws_lds[buf][(wave - 4) * 64], (uint32_t)(i * 4) | (i < 2 * nH ? 0u : 0x80000000u), 0u);
    }
  };
  auto wrsrc = [&](const Item& it) __attribute__((always_inline)) {
    return make_rsrc(a.w13 + (size_t)(it.e * NB + it.nb) * nH * kGateUpChunk, (uint32_t)(nH * kGateUpChunk));
  };
  // DMA instruction q of wave w moves LDS block b = 8q + w (1 KiB): rows
  // 8b .. 8b + 7 of the activation tile (lane: row 8b + l/8, swizzled slot
  // l % 8) and bytes 1024 b .. of the weight chunk; rows past the tile read
  // out of range (zeros).  Row scales: waves 0-3 load rows 64w + lane, waves
  // 4-7 out of range.
  struct Src {
    rsrc_t wr;
    uint32_t avo[4], svo, wlo;
  };
  auto src_of = [&](int buf, const Item& it) __attribute__((always_inline)) {
    Src q;
    q.wr = wrsrc(it);
    // lane terms from an opaque thread id: not shared with (and kept live
    // from) the other call
    int ltid = (int)threadIdx.x;
    asm volatile("" : "+v"(ltid));
    const int lane = ltid & 63;
    q.wlo = (uint32_t)(lane * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = (j * 8 + wave) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(row);
      q.avo[j] = (uint32_t)(tok_lds[buf][row] / a.k * H + c * 16) | (row < it.rows ? 0u : 0x80000000u);
    }
    const int srow = (wave & 3) * 64 + lane;
    q.svo = (uint32_t)(tok_lds[buf][srow] / a.k * 4) | (srow < it.rows && wave < 4 ? 0u : 0x80000000u);
    return q;
  };
  // K block kb's loads in two-instruction parts 0-3 (weights, activations)
  // and part 4 (row scales); past the last block every load
  // reads out of range (zeros into the unused stage)
  auto issue_part = [&](auto ST, auto PT, int kb, const Src& q) __attribute__((always_inline)) {
    constexpr int st = decltype(ST)::value, p = decltype(PT)::value;
    const bool in = kb < nH;
    const uint32_t oob = in ? 0u : 0x80000000u;
    if constexpr (p < 2) {
      uint8_t* wl = st == 0 ? w_lds0 : w_lds1;
      const uint32_t sw = in ? (uint32_t)(kb * kGateUpChunk) : 0u;
#pragma unroll
      for (int j = 2 * p; j < 2 * p + 2; ++j)
        dma16<0>(q.wr, wl + (j * 8 + wave) * 1024, ((uint32_t)((j * 8 + wave) * 1024) + q.wlo) | oob, sw);
    } else if constexpr (p < 4) {
      uint8_t* al = st == 0 ? a_lds0 : a_lds1;
      const uint32_t sa = in ? (uint32_t)(kb * kBlock) : 0u;
#pragma unroll
      for (int j = 2 * (p - 2); j < 2 * (p - 2) + 2; ++j) dma16<0>(xr, al + (j * 8 + wave) * 1024, q.avo[j] | oob, sa);
    } else {
      static_assert(st == 0, "block 0's row scales only");
      dma4(sr, sx0_lds + wave * 64, q.svo | oob, in ? (uint32_t)(kb * a.T * 4) : 0u);
    }
  };
  // block kb's row scale of row 64w + lane (waves 0-3; 0 past the last block)
  auto row_scale = [&](int kb, const Src& q) __attribute__((always_inline)) {
    const bool in = kb < nH;
    return bloadf(sr, q.svo | (in ? 0u : 0x80000000u), in ? (uint32_t)(kb * a.T * 4) : 0u);
  };
  auto issue = [&](auto ST, int kb, const Src& q) __attribute__((always_inline)) {
    static_for<5>([&](auto PT) __attribute__((always_inline)) { issue_part(ST, PT, kb, q); });
  };

  int item = item_index(0);
  if (item >= n_items) return;
  Item it = item_of(item, NB, a.tiles);
  meta_dma(0, it);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  ring_barrier();
  issue(std::integral_constant<int, 0>{}, 0, src_of(0, it));

  for (int r = 0;; ++r) {
    const int e = it.e, p0 = it.p0, rows = it.rows, nb = it.nb;
    const int buf = r & 1;
    const int next = item_index(r + 1);
    const bool has_next = next < n_items;
    const Item nit = item_of(has_next ? next : item, NB, a.tiles);
    // 16-row subtiles of this wave's half that hold rows (wave-uniform)
    const int rows_h = rows - mh * 128 < 0 ? 0 : (rows - mh * 128 > 128 ? 128 : rows - mh * 128);
    const int mtw = (rows_h + 15) >> 4;

    // The first item waits here for its block 0 and slot list.  A later
    // item's block 0 (and its row scales) landed in the previous item's last
    // K step, and the previous epilogue ended with a barrier after its last
    // LDS read, so its h stores are not waited for.
    if (r == 0) {
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      ring_barrier();
    }
    const Src cur = src_of(buf, it);
    // the next item's slots and weight scales into the other buffer (they
    // land with block 1)
    if (has_next) meta_dma(buf ^ 1, nit);
    // block kb's promotion factors from row scale v into cs (waves 0-3, each
    // its own 64 rows; the same FP32 products the promotion would form)
    auto put_cs = [&](float* cs, int kb, float v) __attribute__((always_inline)) {
      const int kc = kb < nH ? kb : nH - 1;
      const int r = wave * 64 + lane;
      cs[r] = v * ws_lds[buf][2 * kc];
      cs[BM + r] = v * ws_lds[buf][2 * kc + 1];
    };
    if (wave < 4) put_cs(cs_lds0, 0, sx0_lds[wave * 64 + lane]);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    ring_barrier();

    // acc[m][t]: row 128 mh + 16 m + lane % 16, columns 4 (lane / 16) .. + 3
    // of n-tile t (gate 0-1, up 2-3): the weights are the MFMA's A operand,
    // so a lane's row needs one promotion factor per subtile, not four
    f32x4 acc[8][4];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // one K block over MT subtiles: issue block kb + 1 into the other stage
    // (read last step), multiply block kb out of stage s, wait for kb + 1,
    // then (waves 0-3) form block kb + 1's promotion factors
    // LC: the last pair of steps, whose second step (next stage 0, read in
    // the step before) loads the next item's block 0 and its row scales
    // instead of the out-of-range block past this item's last one, so that
    // block lands under this step's MFMAs rather than after the epilogue.
    auto step = [&](auto S, auto MTC, auto LC, int kb0) __attribute__((always_inline)) {
      constexpr int s = decltype(S)::value, MT = decltype(MTC)::value;
      constexpr bool kNextItem = decltype(LC)::value && s == 1;
      const int kb = kb0 + s;
      constexpr auto NEXT = std::integral_constant<int, 1 - s>{};
      const Src src = kNextItem ? src_of(buf ^ 1, nit) : cur;
      const int kn = kNextItem ? (has_next ? 0 : nH) : kb + 1;
      if constexpr (kNextItem) issue_part(NEXT, std::integral_constant<int, 4>{}, kn, src);
      float rs = 0.f;
      // without subtiles to interleave with, block kb + 1's loads go first
      if constexpr (MT == 0) {
        static_for<4>([&](auto PT) __attribute__((always_inline)) { issue_part(NEXT, PT, kn, src); });
        if (wave < 4) rs = row_scale(kb + 1, cur);
      }
      if (MT > 0 && kb < nH) {
        const uint8_t* wbuf = (s == 0 ? w_lds0 : w_lds1) + w_rd;
        const uint8_t* abuf = (s == 0 ? a_lds0 : a_lds1) + afr;
        const float* crow = (s == 0 ? cs_lds0 : cs_lds1) + mh * 128 + (lane & 15);
        i32x8 B[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) B[t] = cat(ld16(wbuf + t * 2048), ld16(wbuf + t * 2048 + 1024));
        // Subtile m: its factor reads and the next subtile's fragment reads,
        // its four MFMAs, a part of block kb + 1's loads under them, then the
        // promotion of its own products (the other wave of the SIMD
        // multiplies meanwhile).
        i32x8 A2[2];
        float CG, CU;
        f32x4 P[4];
        A2[0] = cat(ld16(abuf + afc0), ld16(abuf + afc1));
        static_for<MT>([&](auto M) __attribute__((always_inline)) {
          constexpr int m = decltype(M)::value;
          constexpr int per = MT >= 4 ? 1 : 4 / (MT > 0 ? MT : 1);  // load parts per subtile
          CG = crow[m * 16];
          CU = crow[BM + m * 16];
          if constexpr (m + 1 < MT)
            A2[(m + 1) & 1] = cat(ld16(abuf + (m + 1) * 2048 + afc0), ld16(abuf + (m + 1) * 2048 + afc1));
#pragma unroll
          for (int t = 0; t < 4; ++t) P[t] = mfma_e4m3(B[t], A2[m & 1]);
          static_for<per>([&](auto J) __attribute__((always_inline)) {
            constexpr int q = m * per + decltype(J)::value;
            if constexpr (q < 4) issue_part(NEXT, std::integral_constant<int, q>{}, kn, src);
          });
          if constexpr (m == 0) {
            if (wave < 4) rs = row_scale(kb + 1, cur);
          }
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[m][t][i] = __builtin_fmaf(P[t][i], t < 2 ? CG : CU, acc[m][t][i]);
          pin_in_place(acc[m]);
          constexpr int nl = (m * per < 4 ? 2 * per : 0) + (m == 0 ? 1 : 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // DS reads (next subtile)
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, nl, 0);  // VMEM reads
          __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // VALU
          __builtin_amdgcn_sched_barrier(0);
        });
      } else if constexpr (MT > 0) {
        static_for<4>([&](auto PT) __attribute__((always_inline)) { issue_part(NEXT, PT, kn, src); });
        if (wave < 4) rs = row_scale(kb + 1, cur);
      }
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): block kb + 1 has landed
      if (wave < 4) put_cs(s == 0 ? cs_lds1 : cs_lds0, kb + 1, rs);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the factors are in LDS
      ring_barrier();
    };
    auto kloop = [&](auto MTC) __attribute__((always_inline)) {
      static_assert(NS == 2, "the K loop is unrolled by the stage count");
      int kb0 = 0;
      for (; kb0 + NS < nH; kb0 += NS) {
        step(std::integral_constant<int, 0>{}, MTC, std::false_type{}, kb0);
        step(std::integral_constant<int, 1>{}, MTC, std::false_type{}, kb0);
      }
      step(std::integral_constant<int, 0>{}, MTC, std::true_type{}, kb0);
      step(std::integral_constant<int, 1>{}, MTC, std::true_type{}, kb0);
    };
    // every wave runs the same K loop and barriers; a half with few rows
    // multiplies fewer subtiles
    if (mtw > 4)
      kloop(std::integral_constant<int, 8>{});
    else if (mtw > 0)
      kloop(std::integral_constant<int, 4>{});
    else
      kloop(std::integral_constant<int, 0>{});

    // The epilogue's lane indices are re-derived from an opaque copy of the
    // thread id, so the compiler cannot compute epilogue addresses before the
    // K loop and keep them live (spilled) across it.
    int etid = (int)threadIdx.x;
    asm volatile("" : "+v"(etid));
    const int ecol = etid & 15, egrp = (etid >> 4) & 3;
    if constexpr (kDbg) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int row = mh * 128 + m * 16 + ecol;
        if (m < mtw && row < rows) {
          float* g = a.gu_dbg + (size_t)(p0 + row) * 2 * Ip + nb * kBlock + wn * 32 + egrp * 4;
          *reinterpret_cast<f32x4*>(g) = acc[m][0];
          *reinterpret_cast<f32x4*>(g + 16) = acc[m][1];
          *reinterpret_cast<f32x4*>(g + Ip) = acc[m][2];
          *reinterpret_cast<f32x4*>(g + Ip + 16) = acc[m][3];
        }
      }
    }
    // h = silu(g) * u in FP32, one 128-row half at a time (the half's waves
    // write it to stage 1: a_lds1 rows 0-63, w_lds1 rows 64-127, 512 bytes
    // each), then four threads per row quantise it: thread t takes 16-byte
    // chunks 8 (t % 4) .. + 7 (32 columns) of row t / 4.  Chunk c of row r sits
    // in slot c ^ (r % 32) ^ 8 (c / 16), so the 16-byte stores of one
    // instruction (16 rows, one chunk each) fill distinct banks.
    auto hslot = [](int rr, int c) __attribute__((always_inline)) { return c ^ (rr & 31) ^ ((c >> 4) << 3); };
    // h of this wave's rows in registers first (the accumulators die here)
    float hv[8][4][2];
    auto act = [&](auto CL) __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (decltype(CL)::value) {
            hv[m][i][0] = silu_mul_act(acc[m][0][i], acc[m][2][i], a.act_limit);
            hv[m][i][1] = silu_mul_act(acc[m][1][i], acc[m][3][i], a.act_limit);
          } else {
            hv[m][i][0] = silu_mul(acc[m][0][i], acc[m][2][i]);
            hv[m][i][1] = silu_mul(acc[m][1][i], acc[m][3][i]);
          }
        }
    };
    if (a.act_limit > 0.0f)
      act(std::true_type{});
    else
      act(std::false_type{});
    // (the next item's first K block is in stage 0 already; this epilogue
    // stages h in stage 1)
    for (int half = 0; half < 2 && half * 128 < rows; ++half) {
      if (mh == half) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          if (m < mtw) {
            uint8_t* hb = m < 4 ? a_lds1 : w_lds1;
            {
              const int rr = (m & 3) * 16 + ecol;
              const int c0 = wn * 8 + egrp, c1 = c0 + 4;
              *reinterpret_cast<f32x4*>(hb + rr * 512 + (hslot(rr, c0) << 4)) =
                  f32x4{hv[m][0][0], hv[m][1][0], hv[m][2][0], hv[m][3][0]};
              *reinterpret_cast<f32x4*>(hb + rr * 512 + (hslot(rr, c1) << 4)) =
                  f32x4{hv[m][0][1], hv[m][1][1], hv[m][2][1], hv[m][3][1]};
            }
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's h stores are done
      ring_barrier();
      {
        const int row = etid >> 2, qt = etid & 3, rr = row & 63;
        const uint8_t* hb = (__builtin_amdgcn_readfirstlane(etid >> 8) == 0 ? a_lds1 : w_lds1) + rr * 512;
        float v[32];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const f32x4 q = ld16f(reinterpret_cast<const float*>(hb + (hslot(rr, qt * 8 + j) << 4)));
#pragma unroll
          for (int k = 0; k < 4; ++k) v[4 * j + k] = q[k];
        }
        uint32_t mb = 0;
#pragma unroll
        for (int k = 0; k < 32; ++k) mb = umax(mb, abs_bits(v[k]));
        // the row's other three quarters: lanes 4 (row % 16) .. + 3
        mb = umax(mb, (uint32_t)__builtin_amdgcn_mov_dpp((int)mb, 0xB1, 0xF, 0xF, false));
        mb = umax(mb, (uint32_t)__builtin_amdgcn_mov_dpp((int)mb, 0x4E, 0xF, 0xF, false));
        const float amax = __uint_as_float(mb);
        const float sc = __fdiv_rn(amax, 448.0f), y = __fdiv_rn(1.0f, sc);
        uint32_t w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t lo = e4m3_pair(row_div(v[4 * k], sc, y), row_div(v[4 * k + 1], sc, y));
          const uint32_t hi = e4m3_pair(row_div(v[4 * k + 2], sc, y), row_div(v[4 * k + 3], sc, y));
          // branch-free: an all-zero row (sc = 0) takes code 0 by the select
          w[k] = amax != 0.0f ? (lo | (hi << 16)) : 0u;
        }
        if (amax != 0.0f && amax < kRowDivMin) {  // tiny rows (never seen in practice): divide
#pragma unroll
          for (int k = 0; k < 8; ++k)
            w[k] = e4m3_pair(__fdiv_rn(v[4 * k], sc), __fdiv_rn(v[4 * k + 1], sc)) |
                   (e4m3_pair(__fdiv_rn(v[4 * k + 2], sc), __fdiv_rn(v[4 * k + 3], sc)) << 16);
        }
        const int trow = half * 128 + row;
        if (trow < rows) {
          uint8_t* dst = a.hq + (size_t)(p0 + trow) * Ip + nb * kBlock + qt * 32;
          st16(dst, i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]});
          st16(dst + 16, i32x4{(int)w[4], (int)w[5], (int)w[6], (int)w[7]});
          if (qt == 0) {
            a.sh[(size_t)(p0 + trow) * NB + nb] = sc;
            a.shT[(size_t)nb * a.P + p0 + trow] = sc;
          }
        }
      }
      // the staged half has been read before the next one overwrites it
      __builtin_amdgcn_s_waitcnt(0xC07F);
      ring_barrier();
    }
    if (!has_next) break;
    item = next;
    it = nit;
  }
}
// gate_up for experts with 17..128 rows: one 128-row tile per (expert,
// 128-column block), bound by the weight stream.  Waves 0-3 multiply (one
// per SIMD, 128 rows x 32 gate + 32 up columns each) out of three LDS
// stages; waves 4-7 only move data.  Producer pair kb % 2 issues block
// kb + 2 (weights, activation rows gathered through the plan, row scales)
// into the stage read in step kb - 1, while the other pair waits for block
// kb + 1 (which it issued the step before) and forms that block's promotion
// factors in LDS, so every wait is a plain vmcnt(0) on the waiting wave's
// own loads and the matrix waves never wait on memory.  While the matrix
// waves quantise one item's h, the producers already fetch the next item's
// row list, weight scales and first K block, so the weight stream does not
// stop between items.
template <bool kDbg>
__global__ __launch_bounds__(kWideThreads, 1) void gate_up_narrow_kernel(GateUpArgs a) {
  constexpr int BM = kNarrowRows;
  // one LDS object per stage, indexed only by compile-time stage numbers
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds0[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds1[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds2[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t w_lds0[kGateUpChunk];
  __shared__ __attribute__((aligned(1024))) uint8_t w_lds1[kGateUpChunk];
  __shared__ __attribute__((aligned(1024))) uint8_t w_lds2[kGateUpChunk];
  __shared__ __attribute__((aligned(256))) float sx_lds0[BM];
  __shared__ __attribute__((aligned(256))) float sx_lds1[BM];
  __shared__ __attribute__((aligned(256))) float sx_lds2[BM];
  __shared__ float ws_lds[2 * kMaxKBlocks];
  __shared__ int tok_lds[BM];
  // promotion factors per stage: row scale x gate weight scale (rows 0-127),
  // then x up weight scale, formed by the producer pair that waited for the
  // block (the matrix waves then read two factors per row)
  __shared__ __attribute__((aligned(256))) float cs_lds0[2 * BM];
  __shared__ __attribute__((aligned(256))) float cs_lds1[2 * BM];
  __shared__ __attribute__((aligned(256))) float cs_lds2[2 * BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool mma = wave < 4;  // matrix waves (32-column group wn = wave)
  const int wn = wave & 3, pair = (wave >> 1) & 1, pw = wave & 1;
  const int ptid = tid - 256;  // producer thread index
  const int H = a.H, Ip = a.Ip, nH = H / kBlock, NB = Ip / kBlock;
  const int n_items = a.n_tiles[0] * NB;
  const rsrc_t xr = make_rsrc(a.xq, (uint32_t)a.xq_bytes);
  const rsrc_t sr = make_rsrc(a.sxT, (uint32_t)a.sxT_bytes);
  auto hslot = [](int rr, int c) __attribute__((always_inline)) { return c ^ (rr & 31) ^ ((c >> 4) << 3); };

  // an item's row list and weight scales into LDS (producer threads)
  auto load_meta = [&](const Item& it) __attribute__((always_inline)) {
    if (ptid < BM) tok_lds[ptid] = a.perm[it.p0 + (ptid < it.rows ? ptid : 0)] / a.k;
    const float* ws = a.s13 + (size_t)(it.e * NB + it.nb) * nH * 2;
    for (int i = ptid; i < 2 * nH; i += 256) ws_lds[i] = ws[i];
  };
  auto wrsrc = [&](const Item& it) __attribute__((always_inline)) {
    return make_rsrc(a.w13 + (size_t)(it.e * NB + it.nb) * nH * kGateUpChunk, (uint32_t)(nH * kGateUpChunk));
  };
  // producer pw of a pair moves the 1 KiB LDS blocks b = 2q + pw: weights
  // q = 0..15, activation rows 8b .. 8b + 7 for q = 0..7 (lane: row 8b + l/8,
  // swizzled slot l % 8), row scales 64 pw .. +63; past the last K block the
  // loads read out of range (zeros)
  auto issue = [&](auto ST, int kb, rsrc_t wr, int rows) __attribute__((always_inline)) {
    constexpr int st = decltype(ST)::value;
    uint8_t* wl = st == 0 ? w_lds0 : (st == 1 ? w_lds1 : w_lds2);
    uint8_t* al = st == 0 ? a_lds0 : (st == 1 ? a_lds1 : a_lds2);
    float* sl = st == 0 ? sx_lds0 : (st == 1 ? sx_lds1 : sx_lds2);
    const bool in = kb < nH;
    const uint32_t oob = in ? 0u : 0x80000000u;
    const uint32_t sw = in ? (uint32_t)(kb * kGateUpChunk) : 0u, sa = in ? (uint32_t)(kb * kBlock) : 0u;
    // lane offsets derived here from an opaque thread id, so that they are
    // not kept live (and spilled) across the whole item loop
    int ltid = (int)threadIdx.x;
    asm volatile("" : "+v"(ltid));
    const int lane = ltid & 63;
    // weights with the streaming kernels' cache policy (read once per pass;
    // 10% faster on the E=160 I=192 T=1024 slice than the default policy)
#pragma unroll
    for (int q = 0; q < 16; ++q)
      dma16<kWeightAux>(wr, wl + (2 * q + pw) * 1024, (uint32_t)((2 * q + pw) * 1024 + lane * 16) | oob, sw);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = (2 * q + pw) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(row);
      const uint32_t avo = (uint32_t)(tok_lds[row] * H + c * 16) | (row < rows ? 0u : 0x80000000u);
      dma16<0>(xr, al + (2 * q + pw) * 1024, avo | oob, sa);
    }
    const int srow = pw * 64 + lane;
    const uint32_t svo = (uint32_t)(tok_lds[srow] * 4) | (srow < rows ? 0u : 0x80000000u);
    dma4(sr, sl + pw * 64, svo | oob, in ? (uint32_t)(kb * a.T * 4) : 0u);
  };

  // block kb's factors of row 64 pw + lane into stage ST (producer pair that
  // waited for the block; past the last block the last weight scales)
  auto put_cs = [&](auto ST, int kb) __attribute__((always_inline)) {
    constexpr int st = decltype(ST)::value;
    const float* sl = st == 0 ? sx_lds0 : (st == 1 ? sx_lds1 : sx_lds2);
    float* cs = st == 0 ? cs_lds0 : (st == 1 ? cs_lds1 : cs_lds2);
    int ltid = (int)threadIdx.x;
    asm volatile("" : "+v"(ltid));
    const int row = pw * 64 + (ltid & 63);
    const int kc = kb < nH ? kb : nH - 1;
    const float v = sl[row];
    cs[row] = v * ws_lds[2 * kc];
    cs[BM + row] = v * ws_lds[2 * kc + 1];
  };

  int item = item_index(0);
  if (item >= n_items) return;
  Item it = item_of(item, NB, a.tiles);
  if (!mma) load_meta(it);
  __syncthreads();
  if (!mma && pair == 0) issue(std::integral_constant<int, 0>{}, 0, wrsrc(it), it.rows);

  for (int r = 0;; ++r) {
    const int e = it.e, p0 = it.p0, rows = it.rows, nb = it.nb;
    const int mt = (rows + 15) >> 4;
    const int next = item_index(r + 1);
    int etid = (int)threadIdx.x;

    // The two roles run separate loops with the same barriers: the matrix
    // waves' accumulators are not live in the producers' code, which keeps
    // both within 256 registers.
    if (mma) {
      // acc[m][t]: row 16 m + lane % 16, columns 4 (lane / 16) .. + 3 of
      // n-tile t (weights as the MFMA's A operand, as in gate_up_wide_kernel)
      f32x4 acc[8][4];
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      // block kb out of stage s, then the step barrier
      auto step = [&](auto S, auto MTC, int kb) __attribute__((always_inline)) {
        constexpr int s = decltype(S)::value, MT = decltype(MTC)::value;
        if (kb < nH) {
          // lane offsets re-derived each step from an opaque thread id:
          // cheaper than keeping them in registers across the K loop
          int ltid = (int)threadIdx.x;
          asm volatile("" : "+v"(ltid));
          const int ll = ltid & 63, lg = (ll >> 4) & 3;
          const int afc0 = ((2 * lg) ^ swz(ll)) << 4, afc1 = ((2 * lg + 1) ^ swz(ll)) << 4;
          const uint8_t* wbuf = (s == 0 ? w_lds0 : (s == 1 ? w_lds1 : w_lds2)) + wn * 8192 + ll * 16;
          const uint8_t* abuf = (s == 0 ? a_lds0 : (s == 1 ? a_lds1 : a_lds2)) + (ll & 15) * 128;
          const float* crow = (s == 0 ? cs_lds0 : (s == 1 ? cs_lds1 : cs_lds2)) + (ll & 15);
          i32x8 B[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) B[t] = cat(ld16(wbuf + t * 2048), ld16(wbuf + t * 2048 + 1024));
          // software pipeline over the subtiles: subtile m's MFMAs run while
          // the VALU promotes subtile m - 1 (the matrix wave is alone on its
          // SIMD, so nothing else would fill the MFMA pipe meanwhile)
          i32x8 A2[2];
          f32x4 P[2][4];
          A2[0] = cat(ld16(abuf + afc0), ld16(abuf + afc1));
          float G3[3], U3[3];
          G3[0] = crow[0];
          U3[0] = crow[BM];
          auto promote = [&](auto J) __attribute__((always_inline)) {
            constexpr int j = decltype(J)::value;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float cg = G3[j % 3], cu = U3[j % 3];
              acc[j][0][i] = __builtin_fmaf(P[j & 1][0][i], cg, acc[j][0][i]);
              acc[j][1][i] = __builtin_fmaf(P[j & 1][1][i], cg, acc[j][1][i]);
              acc[j][2][i] = __builtin_fmaf(P[j & 1][2][i], cu, acc[j][2][i]);
              acc[j][3][i] = __builtin_fmaf(P[j & 1][3][i], cu, acc[j][3][i]);
            }
            pin_in_place(acc[j]);
          };
          static_for<MT>([&](auto M) __attribute__((always_inline)) {
            constexpr int m = decltype(M)::value;
            if constexpr (m + 1 < MT) {
              A2[(m + 1) & 1] = cat(ld16(abuf + (m + 1) * 2048 + afc0), ld16(abuf + (m + 1) * 2048 + afc1));
              G3[(m + 1) % 3] = crow[(m + 1) * 16];
              U3[(m + 1) % 3] = crow[BM + (m + 1) * 16];
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) P[m & 1][t] = mfma_e4m3(B[t], A2[m & 1]);
            if constexpr (m > 0) promote(std::integral_constant<int, m - 1>{});
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS reads (next subtile)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
              __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
            }
            __builtin_amdgcn_sched_barrier(0);
          });
          promote(std::integral_constant<int, MT - 1>{});
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this step's LDS reads are done
        ring_barrier();
      };
      auto kloop = [&](auto MTC) __attribute__((always_inline)) {
        for (int kb0 = 0; kb0 < nH; kb0 += 3) {
          step(std::integral_constant<int, 0>{}, MTC, kb0);
          step(std::integral_constant<int, 1>{}, MTC, kb0 + 1);
          step(std::integral_constant<int, 2>{}, MTC, kb0 + 2);
        }
      };
      ring_barrier();  // block 0 has landed
      if (mt > 4)
        kloop(std::integral_constant<int, 8>{});
      else
        kloop(std::integral_constant<int, 4>{});
      ring_barrier();  // the producers' last loads have landed

      // epilogue: h in FP32 staged in w_lds1 (rows 0-63) and w_lds2 (rows
      // 64-127; stage 0 takes the next item's first block meanwhile), then
      // two matrix threads per row quantise it (16-byte chunk c of row r in
      // slot c ^ (r % 32) ^ 8 (c / 16), as in gate_up_wide_kernel)
      asm volatile("" : "+v"(etid));
      const int ecol = etid & 15, egrp = (etid >> 4) & 3;
      if constexpr (kDbg) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int row = m * 16 + ecol;
          if (m < mt && row < rows) {
            float* g = a.gu_dbg + (size_t)(p0 + row) * 2 * Ip + nb * kBlock + wn * 32 + egrp * 4;
            *reinterpret_cast<f32x4*>(g) = acc[m][0];
            *reinterpret_cast<f32x4*>(g + 16) = acc[m][1];
            *reinterpret_cast<f32x4*>(g + Ip) = acc[m][2];
            *reinterpret_cast<f32x4*>(g + Ip + 16) = acc[m][3];
          }
        }
      }
      auto act = [&](auto CL) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          if (m < mt) {
            uint8_t* hb = m < 4 ? w_lds1 : w_lds2;
            f32x4 h0, h1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if constexpr (decltype(CL)::value) {
                h0[i] = silu_mul_act(acc[m][0][i], acc[m][2][i], a.act_limit);
                h1[i] = silu_mul_act(acc[m][1][i], acc[m][3][i], a.act_limit);
              } else {
                h0[i] = silu_mul(acc[m][0][i], acc[m][2][i]);
                h1[i] = silu_mul(acc[m][1][i], acc[m][3][i]);
              }
            }
            // row (m % 4) 16 + lane % 16, columns 32 wn + 4 (lane / 16) .. + 3
            // (chunk c0) and 16 further (chunk c1)
            const int rr = (m & 3) * 16 + ecol;
            const int c0 = wn * 8 + egrp, c1 = c0 + 4;
            *reinterpret_cast<f32x4*>(hb + rr * 512 + (hslot(rr, c0) << 4)) = h0;
            *reinterpret_cast<f32x4*>(hb + rr * 512 + (hslot(rr, c1) << 4)) = h1;
          }
        }
      };
      if (a.act_limit > 0.0f)
        act(std::true_type{});
      else
        act(std::false_type{});
      __syncthreads();  // h staged
      {
        const int row = etid >> 1, half = etid & 1, rr = row & 63;
        const uint8_t* hb = (row < 64 ? w_lds1 : w_lds2) + rr * 512;
        float v[64];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const f32x4 q = ld16f(reinterpret_cast<const float*>(hb + (hslot(rr, half * 16 + j) << 4)));
#pragma unroll
          for (int k = 0; k < 4; ++k) v[4 * j + k] = q[k];
        }
        uint32_t mb = 0;
#pragma unroll
        for (int k = 0; k < 64; ++k) mb = umax(mb, abs_bits(v[k]));
        mb = umax(mb, (uint32_t)__builtin_amdgcn_mov_dpp((int)mb, 0xB1, 0xF, 0xF, false));  // the other half
        const float amax = __uint_as_float(mb);
        const float sc = __fdiv_rn(amax, 448.0f), y = __fdiv_rn(1.0f, sc);
        uint32_t w[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const uint32_t lo = e4m3_pair(row_div(v[4 * k], sc, y), row_div(v[4 * k + 1], sc, y));
          const uint32_t hi = e4m3_pair(row_div(v[4 * k + 2], sc, y), row_div(v[4 * k + 3], sc, y));
          // branch-free: an all-zero row (sc = 0) takes code 0 by the select
          w[k] = amax != 0.0f ? (lo | (hi << 16)) : 0u;
        }
        if (amax != 0.0f && amax < kRowDivMin) {  // tiny rows (never seen in practice): divide
#pragma unroll
          for (int k = 0; k < 16; ++k)
            w[k] = e4m3_pair(__fdiv_rn(v[4 * k], sc), __fdiv_rn(v[4 * k + 1], sc)) |
                   (e4m3_pair(__fdiv_rn(v[4 * k + 2], sc), __fdiv_rn(v[4 * k + 3], sc)) << 16);
        }
        if (row < rows) {
          uint8_t* dst = a.hq + (size_t)(p0 + row) * Ip + nb * kBlock + half * 64;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            st16(dst + q * 16, i32x4{(int)w[4 * q], (int)w[4 * q + 1], (int)w[4 * q + 2], (int)w[4 * q + 3]});
          if (half == 0) {
            a.sh[(size_t)(p0 + row) * NB + nb] = sc;
            a.shT[(size_t)nb * a.P + p0 + row] = sc;
          }
        }
      }
      __syncthreads();  // h read: stages 1-2 are free for the next item
    } else {
      // producers: pair kb % 2 loads block kb + 2 into the stage read last
      // step while the other pair waits for block kb + 1
      const rsrc_t wr = wrsrc(it);
      auto pstep = [&](auto S, int kb) __attribute__((always_inline)) {
        constexpr int s = decltype(S)::value;
        if (pair == (kb & 1)) {
          issue(std::integral_constant<int, (s + 2) % 3>{}, kb + 2, wr, rows);
        } else {
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): block kb + 1 has landed
          put_cs(std::integral_constant<int, (s + 1) % 3>{}, kb + 1);
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        }
        ring_barrier();
      };
      if (pair == 1) {
        issue(std::integral_constant<int, 1>{}, 1, wr, rows);
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): block 0 has landed
        put_cs(std::integral_constant<int, 0>{}, 0);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      }
      ring_barrier();
      for (int kb0 = 0; kb0 < nH; kb0 += 3) {
        pstep(std::integral_constant<int, 0>{}, kb0);
        pstep(std::integral_constant<int, 1>{}, kb0 + 1);
        pstep(std::integral_constant<int, 2>{}, kb0 + 2);
      }
      // the out-of-range loads issued past the last block still write zeros
      // to their stages: let them land before the stages are reused
      __builtin_amdgcn_s_waitcnt(0x0F70);
      ring_barrier();
      // the next item's row list and scales (this item's are no longer read)
      if (next < n_items) load_meta(item_of(next, NB, a.tiles));
      __syncthreads();  // h staged; the next item's row list is in LDS
      if (next < n_items && pair == 0) {
        const Item nit = item_of(next, NB, a.tiles);
        issue(std::integral_constant<int, 0>{}, 0, wrsrc(nit), nit.rows);
      }
      __syncthreads();
    }
    if (next >= n_items) break;
    item = next;
    it = item_of(item, NB, a.tiles);
  }
}

hipError_t launch_gate_up(const GateUpArgs& a, int kind, int grid, hipStream_t s) {
  if (kind == kGemmWide && a.gu_dbg)
    hipLaunchKernelGGL(gate_up_wide_kernel<true>, dim3(grid), dim3(kWideThreads), 0, s, a);
  else if (kind == kGemmWide)
    hipLaunchKernelGGL(gate_up_wide_kernel<false>, dim3(grid), dim3(kWideThreads), 0, s, a);
  else if (kind == kGemmNarrow && a.gu_dbg)
    hipLaunchKernelGGL(gate_up_narrow_kernel<true>, dim3(grid), dim3(kWideThreads), 0, s, a);
  else if (kind == kGemmNarrow)
    hipLaunchKernelGGL(gate_up_narrow_kernel<false>, dim3(grid), dim3(kWideThreads), 0, s, a);
  else
    hipLaunchKernelGGL(gate_up_stream_kernel<kStreamDepth>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// -------------------------------------------------------------------- down --
__device__ __forceinline__ int pick3(int i, int v0, int v1, int v2) { return i == 0 ? v0 : (i == 1 ? v1 : v2); }

// Descriptor of the j-th item (b + j * G) of a streaming workgroup, j clamped
// to its last item: weight block index e * NB + nb, first row, rows (uniform).
__device__ __forceinline__ void stream_item(const Tile* tiles, int b, int j, int my_items, int G, int NB, int& wblk,
                                            int& p0, int& rows) {
  const int i = b + (j < my_items ? j : my_items - 1) * G;
  const int t = i / NB;
  wblk = __builtin_amdgcn_readfirstlane(tiles[t].e * NB + (i - t * NB));
  p0 = __builtin_amdgcn_readfirstlane(tiles[t].p0);
  rows = __builtin_amdgcn_readfirstlane(tiles[t].rows);
}

// Streaming down for experts with at most 16 rows (the HBM-bound regime).
// The items (tile, 128-column block) of a workgroup form one flat sequence
// of K steps, and each wave's loads run D - 1 steps ahead of its MFMAs
// across item boundaries, so a workgroup's weight stream does not drain
// between items (an item is only Ip / 128 steps long).  No LDS and no
// barrier: every wave loads its activation fragment, its two weight
// fragments, the scales of its four rows (from the K-block-major copy) and
// the step's weight scale straight into registers.  Same MFMA, promotion
// order and arithmetic as down_wide_kernel.
//
// The MFMA side finishes an item at most two items behind the load side
// when D <= 2 Ip / 128, so the load side keeps the last three items' row
// ranges for the output stores.
template <int D>
__global__ __launch_bounds__(kThreads, kDownWgPerCu) void down_stream_kernel(DownArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int H = a.H, Ip = a.Ip, nI = Ip / kBlock, NB = H / kBlock;
  const int n_items = a.n_tiles[0] * NB;
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  if (b >= n_items) return;
  const int my_items = (n_items - 1 - b) / G + 1;
  const int S = my_items * nI;  // K steps of this workgroup
  const rsrc_t hr = make_rsrc(a.hq, (uint32_t)a.hq_bytes);
  const rsrc_t shr = make_rsrc(a.shT, (uint32_t)a.shT_bytes);
  const uint32_t bvoff = (uint32_t)(wave * 4096 + lane * 16);

  // load side: step gl = item jl, block kbl.  Item descriptors (weight block
  // e * NB + nb, first row p0, rows): c = current, n = next (prefetched),
  // 1 and 2 = the two before c (for the MFMA side's stores)
  int gl = 0, jl = 0, kbl = 0;
  int c_w, c_p0, c_rows, n_w, n_p0, n_rows, w1 = 0, p1 = 0, r1 = 0, w2 = 0, p2 = 0, r2 = 0;
  stream_item(a.tiles, b, 0, my_items, G, NB, c_w, c_p0, c_rows);
  stream_item(a.tiles, b, 1, my_items, G, NB, n_w, n_p0, n_rows);
  uint32_t avo = (uint32_t)((c_p0 + (col < c_rows ? col : 0)) * Ip + grp * 32);
  uint32_t sho = (uint32_t)((c_p0 + grp * 4) * 4);

  i32x8 A[D], B[D][2];
  f32x4 R[D];
  float W[D];
  // the buffer resources are rebuilt per load from the uniform block index
  // (a resource carried around the loop would be kept in VGPRs)
  auto load = [&](auto SL) __attribute__((always_inline)) {
    constexpr int s = decltype(SL)::value;
    const bool in = gl < S;
    const uint32_t oob = in ? 0u : 0x80000000u;
    const uint32_t sa = in ? (uint32_t)(kbl * kBlock) : 0u, so = in ? (uint32_t)(kbl * kDownChunk) : 0u;
    const rsrc_t wr = make_rsrc(a.w2 + (size_t)c_w * nI * kDownChunk, (uint32_t)(nI * kDownChunk));
    const rsrc_t sr = make_rsrc(a.s2 + (size_t)c_w * nI, (uint32_t)(nI * 4));
    A[s] = cat(bload16(hr, avo + oob, sa), bload16(hr, avo + oob, sa + 16));
#pragma unroll
    for (int t = 0; t < 2; ++t)
      B[s][t] = cat(wload16(wr, bvoff + oob, so + t * 2048), wload16(wr, bvoff + oob, so + t * 2048 + 1024));
    const uint32_t ss = in ? (uint32_t)(kbl * a.P * 4) : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) R[s][i] = bloadf(shr, (sho + 4 * i) + oob, ss);
    W[s] = bloadf(sr, oob, in ? (uint32_t)(kbl * 4) : 0u);
    // advance the load side
    ++gl;
    if (++kbl == nI && gl < S) {
      kbl = 0;
      ++jl;
      w2 = w1, p2 = p1, r2 = r1;
      w1 = c_w, p1 = c_p0, r1 = c_rows;
      c_w = n_w, c_p0 = n_p0, c_rows = n_rows;
      stream_item(a.tiles, b, jl + 1, my_items, G, NB, n_w, n_p0, n_rows);
      avo = (uint32_t)((c_p0 + (col < c_rows ? col : 0)) * Ip + grp * 32);
      sho = (uint32_t)((c_p0 + grp * 4) * 4);
    }
  };

  // MFMA side: item jc, block kbc
  int jc = 0, kbc = 0;
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  auto compute = [&](auto SL) __attribute__((always_inline)) {
    constexpr int s = decltype(SL)::value;
    const f32x4 q0 = mfma_e4m3(A[s], B[s][0]);
    const f32x4 q1 = mfma_e4m3(A[s], B[s][1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sc = R[s][i] * W[s];
      acc[0][i] = __builtin_fmaf(q0[i], sc, acc[0][i]);
      acc[1][i] = __builtin_fmaf(q1[i], sc, acc[1][i]);
    }
    if (++kbc == nI) {
      const int lag = jl - jc;  // 0, 1 or 2
      // (selects of values: a select of the variables' addresses would keep
      // them all in scratch memory)
      const int wb = pick3(lag, c_w, w1, w2);
      const int p0 = pick3(lag, c_p0, p1, p2);
      const int rows = pick3(lag, c_rows, r1, r2);
      const int nb = wb % NB;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = grp * 4 + i;
        if (r < rows) {
          float* dst = a.y + (size_t)(p0 + r) * H + nb * kBlock + wave * 32 + col;
          dst[0] = acc[0][i];
          dst[16] = acc[1][i];
        }
        acc[0][i] = 0.f;
        acc[1][i] = 0.f;
      }
      kbc = 0;
      ++jc;
    }
  };

  static_for<D - 1>([&](auto SL) __attribute__((always_inline)) { load(SL); });
  for (int g0 = 0; g0 < S; g0 += D) {
    static_for<D>([&](auto SL) __attribute__((always_inline)) {
      constexpr int s = decltype(SL)::value;
      load(std::integral_constant<int, (s + D - 1) % D>{});
      if (g0 + s < S) compute(SL);
    });
  }
}

// down for experts with more than kSmallRows rows (the 128-row and the
// 256-row tile lists, in one launch): a 512-thread workgroup computes up to
// 256 rows x 256 hidden columns (weight blocks nb2, nb2 + 1),
// both operands double-buffered in LDS by buffer-load-to-LDS as in
// gate_up_wide_kernel.  Wave w = 4 mh + wn owns rows 128 mh .. +127 and 64
// columns: block nb2 + wn / 2, 32-column groups 2 (wn % 2) and 2 (wn % 2) + 1.
__global__ __launch_bounds__(kWideThreads, 1) void down_wide_kernel(DownArgs a) {
  constexpr int BM = kWideRows;
  constexpr int NS = 2;
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds0[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds1[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t w_lds0[2 * kDownChunk];
  __shared__ __attribute__((aligned(1024))) uint8_t w_lds1[2 * kDownChunk];
  __shared__ __attribute__((aligned(256))) float s_lds0[2 * BM];
  __shared__ __attribute__((aligned(256))) float s_lds1[2 * BM];
  // weight scales of blocks nb2 and nb2 + 1, for the current item and the next
  __shared__ __attribute__((aligned(256))) float ws_lds[2][2][kMaxKBlocks];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mh = wave >> 2, wn = wave & 3, half = wn >> 1;
  const int col = lane & 15, grp = lane >> 4;
  const int H = a.H, Ip = a.Ip, nI = Ip / kBlock, NB = H / kBlock;
  const int NB2 = (NB + 1) >> 1;
  // items of the first list, then those of the second (one launch covers
  // the 128-row and the 256-row tiles, so only one launch ends with a tail)
  const int n_first = a.n_tiles[0] * NB2;
  const int n_items = n_first + (a.tiles2 != nullptr ? a.n_tiles[1] * NB2 : 0);
  auto item_at = [&](int i) __attribute__((always_inline)) {
    return i < n_first ? item_of(i, NB2, a.tiles) : item_of(i - n_first, NB2, a.tiles2);
  };
  const rsrc_t hr = make_rsrc(a.hq, (uint32_t)a.hq_bytes);
  const rsrc_t sr = make_rsrc(a.shT, (uint32_t)a.shT_bytes);
  // the wave's 8 KiB of the stage: block wn / 2, groups 2 (wn % 2), +1
  const int w_rd = wn * 8192 + lane * 16;
  const int afr = (mh * 128 + (lane & 15)) * 128;
  const int afc0 = ((2 * grp) ^ swz(lane)) << 4, afc1 = ((2 * grp + 1) ^ swz(lane)) << 4;

  // An item's weight scales straight into LDS buffer buf: waves 0-1 block
  // nb2, waves 2-3 block nb2 + 1 (out of range when it is missing or past nI)
  auto ws_dma = [&](int buf, const Item& it) __attribute__((always_inline)) {
    if (wave < 4) {
      const int nb2 = it.nb * 2, hb = wave >> 1, i = (wave & 1) * 64 + lane;
      const bool ok = i < nI && nb2 + hb < NB;
      const rsrc_t wsr = make_rsrc(a.s2 + (size_t)(it.e * NB + nb2) * nI, (uint32_t)(2 * nI * 4));
      dma4(wsr, &ws_lds[buf][hb][(wave & 1) * 64], (uint32_t)((hb * nI + i) * 4) | (ok ? 0u : 0x80000000u), 0u);
    }
  };
  // DMA sources of an item: LDS block b = 8q + w (1 KiB) of instruction q
  // of wave w; blocks nb2 and nb2 + 1 are nI * kDownChunk bytes apart and a
  // missing second block reads out of range
  struct Src {
    rsrc_t wr;
    uint32_t wvo[4], avo[4], svo;
    int g8;  // 8-row groups of the tile that hold rows
  };
  auto src_of = [&](const Item& it) __attribute__((always_inline)) {
    Src q;
    const int nb2 = it.nb * 2;
    const bool two = nb2 + 1 < NB;
    const int wblk = __builtin_amdgcn_readfirstlane(it.e * NB + nb2);
    const int wbytes = __builtin_amdgcn_readfirstlane((two ? 2 : 1) * nI * kDownChunk);
    q.wr = make_rsrc(a.w2 + (size_t)wblk * nI * kDownChunk, (uint32_t)wbytes);
    q.g8 = (it.rows + 7) >> 3;
    // lane terms from an opaque thread id: not shared with (and kept live
    // from) the other call
    int ltid = (int)threadIdx.x;
    asm volatile("" : "+v"(ltid));
    const int ln = ltid & 63;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = j * 8 + wave;
      q.wvo[j] = (uint32_t)((b >> 4) * nI * kDownChunk + (b & 15) * 1024 + ln * 16);
      const int row = b * 8 + (ln >> 3);
      const int c = (ln & 7) ^ swz(row);
      q.avo[j] = (uint32_t)((it.p0 + (row < it.rows ? row : 0)) * Ip + c * 16) | (row < it.rows ? 0u : 0x80000000u);
    }
    const int srow = (wave & 3) * 64 + ln;
    q.svo = (uint32_t)((it.p0 + (srow < it.rows ? srow : 0)) * 4) | (srow < it.rows && wave < 4 ? 0u : 0x80000000u);
    return q;
  };
  // loads of K block kb in parts, as in gate_up_wide_kernel
  auto issue_part = [&](auto ST, auto PT, int kb, const Src& q) __attribute__((always_inline)) {
    constexpr int st = decltype(ST)::value, p = decltype(PT)::value;
    const bool in = kb < nI;
    const uint32_t oob = in ? 0u : 0x80000000u;
    if constexpr (p < 2) {
      uint8_t* wl = st == 0 ? w_lds0 : w_lds1;
      const uint32_t sw = in ? (uint32_t)(kb * kDownChunk) : 0u;
#pragma unroll
      for (int j = 2 * p; j < 2 * p + 2; ++j) dma16<0>(q.wr, wl + (j * 8 + wave) * 1024, q.wvo[j] | oob, sw);
    } else if constexpr (p < 4) {
      uint8_t* al = st == 0 ? a_lds0 : a_lds1;
      const uint32_t sa = in ? (uint32_t)(kb * kBlock) : 0u;
#pragma unroll
      // no DMA for 8-row groups past the tile's rows: those LDS rows keep
      // stale bytes, which reach only output rows that are never stored (a
      // row of the product depends on its own activation row alone); 2-5%
      // faster where tiles are half full (T = 4096, E=160 T=1024)
      for (int j = 2 * (p - 2); j < 2 * (p - 2) + 2; ++j)
        if (j * 8 + wave < q.g8) dma16<0>(hr, al + (j * 8 + wave) * 1024, q.avo[j] | oob, sa);
    } else {
      float* sl = st == 0 ? s_lds0 : s_lds1;
      dma4(sr, sl + wave * 64, q.svo | oob, in ? (uint32_t)(kb * a.P * 4) : 0u);
    }
  };
  auto issue = [&](auto ST, int kb, const Src& q) __attribute__((always_inline)) {
    static_for<5>([&](auto PT) __attribute__((always_inline)) { issue_part(ST, PT, kb, q); });
  };

  const MixedItems mix(n_first, n_items - n_first);
  int q = 0;
  int item = mix.next(q);
  if (item >= n_items) return;
  Item it = item_at(item);
  ws_dma(0, it);
  issue(std::integral_constant<int, 0>{}, 0, src_of(it));

  for (int r = 0;; ++r) {
    const int buf = r & 1;
    const int next = mix.next(q);
    const bool has_next = next < n_items;
    const Item nit = item_at(has_next ? next : item);
    const int nb2 = it.nb * 2;
    const bool two = nb2 + 1 < NB;  // second weight block present
    const int p0 = it.p0, rows = it.rows;
    const int rows_h = rows - mh * 128 < 0 ? 0 : (rows - mh * 128 > 128 ? 128 : rows - mh * 128);
    const int mtw = (half == 1 && !two) ? 0 : (rows_h + 15) >> 4;

    // The first item waits here for its block 0 and weight scales; a later
    // item's block 0 landed in the previous item's last step, its weight
    // scales in that item's first step, and every wave passed that last
    // step's barrier after its final LDS read.  So the previous item's y
    // stores are not waited for: they drain under step 0, whose closing
    // vmcnt(0) covers them (stores and loads complete in issue order).
    if (r == 0) {
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      ring_barrier();
    }
    const Src cur = src_of(it);
    // the next item's weight scales into the other buffer (they land with block 1)
    if (has_next) ws_dma(buf ^ 1, nit);

    // acc[m][t]: row 128 mh + 16 m + lane % 16, columns 4 (lane / 16) .. + 3
    // of n-tile t, so each lane stores 16 contiguous bytes of y per n-tile
    f32x4 acc[8][4];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LC: the last pair of steps.  Its second step (whose next stage is
    // stage 0, read in the step before) loads the next item's block 0
    // instead of the out-of-range block past this item's last one, so that
    // block lands under this step's MFMAs rather than after the y stores.
    auto step = [&](auto S, auto MTC, auto LC, int kb0) __attribute__((always_inline)) {
      constexpr int s = decltype(S)::value, MT = decltype(MTC)::value;
      constexpr bool kNextItem = decltype(LC)::value && s == 1;
      const int kb = kb0 + s;
      constexpr auto NEXT = std::integral_constant<int, 1 - s>{};
      const Src src = kNextItem ? src_of(nit) : cur;
      const int kn = kNextItem ? (has_next ? 0 : nI) : kb + 1;
      if constexpr (MT == 0) issue(NEXT, kn, src);
      if (MT > 0 && kb < nI) {
        const float wsc = ws_lds[buf][half][kb];
        const uint8_t* wbuf = (s == 0 ? w_lds0 : w_lds1) + w_rd;
        const uint8_t* abuf = (s == 0 ? a_lds0 : a_lds1) + afr;
        const float* srw = (s == 0 ? s_lds0 : s_lds1) + mh * 128 + (lane & 15);
        i32x8 B[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) B[t] = cat(ld16(wbuf + t * 2048), ld16(wbuf + t * 2048 + 1024));
        // subtile by subtile as in gate_up_wide_kernel
        i32x8 A2[2];
        float R2[2];
        f32x4 Q[4];
        A2[0] = cat(ld16(abuf + afc0), ld16(abuf + afc1));
        R2[0] = srw[0];
        static_for<MT>([&](auto M) __attribute__((always_inline)) {
          constexpr int m = decltype(M)::value;
          constexpr int per = MT >= 4 ? 1 : 4 / (MT > 0 ? MT : 1);
          if constexpr (m + 1 < MT) {
            A2[(m + 1) & 1] = cat(ld16(abuf + (m + 1) * 2048 + afc0), ld16(abuf + (m + 1) * 2048 + afc1));
            R2[(m + 1) & 1] = srw[(m + 1) * 16];
          }
          // weights as the A operand: lane l gets row l % 16 of the subtile
          // and columns 4 (l / 16) .. + 3 of n-tile t
#pragma unroll
          for (int t = 0; t < 4; ++t) Q[t] = mfma_e4m3(B[t], A2[m & 1]);
          static_for<per>([&](auto J) __attribute__((always_inline)) {
            constexpr int qp = m * per + decltype(J)::value;
            if constexpr (qp < 4) issue_part(NEXT, std::integral_constant<int, qp>{}, kn, src);
          });
          if constexpr (m == 0) issue_part(NEXT, std::integral_constant<int, 4>{}, kn, src);
          const float sc = R2[m & 1] * wsc;
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][t][i] = __builtin_fmaf(Q[t][i], sc, acc[m][t][i]);
          pin_in_place(acc[m]);
          constexpr int nl = (m * per < 4 ? 2 * per : 0) + (m == 0 ? 1 : 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // DS reads (next subtile)
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, nl, 0);  // VMEM reads
          __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);  // VALU
          __builtin_amdgcn_sched_barrier(0);
        });
      } else if constexpr (MT > 0) {
        issue(NEXT, kn, src);
      }
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): block kn has landed
      ring_barrier();
    };
    auto kloop = [&](auto MTC) __attribute__((always_inline)) {
      static_assert(NS == 2, "the K loop is unrolled by the stage count");
      int kb0 = 0;
      for (; kb0 + NS < nI; kb0 += NS) {
        step(std::integral_constant<int, 0>{}, MTC, std::false_type{}, kb0);
        step(std::integral_constant<int, 1>{}, MTC, std::false_type{}, kb0);
      }
      step(std::integral_constant<int, 0>{}, MTC, std::true_type{}, kb0);
      step(std::integral_constant<int, 1>{}, MTC, std::true_type{}, kb0);
    };
    if (mtw > 4)
      kloop(std::integral_constant<int, 8>{});
    else if (mtw > 0)
      kloop(std::integral_constant<int, 4>{});
    else
      kloop(std::integral_constant<int, 0>{});

    int etid = (int)threadIdx.x;
    asm volatile("" : "+v"(etid));
    const int ecol = etid & 15, egrp = (etid >> 4) & 3;
    // y leaves through this wave's own four 1 KiB blocks of stage 1 (those
    // its DMA fills next), 16 rows at a time, alternating between the a and
    // the w blocks so one subtile's LDS writes need not wait for the previous
    // one's reads: lane (r, g) writes chunks 4 t + g of row r, then reads back
    // 4 rows x 16 chunks, so each store writes four whole 256-byte row
    // segments (16-byte stores straight from the MFMA layout cover 16 rows x
    // 64 bytes each and measured 4-6% slower for the whole kernel).  Chunk c
    // of row r sits in slot c ^ r; row r is at (r / 4) x 8 KiB + (r % 4) x
    // 256.  The stores go through a buffer descriptor of this item's rows, so
    // stores to rows past the tile fall outside it and are dropped (no branch
    // per store), with the non-temporal policy: the combine that reads y runs
    // 3-19% faster when no dirty y lines are left in the caches to be written
    // back under it.
    const rsrc_t yr = make_rsrc(a.y + (size_t)p0 * H, (uint32_t)(rows * H * 4));
    const uint32_t ycol = (uint32_t)((nb2 + half) * kBlock + (wn & 1) * 64 + ecol * 4) * 4u;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m < mtw) {
        uint8_t* yst = ((m & 1) ? w_lds1 : a_lds1) + wave * 1024;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          *reinterpret_cast<f32x4*>(yst + (ecol >> 2) * 8192 + (ecol & 3) * 256 + (((4 * t + egrp) ^ ecol) << 4)) =
              acc[m][t];
        f32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          v[j] = *reinterpret_cast<const f32x4*>(yst + j * 8192 + egrp * 256 + ((ecol ^ (4 * j + egrp)) << 4));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t row = (uint32_t)(mh * 128 + m * 16 + 4 * j + egrp);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v[j]), yr, row * (uint32_t)H * 4u + ycol, 0,
                                                 kWeightAux);
        }
      }
    }
    if (!has_next) break;
    item = next;
    it = nit;
  }
}

hipError_t launch_down(const DownArgs& a, int kind, int grid, hipStream_t s) {
  if (kind == kGemmWide || kind == kGemmNarrow)
    hipLaunchKernelGGL(down_wide_kernel, dim3(grid), dim3(kWideThreads), 0, s, a);
  // the loads may run at most 2 Ip / 128 - 1 steps ahead
  else if (2 * (a.Ip / kBlock) >= kStreamDepthDown)
    hipLaunchKernelGGL(down_stream_kernel<kStreamDepthDown>, dim3(grid), dim3(kThreads), 0, s, a);
  else if (a.Ip >= 2 * kBlock)
    hipLaunchKernelGGL(down_stream_kernel<(kStreamDepthDown < 4 ? kStreamDepthDown : 4)>, dim3(grid), dim3(kThreads), 0, s,
                       a);
  else
    hipLaunchKernelGGL(down_stream_kernel<2>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------- W8A16 decode path --
// The pages' path for decode and short continuations keeps the activations
// 16-bit ("ktransformers #2244", Design): x enters gate_up as BF16 and h
// enters down as BF16 (rounded to nearest even from FP32), against the same
// E4M3 weights and 128x128 block scales.  The products run on the BF16
// MFMA (16x16x32): a lane's 32-byte FP8 weight fragment (K 32g .. 32g + 31
// of the 16x16x128 layout, g = lane / 16) is converted exactly to BF16 eight
// codes at a time, and the four MFMAs of a 128-wide K block each take K
// 32g + 8j .. + 7 from every lane (j = 0..3), so the activation fragment is
// the matching 16 bytes of the row, read straight from memory and no weight
// byte crosses lanes.  Per K block: p = sum over the four MFMAs, then
// acc = fma(p, weight block scale, acc) in ascending K-block order.  Every
// tile of the plan's three lists is taken 16 rows at a time by 4-wave
// workgroups (weights streamed into registers D blocks deep, as in the
// streaming W8A8 kernels), so a row's bits do not depend on its neighbours.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// FP8 bytes 0..7 of (lo, hi) as BF16 (exact: E4M3 values fit BF16)
__device__ __forceinline__ bf16x8 fp8x8_bf16(int lo, int hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One 128-wide K block of a 16x16 output tile: activation fragments A[j]
// (8 BF16 each) against the lane's FP8 weight fragment.
__device__ __forceinline__ f32x4 mfma_a16_block(const i32x4 (&A)[4], const i32x8& B) {
  f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[j]), fp8x8_bf16(B[2 * j], B[2 * j + 1]),
                                                p, 0, 0, 0);
  return p;
}

// Tile ti of the three lists taken in order (small, narrow, wide).
__device__ __forceinline__ const Tile* a16_tile(const Tile* const (&lists)[3], int n0, int n1, int ti) {
  return ti < n0 ? lists[0] + ti : (ti < n0 + n1 ? lists[1] + (ti - n0) : lists[2] + (ti - n0 - n1));
}

// gate_up: item (tile, 128-column block nb); wave w owns n-tiles g0, g1, u0,
// u1 of 32-column group w (as gate_up_stream_kernel).
template <int D>
__global__ __launch_bounds__(kThreads, kDecodeWgPerCu) void gate_up_a16_kernel(GateUpA16Args a) {
  __shared__ float ws_lds[2 * kMaxKBlocks];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int H = a.H, Ip = a.Ip, nH = H / kBlock, NB = Ip / kBlock;
  const int n0 = a.n_tiles[0], n1 = a.n_tiles[1], n2 = a.n_tiles[2];
  const int n_items = (n0 + n1 + n2) * NB;
  const rsrc_t xr = make_rsrc(a.x, (uint32_t)a.x_bytes);
  const uint32_t bvoff = (uint32_t)(wave * 8192 + lane * 16);

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int ti = item / NB, nb = item - ti * NB;
    const Tile* tp = a16_tile(a.tiles, n0, n1, ti);
    const int e = __builtin_amdgcn_readfirstlane(tp->e), p0 = __builtin_amdgcn_readfirstlane(tp->p0);
    const int rows = __builtin_amdgcn_readfirstlane(tp->rows);
    __syncthreads();  // the previous item's scales are no longer read
    {
      const float* ws = a.s13 + (size_t)(e * NB + nb) * nH * 2;
      for (int i = tid; i < 2 * nH; i += kThreads) ws_lds[i] = ws[i];
    }
    __syncthreads();
    const rsrc_t wr = make_rsrc(a.w13 + (size_t)(e * NB + nb) * nH * kGateUpChunk, (uint32_t)(nH * kGateUpChunk));

    for (int c0 = 0; c0 < rows; c0 += 16) {
      const int r = c0 + col;
      const int tok = a.perm[p0 + (r < rows ? r : c0)] / a.k;
      const uint32_t avo = (uint32_t)(tok * H * 2 + grp * 64);
      f32x4 acc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      i32x4 A[D][4];
      i32x8 B[D][4];
      // block kb's operands; kb >= nH reads out of range (zeros, no access)
      auto load = [&](int kb, i32x4(&af)[4], i32x8(&bf)[4]) {
        const bool in = kb < nH;
        const uint32_t oob = in ? 0u : 0x80000000u;
        const uint32_t sa = in ? (uint32_t)(kb * kBlock * 2) : 0u, so = in ? (uint32_t)(kb * kGateUpChunk) : 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) af[j] = bload16(xr, avo + oob, sa + j * 16);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          bf[t] = cat(wload16(wr, bvoff + oob, so + t * 2048), wload16(wr, bvoff + oob, so + t * 2048 + 1024));
      };
      auto compute = [&](int kb, const i32x4(&af)[4], const i32x8(&bf)[4]) {
        const float wsg = ws_lds[2 * kb], wsu = ws_lds[2 * kb + 1];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4 p = mfma_a16_block(af, bf[t]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(p[i], t < 2 ? wsg : wsu, acc[t][i]);
        }
      };
#pragma unroll
      for (int s = 0; s < D - 1; ++s) load(s, A[s], B[s]);
      for (int kb0 = 0; kb0 < nH; kb0 += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
          load(kb0 + s + D - 1, A[(s + D - 1) % D], B[(s + D - 1) % D]);
          if (kb0 + s < nH) compute(kb0 + s, A[s], B[s]);
        }
      }
      // h = silu(gate) * up in FP32, stored as BF16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = c0 + grp * 4 + i;
        if (row < rows) {
          const float h0 = silu_mul_act(acc[0][i], acc[2][i], a.act_limit);
          const float h1 = silu_mul_act(acc[1][i], acc[3][i], a.act_limit);
          uint16_t* dst = a.hb + (size_t)(p0 + row) * Ip + nb * kBlock + wave * 32 + col;
          dst[0] = (uint16_t)f32_to_bf16(h0);
          dst[16] = (uint16_t)f32_to_bf16(h1);
        }
      }
    }
  }
}

// down: item (tile, 128-column block nb of H); wave w owns 32 columns (two
// n-tiles), as down_stream_kernel.
template <int D>
__global__ __launch_bounds__(kThreads, kDecodeWgPerCu) void down_a16_kernel(DownA16Args a) {
  __shared__ float ws_lds[kMaxKBlocks];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int H = a.H, Ip = a.Ip, nI = Ip / kBlock, NB = H / kBlock;
  const int n0 = a.n_tiles[0], n1 = a.n_tiles[1], n2 = a.n_tiles[2];
  const int n_items = (n0 + n1 + n2) * NB;
  const rsrc_t hr = make_rsrc(a.hb, (uint32_t)a.hb_bytes);
  const uint32_t bvoff = (uint32_t)(wave * 4096 + lane * 16);

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int ti = item / NB, nb = item - ti * NB;
    const Tile* tp = a16_tile(a.tiles, n0, n1, ti);
    const int e = __builtin_amdgcn_readfirstlane(tp->e), p0 = __builtin_amdgcn_readfirstlane(tp->p0);
    const int rows = __builtin_amdgcn_readfirstlane(tp->rows);
    __syncthreads();
    {
      const float* ws = a.s2 + (size_t)(e * NB + nb) * nI;
      for (int i = tid; i < nI; i += kThreads) ws_lds[i] = ws[i];
    }
    __syncthreads();
    const rsrc_t wr = make_rsrc(a.w2 + (size_t)(e * NB + nb) * nI * kDownChunk, (uint32_t)(nI * kDownChunk));

    for (int c0 = 0; c0 < rows; c0 += 16) {
      const int r = c0 + col;
      const uint32_t avo = (uint32_t)((p0 + (r < rows ? r : c0)) * Ip * 2 + grp * 64);
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      i32x4 A[D][4];
      i32x8 B[D][2];
      auto load = [&](int kb, i32x4(&af)[4], i32x8(&bf)[2]) {
        const bool in = kb < nI;
        const uint32_t oob = in ? 0u : 0x80000000u;
        const uint32_t sa = in ? (uint32_t)(kb * kBlock * 2) : 0u, so = in ? (uint32_t)(kb * kDownChunk) : 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) af[j] = bload16(hr, avo + oob, sa + j * 16);
#pragma unroll
        for (int t = 0; t < 2; ++t)
          bf[t] = cat(wload16(wr, bvoff + oob, so + t * 2048), wload16(wr, bvoff + oob, so + t * 2048 + 1024));
      };
      auto compute = [&](int kb, const i32x4(&af)[4], const i32x8(&bf)[2]) {
        const float wsc = ws_lds[kb];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f32x4 p = mfma_a16_block(af, bf[t]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(p[i], wsc, acc[t][i]);
        }
      };
#pragma unroll
      for (int s = 0; s < D - 1; ++s) load(s, A[s], B[s]);
      for (int kb0 = 0; kb0 < nI; kb0 += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
          load(kb0 + s + D - 1, A[(s + D - 1) % D], B[(s + D - 1) % D]);
          if (kb0 + s < nI) compute(kb0 + s, A[s], B[s]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = c0 + grp * 4 + i;
        if (row < rows) {
          float* dst = a.y + (size_t)(p0 + row) * H + nb * kBlock + wave * 32 + col;
          dst[0] = acc[0][i];
          dst[16] = acc[1][i];
        }
      }
    }
  }
}

// down, one flat sequence per workgroup: its units (item, 16-row subtile of
// the item's tile) in order, each Ip / 128 K steps, with the loads of the
// next unit's first D - 1 blocks issued during the current unit's last
// steps (D divides Ip / 128, so a block's ring slot is its index mod D in
// every unit).  The weight scale of a step is a scalar load.  Same
// arithmetic, in the same order, as down_a16_kernel.
template <int D>
__global__ __launch_bounds__(kThreads, kDecodeWgPerCu) void down_a16_flat_kernel(DownA16Args a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int H = a.H, Ip = a.Ip, nI = Ip / kBlock, NB = H / kBlock;
  const int n0 = a.n_tiles[0], n1 = a.n_tiles[1], n2 = a.n_tiles[2];
  const int n_items = (n0 + n1 + n2) * NB;
  const int G = (int)gridDim.x;
  if ((int)blockIdx.x >= n_items) return;
  const rsrc_t hr = make_rsrc(a.hb, (uint32_t)a.hb_bytes);
  const uint32_t bvoff = (uint32_t)(wave * 4096 + lane * 16);

  struct Unit {
    int item, wblk, p0, rows, c0;  // wblk = e * NB + nb; item >= n_items: past the end
  };
  auto first_unit = [&](int it) __attribute__((always_inline)) {
    Unit u{it, 0, 0, 0, 0};
    if (it < n_items) {
      const int ti = it / NB, nb = it - ti * NB;
      const Tile* tp = a16_tile(a.tiles, n0, n1, ti);
      u.wblk = __builtin_amdgcn_readfirstlane(tp->e) * NB + nb;
      u.p0 = __builtin_amdgcn_readfirstlane(tp->p0);
      u.rows = __builtin_amdgcn_readfirstlane(tp->rows);
    }
    return u;
  };
  auto next_unit = [&](const Unit& u) __attribute__((always_inline)) {
    if (u.c0 + 16 < u.rows) {
      Unit v = u;
      v.c0 += 16;
      return v;
    }
    return first_unit(u.item + G);
  };
  auto load = [&](const Unit& u, int kb, i32x4(&af)[4], i32x8(&bf)[2]) __attribute__((always_inline)) {
    const bool in = u.item < n_items;
    const uint32_t oob = in ? 0u : 0x80000000u;
    const uint32_t sa = in ? (uint32_t)(kb * kBlock * 2) : 0u, so = in ? (uint32_t)(kb * kDownChunk) : 0u;
    const rsrc_t wr = make_rsrc(a.w2 + (size_t)u.wblk * nI * kDownChunk, (uint32_t)(nI * kDownChunk));
    const int r = u.c0 + col;
    const uint32_t avo = (uint32_t)((u.p0 + (r < u.rows ? r : u.c0)) * Ip * 2 + grp * 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) af[j] = bload16(hr, avo + oob, sa + j * 16);
#pragma unroll
    for (int t = 0; t < 2; ++t)
      bf[t] = cat(wload16(wr, bvoff + oob, so + t * 2048), wload16(wr, bvoff + oob, so + t * 2048 + 1024));
  };

  // a unit's weight scales, lane l holding blocks l and l + 64; the next
  // unit's are loaded at the start of the current one, so their wait does
  // not hold up the blocks in flight
  auto load_ws = [&](const Unit& u, float& w0, float& w1) __attribute__((always_inline)) {
    const bool in = u.item < n_items;
    const rsrc_t sr = make_rsrc(a.s2 + (size_t)u.wblk * nI, (uint32_t)(nI * 4));
    w0 = bloadf(sr, (uint32_t)(lane * 4) | (in && lane < nI ? 0u : 0x80000000u), 0u);
    w1 = bloadf(sr, (uint32_t)((lane + 64) * 4) | (in && lane + 64 < nI ? 0u : 0x80000000u), 0u);
  };
  Unit cu = first_unit((int)blockIdx.x);
  Unit nu = next_unit(cu);
  float ws0, ws1, wn0, wn1;
  load_ws(cu, ws0, ws1);
  i32x4 A[D][4];
  i32x8 B[D][2];
#pragma unroll
  for (int s = 0; s < D - 1; ++s) load(cu, s, A[s], B[s]);
  while (cu.item < n_items) {
    load_ws(nu, wn0, wn1);
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int kb0 = 0; kb0 < nI; kb0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        const int lk = kb0 + s + D - 1;
        if (lk < nI)
          load(cu, lk, A[(s + D - 1) % D], B[(s + D - 1) % D]);
        else
          load(nu, lk - nI, A[(s + D - 1) % D], B[(s + D - 1) % D]);
        const int kb = kb0 + s;
        const float wsc = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, kb < 64 ? ws0 : ws1), kb & 63));
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f32x4 p = mfma_a16_block(A[s], B[s][t]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(p[i], wsc, acc[t][i]);
        }
      }
    }
    const int nb = cu.wblk % NB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = cu.c0 + grp * 4 + i;
      if (row < cu.rows) {
        float* dst = a.y + (size_t)(cu.p0 + row) * H + nb * kBlock + wave * 32 + col;
        dst[0] = acc[0][i];
        dst[16] = acc[1][i];
      }
    }
    cu = nu;
    nu = next_unit(cu);
    ws0 = wn0;
    ws1 = wn1;
  }
}

hipError_t launch_gate_up_a16(const GateUpA16Args& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL(gate_up_a16_kernel<3>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_a16(const DownA16Args& a, int grid, hipStream_t s) {
  const int nI = a.Ip / kBlock;
  if (nI % 4 == 0)
    hipLaunchKernelGGL(down_a16_flat_kernel<4>, dim3(grid), dim3(kThreads), 0, s, a);
  else if (nI % 2 == 0)
    hipLaunchKernelGGL(down_a16_flat_kernel<2>, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(down_a16_kernel<4>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// ----------------------------------------------------------------- combine --
// A workgroup per token and 2048 columns; 8 consecutive columns per thread.
// All of a token's y loads are issued before the sums (a skipped slot reads
// row 0 and contributes through a select, never through arithmetic), so each
// thread has its k rows in flight at once; the sums keep the slot order.

constexpr int kCombineSlots = 8;  // routed slots loaded together (more: in groups of 8)
constexpr int kCombineMaxSlots = 257;  // top_k <= 256, plus the shared slot

__device__ __forceinline__ void acc_slot(f32x4 (&acc)[2], const f32x4 (&v)[2], float wj, bool on) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float term = wj * v[h][q];
      acc[h][q] = on ? acc[h][q] + term : acc[h][q];
    }
}

// At most three waves per SIMD: fewer y rows in flight at once read faster
// (T=8192 Zipf 0.324 -> 0.308 ms against six waves; two or four: 0.312, 0.320)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 3))) void combine_kernel(CombineArgs a) {
  // a token's column blocks are consecutive blocks, so each y row is read
  // within a short window (3-6% faster than one column block of every token
  // after another)
  const int n_cb = (a.H + 2047) / 2048;
  const int t = (int)(blockIdx.x / (unsigned)n_cb), cb = (int)(blockIdx.x % (unsigned)n_cb);
  const int k = a.k, H = a.H;
  // a token's slots: up to 256 routed ones and the shared one
  __shared__ int pos[kCombineMaxSlots];
  __shared__ float wt[kCombineMaxSlots];
  const int kr = a.k_routed;
  for (int j = threadIdx.x; j < k; j += 256) {
    pos[j] = a.inv[(size_t)t * k + j];
    wt[j] = j < kr ? a.w[(size_t)t * kr + j] : 1.0f;
  }
  __syncthreads();
  const int c = (cb * 256 + threadIdx.x) * 8;
  if (c >= H) return;
  auto load = [&](int j, f32x4 (&v)[2]) __attribute__((always_inline)) {
    const int p = pos[j];
    const f32x4* src = reinterpret_cast<const f32x4*>(a.y + (size_t)(p >= 0 ? p : 0) * H + c);
    // plain loads (non-temporal ones measured 3-7% slower)
    v[0] = src[0];
    v[1] = src[1];
  };
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // routed slots, in order
  for (int j0 = 0; j0 < kr; j0 += kCombineSlots) {
    f32x4 v[kCombineSlots][2];
#pragma unroll
    for (int j = 0; j < kCombineSlots; ++j)
      if (j0 + j < kr) load(j0 + j, v[j]);
#pragma unroll
    for (int j = 0; j < kCombineSlots; ++j)
      if (j0 + j < kr) acc_slot(acc, v[j], wt[j0 + j], pos[j0 + j] >= 0);
  }
  f32x4 o[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) o[h] = f32x4{a.rho * acc[h][0], a.rho * acc[h][1], a.rho * acc[h][2], a.rho * acc[h][3]};
  // the shared-expert slot is added after the routed sum is scaled
  for (int j = kr; j < k; ++j) {
    f32x4 v[2];
    load(j, v);
    acc_slot(o, v, wt[j], pos[j] >= 0);
  }
  if (a.out_f32) {
    f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + (size_t)t * H + c);
    dst[0] = o[0];
    dst[1] = o[1];
  } else {
    i32x4 b;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      b[2 * h] = (int)(f32_to_bf16(o[h][0]) | (f32_to_bf16(o[h][1]) << 16));
      b[2 * h + 1] = (int)(f32_to_bf16(o[h][2]) | (f32_to_bf16(o[h][3]) << 16));
    }
    st16(reinterpret_cast<uint16_t*>(a.out) + (size_t)t * H + c, b);
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(a.T * ((a.H + 2047) / 2048)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ layout --
// Canonical codes -> MFMA-operand order, one 16-byte output chunk per thread.
//   w13: [e][nb][kb][wave 4][tile 4: g0 g1 u0 u1][half 2][lane 64][16 B]
//   w2 : [e][nb][kb][wave 4][tile 2][half 2][lane 64][16 B]
// Lane l of tile t covers output row 16*(t&1) + l%16 of the wave's 32 rows
// and K bytes 32*(l/16) + 16*half + [0, 16) of the 128-wide block.  Rows or
// columns at or beyond I are zero; NaN codes 0x7F / 0xFF become 0x00 / 0x80.

__device__ __forceinline__ uint8_t clean(uint8_t b) { return (b & 0x7F) == 0x7F ? (uint8_t)(b & 0x80) : b; }

__global__ void layout_w13_kernel(LayoutArgs a) {
  const int nH = a.H / kBlock, NB = a.Ip / kBlock;
  const int64_t per_e = (int64_t)NB * nH * (kGateUpChunk / 16);
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= per_e * a.n) return;
  const int le = (int)(q / per_e);
  int64_t r = q - le * per_e;
  const int lane = (int)(r & 63); r >>= 6;
  const int half = (int)(r & 1); r >>= 1;
  const int t = (int)(r & 3); r >>= 2;
  const int w = (int)(r & 3); r >>= 2;
  const int kb = (int)(r % nH);
  const int nb = (int)(r / nH);
  const int row = nb * kBlock + w * 32 + (t & 1) * 16 + (lane & 15);
  const int k0 = kb * kBlock + (lane >> 4) * 32 + half * 16;
  const uint8_t* src = (t < 2 ? a.gate : a.up) + ((size_t)le * a.I + row) * a.H + k0;
  uint8_t v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = row < a.I ? clean(src[i]) : (uint8_t)0;
  uint8_t* dst = a.w13 + ((size_t)(a.e0 + le) * per_e + (q - le * per_e)) * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) dst[i] = v[i];
}

__global__ void layout_w2_kernel(LayoutArgs a) {
  const int nI = a.Ip / kBlock, NB = a.H / kBlock;
  const int64_t per_e = (int64_t)NB * nI * (kDownChunk / 16);
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= per_e * a.n) return;
  const int le = (int)(q / per_e);
  int64_t r = q - le * per_e;
  const int lane = (int)(r & 63); r >>= 6;
  const int half = (int)(r & 1); r >>= 1;
  const int t = (int)(r & 1); r >>= 1;
  const int w = (int)(r & 3); r >>= 2;
  const int kb = (int)(r % nI);
  const int nb = (int)(r / nI);
  const int row = nb * kBlock + w * 32 + t * 16 + (lane & 15);
  const int k0 = kb * kBlock + (lane >> 4) * 32 + half * 16;
  const uint8_t* src = a.down + ((size_t)le * a.H + row) * a.I;
  uint8_t v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = (k0 + i) < a.I ? clean(src[k0 + i]) : (uint8_t)0;
  uint8_t* dst = a.w2 + ((size_t)(a.e0 + le) * per_e + (q - le * per_e)) * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) dst[i] = v[i];
}

__global__ void layout_scales_kernel(LayoutArgs a) {
  const int nH = a.H / kBlock, nI = a.Ip / kBlock;
  const int64_t n13 = (int64_t)a.n * nI * nH;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n13) {
    const size_t base = (size_t)a.e0 * nI * nH;
    a.s13[(base + i) * 2] = a.gate_scale[i];
    a.s13[(base + i) * 2 + 1] = a.up_scale[i];
    a.s2[base + i] = a.down_scale[i];  // same element count, [nH][nI] order kept
  }
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t s) {
  const int nH = a.H / kBlock, NB = a.Ip / kBlock;
  const int64_t c13 = (int64_t)a.n * NB * nH * (kGateUpChunk / 16);
  const int64_t c2 = (int64_t)a.n * nH * NB * (kDownChunk / 16);
  const int64_t cs = (int64_t)a.n * NB * nH;
  hipLaunchKernelGGL(layout_w13_kernel, dim3((unsigned)((c13 + 255) / 256)), dim3(256), 0, s, a);
  hipLaunchKernelGGL(layout_w2_kernel, dim3((unsigned)((c2 + 255) / 256)), dim3(256), 0, s, a);
  hipLaunchKernelGGL(layout_scales_kernel, dim3((unsigned)((cs + 255) / 256)), dim3(256), 0, s, a);
  if (a.n13) {
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_wnorm(a, s);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------- slice --
// Load-time share of the intermediate dimension: one workgroup per 128x128
// block of the share.  A share that starts on a 128 boundary keeps the
// checkpoint's codes and block scales; otherwise the block is requantised:
// v = dec(code) * S (FP32), s = max|v| / 448, code = E4M3(v / s).

__device__ __forceinline__ float e4m3_dec(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (e == 15u && m == 7u)
    v = 0.0f;  // NaN codes act as signed zeros
  else if (e == 0u)
    v = (float)m * 0x1p-9f;
  else
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (b & 0x80u) ? -v : v;
}

__global__ __launch_bounds__(256) void slice_kernel(SliceArgs a) {
  __shared__ uint32_t red[4];
  const int tid = threadIdx.x;
  const int oR = a.axis == 0 ? a.len : a.R, oC = a.axis == 0 ? a.C : a.len;
  const int orb = (oR + 127) / 128, ocb = (oC + 127) / 128, cb = (a.C + 127) / 128;
  int b = blockIdx.x;
  const int e = b / (orb * ocb);
  b -= e * orb * ocb;
  const int bi = b / ocb, bj = b - (b / ocb) * ocb;
  const int r0 = bi * 128, c0 = bj * 128;
  const int nr = min(128, oR - r0), nc = min(128, oC - c0);
  const uint8_t* src = a.src + (size_t)e * a.R * a.C;
  const float* src_s = a.src_s + (size_t)e * ((a.R + 127) / 128) * cb;
  uint8_t* dst = a.dst + (size_t)e * oR * oC;
  const bool requant = (a.off & 127) != 0;
  auto at = [&](int i, int& gr, int& gc, int& r, int& c) {
    r = r0 + i / nc;
    c = c0 + i - (i / nc) * nc;
    gr = a.axis == 0 ? r + a.off : r;
    gc = a.axis == 0 ? c : c + a.off;
  };
  float s;
  if (requant) {
    uint32_t m = 0;
    for (int i = tid; i < nr * nc; i += 256) {
      int gr, gc, r, c;
      at(i, gr, gc, r, c);
      const float v = e4m3_dec(src[(size_t)gr * a.C + gc]) * src_s[(gr / 128) * cb + gc / 128];
      m = umax(m, abs_bits(v));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = umax(m, (uint32_t)__shfl_xor((int)m, o));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    const float amax = __uint_as_float(umax(umax(red[0], red[1]), umax(red[2], red[3])));
    s = __fdiv_rn(amax, 448.0f);
    for (int i = tid; i < nr * nc; i += 256) {
      int gr, gc, r, c;
      at(i, gr, gc, r, c);
      const float v = e4m3_dec(src[(size_t)gr * a.C + gc]) * src_s[(gr / 128) * cb + gc / 128];
      dst[(size_t)r * oC + c] = (uint8_t)(amax != 0.0f ? to_e4m3(__fdiv_rn(v, s)) : 0u);
    }
  } else {
    const int sr = a.axis == 0 ? (r0 + a.off) / 128 : bi, sc = a.axis == 0 ? bj : (c0 + a.off) / 128;
    s = src_s[sr * cb + sc];
    for (int i = tid; i < nr * nc; i += 256) {
      int gr, gc, r, c;
      at(i, gr, gc, r, c);
      dst[(size_t)r * oC + c] = src[(size_t)gr * a.C + gc];
    }
  }
  if (tid == 0) a.dst_s[(size_t)e * orb * ocb + bi * ocb + bj] = s;
}

hipError_t launch_slice(const SliceArgs& a, hipStream_t s) {
  const int oR = a.axis == 0 ? a.len : a.R, oC = a.axis == 0 ? a.C : a.len;
  const int64_t blocks = (int64_t)a.n * ((oR + 127) / 128) * ((oC + 127) / 128);
  hipLaunchKernelGGL(slice_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// -------------------------------------------------------------- exact ties --
// Layers whose intermediate width fits one 128-wide block (Ip = 128) have a
// single E4M3 group of h per row, so one h code decided on the other side of
// a rounding midpoint moves a row by about 1% (one of 128 values, changed by
// up to 1/16 of its size).  The FP8 MFMA keeps only about 13 bits below the
// largest product of a block dot, so its gate/up differ from the definition's
// ascending FP32 sums by up to ~1e-5 of |x| |w| / sqrt(H / 128) (measured
// over 2.3 M elements, H = 256 .. 6144), which decides ~0.2% of these codes
// differently.  For such layers the GEMM stage writes FP32 gate/up and this
// kernel quantises h, one 128-thread workgroup per slot row, thread n on
// column n:
//   1. h = silu(g) * u from the GEMM's gate/up, with the error bound
//        dh = m |x| (|silu'(g) u| |w_g| + |silu(g)| |w_u|) + 2^-17 |h|,
//      |x| the L2 norm of the dequantised activation row, |w_g|, |w_u| those
//      of the dequantised weight rows (computed at load), m = kTieMargin /
//      sqrt(H / 128), 14 times the largest measured ratio, and the last term
//      for the fast SiLU;
//   2. the elements that may hold the group's max |h| (|h| >= max|h| -
//      2 max dh) are recomputed in the definition's order: per K block an
//      FP32 sum of the exact products in ascending column order, then
//      acc + p * (s_x * s_w), and SiLU with the correctly rounded FP32 e^-g;
//      their largest |h| gives the scale s = max|h| / 448 of the definition;
//   3. every other element whose |h| / s lies within dh / s of a midpoint
//      between two E4M3 values, or whose |h| is within dh of zero (the sign
//      of a zero code), is recomputed the same way;
//   4. codes = E4M3(h / s) (IEEE division), from the recomputed h where
//      there is one.
// An element outside both sets is farther from every decision than its error
// bound, so every code and the scale are those of the definition.  Rows with
// a NaN or infinite h take s = max|h| / 448 and the codes of h / s directly.

__device__ __forceinline__ float tie_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1];
}

__device__ __forceinline__ uint32_t tie_umax(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = umax(v, (uint32_t)__shfl_xor((int)v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return umax(red[0], red[1]);
}

__device__ __forceinline__ uint32_t byte_of(const i32x4& v, int i) {
  return ((uint32_t)v[i >> 2] >> (8 * (i & 3))) & 0xFFu;
}

// silu(g) * u of the definition: the clamp of the activation, then
// (g / (1 + e)) * u with e the correctly rounded FP32 e^-g, IEEE operations.
__device__ __forceinline__ float exact_silu_mul(float g, float u, float L) {
  if (L > 0.0f) {
    g = g > L ? L : g;
    u = u > L ? L : (u < -L ? -L : u);
  }
  const float e = (float)exp(-(double)g);
  return __fmul_rn(__fdiv_rn(g, __fadd_rn(1.0f, e)), u);
}

// Gate and up of column n (< 128) of expert e for the activation row in LDS,
// in the definition's order, read from the MFMA-operand weight layout: row n
// of the block lives in wave n / 32, tile (n / 16) & 1 (gate) or 2 + that
// (up), lane n % 16 + 16 g, half h, for K bytes 32 g + 16 h .. + 15.
__device__ __noinline__ float exact_h(const TieArgs& a, const uint8_t* xs, const float* sxs, int e, int n,
                                      int nH) {
  const uint8_t* wb = a.w13 + (size_t)e * nH * kGateUpChunk;
  const float* ws = a.s13 + (size_t)e * nH * 2;
  const int w = n >> 5, tt = (n >> 4) & 1, r16 = n & 15;
  float ag = 0.0f, au = 0.0f;
  for (int kb = 0; kb < nH; ++kb) {
    const uint8_t* cb = wb + (size_t)kb * kGateUpChunk;
    float pg = 0.0f, pu = 0.0f;
    for (int g4 = 0; g4 < 4; ++g4) {
      for (int half = 0; half < 2; ++half) {
        const int lo = (g4 * 16 + r16) * 16;
        const i32x4 G = ld16(cb + ((w * 4 + tt) * 2 + half) * 1024 + lo);
        const i32x4 U = ld16(cb + ((w * 4 + 2 + tt) * 2 + half) * 1024 + lo);
        const uint8_t* x = xs + kb * kBlock + g4 * 32 + half * 16;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float xa = e4m3_dec(x[i]);
          pg = __fadd_rn(pg, __fmul_rn(xa, e4m3_dec(byte_of(G, i))));
          pu = __fadd_rn(pu, __fmul_rn(xa, e4m3_dec(byte_of(U, i))));
        }
      }
    }
    ag = __fadd_rn(ag, __fmul_rn(pg, __fmul_rn(sxs[kb], ws[2 * kb])));
    au = __fadd_rn(au, __fmul_rn(pu, __fmul_rn(sxs[kb], ws[2 * kb + 1])));
  }
  return exact_silu_mul(ag, au, a.act_limit);
}

__global__ __launch_bounds__(128) void tie_exact_kernel(TieArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[kMaxKBlocks * kBlock];
  __shared__ float sxs[kMaxKBlocks];
  __shared__ float redf[2];
  __shared__ uint32_t redu[2];
  const int p = blockIdx.x, n = threadIdx.x;
  if (p >= a.offsets[a.E]) return;  // past the routed slots (whole workgroup)
  // the expert of sorted slot p: the largest e with offsets[e] <= p (that
  // expert is not empty, because offsets[e + 1] > p)
  int lo = 0, hi = a.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.offsets[mid] <= p) lo = mid; else hi = mid;
  }
  const int e = lo, H = a.H, nH = H / kBlock;
  const int64_t t = a.perm[p] / a.k;
  for (int i = n * 16; i < H; i += 128 * 16) st16(&xs[i], ld16(a.xq + t * H + i));
  for (int i = n; i < nH; i += 128) sxs[i] = a.sx[t * nH + i];
  __syncthreads();
  float ss = 0.0f;
  for (int i = n; i < H; i += 128) {
    const float v = e4m3_dec(xs[i]) * sxs[i >> 7];
    ss = __builtin_fmaf(v, v, ss);
  }
  const float xnorm = sqrtf(tie_sum(ss, redf));

  const float L = a.act_limit;
  float g = a.gu[(size_t)p * 2 * kBlock + n], u = a.gu[(size_t)p * 2 * kBlock + kBlock + n];
  if (L > 0.0f) {
    g = g > L ? L : g;
    u = u > L ? L : (u < -L ? -L : u);
  }
  const float hg = silu_mul(g, u);
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f));
  const float ds = sg * (1.0f + g * (1.0f - sg));
  const float wg = a.n13[(size_t)e * 2 * kBlock + n], wu = a.n13[(size_t)e * 2 * kBlock + kBlock + n];
  const float dh = a.margin * xnorm * (fabsf(ds * u) * wg + fabsf(g * sg) * wu) + fabsf(hg) * 0x1p-17f;
  const float amax_g = __uint_as_float(tie_umax(abs_bits(hg), redu));
  const float dh_max = __uint_as_float(tie_umax(abs_bits(dh), redu));

  uint32_t code;
  float s;
  if (!(amax_g <= 3.4028234663852886e38f) || !(dh_max <= 3.4028234663852886e38f)) {
    // NaN or infinity in the row: no decision is near a finite tie
    s = __fdiv_rn(amax_g, 448.0f);
    code = to_e4m3(__fdiv_rn(hg, s));
  } else if (amax_g == 0.0f) {
    // every h is zero (the MFMA keeps the largest product of a nonzero dot)
    s = 0.0f;
    code = 0u;
  } else {
    float hx = hg;
    bool exact = false;
    if (fabsf(hg) >= amax_g - 2.0f * dh_max) {
      hx = exact_h(a, xs, sxs, e, n, nH);
      exact = true;
    }
    const float amax = __uint_as_float(tie_umax(exact ? abs_bits(hx) : 0u, redu));
    s = __fdiv_rn(amax, 448.0f);
    if (amax == 0.0f) {
      code = 0u;
    } else {
      if (!exact) {
        const float v = __fdiv_rn(fabsf(hg), s), dv = __fdiv_rn(dh, s);
        const uint32_t c = to_e4m3(v);
        const float mc = e4m3_dec(c);
        const bool near_lo = c > 0u && v - 0.5f * (e4m3_dec(c - 1u) + mc) <= dv;
        const bool near_hi = c < 0x7Eu && 0.5f * (mc + e4m3_dec(c + 1u)) - v <= dv;
        // |h| within its bound of 0: the sign, hence +0 / -0, is undecided
        const bool near_zero = fabsf(hg) <= dh;
        if (near_lo || near_hi || near_zero) {
          hx = exact_h(a, xs, sxs, e, n, nH);
          exact = true;
        }
      }
      code = to_e4m3(__fdiv_rn(exact ? hx : hg, s));
    }
  }
  a.hq[(size_t)p * kBlock + n] = (uint8_t)code;
  if (n == 0) {
    a.sh[p] = s;
    a.shT[p] = s;
  }
}

hipError_t launch_tie_exact(const TieArgs& a, int64_t max_slots, hipStream_t s) {
  if (max_slots <= 0) return hipSuccess;
  hipLaunchKernelGGL(tie_exact_kernel, dim3((unsigned)max_slots), dim3(128), 0, s, a);
  return hipGetLastError();
}

// L2 norms of the dequantised gate and up rows of experts [e0, e0 + n) from
// the canonical codes and scales: n13[e][r] for gate row r < Ip, up row r - Ip
// otherwise; padding rows get 0.  Used only by the exact-tie quantiser.
__global__ void wnorm_kernel(LayoutArgs a) {
  const int Ip = a.Ip, nH = a.H / kBlock, nIc = (a.I + kBlock - 1) / kBlock;
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= (int64_t)a.n * 2 * Ip) return;
  const int le = (int)(q / (2 * Ip)), r = (int)(q - (int64_t)le * 2 * Ip);
  const int row = r < Ip ? r : r - Ip;
  float ss = 0.0f;
  if (row < a.I) {
    const uint8_t* src = (r < Ip ? a.gate : a.up) + ((size_t)le * a.I + row) * a.H;
    const float* sc = (r < Ip ? a.gate_scale : a.up_scale) + ((size_t)le * nIc + row / kBlock) * nH;
    for (int kb = 0; kb < nH; ++kb) {
      float bs = 0.0f;
      for (int c = 0; c < kBlock; ++c) {
        const float v = e4m3_dec(src[kb * kBlock + c]);
        bs = __builtin_fmaf(v, v, bs);
      }
      ss = __builtin_fmaf(bs, sc[kb] * sc[kb], ss);
    }
  }
  a.n13[(size_t)(a.e0 + le) * 2 * Ip + r] = sqrtf(ss);
}

hipError_t launch_wnorm(const LayoutArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.n * 2 * a.Ip;
  hipLaunchKernelGGL(wnorm_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------- static scratch --
// The per-pass workspace of moe_fp8_prefill_run_static, for callers that
// cannot allocate: one array per device, held until the process ends and
// shared by every handle and call on that device.  On the host the array's
// name is a host-side stand-in, not a device address; host code uses only the
// address hipGetSymbolAddress returns for the current device, looked up once
// per device and kept.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t static_scratch(uint8_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static uint8_t* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = (uint8_t*)p;
  }
  *out = addr[dev];
  return hipSuccess;
}

// ------------------------------------------------------------- calibration --
// Measured ceilings for the rooflines: independent chains of the GEMMs' own
// 16x16x128 FP8 MFMA (two waves per SIMD, eight chains per wave, nothing
// else in the loop), and a streaming read of a device buffer with 16-byte
// non-temporal loads, four in flight per thread.

__global__ __launch_bounds__(256) void peak_mfma_kernel(int32_t iters, float* out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // E4M3 operands 1.0 (0x38) and 0.5 (0x30): the chains stay finite
  const i32x8 a = {0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, lane};
  const i32x8 b = {0x30303030, 0x30303030, 0x30303030, 0x30303030, 0x30303030, 0x30303030, 0x30303030, 0x30303030};
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int32_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 0, 0, 0);
  }
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) sum += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (lane == 0) out[blockIdx.x * 4 + wave] = sum;
}

// Work group g streams 32 KiB chunks g, g + G, ...: eight 16-byte buffer
// loads per thread (each wave instruction one contiguous KiB), with the next
// chunk's eight loads issued before the current chunk is consumed.
constexpr uint32_t kPeakChunk = 256 * 16 * 8;

__global__ __launch_bounds__(256) void peak_stream_kernel(const uint8_t* src, uint32_t n_chunks, int32_t* out) {
  const rsrc_t r = make_rsrc(src, n_chunks * kPeakChunk);
  const uint32_t t16 = threadIdx.x * 16u;
  i32x4 acc = {0, 0, 0, 0};
  i32x4 a[8], b[8];
  uint32_t c = blockIdx.x;
  if (c < n_chunks) {
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = wload16(r, t16 + j * 4096u, c * kPeakChunk);
  }
  for (; c < n_chunks; c += gridDim.x) {
    const uint32_t nc = c + gridDim.x;
    if (nc < n_chunks) {
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = wload16(r, t16 + j * 4096u, nc * kPeakChunk);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc ^= a[j];
      a[j] = b[j];
    }
  }
  const int32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (v == 0x5EED1234) out[blockIdx.x] = v;  // depends on the data: the loads stay
}

hipError_t launch_peak_mfma(int32_t iters, int grid, float* out, hipStream_t s) {
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(grid), dim3(256), 0, s, iters, out);
  return hipGetLastError();
}

// Streams the first n_chunks * 32 KiB bytes of src (under 4 GiB); returns
// the bytes read in *bytes.
hipError_t launch_peak_stream(const void* src, int64_t max_bytes, int grid, int32_t* out, int64_t* bytes,
                              hipStream_t s) {
  const int64_t cap = std::min<int64_t>(max_bytes, (int64_t(1) << 32) - kPeakChunk);
  const uint32_t n_chunks = (uint32_t)(cap / kPeakChunk);
  *bytes = (int64_t)n_chunks * kPeakChunk;
  hipLaunchKernelGGL(peak_stream_kernel, dim3(grid), dim3(256), 0, s, (const uint8_t*)src, n_chunks, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------- probe --

__global__ __launch_bounds__(64) void mfma_probe_kernel(const uint8_t* a, const uint8_t* b, float* d) {
  const int lane = threadIdx.x, g = lane >> 4, c = lane & 15;
  const i32x8 af = cat(ld16(a + c * 128 + g * 32), ld16(a + c * 128 + g * 32 + 16));
  const i32x8 bf = cat(ld16(b + c * 128 + g * 32), ld16(b + c * 128 + g * 32 + 16));
  const f32x4 r = mfma_e4m3(af, bf);
#pragma unroll
  for (int i = 0; i < 4; ++i) d[(g * 4 + i) * 16 + c] = r[i];
  // second result: the same product as four K=32 FP8 MFMAs chained through
  // the accumulator (lane l holds 8 K bytes 8*(l/16).. of each 32-wide slice)
  f32x4 r2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const long av = *reinterpret_cast<const long*>(a + c * 128 + s * 32 + g * 8);
    const long bv = *reinterpret_cast<const long*>(b + c * 128 + s * 32 + g * 8);
    r2 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(av, bv, r2, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) d[256 + (g * 4 + i) * 16 + c] = r2[i];
  // third result: four independent K=32 MFMAs, each promoted to FP32
  f32x4 r3 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const long av = *reinterpret_cast<const long*>(a + c * 128 + s * 32 + g * 8);
    const long bv = *reinterpret_cast<const long*>(b + c * 128 + s * 32 + g * 8);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const f32x4 part = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(av, bv, z, 0, 0, 0);
    r3 = r3 + part;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) d[512 + (g * 4 + i) * 16 + c] = r3[i];
}

hipError_t launch_mfma_probe(const uint8_t* a, const uint8_t* b, float* d, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(1), dim3(64), 0, s, a, b, d);
  return hipGetLastError();
}

}  // namespace moe
