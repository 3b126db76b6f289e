// Internal interface between the C-ABI host code (moe_api.cpp) and the HIP
// kernels (moe_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kBlock = 128;          // weight block edge and activation group
constexpr int kWaves = 4;            // waves per GEMM workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kSmallRows = 16;       // experts with <= this many rows use the 1-subtile GEMM
constexpr int kNarrowRows = 128;     // experts with kSmallRows < rows <= kNarrowRows: one tile, 3-stage GEMMs
constexpr int kWideRows = 256;       // rows per tile of the 8-wave GEMMs for experts with more rows
#ifndef MOE_STREAM_DEPTH
#define MOE_STREAM_DEPTH 5
#endif
#ifndef MOE_STREAM_DEPTH_DOWN
#define MOE_STREAM_DEPTH_DOWN 6
#endif
#ifndef MOE_WEIGHT_AUX
#define MOE_WEIGHT_AUX 2
#endif
#ifndef MOE_GU_WG_PER_CU
#define MOE_GU_WG_PER_CU 2
#endif
#ifndef MOE_MIX_LISTS
#define MOE_MIX_LISTS 1  // interleave two tile lists of one launch by XCD runs
#endif
#ifndef MOE_DN_WG_PER_CU
#define MOE_DN_WG_PER_CU 2
#endif
constexpr int kWeightAux = MOE_WEIGHT_AUX;          // cache-policy bits of the weight loads
constexpr int kGateUpWgPerCu = MOE_GU_WG_PER_CU;  // persistent grid of the streaming gate_up
constexpr int kDownWgPerCu = MOE_DN_WG_PER_CU;    // persistent grid of the streaming down
constexpr bool kMixLists = MOE_MIX_LISTS != 0;
constexpr int kStreamDepth = MOE_STREAM_DEPTH;           // K blocks in flight per wave, streaming gate_up
constexpr int kStreamDepthDown = MOE_STREAM_DEPTH_DOWN;  // K blocks in flight per wave, streaming down
constexpr int kMaxExperts = 1024;
constexpr int kMaxKBlocks = 128;     // H/128 and Ip/128 limit (LDS-staged weight scales)

// Bytes of swizzled weights per (expert, 128-row output block, 128-wide K block).
constexpr int kGateUpChunk = kWaves * 4 * 2048;  // gate 128 rows + up 128 rows
constexpr int kDownChunk = kWaves * 2 * 2048;    // 128 rows of down

// A GEMM work tile: rows [p0, p0+rows) of the sorted slot order, all of
// expert e, whose large-expert tiles are first .. first+count-1.
struct Tile {
  int32_t e, p0, rows, first, count, pad0, pad1, pad2;
};

struct PlanArgs {
  const int32_t* ids;  // [T][k_routed]
  int32_t T, k, E;     // slots per token and experts, a shared expert included
  int32_t k_routed, E_routed;  // slots k_routed..k-1 of a token are the shared expert E-1
  int32_t* counts;     // [E]
  int32_t* offsets;    // [E+1]
  int32_t* perm;       // [T*k]
  int32_t* inv;        // [T*k]
  Tile* small_tiles;   // [E]
  Tile* narrow_tiles;  // [E]: experts with kSmallRows < rows <= kNarrowRows, one tile each
  Tile* wide_tiles;    // [T*k/kWideRows + E]: experts with more rows, tiles of <= kWideRows
  int32_t* n_tiles;    // [3]: small, narrow, wide
  int32_t* err;        // sticky bad-id flag
  int32_t* chunk;      // [ceil(T*k/1024)][E] scratch: per-chunk counts, then first positions
};

struct RouteArgs {
  const float* logits;  // [T][E]
  int64_t T;
  int32_t E, k, kind;   // kind: 0 softmax, 1 sigmoid
  int32_t* ids;         // [T][k]
  float* w;             // [T][k]
};
constexpr int kRouteMaxK = 64;           // one lane per chosen slot
constexpr int kRoutePerLane = kMaxExperts / 64;
struct QuantArgs {
  const uint16_t* x;   // bf16 [T][H]
  int32_t T, H;
  uint8_t* xq;         // [T][H]
  float* sx;           // [T][H/128]
  float* sxT;          // [H/128][T]: the same scales, K-block major
};

struct GateUpArgs {
  const uint8_t* xq;   // [T][H]
  const float* sx;     // [T][H/128]
  int64_t xq_bytes, sx_bytes;  // extents of xq and sx (buffer bounds)
  const int32_t* perm;
  int32_t k, H, Ip;
  const uint8_t* w13;  // swizzled
  const float* s13;    // [E][Ip/128][H/128][2]
  const Tile* tiles;
  const int32_t* n_tiles;
  uint8_t* hq;         // [P][Ip]
  float* sh;           // [P][Ip/128]
  float* gu_dbg;       // optional [P][2*Ip] FP32 gate|up before the epilogue
  float act_limit;     // > 0: clamped SiLU (gate <= L, |up| <= L); 0: unclamped
  // K-block-major copies of the row scales: a tile's rows for one K block are
  // then adjacent words rather than one cache line per row
  const float* sxT;    // [H/128][T]
  int64_t sxT_bytes;
  int32_t T, P;        // rows and slots of the pass (pitches of sxT and shT)
  float* shT;          // [Ip/128][P]
};

struct DownArgs {
  const uint8_t* hq;   // [P][Ip]
  const float* sh;     // [P][Ip/128]
  int64_t hq_bytes, sh_bytes;  // extents of hq and sh (buffer bounds)
  int32_t H, Ip;
  const uint8_t* w2;   // swizzled
  const float* s2;     // [E][H/128][Ip/128]
  const Tile* tiles;
  const int32_t* n_tiles;
  float* y;            // [P][H]
  const float* shT;    // [Ip/128][P], K-block major
  int64_t shT_bytes;
  int32_t P;
  // down_wide_kernel: a second tile list whose items follow the first list's
  // (count n_tiles[1]), or null
  const Tile* tiles2;
};

struct CombineArgs {
  const float* y;      // [P][H]
  const int32_t* inv;  // [T*k]
  const float* w;      // [T][k_routed]
  int32_t T, k, H;     // k: slots per token, the shared slot (weight 1) last
  int32_t k_routed;
  float rho;
  int32_t out_f32;
  void* out;
};

struct LayoutArgs {
  // canonical codes of experts [e0, e0 + n) on the device
  const uint8_t* gate;  // [n][I][H]
  const uint8_t* up;    // [n][I][H]
  const uint8_t* down;  // [n][H][I]
  const float* gate_scale;  // [n][nI][nH]
  const float* up_scale;
  const float* down_scale;  // [n][nH][nI]
  int32_t e0, n, H, I, Ip;
  uint8_t* w13;
  float* s13;
  uint8_t* w2;
  float* s2;
  float* n13;  // [E][2*Ip] gate|up row norms for the exact-tie quantiser, or null
};

// The exact-tie quantiser of h for layers with Ip == 128 (tie_exact_kernel).
constexpr float kTieMargin = 1.5e-4f;
struct TieArgs {
  const float* gu;         // [P][256] FP32 gate | up from the GEMM
  const uint8_t* xq;       // [T][H]
  const float* sx;         // [T][H/128]
  const int32_t* perm;     // sorted position -> slot t*k+j
  const int32_t* offsets;  // [E+1]
  int32_t E, k, H;
  const uint8_t* w13;      // swizzled
  const float* s13;        // [E][1][H/128][2]
  const float* n13;        // [E][256]
  uint8_t* hq;             // [P][128]
  float* sh;               // [P]
  float* shT;              // [P]
  float act_limit;
  float margin;            // kTieMargin / sqrt(H / 128)
};

struct SliceArgs {
  // n experts' matrices [R][C] (codes) with block scales [ceil(R/128)][ceil(C/128)],
  // sliced along rows (axis 0) or columns (axis 1) to [off, off + len)
  const uint8_t* src;
  const float* src_s;
  int32_t n, R, C, axis, off, len;
  uint8_t* dst;    // [n][oR][oC]
  float* dst_s;    // [n][ceil(oR/128)][ceil(oC/128)]
};

// GEMM variants (launch_gate_up / launch_down kind)
constexpr int kGemmStream = 0, kGemmNarrow = 1, kGemmWide = 2;

// The W8A16 decode path: activations stay BF16 (x as given, h rounded to
// BF16); every tile of the three lists is taken 16 rows at a time.
constexpr int kDecodeRows = 1024;  // rows per decode pass
constexpr int kDecodeWgPerCu = 2;
struct GateUpA16Args {
  const uint16_t* x;     // bf16 [T][H]
  int64_t x_bytes;
  const int32_t* perm;
  int32_t k, H, Ip;
  const uint8_t* w13;    // swizzled
  const float* s13;
  const Tile* tiles[3];  // small, narrow, wide lists
  const int32_t* n_tiles;
  uint16_t* hb;          // bf16 [P][Ip]
  float act_limit;
};
struct DownA16Args {
  const uint16_t* hb;    // bf16 [P][Ip]
  int64_t hb_bytes;
  int32_t H, Ip;
  const uint8_t* w2;     // swizzled
  const float* s2;
  const Tile* tiles[3];
  const int32_t* n_tiles;
  float* y;              // [P][H]
};

// Launchers (return the launch status).
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_quant(const QuantArgs& a, hipStream_t s);
hipError_t launch_gate_up(const GateUpArgs& a, int kind, int grid, hipStream_t s);
hipError_t launch_down(const DownArgs& a, int kind, int grid, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_gate_up_a16(const GateUpA16Args& a, int grid, hipStream_t s);
hipError_t launch_down_a16(const DownA16Args& a, int grid, hipStream_t s);
hipError_t launch_layout(const LayoutArgs& a, hipStream_t s);
hipError_t launch_slice(const SliceArgs& a, hipStream_t s);
hipError_t launch_tie_exact(const TieArgs& a, int64_t max_slots, hipStream_t s);
hipError_t launch_wnorm(const LayoutArgs& a, hipStream_t s);
// run_static(): the static per-device workspace array and its address on the
// current device (looked up once per device).
constexpr int64_t kStaticScratchBytes = int64_t(64) << 20;
hipError_t static_scratch(uint8_t** out);
hipError_t launch_peak_mfma(int32_t iters, int grid, float* out, hipStream_t s);
hipError_t launch_peak_stream(const void* src, int64_t max_bytes, int grid, int32_t* out, int64_t* bytes,
                              hipStream_t s);
hipError_t launch_mfma_probe(const uint8_t* a, const uint8_t* b, float* d, hipStream_t s);

}  // namespace moe
