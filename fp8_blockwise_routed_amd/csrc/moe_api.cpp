// C-ABI entry points of the routed-expert FP8 MoE prefill library.  Host code
// only: argument checks, device memory, weight upload, the per-pass launch
// sequence and the handle's fail-closed state.  Kernels are in
// moe_kernels.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstddef>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/moe_fp8_prefill.h"
#include "moe_internal.h"

using namespace moe;

namespace {

struct Dims {
  // E, k count the shared expert and its slot; Er, kr are the routed ones
  int64_t E, k, H, I, Ip, nH, nI, max_rows, P;  // P = max_rows * k
  int64_t Er, kr, shared;
  int64_t I_full, I_off;  // checkpoint width and the share's start (I_full == I: no share)
  // one 128-wide h group per row: h is quantised by the exact-tie quantiser
  bool exact_ties() const { return nI == 1; }
};

// Description sizes of older callers: without shared_experts, and without
// activation_limit.  Fields past a caller's struct_size read as 0.
constexpr int32_t kDescNoShared = (int32_t)offsetof(moe_fp8_prefill_desc, shared_experts);
constexpr int32_t kDescNoLimit = (int32_t)offsetof(moe_fp8_prefill_desc, activation_limit);
constexpr int32_t kDescNoShare = (int32_t)offsetof(moe_fp8_prefill_desc, inter_full);

bool desc_size_ok(const moe_fp8_prefill_desc* d) {
  return d->struct_size == (int32_t)sizeof(moe_fp8_prefill_desc) || d->struct_size == kDescNoShare ||
         d->struct_size == kDescNoLimit || d->struct_size == kDescNoShared;
}
int32_t desc_inter_full(const moe_fp8_prefill_desc* d) {
  return d->struct_size > kDescNoShare ? d->inter_full : 0;
}
int32_t desc_inter_offset(const moe_fp8_prefill_desc* d) {
  return d->struct_size > kDescNoShare ? d->inter_offset : 0;
}
int32_t desc_shared(const moe_fp8_prefill_desc* d) {
  return d->struct_size > kDescNoShared ? d->shared_experts : 0;
}
float desc_limit(const moe_fp8_prefill_desc* d) {
  return d->struct_size > kDescNoLimit ? d->activation_limit : 0.0f;
}

Dims dims_of(const moe_fp8_prefill_desc* d) {
  Dims m;
  m.shared = desc_shared(d);
  m.I_full = desc_inter_full(d) > 0 ? desc_inter_full(d) : d->inter;
  m.I_off = desc_inter_full(d) > 0 ? desc_inter_offset(d) : 0;
  m.Er = d->num_experts;
  m.kr = d->top_k;
  m.E = m.Er + m.shared;
  m.k = m.kr + m.shared;
  m.H = d->hidden;
  m.I = d->inter;
  m.Ip = kBlock * ((m.I + kBlock - 1) / kBlock);
  m.nH = m.H / kBlock;
  m.nI = m.Ip / kBlock;
  m.max_rows = d->max_rows;
  m.P = m.max_rows * m.k;
  return m;
}

int64_t align256(int64_t n) { return (n + 255) & ~int64_t(255); }

// Workspace pieces, in allocation order.
struct WsSizes {
  int64_t xq, sx, sxT, hq, sh, shT, y, counts, offsets, perm, inv, small_tiles, narrow_tiles, wide_tiles, n_tiles, chunk,
      err, rids, rw, hb, gu;
  int64_t total() const {
    return align256(xq) + align256(sx) + align256(sxT) + align256(hq) + align256(sh) + align256(shT) +
           align256(y) +
           align256(counts) + align256(offsets) + align256(perm) + align256(inv) +
           align256(small_tiles) + align256(narrow_tiles) + align256(wide_tiles) + align256(n_tiles) + align256(chunk) +
           align256(err) +
           align256(rids) + align256(rw) + align256(hb) + align256(gu);
  }
};

WsSizes ws_sizes(const Dims& m) {
  WsSizes w;
  w.xq = m.max_rows * m.H;
  w.sx = m.max_rows * m.nH * 4;
  w.sxT = w.sx;
  w.hq = m.P * m.Ip;
  w.sh = m.P * m.nI * 4;
  w.shT = w.sh;
  w.y = m.P * m.H * 4;
  w.counts = m.E * 4;
  w.offsets = (m.E + 1) * 4;
  w.perm = m.P * 4;
  w.inv = m.P * 4;
  w.small_tiles = m.E * (int64_t)sizeof(Tile);
  w.narrow_tiles = m.E * (int64_t)sizeof(Tile);
  w.wide_tiles = (m.P / kWideRows + m.E + 1) * (int64_t)sizeof(Tile);
  w.n_tiles = 4 * 4;
  w.chunk = (m.P + 1023) / 1024 * m.E * 4;  // the plan's per-chunk counts
  w.err = 4;
  w.rids = m.max_rows * m.kr * 4;  // one pass's routed ids and weights (run_logits)
  w.rw = m.max_rows * m.kr * 4;
  // BF16 h of one W8A16 decode pass (at most kDecodeRows rows)
  w.hb = std::min<int64_t>(m.max_rows, kDecodeRows) * m.k * m.Ip * 2;
  // FP32 gate|up of one pass for the exact-tie quantiser (Ip == 128 only)
  w.gu = m.exact_ties() ? m.P * 2 * m.Ip * 4 : 0;
  return w;
}

// Gate|up row norms kept with the weights for the exact-tie quantiser.
int64_t norm_bytes_of(const Dims& m) { return m.exact_ties() ? m.E * 2 * m.Ip * 4 : 0; }

int64_t weight_bytes_of(const Dims& m) {
  const int64_t codes = m.E * (2 * m.Ip * m.H + m.H * m.Ip);
  const int64_t scales = m.E * (2 * m.nI * m.nH + m.nH * m.nI) * 4;
  return align256(codes) + align256(scales) + align256(norm_bytes_of(m));
}

struct StageEvents {
  hipEvent_t ev[MOE_NUM_STAGES + 1];
  uint32_t mask;  // stages timed in this pass
};

// Event b sits between stage b - 1 and stage b; it is needed when either is timed.
bool boundary_needed(uint32_t mask, int b) {
  return (b > 0 && ((mask >> (b - 1)) & 1u)) || (b < MOE_NUM_STAGES && ((mask >> b) & 1u));
}

// Per-pass device buffers (pieces of WsSizes).
struct Workspace {
  uint8_t* xq = nullptr;
  float* sx = nullptr;
  float* sxT = nullptr;
  uint8_t* hq = nullptr;
  uint16_t* hb = nullptr;  // W8A16 decode: BF16 h
  float* sh = nullptr;
  float* shT = nullptr;
  float* y = nullptr;
  int32_t* counts = nullptr;
  int32_t* offsets = nullptr;
  int32_t* perm = nullptr;
  int32_t* inv = nullptr;
  Tile* small_tiles = nullptr;
  Tile* narrow_tiles = nullptr;
  Tile* wide_tiles = nullptr;
  int32_t* n_tiles = nullptr;
  int32_t* chunk = nullptr;
  int32_t* rids = nullptr;
  float* rw = nullptr;
  float* gu = nullptr;  // exact-tie layers: FP32 gate|up of a pass
};

// The pieces of w laid out one after the other (256-byte aligned) from base.
Workspace carve(const WsSizes& w, uint8_t* base) {
  Workspace ws;
  auto take = [&](int64_t bytes) -> void* {
    void* p = bytes > 0 ? (void*)base : nullptr;
    base += align256(bytes);
    return p;
  };
  ws.xq = (uint8_t*)take(w.xq);
  ws.sx = (float*)take(w.sx);
  ws.sxT = (float*)take(w.sxT);
  ws.hq = (uint8_t*)take(w.hq);
  ws.sh = (float*)take(w.sh);
  ws.shT = (float*)take(w.shT);
  ws.y = (float*)take(w.y);
  ws.counts = (int32_t*)take(w.counts);
  ws.offsets = (int32_t*)take(w.offsets);
  ws.perm = (int32_t*)take(w.perm);
  ws.inv = (int32_t*)take(w.inv);
  ws.small_tiles = (Tile*)take(w.small_tiles);
  ws.narrow_tiles = (Tile*)take(w.narrow_tiles);
  ws.wide_tiles = (Tile*)take(w.wide_tiles);
  ws.n_tiles = (int32_t*)take(w.n_tiles);
  ws.chunk = (int32_t*)take(w.chunk);
  take(w.err);
  ws.rids = (int32_t*)take(w.rids);
  ws.rw = (float*)take(w.rw);
  ws.hb = (uint16_t*)take(w.hb);
  ws.gu = (float*)take(w.gu);
  return ws;
}

// The workspace of run_static() for passes of `rows` rows: run()'s pieces
// without those of run_logits() and the decode path.
WsSizes static_sizes(const Dims& m, int64_t rows) {
  Dims r = m;
  r.max_rows = rows;
  r.P = rows * m.k;
  WsSizes w = ws_sizes(r);
  w.rids = w.rw = w.hb = 0;
  return w;
}

// The most rows (<= max_rows) whose static_sizes fit kStaticScratchBytes, or 0.
int64_t static_rows_of(const Dims& m) {
  int64_t lo = 0, hi = m.max_rows;  // fits(lo) (or lo == 0), find the largest
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (static_sizes(m, mid).total() <= kStaticScratchBytes) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace

struct moe_fp8_prefill {
  moe_fp8_prefill_desc desc;
  Dims m;
  int device = 0;
  int num_cus = 256;
  // weights
  uint8_t* w13 = nullptr;
  float* s13 = nullptr;
  uint8_t* w2 = nullptr;
  float* s2 = nullptr;
  float* n13 = nullptr;  // exact-tie layers: gate|up row norms
  // workspace for max_rows rows (allocated in create) and the bad-id flag
  Workspace ws;
  int32_t* err = nullptr;
  // run_static(): this device's static scratch array and the rows per pass
  // its workspace holds
  uint8_t* scratch = nullptr;
  int64_t static_rows = 0;
  std::vector<void*> allocations;
  // state
  std::atomic<int> busy{0};
  bool failed = false;
  bool inject_failure = false;
  hipEvent_t done = nullptr;
  // streamed layer slots (create_streamed); n_slots == 0 for a resident handle
  struct Slot {
    uint8_t* w13 = nullptr;
    float* s13 = nullptr;
    uint8_t* w2 = nullptr;
    float* s2 = nullptr;
    float* n13 = nullptr;
    hipEvent_t ready = nullptr;  // recorded when its staging has been enqueued
    hipEvent_t free = nullptr;   // recorded after the last pass that read it
    bool staged = false;
    bool used = false;
  };
  int n_slots = 0;
  int active = 0;
  Slot slots[2];
  uint8_t* stage_codes = nullptr;  // one group of experts in the canonical layout
  float* stage_scales = nullptr;
  uint8_t* stage_full_codes = nullptr;  // the same at full checkpoint width (shares)
  float* stage_full_scales = nullptr;
  hipEvent_t stage_done = nullptr;  // orders stage() calls made on different streams
  bool staged_once = false;
  hipStream_t last_stream = nullptr;
  bool has_last = false;
  int64_t last_T = 0;  // rows of the last pass
  // timing
  uint32_t timing = 0;  // mask of timed stages
  std::vector<StageEvents> pending;
  std::vector<StageEvents> free_events;
};

namespace {

int fail(moe_fp8_prefill* h, int code = MOE_ERR_DEVICE) {
  if (h) h->failed = true;
  return code;
}

hipError_t dalloc(moe_fp8_prefill* h, void** p, int64_t bytes) {
  *p = nullptr;
  hipError_t e = hipMalloc(p, (size_t)(bytes > 0 ? bytes : 1));
  if (e == hipSuccess) h->allocations.push_back(*p);
  return e;
}

void free_all(moe_fp8_prefill* h) {
  for (void* p : h->allocations) (void)hipFree(p);
  h->allocations.clear();
  if (h->done) (void)hipEventDestroy(h->done);
  for (auto& sl : h->slots) {
    if (sl.ready) (void)hipEventDestroy(sl.ready);
    if (sl.free) (void)hipEventDestroy(sl.free);
  }
  if (h->stage_done) (void)hipEventDestroy(h->stage_done);
  for (auto& s : h->pending)
    for (auto ev : s.ev) (void)hipEventDestroy(ev);
  for (auto& s : h->free_events)
    for (auto ev : s.ev) (void)hipEventDestroy(ev);
  h->pending.clear();
  h->free_events.clear();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Upload experts [e0, e0+n) from canonical buffers (host or device) and
// re-lay them out into the handle's weight arrays.
constexpr int64_t kStageGroup = 8;  // experts per staging copy

// Staging buffers for one group of experts: the canonical layout of the
// handle's I (`codes`, `scales`), and, when the handle takes a share of a
// wider checkpoint, of the full width (`full_codes`, `full_scales`).
struct Staging {
  uint8_t* codes = nullptr;
  float* scales = nullptr;
  uint8_t* full_codes = nullptr;
  float* full_scales = nullptr;
};

bool slicing(const Dims& m) { return m.I_full != m.I; }

// Device bytes of the staging buffers (codes, scales, full codes, full scales).
void staging_bytes(const Dims& m, bool src_on_device, int64_t out[4]) {
  const int64_t n = m.E < kStageGroup ? m.E : kStageGroup;
  const int64_t sc = (m.I + 127) / 128 * m.nH, scf = (m.I_full + 127) / 128 * m.nH;
  out[0] = 3 * m.I * m.H * n;
  out[1] = 3 * sc * n * 4;
  out[2] = slicing(m) && !src_on_device ? 3 * m.I_full * m.H * n : 0;
  out[3] = slicing(m) && !src_on_device ? 3 * scf * n * 4 : 0;
}

// Experts [0, E) of a layer in the checkpoint layout (the full width I_full
// when the handle takes a share) -> (w13, s13, w2, s2), a group of experts at
// a time: copied to the device (host source), cut to the share and
// requantised if it is unaligned, re-laid out.  Everything is enqueued on s
// in order, so each staging buffer is reused only after the kernels that
// read it; no host synchronisation.
int enqueue_upload(moe_fp8_prefill* h, const uint8_t* gate, const uint8_t* up, const uint8_t* down,
                   const float* gate_scale, const float* up_scale, const float* down_scale,
                   bool src_on_device, uint8_t* w13, float* s13, uint8_t* w2, float* s2, float* n13,
                   const Staging& st, hipStream_t s) {
  const Dims& m = h->m;
  const int64_t wfull = m.I_full * m.H, sfull = (m.I_full + 127) / 128 * m.nH;
  const int64_t wcode = m.I * m.H, wscale = (m.I + 127) / 128 * m.nH;
  const hipMemcpyKind kind = src_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;
  for (int64_t e0 = 0; e0 < m.E; e0 += kStageGroup) {
    const int64_t n = (m.E - e0) < kStageGroup ? (m.E - e0) : kStageGroup;
    // this group's source, in the checkpoint layout at full width
    const uint8_t* src[3] = {gate + e0 * wfull, up + e0 * wfull, down + e0 * wfull};
    const float* ssrc[3] = {gate_scale + e0 * sfull, up_scale + e0 * sfull, down_scale + e0 * sfull};
    uint8_t* dst[3] = {st.codes, st.codes + wcode * n, st.codes + 2 * wcode * n};
    float* sdst[3] = {st.scales, st.scales + wscale * n, st.scales + 2 * wscale * n};
    if (!slicing(m) && src_on_device) {
      for (int i = 0; i < 3; ++i) {
        dst[i] = const_cast<uint8_t*>(src[i]);
        sdst[i] = const_cast<float*>(ssrc[i]);
      }
    } else if (!slicing(m)) {
      for (int i = 0; i < 3; ++i)
        if (hipMemcpyAsync(dst[i], src[i], (size_t)(wcode * n), kind, s) != hipSuccess ||
            hipMemcpyAsync(sdst[i], ssrc[i], (size_t)(wscale * n * 4), kind, s) != hipSuccess)
          return MOE_ERR_DEVICE;
    } else {
      if (!src_on_device) {
        for (int i = 0; i < 3; ++i) {
          uint8_t* fc = st.full_codes + i * wfull * n;
          float* fs = st.full_scales + i * sfull * n;
          if (hipMemcpyAsync(fc, src[i], (size_t)(wfull * n), kind, s) != hipSuccess ||
              hipMemcpyAsync(fs, ssrc[i], (size_t)(sfull * n * 4), kind, s) != hipSuccess)
            return MOE_ERR_DEVICE;
          src[i] = fc;
          ssrc[i] = fs;
        }
      }
      for (int i = 0; i < 3; ++i) {
        // gate / up: [I][H], share of the rows; down: [H][I], share of the columns
        SliceArgs sa{src[i], ssrc[i], (int32_t)n, (int32_t)(i < 2 ? m.I_full : m.H),
                     (int32_t)(i < 2 ? m.H : m.I_full), i < 2 ? 0 : 1, (int32_t)m.I_off, (int32_t)m.I,
                     dst[i], sdst[i]};
        if (launch_slice(sa, s) != hipSuccess) return MOE_ERR_DEVICE;
      }
    }
    LayoutArgs a{dst[0], dst[1], dst[2], sdst[0], sdst[1], sdst[2], (int32_t)e0, (int32_t)n, (int32_t)m.H,
                 (int32_t)m.I, (int32_t)m.Ip, w13, s13, w2, s2, n13};
    if (launch_layout(a, s) != hipSuccess) return MOE_ERR_DEVICE;
  }
  return MOE_OK;
}

// Allocates `st` (recorded in the handle's allocation list if `keep`, else
// in `temp` for the caller to free).
int alloc_staging(moe_fp8_prefill* h, bool src_on_device, Staging* st, std::vector<void*>* temp) {
  int64_t bytes[4];
  staging_bytes(h->m, src_on_device, bytes);
  void** slots[4] = {(void**)&st->codes, (void**)&st->scales, (void**)&st->full_codes,
                     (void**)&st->full_scales};
  for (int i = 0; i < 4; ++i) {
    if (bytes[i] == 0) continue;
    if (hipMalloc(slots[i], (size_t)bytes[i]) != hipSuccess) return MOE_ERR_OUT_OF_MEMORY;
    (temp ? *temp : h->allocations).push_back(*slots[i]);
  }
  return MOE_OK;
}

int upload_weights(moe_fp8_prefill* h, hipStream_t s) {
  const moe_fp8_prefill_desc* d = &h->desc;
  const bool on_dev = d->weights_on_device != 0;
  Staging st;
  std::vector<void*> temp;
  int rc = MOE_OK;
  if (!(on_dev && !slicing(h->m))) rc = alloc_staging(h, on_dev, &st, &temp);
  if (rc == MOE_OK)
    rc = enqueue_upload(h, d->gate, d->up, d->down, d->gate_scale, d->up_scale, d->down_scale, on_dev,
                        h->w13, h->s13, h->w2, h->s2, h->n13, st, s);
  if (hipStreamSynchronize(s) != hipSuccess && rc == MOE_OK) rc = MOE_ERR_DEVICE;
  for (void* p : temp) (void)hipFree(p);
  return rc;
}

// Grid of a persistent GEMM launch: enough resident workgroups to fill the
// chip, never more than the largest possible number of work items.
int gemm_grid(const moe_fp8_prefill* h, int64_t max_items, int kind, bool gate_up) {
  const int64_t per_cu = kind != kGemmStream ? 1 : (gate_up ? kGateUpWgPerCu : kDownWgPerCu);
  return (int)std::max<int64_t>(1, std::min<int64_t>(max_items, h->num_cus * per_cu));
}

// Most tiles of one pass in each list (the kernels read the real counts).
int64_t max_tiles(const Dims& m, int64_t P, int kind) {
  if (kind == kGemmStream) return std::min<int64_t>(m.E, P);
  if (kind == kGemmNarrow) return std::min<int64_t>(m.E, P / (kSmallRows + 1));
  return P / kWideRows + std::min<int64_t>(m.E, P / (kNarrowRows + 1));
}

// The gate_up launches of a pass over t rows / P slots whose plan and
// activations are in the workspace: streaming tiles (experts with 1..16
// rows), 128-row tiles (17..128 rows), then tiles of up to 256 rows.
// after[kind], if given and not null, is recorded after each of the three
// (also when a launch is skipped for lack of work).
hipError_t launch_gate_up_all(moe_fp8_prefill* h, const Workspace& ws, int64_t t, int64_t P, float* gu_dbg, hipStream_t s,
                              hipEvent_t* after = nullptr) {
  const Dims& m = h->m;
  const int64_t nb = m.Ip / kBlock;
  // layers with one h group per row: the GEMMs write FP32 gate|up, which the
  // exact-tie quantiser turns into h codes and scales after the last launch
  if (m.exact_ties() && !gu_dbg) gu_dbg = ws.gu;
  GateUpArgs ga{ws.xq, ws.sx, t * m.H, t * m.nH * 4, ws.perm, (int32_t)m.k, (int32_t)m.H, (int32_t)m.Ip,
                h->w13, h->s13, ws.small_tiles, ws.n_tiles, ws.hq, ws.sh, gu_dbg,
                h->desc.activation == MOE_ACT_SILU_CLAMPED ? h->desc.activation_limit : 0.0f,
                ws.sxT, t * m.nH * 4, (int32_t)t, (int32_t)P, ws.shT};
  Tile* lists[3] = {ws.small_tiles, ws.narrow_tiles, ws.wide_tiles};
  for (int kind = kGemmStream; kind <= kGemmWide; ++kind) {
    const int64_t items = max_tiles(m, P, kind) * nb;
    if (items > 0) {
      ga.tiles = lists[kind];
      ga.n_tiles = ws.n_tiles + kind;
      hipError_t e = launch_gate_up(ga, kind, gemm_grid(h, items, kind, true), s);
      if (e != hipSuccess) return e;
    }
    if (kind == kGemmWide && m.exact_ties()) {
      const float limit = h->desc.activation == MOE_ACT_SILU_CLAMPED ? h->desc.activation_limit : 0.0f;
      TieArgs ta{gu_dbg, ws.xq, ws.sx, ws.perm, ws.offsets, (int32_t)m.E, (int32_t)m.k, (int32_t)m.H,
                 h->w13, h->s13, h->n13, ws.hq, ws.sh, ws.shT, limit,
                 kTieMargin / sqrtf((float)m.nH)};
      hipError_t e = launch_tie_exact(ta, P, s);
      if (e != hipSuccess) return e;
    }
    if (after && after[kind]) {
      hipError_t e = hipEventRecord(after[kind], s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// The down launches, in the same order.
hipError_t launch_down_all(moe_fp8_prefill* h, const Workspace& ws, int64_t P, hipStream_t s, hipEvent_t* after = nullptr) {
  const Dims& m = h->m;
  const int64_t nb = m.H / kBlock, nb2 = (nb + 1) / 2;
  DownArgs da{ws.hq, ws.sh, P * m.Ip, P * m.nI * 4, (int32_t)m.H, (int32_t)m.Ip, h->w2, h->s2,
              ws.small_tiles, ws.n_tiles, ws.y, ws.shT, P * m.nI * 4, (int32_t)P, nullptr};
  Tile* lists[3] = {ws.small_tiles, ws.narrow_tiles, ws.wide_tiles};
  for (int kind = kGemmStream; kind <= kGemmWide; ++kind) {
    // the 128-row and the 256-row tiles run in one launch of the same
    // kernel (after[kGemmNarrow] is then recorded before it)
    const int64_t items = kind == kGemmStream ? max_tiles(m, P, kind) * nb
                          : kind == kGemmWide ? (max_tiles(m, P, kGemmNarrow) + max_tiles(m, P, kGemmWide)) * nb2
                                              : 0;
    if (items > 0) {
      da.tiles = lists[kind == kGemmWide ? kGemmNarrow : kind];
      da.n_tiles = ws.n_tiles + (kind == kGemmWide ? kGemmNarrow : kind);
      da.tiles2 = kind == kGemmWide ? ws.wide_tiles : nullptr;
      hipError_t e = launch_down(da, kind, gemm_grid(h, items, kind, false), s);
      if (e != hipSuccess) return e;
    }
    if (after && after[kind]) {
      hipError_t e = hipEventRecord(after[kind], s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

#ifndef MOE_STAGE_EVENT_FLAGS
#define MOE_STAGE_EVENT_FLAGS hipEventDisableSystemFence
#endif
constexpr unsigned kStageEventFlags = MOE_STAGE_EVENT_FLAGS;

int get_stage_events(moe_fp8_prefill* h, StageEvents* out) {
  if (!h->free_events.empty()) {
    *out = h->free_events.back();
    h->free_events.pop_back();
    return MOE_OK;
  }
  // timing only, on this device: no system-scope release (which would write
  // the L2 back at every stage boundary and slow the next launch)
  for (int i = 0; i <= MOE_NUM_STAGES; ++i)
    if (hipEventCreateWithFlags(&out->ev[i], kStageEventFlags) != hipSuccess) return MOE_ERR_DEVICE;
  return MOE_OK;
}

// Checks and per-call stream handling shared by run() and run_logits(),
// then the passes.  Exactly one of (ids, w) and logits is given.
// The W8A16 gate_up and down of one pass over t rows / P slots (the plan is
// in the workspace), with the events of the timed stages: gate_up and down
// take the streaming slots, the other GEMM slots record empty intervals.
hipError_t launch_a16(moe_fp8_prefill* h, const Workspace& ws, const uint16_t* x, int64_t t, int64_t P, hipStream_t s, hipEvent_t* at) {
  const Dims& m = h->m;
  const int64_t max_tiles16 = P / 16 + m.E;  // tiles of <= 16 rows over all lists
  GateUpA16Args ga{x, t * m.H * 2, ws.perm, (int32_t)m.k, (int32_t)m.H, (int32_t)m.Ip, h->w13, h->s13,
                   {ws.small_tiles, ws.narrow_tiles, ws.wide_tiles}, ws.n_tiles, ws.hb,
                   h->desc.activation == MOE_ACT_SILU_CLAMPED ? h->desc.activation_limit : 0.0f};
  const int64_t cap = h->num_cus * kDecodeWgPerCu;
  hipError_t e = launch_gate_up_a16(ga, (int)std::max<int64_t>(1, std::min<int64_t>(max_tiles16 * (m.Ip / kBlock), cap)), s);
  if (e != hipSuccess) return e;
  for (int b = 3; b <= 5; ++b)
    if (at[b] && (e = hipEventRecord(at[b], s)) != hipSuccess) return e;
  DownA16Args da{ws.hb, P * m.Ip * 2, (int32_t)m.H, (int32_t)m.Ip, h->w2, h->s2,
                 {ws.small_tiles, ws.narrow_tiles, ws.wide_tiles}, ws.n_tiles, ws.y};
  e = launch_down_a16(da, (int)std::max<int64_t>(1, std::min<int64_t>(max_tiles16 * (m.H / kBlock), cap)), s);
  if (e != hipSuccess) return e;
  for (int b = 6; b <= 8; ++b)
    if (at[b] && (e = hipEventRecord(at[b], s)) != hipSuccess) return e;
  return hipSuccess;
}

int run_passes(moe_fp8_prefill* h, const Workspace& ws, int64_t pass_limit, const void* x, const int32_t* ids, const float* w,
               const float* logits, int32_t router, int64_t T, void* out, void* stream_, bool a16 = false) {
  if (!h) return MOE_ERR_INVALID_ARG;
  if (h->failed) return MOE_ERR_FAILED_STATE;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !out || !aligned16(x) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  if (logits ? (router != MOE_ROUTER_SOFTMAX && router != MOE_ROUTER_SIGMOID) : (!ids || !w))
    return MOE_ERR_INVALID_ARG;
  if (logits && h->m.kr > kRouteMaxK) return MOE_ERR_UNSUPPORTED;
  int expected = 0;
  if (!h->busy.compare_exchange_strong(expected, 1)) return MOE_ERR_BUSY;
  struct Release {
    std::atomic<int>& b;
    ~Release() { b.store(0); }
  } release{h->busy};

  hipStream_t s = (hipStream_t)stream_;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) return fail(h);
  if (cap != hipStreamCaptureStatusNone) return MOE_ERR_UNSUPPORTED;
  if (h->inject_failure) {
    h->inject_failure = false;
    return fail(h);
  }
  if (h->has_last && h->last_stream != s && hipStreamWaitEvent(s, h->done, 0) != hipSuccess)
    return fail(h);
  moe_fp8_prefill::Slot* slot = nullptr;
  if (h->n_slots) {
    slot = &h->slots[h->active];
    if (!slot->staged) return MOE_ERR_INVALID_ARG;
    if (hipStreamWaitEvent(s, slot->ready, 0) != hipSuccess) return fail(h);
  }

  const Dims& m = h->m;
  const int64_t out_elem = h->desc.out_dtype == MOE_DTYPE_F32 ? 4 : 2;

  const int64_t pass_rows = std::min<int64_t>(pass_limit, a16 ? std::min<int64_t>(m.max_rows, kDecodeRows) : m.max_rows);
  for (int64_t r0 = 0; r0 < T; r0 += pass_rows) {
    const int64_t t = (T - r0) < pass_rows ? (T - r0) : pass_rows;
    const int64_t P = t * m.k;
    StageEvents ev{};
    hipEvent_t at[MOE_NUM_STAGES + 1] = {};  // the boundaries this pass records
    if (h->timing) {
      if (get_stage_events(h, &ev) != MOE_OK) return fail(h);
      ev.mask = h->timing;
      for (int b = 0; b <= MOE_NUM_STAGES; ++b)
        if (boundary_needed(ev.mask, b)) at[b] = ev.ev[b];
      if (at[0] && hipEventRecord(at[0], s) != hipSuccess) return fail(h);
    }
    const int32_t* ids_p = ids ? ids + r0 * m.kr : ws.rids;
    const float* w_p = w ? w + r0 * m.kr : ws.rw;
    if (logits) {
      RouteArgs ra{logits + r0 * m.Er, t, (int32_t)m.Er, (int32_t)m.kr, router, ws.rids, ws.rw};
      if (launch_route(ra, s) != hipSuccess) return fail(h);
    }
    PlanArgs pa{ids_p, (int32_t)t, (int32_t)m.k, (int32_t)m.E, (int32_t)m.kr, (int32_t)m.Er,
                ws.counts, ws.offsets, ws.perm, ws.inv, ws.small_tiles,
                ws.narrow_tiles, ws.wide_tiles, ws.n_tiles, h->err, ws.chunk};
    if (launch_plan(pa, s) != hipSuccess) return fail(h);
    if (at[1] && hipEventRecord(at[1], s) != hipSuccess) return fail(h);

    if (a16) {
      // W8A16: no activation quantisation; one gate_up and one down launch
      // over all tiles (timed in the streaming slots)
      if (at[2] && hipEventRecord(at[2], s) != hipSuccess) return fail(h);
      if (launch_a16(h, ws, (const uint16_t*)x + r0 * m.H, t, P, s, at) != hipSuccess) return fail(h);
    } else {
      QuantArgs qa{(const uint16_t*)x + r0 * m.H, (int32_t)t, (int32_t)m.H, ws.xq, ws.sx, ws.sxT};
      if (launch_quant(qa, s) != hipSuccess) return fail(h);
      if (at[2] && hipEventRecord(at[2], s) != hipSuccess) return fail(h);

      if (launch_gate_up_all(h, ws, t, P, nullptr, s, &at[3]) != hipSuccess) return fail(h);
      if (launch_down_all(h, ws, P, s, &at[6]) != hipSuccess) return fail(h);
    }

    CombineArgs ca{ws.y, ws.inv, w_p, (int32_t)t, (int32_t)m.k, (int32_t)m.H, (int32_t)m.kr,
                   h->desc.routed_scale, h->desc.out_dtype == MOE_DTYPE_F32 ? 1 : 0,
                   (uint8_t*)out + r0 * m.H * out_elem};
    if (launch_combine(ca, s) != hipSuccess) return fail(h);
    if (h->timing) {
      if (at[MOE_NUM_STAGES] && hipEventRecord(at[MOE_NUM_STAGES], s) != hipSuccess) return fail(h);
      h->pending.push_back(ev);
    }
    if (&ws == &h->ws) h->last_T = t;  // the inspection calls read the handle's workspace
  }
  if (hipEventRecord(h->done, s) != hipSuccess) return fail(h);
  if (slot) {
    if (hipEventRecord(slot->free, s) != hipSuccess) return fail(h);
    slot->used = true;
  }
  h->last_stream = s;
  h->has_last = true;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_fp8_prefill_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_OUT_OF_MEMORY: return "device out of memory";
    case MOE_ERR_DEVICE: return "device (HIP) error; handle failed";
    case MOE_ERR_FAILED_STATE: return "handle failed earlier and refuses work";
    case MOE_ERR_BUSY: return "handle is in use by another call";
    case MOE_ERR_BAD_EXPERT_ID: return "expert id >= number of experts (slot skipped)";
    default: return "unknown error code";
  }
}

int moe_fp8_prefill_validate(const moe_fp8_prefill_desc* d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (!desc_size_ok(d)) return MOE_ERR_INVALID_ARG;
  const int32_t shared = desc_shared(d);
  const float limit = desc_limit(d);
  const int32_t i_full = desc_inter_full(d), i_off = desc_inter_offset(d);
  if (i_full < 0 || (i_full == 0 && i_off != 0)) return MOE_ERR_INVALID_ARG;
  if (i_full > 0 && (i_off < 0 || d->inter < 1 || (int64_t)i_off + d->inter > i_full)) return MOE_ERR_INVALID_ARG;
  if (i_full > kMaxKBlocks * kBlock) return MOE_ERR_UNSUPPORTED;
  if (shared != 0 && shared != 1) return MOE_ERR_UNSUPPORTED;
  if (!d->gate || !d->up || !d->down || !d->gate_scale || !d->up_scale || !d->down_scale)
    return MOE_ERR_INVALID_ARG;
  if (d->num_experts < 1 || d->top_k < 1 || d->hidden < 1 || d->inter < 1 || d->max_rows < 1)
    return MOE_ERR_INVALID_ARG;
  if (d->block != kBlock) return MOE_ERR_UNSUPPORTED;
  if (d->activation != MOE_ACT_SILU_UNCLAMPED && d->activation != MOE_ACT_SILU_CLAMPED)
    return MOE_ERR_UNSUPPORTED;
  if (d->activation == MOE_ACT_SILU_CLAMPED ? !(std::isfinite(limit) && limit > 0.0f) : limit != 0.0f)
    return MOE_ERR_INVALID_ARG;
  if (d->out_dtype != MOE_DTYPE_BF16 && d->out_dtype != MOE_DTYPE_F32) return MOE_ERR_UNSUPPORTED;
  if (d->hidden % kBlock != 0) return MOE_ERR_UNSUPPORTED;
  if (d->hidden > kMaxKBlocks * kBlock || d->inter > kMaxKBlocks * kBlock) return MOE_ERR_UNSUPPORTED;
  if (d->num_experts + shared > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (d->top_k > d->num_experts || d->top_k > 256) return MOE_ERR_UNSUPPORTED;
  if (!std::isfinite(d->routed_scale)) return MOE_ERR_INVALID_ARG;
  const Dims m = dims_of(d);
  // 32-bit buffer offsets inside one pass: activations, h, and one expert's
  // weight block row
  if (m.P >= (int64_t(1) << 31) || m.max_rows * m.H >= (int64_t(1) << 31) ||
      m.P * m.Ip >= (int64_t(1) << 31) || m.Ip * m.H >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int64_t moe_fp8_prefill_workspace_bytes(const moe_fp8_prefill_desc* d) {
  const int rc = moe_fp8_prefill_validate(d);
  if (rc != MOE_OK) return -rc;
  return ws_sizes(dims_of(d)).total();
}

int64_t moe_fp8_prefill_weight_bytes(const moe_fp8_prefill_desc* d) {
  const int rc = moe_fp8_prefill_validate(d);
  if (rc != MOE_OK) return -rc;
  return weight_bytes_of(dims_of(d));
}

int moe_fp8_prefill_create(const moe_fp8_prefill_desc* d, moe_fp8_prefill** out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  const int rc = moe_fp8_prefill_validate(d);
  if (rc != MOE_OK) return rc;
  moe_fp8_prefill* h = new (std::nothrow) moe_fp8_prefill();
  if (!h) return MOE_ERR_OUT_OF_MEMORY;
  // a caller's description may end before shared_experts: copy what it has
  memcpy(&h->desc, d, (size_t)d->struct_size);
  h->desc.shared_experts = desc_shared(d);
  h->desc.activation_limit = desc_limit(d);
  h->desc.inter_full = desc_inter_full(d);
  h->desc.inter_offset = desc_inter_offset(d);
  h->desc.struct_size = (int32_t)sizeof(moe_fp8_prefill_desc);
  h->m = dims_of(d);
  const Dims& m = h->m;
  if (hipGetDevice(&h->device) != hipSuccess) {
    delete h;
    return MOE_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, h->device) == hipSuccess && prop.multiProcessorCount > 0)
    h->num_cus = prop.multiProcessorCount;
  if (static_scratch(&h->scratch) != hipSuccess) h->scratch = nullptr;  // run_static() then refuses
  h->static_rows = static_rows_of(m);

  const WsSizes w = ws_sizes(m);
  void* p;
  bool ok = true;
  auto get = [&](int64_t bytes) -> void* {
    if (!ok) return nullptr;
    if (dalloc(h, &p, bytes) != hipSuccess) {
      ok = false;
      return nullptr;
    }
    return p;
  };
  h->w13 = (uint8_t*)get(m.E * 2 * m.Ip * m.H);
  h->s13 = (float*)get(m.E * m.nI * m.nH * 2 * 4);
  h->w2 = (uint8_t*)get(m.E * m.H * m.Ip);
  h->s2 = (float*)get(m.E * m.nH * m.nI * 4);
  if (m.exact_ties()) h->n13 = (float*)get(norm_bytes_of(m));
  h->ws.xq = (uint8_t*)get(w.xq);
  h->ws.sx = (float*)get(w.sx);
  h->ws.sxT = (float*)get(w.sxT);
  h->ws.hq = (uint8_t*)get(w.hq);
  h->ws.sh = (float*)get(w.sh);
  h->ws.shT = (float*)get(w.shT);
  h->ws.y = (float*)get(w.y);
  h->ws.counts = (int32_t*)get(w.counts);
  h->ws.offsets = (int32_t*)get(w.offsets);
  h->ws.perm = (int32_t*)get(w.perm);
  h->ws.inv = (int32_t*)get(w.inv);
  h->ws.small_tiles = (Tile*)get(w.small_tiles);
  h->ws.narrow_tiles = (Tile*)get(w.narrow_tiles);
  h->ws.wide_tiles = (Tile*)get(w.wide_tiles);
  h->ws.n_tiles = (int32_t*)get(w.n_tiles);
  h->ws.chunk = (int32_t*)get(w.chunk);
  h->err = (int32_t*)get(w.err);
  h->ws.rids = (int32_t*)get(w.rids);
  h->ws.rw = (float*)get(w.rw);
  h->ws.hb = (uint16_t*)get(w.hb);
  if (m.exact_ties()) h->ws.gu = (float*)get(w.gu);
  if (!ok) {
    free_all(h);
    delete h;
    return MOE_ERR_OUT_OF_MEMORY;
  }
  hipStream_t s = (hipStream_t)d->stream;
  if (hipEventCreateWithFlags(&h->done, hipEventDisableTiming) != hipSuccess ||
      hipMemsetAsync(h->err, 0, 4, s) != hipSuccess) {
    free_all(h);
    delete h;
    return MOE_ERR_DEVICE;
  }
  const int up = upload_weights(h, s);
  if (up != MOE_OK || hipStreamSynchronize(s) != hipSuccess) {
    free_all(h);
    delete h;
    return up != MOE_OK ? up : MOE_ERR_DEVICE;
  }
  // the caller's weight pointers are not kept
  h->desc.gate = h->desc.up = h->desc.down = nullptr;
  h->desc.gate_scale = h->desc.up_scale = h->desc.down_scale = nullptr;
  *out = h;
  return MOE_OK;
}

int moe_fp8_prefill_run(moe_fp8_prefill* h, const void* x, const int32_t* ids, const float* w,
                        int64_t T, void* out, void* stream) {
  if (!h) return MOE_ERR_INVALID_ARG;
  return run_passes(h, h->ws, h->m.max_rows, x, ids, w, nullptr, 0, T, out, stream);
}

int moe_fp8_prefill_run_static(moe_fp8_prefill* h, const void* x, const int32_t* ids, const float* w,
                               int64_t T, void* out, void* stream) {
  if (!h) return MOE_ERR_INVALID_ARG;
  if (!h->scratch) return h->failed ? MOE_ERR_FAILED_STATE : MOE_ERR_DEVICE;  // its address was not found
  if (h->static_rows < 1) return MOE_ERR_UNSUPPORTED;  // not one row's workspace fits the array
  const Workspace ws = carve(static_sizes(h->m, h->static_rows), h->scratch);
  return run_passes(h, ws, h->static_rows, x, ids, w, nullptr, 0, T, out, stream);
}

int moe_fp8_prefill_run_decode(moe_fp8_prefill* h, const void* x, const int32_t* ids, const float* w,
                               int64_t T, void* out, void* stream) {
  if (!h) return MOE_ERR_INVALID_ARG;
  return run_passes(h, h->ws, h->m.max_rows, x, ids, w, nullptr, 0, T, out, stream, true);
}

int moe_fp8_prefill_run_logits(moe_fp8_prefill* h, const void* x, const float* logits,
                               int32_t router, int64_t T, void* out, void* stream) {
  if (!logits) return MOE_ERR_INVALID_ARG;
  if (!h) return MOE_ERR_INVALID_ARG;
  return run_passes(h, h->ws, h->m.max_rows, x, nullptr, nullptr, logits, router, T, out, stream);
}

int moe_fp8_prefill_route(moe_fp8_prefill* h, const float* logits, int32_t router, int64_t T,
                          int32_t* ids, float* w, void* stream) {
  if (!h) return MOE_ERR_INVALID_ARG;
  if (h->failed) return MOE_ERR_FAILED_STATE;
  if (T < 0 || (T > 0 && (!logits || !ids || !w))) return MOE_ERR_INVALID_ARG;
  if (router != MOE_ROUTER_SOFTMAX && router != MOE_ROUTER_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (h->m.kr > kRouteMaxK) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  RouteArgs ra{logits, T, (int32_t)h->m.Er, (int32_t)h->m.kr, router, ids, w};
  if (launch_route(ra, (hipStream_t)stream) != hipSuccess) return fail(h);
  return MOE_OK;
}

int moe_fp8_prefill_status(moe_fp8_prefill* h) {
  if (!h) return MOE_ERR_INVALID_ARG;
  if (h->failed) return MOE_ERR_FAILED_STATE;
  if (h->has_last && hipEventSynchronize(h->done) != hipSuccess) return fail(h);
  int32_t e = 0;
  if (hipMemcpy(&e, h->err, 4, hipMemcpyDeviceToHost) != hipSuccess) return fail(h);
  if (e) {
    if (hipMemset(h->err, 0, 4) != hipSuccess) return fail(h);
    return MOE_ERR_BAD_EXPERT_ID;
  }
  return MOE_OK;
}

void moe_fp8_prefill_destroy(moe_fp8_prefill* h) {
  if (!h) return;
  if (h->has_last) (void)hipEventSynchronize(h->done);
  (void)hipDeviceSynchronize();
  free_all(h);
  delete h;
}

int moe_fp8_prefill_debug_plan(moe_fp8_prefill* h, int32_t* counts, int32_t* offsets, int32_t* perm,
                               int32_t* inv, int64_t cap) {
  if (!h || !counts || !offsets || !perm || !inv) return MOE_ERR_INVALID_ARG;
  if (h->failed) return MOE_ERR_FAILED_STATE;
  const int64_t P = h->last_T * h->m.k;
  if (cap < P) return MOE_ERR_INVALID_ARG;
  if (hipDeviceSynchronize() != hipSuccess) return fail(h);
  const int64_t E = h->m.E;
  if (hipMemcpy(counts, h->ws.counts, E * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(offsets, h->ws.offsets, (E + 1) * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(h);
  const int64_t routed = offsets[E];
  if (routed > P) return fail(h);
  if ((routed > 0 && hipMemcpy(perm, h->ws.perm, routed * 4, hipMemcpyDeviceToHost) != hipSuccess) ||
      (P > 0 && hipMemcpy(inv, h->ws.inv, P * 4, hipMemcpyDeviceToHost) != hipSuccess))
    return fail(h);
  return MOE_OK;
}

int moe_fp8_prefill_debug_activations(moe_fp8_prefill* h, uint8_t* xq, float* sx, int64_t rows) {
  if (!h || !xq || !sx || rows < 0 || rows > h->last_T) return MOE_ERR_INVALID_ARG;
  if (h->failed) return MOE_ERR_FAILED_STATE;
  if (hipDeviceSynchronize() != hipSuccess) return fail(h);
  if (rows == 0) return MOE_OK;
  if (hipMemcpy(xq, h->ws.xq, rows * h->m.H, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(sx, h->ws.sx, rows * h->m.nH * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(h);
  return MOE_OK;
}

int moe_fp8_prefill_debug_intermediates(moe_fp8_prefill* h, uint8_t* hq, float* sh, float* y,
                                        int64_t cap_rows, int64_t* n_rows) {
  if (!h || !n_rows) return MOE_ERR_INVALID_ARG;
  if (h->failed) return MOE_ERR_FAILED_STATE;
  if (hipDeviceSynchronize() != hipSuccess) return fail(h);
  int32_t routed = 0;
  if (hipMemcpy(&routed, h->ws.offsets + h->m.E, 4, hipMemcpyDeviceToHost) != hipSuccess) return fail(h);
  *n_rows = routed;
  if (routed > cap_rows) return MOE_ERR_INVALID_ARG;
  if (routed == 0) return MOE_OK;
  const Dims& m = h->m;
  if ((hq && hipMemcpy(hq, h->ws.hq, routed * m.Ip, hipMemcpyDeviceToHost) != hipSuccess) ||
      (sh && hipMemcpy(sh, h->ws.sh, routed * m.nI * 4, hipMemcpyDeviceToHost) != hipSuccess) ||
      (y && hipMemcpy(y, h->ws.y, routed * m.H * 4, hipMemcpyDeviceToHost) != hipSuccess))
    return fail(h);
  return MOE_OK;
}

int moe_fp8_prefill_debug_gate_up(moe_fp8_prefill* h, float* gu, int64_t cap_rows, int64_t* n_rows) {
  if (!h || !gu || !n_rows) return MOE_ERR_INVALID_ARG;
  if (h->failed) return MOE_ERR_FAILED_STATE;
  if (hipDeviceSynchronize() != hipSuccess) return fail(h);
  int32_t routed = 0;
  if (hipMemcpy(&routed, h->ws.offsets + h->m.E, 4, hipMemcpyDeviceToHost) != hipSuccess) return fail(h);
  *n_rows = routed;
  if (routed > cap_rows) return MOE_ERR_INVALID_ARG;
  if (routed == 0) return MOE_OK;
  const int64_t bytes = (int64_t)routed * 2 * h->m.Ip * 4;
  float* dbg = nullptr;
  if (hipMalloc((void**)&dbg, (size_t)bytes) != hipSuccess) return MOE_ERR_OUT_OF_MEMORY;
  // re-run the last pass's gate_up (deterministic: rewrites identical h)
  int rc = MOE_OK;
  if (launch_gate_up_all(h, h->ws, h->last_T, h->last_T * h->m.k, dbg, nullptr) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(gu, dbg, (size_t)bytes, hipMemcpyDeviceToHost) != hipSuccess)
    rc = fail(h);
  (void)hipFree(dbg);
  return rc;
}

int moe_fp8_prefill_debug_unpack(moe_fp8_prefill* h, int32_t e, uint8_t* gate, uint8_t* up,
                                 uint8_t* down, float* gate_scale, float* up_scale, float* down_scale) {
  if (!h || !gate || !up || !down || !gate_scale || !up_scale || !down_scale) return MOE_ERR_INVALID_ARG;
  const Dims& m = h->m;
  if (e < 0 || e >= m.E) return MOE_ERR_INVALID_ARG;
  if (h->failed) return MOE_ERR_FAILED_STATE;
  if (hipDeviceSynchronize() != hipSuccess) return fail(h);
  const int64_t n13 = 2 * m.Ip * m.H, n2 = m.H * m.Ip;
  std::vector<uint8_t> b13((size_t)n13), b2((size_t)n2);
  std::vector<float> s13((size_t)(m.nI * m.nH * 2)), s2((size_t)(m.nH * m.nI));
  if (hipMemcpy(b13.data(), h->w13 + e * n13, n13, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(b2.data(), h->w2 + e * n2, n2, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(s13.data(), h->s13 + e * m.nI * m.nH * 2, s13.size() * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(s2.data(), h->s2 + e * m.nH * m.nI, s2.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(h);
  // inverse of the layout kernels' index map
  const int64_t nH = m.nH, nI = m.nI, NB13 = m.nI, NB2 = m.nH;
  for (int64_t nb = 0; nb < NB13; ++nb)
    for (int64_t kb = 0; kb < nH; ++kb)
      for (int w = 0; w < 4; ++w)
        for (int t = 0; t < 4; ++t)
          for (int half = 0; half < 2; ++half)
            for (int lane = 0; lane < 64; ++lane) {
              const int64_t row = nb * 128 + w * 32 + (t & 1) * 16 + (lane & 15);
              if (row >= m.I) continue;
              const int64_t k0 = kb * 128 + (lane >> 4) * 32 + half * 16;
              const int64_t src = ((((nb * nH + kb) * 4 + w) * 4 + t) * 2 + half) * 1024 + lane * 16;
              uint8_t* dst = (t < 2 ? gate : up) + row * m.H + k0;
              std::memcpy(dst, &b13[(size_t)src], 16);
            }
  for (int64_t nb = 0; nb < NB2; ++nb)
    for (int64_t kb = 0; kb < nI; ++kb)
      for (int w = 0; w < 4; ++w)
        for (int t = 0; t < 2; ++t)
          for (int half = 0; half < 2; ++half)
            for (int lane = 0; lane < 64; ++lane) {
              const int64_t row = nb * 128 + w * 32 + t * 16 + (lane & 15);
              const int64_t k0 = kb * 128 + (lane >> 4) * 32 + half * 16;
              const int64_t src = ((((nb * nI + kb) * 4 + w) * 2 + t) * 2 + half) * 1024 + lane * 16;
              for (int i = 0; i < 16; ++i)
                if (k0 + i < m.I) down[row * m.I + k0 + i] = b2[(size_t)src + i];
            }
  const int64_t nIr = (m.I + 127) / 128;  // == nI
  for (int64_t i = 0; i < nIr * nH; ++i) {
    gate_scale[i] = s13[(size_t)i * 2];
    up_scale[i] = s13[(size_t)i * 2 + 1];
  }
  for (int64_t i = 0; i < nH * nI; ++i) down_scale[i] = s2[(size_t)i];
  return MOE_OK;
}

int moe_fp8_prefill_debug_mfma(const uint8_t* a, const uint8_t* b, float* d) {
  if (!a || !b || !d) return MOE_ERR_INVALID_ARG;
  uint8_t *da = nullptr, *db = nullptr;
  float* dd = nullptr;
  int rc = MOE_OK;
  if (hipMalloc((void**)&da, 2048) != hipSuccess || hipMalloc((void**)&db, 2048) != hipSuccess ||
      hipMalloc((void**)&dd, 3072) != hipSuccess) {
    rc = MOE_ERR_OUT_OF_MEMORY;
  } else if (hipMemcpy(da, a, 2048, hipMemcpyHostToDevice) != hipSuccess ||
             hipMemcpy(db, b, 2048, hipMemcpyHostToDevice) != hipSuccess ||
             launch_mfma_probe(da, db, dd, nullptr) != hipSuccess ||
             hipMemcpy(d, dd, 3072, hipMemcpyDeviceToHost) != hipSuccess) {
    rc = MOE_ERR_DEVICE;
  }
  if (da) (void)hipFree(da);
  if (db) (void)hipFree(db);
  if (dd) (void)hipFree(dd);
  return rc;
}

int moe_fp8_prefill_calibrate(int32_t kind, int64_t n, void* buf, int64_t buf_bytes, void* stream,
                              double* work) {
  constexpr int64_t kResultBytes = 64 * 1024;
  if (kind != MOE_CALIBRATE_MFMA && kind != MOE_CALIBRATE_STREAM) return MOE_ERR_INVALID_ARG;
  if (!buf || !work || ((uintptr_t)buf & 15u) != 0 || buf_bytes < kResultBytes) return MOE_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MOE_ERR_DEVICE;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* result = (uint8_t*)buf + (buf_bytes - kResultBytes);
  if (kind == MOE_CALIBRATE_MFMA) {
    if (n < 1 || n > (int64_t(1) << 30)) return MOE_ERR_INVALID_ARG;
    const int grid = 2 * cus;  // 8 waves per CU: two per SIMD
    if (grid * 4 * 4 > kResultBytes) return MOE_ERR_UNSUPPORTED;
    if (launch_peak_mfma((int32_t)n, grid, (float*)result, s) != hipSuccess) return MOE_ERR_DEVICE;
    *work = (double)grid * 4 * (double)n * 8 * (2.0 * 16 * 16 * 128);
    return MOE_OK;
  }
  if (kind == MOE_CALIBRATE_STREAM) {
    const int64_t bytes = (buf_bytes - kResultBytes) & ~int64_t(15);
    if (bytes <= 0) return MOE_ERR_INVALID_ARG;
    const int grid = 4 * cus;
    if (grid * 4 > kResultBytes) return MOE_ERR_UNSUPPORTED;
    int64_t read = 0;
    if (launch_peak_stream(buf, bytes, grid, (int32_t*)result, &read, s) != hipSuccess) return MOE_ERR_DEVICE;
    *work = (double)read;
    return MOE_OK;
  }
  return MOE_ERR_INVALID_ARG;
}

int moe_fp8_prefill_set_timing(moe_fp8_prefill* h, int32_t enable) {
  if (!h) return MOE_ERR_INVALID_ARG;
  h->timing = enable != 0 ? (1u << MOE_NUM_STAGES) - 1u : 0u;
  return MOE_OK;
}

int moe_fp8_prefill_set_timing_stages(moe_fp8_prefill* h, uint32_t stage_mask) {
  if (!h || (stage_mask >> MOE_NUM_STAGES) != 0) return MOE_ERR_INVALID_ARG;
  h->timing = stage_mask;
  return MOE_OK;
}

int moe_fp8_prefill_read_timing(moe_fp8_prefill* h, float* stage_ms, int32_t max_records,
                                int32_t* n_records) {
  if (!h || !n_records || (max_records > 0 && !stage_ms)) return MOE_ERR_INVALID_ARG;
  if (h->failed) return MOE_ERR_FAILED_STATE;
  int32_t n = 0;
  for (auto& s : h->pending) {
    int last = MOE_NUM_STAGES;
    while (!boundary_needed(s.mask, last)) --last;
    if (hipEventSynchronize(s.ev[last]) != hipSuccess) return fail(h);
    if (n < max_records) {
      for (int i = 0; i < MOE_NUM_STAGES; ++i) {
        float ms = -1.f;
        if (((s.mask >> i) & 1u) && hipEventElapsedTime(&ms, s.ev[i], s.ev[i + 1]) != hipSuccess) return fail(h);
        stage_ms[n * MOE_NUM_STAGES + i] = ms;
      }
      ++n;
    }
    h->free_events.push_back(s);
  }
  h->pending.clear();
  *n_records = n;
  return MOE_OK;
}

int moe_fp8_prefill_debug_inject_failure(moe_fp8_prefill* h) {
  if (!h) return MOE_ERR_INVALID_ARG;
  h->inject_failure = true;
  return MOE_OK;
}

int moe_fp8_prefill_create_streamed(const moe_fp8_prefill_desc* d, int32_t n_slots,
                                    moe_fp8_prefill** out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  if (!d || (n_slots != 1 && n_slots != 2)) return MOE_ERR_INVALID_ARG;
  // the description's weight pointers are not used: validate a copy with
  // placeholders in them
  moe_fp8_prefill_desc v;
  memset(&v, 0, sizeof(v));
  if (!desc_size_ok(d)) return MOE_ERR_INVALID_ARG;
  memcpy(&v, d, (size_t)d->struct_size);
  v.struct_size = (int32_t)sizeof(v);
  v.shared_experts = desc_shared(d);
  v.activation_limit = desc_limit(d);
  v.inter_full = desc_inter_full(d);
  v.inter_offset = desc_inter_offset(d);
  static const uint8_t placeholder[16] = {0};
  v.gate = v.up = v.down = placeholder;
  v.gate_scale = v.up_scale = v.down_scale = (const float*)placeholder;
  v.weights_on_device = 0;
  const int rc = moe_fp8_prefill_validate(&v);
  if (rc != MOE_OK) return rc;
  moe_fp8_prefill* h = new (std::nothrow) moe_fp8_prefill();
  if (!h) return MOE_ERR_OUT_OF_MEMORY;
  h->desc = v;
  h->desc.gate = h->desc.up = h->desc.down = nullptr;
  h->desc.gate_scale = h->desc.up_scale = h->desc.down_scale = nullptr;
  h->m = dims_of(&v);
  const Dims& m = h->m;
  if (hipGetDevice(&h->device) != hipSuccess) {
    delete h;
    return MOE_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, h->device) == hipSuccess && prop.multiProcessorCount > 0)
    h->num_cus = prop.multiProcessorCount;
  if (static_scratch(&h->scratch) != hipSuccess) h->scratch = nullptr;  // run_static() then refuses
  h->static_rows = static_rows_of(m);
  const WsSizes w = ws_sizes(m);
  void* p;
  bool ok = true;
  auto get = [&](int64_t bytes) -> void* {
    if (!ok) return nullptr;
    if (dalloc(h, &p, bytes) != hipSuccess) {
      ok = false;
      return nullptr;
    }
    return p;
  };
  h->n_slots = n_slots;
  for (int i = 0; i < n_slots; ++i) {
    h->slots[i].w13 = (uint8_t*)get(m.E * 2 * m.Ip * m.H);
    h->slots[i].s13 = (float*)get(m.E * m.nI * m.nH * 2 * 4);
    h->slots[i].w2 = (uint8_t*)get(m.E * m.H * m.Ip);
    h->slots[i].s2 = (float*)get(m.E * m.nH * m.nI * 4);
    if (m.exact_ties()) h->slots[i].n13 = (float*)get(norm_bytes_of(m));
  }
  if (ok) {
    Staging st;
    ok = alloc_staging(h, false, &st, nullptr) == MOE_OK;
    h->stage_codes = st.codes;
    h->stage_scales = st.scales;
    h->stage_full_codes = st.full_codes;
    h->stage_full_scales = st.full_scales;
  }
  h->ws.xq = (uint8_t*)get(w.xq);
  h->ws.sx = (float*)get(w.sx);
  h->ws.sxT = (float*)get(w.sxT);
  h->ws.hq = (uint8_t*)get(w.hq);
  h->ws.sh = (float*)get(w.sh);
  h->ws.shT = (float*)get(w.shT);
  h->ws.y = (float*)get(w.y);
  h->ws.counts = (int32_t*)get(w.counts);
  h->ws.offsets = (int32_t*)get(w.offsets);
  h->ws.perm = (int32_t*)get(w.perm);
  h->ws.inv = (int32_t*)get(w.inv);
  h->ws.small_tiles = (Tile*)get(w.small_tiles);
  h->ws.narrow_tiles = (Tile*)get(w.narrow_tiles);
  h->ws.wide_tiles = (Tile*)get(w.wide_tiles);
  h->ws.n_tiles = (int32_t*)get(w.n_tiles);
  h->ws.chunk = (int32_t*)get(w.chunk);
  h->err = (int32_t*)get(w.err);
  h->ws.rids = (int32_t*)get(w.rids);
  h->ws.rw = (float*)get(w.rw);
  h->ws.hb = (uint16_t*)get(w.hb);
  if (m.exact_ties()) h->ws.gu = (float*)get(w.gu);
  if (!ok) {
    free_all(h);
    delete h;
    return MOE_ERR_OUT_OF_MEMORY;
  }
  bool ev_ok = hipEventCreateWithFlags(&h->done, hipEventDisableTiming) == hipSuccess &&
               hipEventCreateWithFlags(&h->stage_done, hipEventDisableTiming) == hipSuccess;
  for (int i = 0; i < n_slots && ev_ok; ++i)
    ev_ok = hipEventCreateWithFlags(&h->slots[i].ready, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&h->slots[i].free, hipEventDisableTiming) == hipSuccess;
  hipStream_t s = (hipStream_t)v.stream;
  if (!ev_ok || hipMemsetAsync(h->err, 0, 4, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess) {
    free_all(h);
    delete h;
    return MOE_ERR_DEVICE;
  }
  h->w13 = h->slots[0].w13;
  h->s13 = h->slots[0].s13;
  h->w2 = h->slots[0].w2;
  h->s2 = h->slots[0].s2;
  h->n13 = h->slots[0].n13;
  *out = h;
  return MOE_OK;
}

int moe_fp8_prefill_stage(moe_fp8_prefill* h, int32_t slot, const uint8_t* gate, const uint8_t* up,
                          const uint8_t* down, const float* gate_scale, const float* up_scale,
                          const float* down_scale, void* stream_) {
  if (!h) return MOE_ERR_INVALID_ARG;
  if (h->failed) return MOE_ERR_FAILED_STATE;
  if (!h->n_slots || slot < 0 || slot >= h->n_slots) return MOE_ERR_INVALID_ARG;
  if (!gate || !up || !down || !gate_scale || !up_scale || !down_scale) return MOE_ERR_INVALID_ARG;
  int expected = 0;
  if (!h->busy.compare_exchange_strong(expected, 1)) return MOE_ERR_BUSY;
  struct Release {
    std::atomic<int>& b;
    ~Release() { b.store(0); }
  } release{h->busy};
  hipStream_t s = (hipStream_t)stream_;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) return fail(h);
  if (cap != hipStreamCaptureStatusNone) return MOE_ERR_UNSUPPORTED;
  if (h->inject_failure) {
    h->inject_failure = false;
    return fail(h);
  }
  moe_fp8_prefill::Slot& sl = h->slots[slot];
  // stream-ordered reuse: the passes that read this slot, and the previous
  // staging (it owns the staging buffers), come first
  if (sl.used && hipStreamWaitEvent(s, sl.free, 0) != hipSuccess) return fail(h);
  if (h->staged_once && hipStreamWaitEvent(s, h->stage_done, 0) != hipSuccess) return fail(h);
  Staging st;
  st.codes = h->stage_codes;
  st.scales = h->stage_scales;
  st.full_codes = h->stage_full_codes;
  st.full_scales = h->stage_full_scales;
  const int rc = enqueue_upload(h, gate, up, down, gate_scale, up_scale, down_scale, false, sl.w13, sl.s13,
                                sl.w2, sl.s2, sl.n13, st, s);
  if (rc != MOE_OK) return fail(h, rc);
  if (hipEventRecord(sl.ready, s) != hipSuccess || hipEventRecord(h->stage_done, s) != hipSuccess)
    return fail(h);
  sl.staged = true;
  h->staged_once = true;
  return MOE_OK;
}

int moe_fp8_prefill_select_slot(moe_fp8_prefill* h, int32_t slot) {
  if (!h) return MOE_ERR_INVALID_ARG;
  if (h->failed) return MOE_ERR_FAILED_STATE;
  if (!h->n_slots || slot < 0 || slot >= h->n_slots || !h->slots[slot].staged) return MOE_ERR_INVALID_ARG;
  int expected = 0;
  if (!h->busy.compare_exchange_strong(expected, 1)) return MOE_ERR_BUSY;
  h->active = slot;
  h->w13 = h->slots[slot].w13;
  h->s13 = h->slots[slot].s13;
  h->w2 = h->slots[slot].w2;
  h->s2 = h->slots[slot].s2;
  h->n13 = h->slots[slot].n13;
  h->busy.store(0);
  return MOE_OK;
}

}  // extern "C"
