/*
 * moe_fp8_prefill: the routed-expert FFN of a top-k mixture-of-experts layer
 * during prompt prefill, on one MI355X (gfx950), as a C-ABI library.
 *
 * The method (sources are the pages' titles and sections):
 *   - "ktransformers #2244" (Full GLM-5.3 streamed FP8 GPU prefill), Design:
 *     prefill runs W8A8 on the GPU: E4M3 expert weights with block scales and
 *     FP8 activations; full GLM uses unclamped SiLU; routed scaling is kept;
 *     all weights and scales are reserved up front in one per-layer slot;
 *     stream-ordered reuse; fail closed after a staging failure; unsupported
 *     dimensions / activation / quantisation and CUDA-graph capture are
 *     rejected; expert arithmetic is tiled without repeating weight transfer.
 *   - "hpc-ops #80" (GLM-4.6-FP8 on H20), gap table row 6: blockwise FP8 MoE
 *     (per-128x128 weight blocks) instead of per-tensor scales, which saturate
 *     on outlier tokens; a non-128-multiple intermediate size is zero-padded.
 *   - "ktransformers #2245" (Exact AVX2 FP8 arithmetic conversion), Semantics
 *     and scope: E4M3 decode; NaN codes act as signed zeros.
 *   - "TensorFold #2852" (a whole prompt pass routes its experts in one call),
 *     description and exactness paragraph: plan, grouped gate+up, gate-up
 *     epilogue, grouped down, combine; a skip id that is never loaded; the
 *     whole K accumulated in one pass (no split-K) and a deterministic member
 *     order, so a row's bits do not depend on how many rows share a call.
 *
 * What run() computes, for token t (rho = routed scale):
 *   out[t] = cast( rho * sum_{j<k} w[t,j] * y[t,j] )            (FP32 sum, ascending j)
 *   y[t,j] = D_e . Q( silu(G_e . Q(x[t])) * (U_e . Q(x[t])) ),  e = ids[t,j]
 * Q = dynamic E4M3 quantisation per row and per 128-column group
 *     (s = max|v| / 448, q = round-to-nearest-even(v / s), saturating at 448);
 * G_e, U_e, D_e = the expert's E4M3 matrices with FP32 128x128 block scales;
 * each product is accumulated in FP32, K block by K block, each block's dot
 * multiplied by (activation scale * weight scale).  silu(z) = z / (1 + e^-z).
 *
 * Error behaviour: every call returns an MOE_* code.  A HIP failure inside
 * create or run leaves the handle FAILED: every later run returns
 * MOE_ERR_FAILED_STATE (fail closed).  Expert ids >= E are skipped and
 * reported by moe_fp8_prefill_status() as MOE_ERR_BAD_EXPERT_ID.
 */
#ifndef MOE_FP8_PREFILL_H_
#define MOE_FP8_PREFILL_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* null / misaligned pointer, negative size, bad struct_size */
  MOE_ERR_UNSUPPORTED = 2,   /* dimensions, activation, block or dtype outside the method */
  MOE_ERR_OUT_OF_MEMORY = 3, /* device allocation failed in create */
  MOE_ERR_DEVICE = 4,        /* a HIP call failed; the handle is now FAILED */
  MOE_ERR_FAILED_STATE = 5,  /* the handle failed earlier and refuses work */
  MOE_ERR_BUSY = 6,          /* another thread is inside run() on this handle */
  MOE_ERR_BAD_EXPERT_ID = 7  /* a routed id was >= E; those slots were skipped */
};

enum { MOE_DTYPE_BF16 = 0, MOE_DTYPE_F32 = 1 };
/* Activations: full GLM's unclamped SiLU ("ktransformers #2244", Design), or
 * the clamped variant GLM-5.3-Flash uses, whose formula the pages leave
 * open; here the limit L is a parameter: gate capped at L, up clipped to
 * [-L, L], then silu(gate) * up (NaN passes through). */
enum { MOE_ACT_SILU_UNCLAMPED = 0, MOE_ACT_SILU_CLAMPED = 1 };
enum { MOE_ROUTER_SOFTMAX = 0, MOE_ROUTER_SIGMOID = 1 };

/*
 * Layer description for create().  Weight layout is the checkpoint's:
 *   gate, up   : u8 [E][I][H]   E4M3 codes, row = intermediate feature
 *   down       : u8 [E][H][I]   E4M3 codes, row = hidden feature
 *   gate_scale, up_scale : f32 [E][ceil(I/128)][H/128]   block (row blk, col blk)
 *   down_scale           : f32 [E][H/128][ceil(I/128)]
 * A block (nb, kb) covers rows 128*nb.. and columns 128*kb..; edge blocks of a
 * non-128-multiple I are partial.  Pointers are host memory unless
 * weights_on_device != 0 (then device memory on the current device).  The
 * library copies and re-lays out the weights; the caller may free its copies
 * once create() returns.
 */
typedef struct moe_fp8_prefill_desc {
  int32_t struct_size;      /* sizeof(moe_fp8_prefill_desc), or the size up to
                               shared_experts, activation_limit or inter_full
                               (older callers) */
  int32_t num_experts;      /* E, 1..1024 */
  int32_t top_k;            /* k, 1..min(E, 256) */
  int32_t hidden;           /* H, multiple of 128 */
  int32_t inter;            /* I >= 1; padded to Ip = 128*ceil(I/128) with zero codes */
  int32_t max_rows;         /* rows per internal pass; run() chunks larger T */
  int32_t out_dtype;        /* MOE_DTYPE_BF16 or MOE_DTYPE_F32 */
  int32_t activation;       /* MOE_ACT_SILU_UNCLAMPED or MOE_ACT_SILU_CLAMPED */
  int32_t block;            /* 128 */
  float routed_scale;       /* rho, finite */
  int32_t weights_on_device;
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  const float* gate_scale;
  const float* up_scale;
  const float* down_scale;
  void* stream;             /* hipStream_t used for the upload; NULL = null stream */
  /* Always-on shared expert, 0 or 1 ("TensorFold #2852": nine slots planned
   * over E+1 expert ids).  With 1, every weight and scale array holds E+1
   * experts and expert E is the shared one: each token gets a (k+1)-th slot
   * on it with weight 1, computed in the same grouped GEMMs and added after
   * the routed sum is scaled by routed_scale:
   *   out[t] = cast( rho * sum_{j<k} w[t,j] * y[t,j]  +  y_shared[t] ).
   * ids and w stay [T][k]; a routed id >= E (including E) is a bad id.  A
   * caller built before this field (struct_size without it) gets 0. */
  int32_t shared_experts;
  /* L of MOE_ACT_SILU_CLAMPED: finite and > 0 (ten for GLM-5.3-Flash); must
   * be 0 with MOE_ACT_SILU_UNCLAMPED.  Absent (older struct_size) = 0. */
  float activation_limit;
  /* Load-time share of a wider checkpoint ("hpc-ops #80", gap table row 6: a
   * tensor-parallel rank's 192 of the intermediate features, zero-padded to
   * 256, with a load-time weight requant).  inter_full > 0: the weight arrays
   * hold inter_full intermediate features (gate/up rows, down columns, scale
   * grids ceil(inter_full/128) wide) and the layer uses features
   * [inter_offset, inter_offset + inter).  A share starting on a multiple of
   * 128 keeps the checkpoint's codes and block scales; otherwise each of its
   * 128x128 blocks is requantised at load: v = dec(code) * S in FP32,
   * s = max|v| / 448, code = E4M3(v / s) (round to nearest even).
   * inter_full = 0 (and inter_offset = 0): the arrays hold exactly inter. */
  int32_t inter_full;
  int32_t inter_offset;
} moe_fp8_prefill_desc;

typedef struct moe_fp8_prefill moe_fp8_prefill;

/* Checks a description on the host: no GPU call, no allocation ("ktransformers
 * #2244", Design: unsupported dimensions, activation or quantisation are
 * rejected up front).  Returns MOE_OK, MOE_ERR_INVALID_ARG or
 * MOE_ERR_UNSUPPORTED. */
int moe_fp8_prefill_validate(const moe_fp8_prefill_desc* d);

/* Device bytes create() will allocate for workspace (all of it is reserved up
 * front; run() allocates nothing: "ktransformers #2244", Design, one slot
 * reserved before anything else claims the memory), and for the re-laid-out
 * weights.  Negative (minus an MOE_* code) for an invalid description. */
int64_t moe_fp8_prefill_workspace_bytes(const moe_fp8_prefill_desc* d);
int64_t moe_fp8_prefill_weight_bytes(const moe_fp8_prefill_desc* d);

/* Validates, allocates weights + workspace on the current device, uploads
 * and re-lays out the weights (NaN codes 0x7F/0xFF become 0x00/0x80:
 * "ktransformers #2245", Semantics and scope; the I edge is zero-padded:
 * "hpc-ops #80", gap table row 6), then synchronises.  *out stays NULL on
 * error. */
int moe_fp8_prefill_create(const moe_fp8_prefill_desc* d, moe_fp8_prefill** out);

/*
 * One prefill pass over T tokens ("TensorFold #2852", description: one call
 * plans, runs the grouped gate+up with its epilogue, the grouped down and the
 * combine for a whole prompt pass; "ktransformers #2244", Design: W8A8 with
 * routed scaling), asynchronous on `stream` (hipStream_t; NULL = null
 * stream).  All pointers are device memory owned by the caller and must
 * stay valid until the stream passes this call:
 *   x     : bf16 [T][H], 16-byte aligned
 *   ids   : i32 [T][k]; id < 0 is a skip slot (never loaded); id >= E is
 *           skipped and flagged (see status)
 *   w     : f32 [T][k] routing weights (used as given)
 *   out   : [T][H] of out_dtype, 16-byte aligned
 * T = 0 is a no-op.  T > max_rows is processed in passes of max_rows rows; a
 * row's result does not depend on T, on the chunking or on the other rows.
 * No allocation, no host synchronisation.  A different stream from the last
 * call waits on that call first.  Returns MOE_ERR_UNSUPPORTED while the stream
 * is capturing, MOE_ERR_BUSY on concurrent use of one handle.
 */
int moe_fp8_prefill_run(moe_fp8_prefill* h, const void* x, const int32_t* ids,
                        const float* w, int64_t T, void* out, void* stream);

/*
 * run() for callers that cannot allocate device memory or whose workspace
 * must not come from the handle: code that records work for later replay,
 * tight serving loops, harnesses that forbid allocation.  Same computation,
 * arguments, stream rules and errors as run(), and the same output bits.
 * The per-pass workspace (activation codes and scales, plan, tile lists, h
 * and y) lives in one static device array of MOE_STATIC_SCRATCH_BYTES that the
 * library holds on every device it runs on until the process ends, instead
 * of the handle's workspace; nothing is allocated and the host does not
 * wait.  T rows run in passes of at most R rows, R the largest row count (at
 * most max_rows) whose workspace fits the array (about 300 rows for E=256,
 * top-8, H=6144, I=2048; every description validate() accepts fits at least
 * three rows); a layer whose single row would not fit is refused with
 * MOE_ERR_UNSUPPORTED.  MOE_ERR_DEVICE if the array's address could not be
 * found when the handle was created.  The array is shared by every handle
 * and call on a device and keeps the last call's contents (no part of it
 * needs to start at zero): calls that overlap on one GPU, from other
 * streams, threads or handles, race, and the caller must order them.  The
 * inspection calls keep describing the last pass run in the handle's own
 * workspace.
 */
#define MOE_STATIC_SCRATCH_BYTES (64ll << 20)
int moe_fp8_prefill_run_static(moe_fp8_prefill* h, const void* x, const int32_t* ids, const float* w,
                               int64_t T, void* out, void* stream);

/*
 * The decode path: the same layer in its W8A16 form, which the pages use for
 * decode and continuations shorter than 256 tokens ("ktransformers #2244",
 * Design: prefill of >= 256 tokens runs W8A8 on the GPU, shorter
 * continuations and decode W8A16).  The activations entering each GEMM stay
 * 16-bit: x as given (BF16) and h = silu(g) * u rounded to BF16 (nearest
 * even); each 128-wide K block is an FP32 dot of activations and decoded
 * weight codes times the weight block scale, accumulated in FP32 in ascending
 * block order; the combine is run()'s.  Arguments, ownership, stream rules
 * and errors as run(); T > min(max_rows, 1024) rows run in passes of that
 * size, and a row's output bits depend on neither its neighbours nor the
 * pass split.  The result differs from run() (no activation quantisation):
 * the two are different methods, each exact to its own definition.
 */
int moe_fp8_prefill_run_decode(moe_fp8_prefill* h, const void* x, const int32_t* ids,
                               const float* w, int64_t T, void* out, void* stream);

/*
 * The top-k router, on the device ("hpc-ops #80", gap table: the router's
 * top-k belongs to the fused MoE step; "TensorFold #2852": routed slots in
 * descending score).  For each token: the k experts with the largest logits,
 * in descending order, ties to the lower expert id, a NaN logit below every
 * number (sigmoid and exp are increasing, so this is the order of the scores;
 * +0 and -0 are equal).  Weights in FP32, normalised over the chosen experts:
 *   MOE_ROUTER_SOFTMAX: s_j = exp(l_j - l_0), w_j = s_j / sum(s)
 *   MOE_ROUTER_SIGMOID: s_j = 1 / (1 + exp(-l_j)), w_j = s_j / sum(s)
 * A chosen set with no mass (sum 0, or softmax with l_0 = -inf) gets zero
 * weights.  logits : f32 [T][E], ids : i32 [T][k], w : f32 [T][k], device
 * memory owned by the caller, on `stream`.  Needs k <= 64 (else
 * MOE_ERR_UNSUPPORTED).  Touches no handle state besides the failed flag.
 */
int moe_fp8_prefill_route(moe_fp8_prefill* h, const float* logits, int32_t router, int64_t T,
                          int32_t* ids, float* w, void* stream);

/*
 * run() from router logits: each pass routes its rows with the router above
 * into the handle's workspace, then runs plan .. combine on those ids and
 * weights.  Same rules as run(); logits : f32 [T][E] device memory.  The
 * output equals run() given the ids and weights moe_fp8_prefill_route()
 * returns for the same logits, bit for bit.
 */
int moe_fp8_prefill_run_logits(moe_fp8_prefill* h, const void* x, const float* logits,
                               int32_t router, int64_t T, void* out, void* stream);

/*
 * Streamed layer slots ("ktransformers #2244", Design: one reusable per-layer
 * slot that the host refills layer after layer; synchronise before reusing a
 * slot; fail closed after a staging failure).  create_streamed() validates
 * like create() but ignores the description's weight pointers, and
 * allocates n_slots (1 or 2) device weight slots plus one staging buffer;
 * nothing is uploaded.
 *
 * stage() copies one layer's weights (host memory in the canonical layout of
 * the description; pinned memory lets the copy overlap other work) into
 * slot `slot` and re-lays them out there, asynchronously on `stream`.  It
 * first makes `stream` wait for the last run() that read that slot and for
 * the previous stage() (they share the staging buffer), so a slot is never
 * overwritten while a queued pass still reads it.  The host arrays must stay
 * valid until the stream passes the call.  A HIP failure leaves the handle
 * FAILED.
 *
 * select_slot() (host only) picks the slot that later run() / run_logits()
 * calls compute with; they wait for that slot's staging.  A slot that was
 * never staged is MOE_ERR_INVALID_ARG.  Slot 0 is selected at creation.
 */
int moe_fp8_prefill_create_streamed(const moe_fp8_prefill_desc* d, int32_t n_slots,
                                    moe_fp8_prefill** out);
int moe_fp8_prefill_stage(moe_fp8_prefill* h, int32_t slot, const uint8_t* gate, const uint8_t* up,
                          const uint8_t* down, const float* gate_scale, const float* up_scale,
                          const float* down_scale, void* stream);
int moe_fp8_prefill_select_slot(moe_fp8_prefill* h, int32_t slot);

/* Synchronises the handle's last stream; returns and clears device-detected
 * errors (MOE_ERR_BAD_EXPERT_ID: "TensorFold #2852", an id outside the layer
 * is never loaded), or MOE_ERR_FAILED_STATE ("ktransformers #2244", Design:
 * fail closed), else MOE_OK. */
int moe_fp8_prefill_status(moe_fp8_prefill* h);

/* NULL-safe.  Synchronises, then frees everything (library plumbing: no
 * passage of the method). */
void moe_fp8_prefill_destroy(moe_fp8_prefill* h);

/* Static string for an MOE_* code. */
const char* moe_fp8_prefill_strerror(int code);

/* ---- inspection (synchronous; for tests and tooling) ------------------ */

/* The last pass's plan ("TensorFold #2852", description: the routing plan
 * that groups a pass's slots by expert), copied to host buffers: counts i32[E], offsets
 * i32[E+1], perm i32[cap] (sorted position -> slot t*k+j), inv i32[cap]
 * (slot -> sorted position or -1).  cap must be >= that pass's T*k.  With a
 * shared expert, E and k here count it (E+1 experts, k+1 slots per token,
 * the shared slot last). */
int moe_fp8_prefill_debug_plan(moe_fp8_prefill* h, int32_t* counts, int32_t* offsets,
                               int32_t* perm, int32_t* inv, int64_t cap);

/* The last pass's quantised activations (Q above: "ktransformers #2244",
 * Design, FP8 activations; "hpc-ops #80", gap table row 6, 128-wide groups):
 * xq u8[rows][H], sx f32[rows][H/128] (token order), rows = that pass's T. */
int moe_fp8_prefill_debug_activations(moe_fp8_prefill* h, uint8_t* xq, float* sx,
                                      int64_t rows);

/* The last pass's per-slot intermediates ("TensorFold #2852", description:
 * the gate-up epilogue's quantised h and the grouped down's FP32 rows) in
 * sorted order: hq u8[n][Ip],
 * sh f32[n][Ip/128], y f32[n][H]; n = number of routed slots (<= cap_rows).
 * Any pointer may be NULL. */
int moe_fp8_prefill_debug_intermediates(moe_fp8_prefill* h, uint8_t* hq, float* sh,
                                        float* y, int64_t cap_rows, int64_t* n_rows);

/* The last pass's FP32 gate and up outputs ("TensorFold #2852", the grouped
 * gate+up) before the SiLU / quantisation epilogue, gu f32[n][2*Ip] (gate columns then up columns, sorted order),
 * recomputed by re-running that pass's gate_up stage into a temporary device
 * buffer (this call allocates; it is an inspection tool). */
int moe_fp8_prefill_debug_gate_up(moe_fp8_prefill* h, float* gu, int64_t cap_rows,
                                  int64_t* n_rows);

/* Expert e's weights back in the canonical layout above (I rows / columns,
 * after NaN-code sanitising: "ktransformers #2245", Semantics and scope): gate, up u8[I][H]; down u8[H][I]; scales as in
 * the description.  Host buffers. */
int moe_fp8_prefill_debug_unpack(moe_fp8_prefill* h, int32_t e, uint8_t* gate, uint8_t* up,
                                 uint8_t* down, float* gate_scale, float* up_scale,
                                 float* down_scale);

/* One 16x16x128 FP8 MFMA through the library's operand convention (a
 * property of the hardware, checked by tests; no passage), on the current
 * device: d[0][i][n] = sum_c dec(a[i][c]) * dec(b[n][c]); d[1] is the
 * same product as four 16x16x32 FP8 MFMAs chained through the accumulator,
 * d[2] as four independent 16x16x32 MFMAs summed in FP32.  Host buffers
 * a u8[16][128], b u8[16][128], d f32[3][16][16]. */
int moe_fp8_prefill_debug_mfma(const uint8_t* a, const uint8_t* b, float* d);

/* Per-launch GPU timing with HIP events on the run stream (measurement
 * plumbing; the per-call protocol of "ktransformers #2245", Real-checkpoint
 * measurements, is the benchmark's).  When enabled,
 * every pass records events between its kernel launches; read_timing()
 * synchronises and returns up to max_records rows (one per pass) of
 * MOE_NUM_STAGES milliseconds: plan (with the router in run_logits),
 * quantise, gate_up of experts with 1-16 rows (streaming), 17-128 rows
 * (128-row tiles) and more rows (256-row tiles), down in the same three
 * groups, combine; then clears the record.  A group with no work in the
 * pass takes the time of an empty stream interval.  down's last two groups
 * run as one launch: its time is reported under the 256-row group and the
 * 128-row group takes an empty interval. */
#define MOE_NUM_STAGES 9
int moe_fp8_prefill_set_timing(moe_fp8_prefill* h, int32_t enable);
/* Timing of some stages only: events are recorded just at the boundaries of
 * the stages whose bit (1 << stage) is set in stage_mask, so a timed loop
 * can measure one launch with two events per pass instead of ten (each event
 * costs the stream ~2 us); read_timing() reports -1 for the other stages.
 * stage_mask 0 turns timing off; set_timing(h, 1) is the mask of all
 * stages.  Errors: MOE_ERR_INVALID_ARG for a NULL handle or bits at or past
 * MOE_NUM_STAGES. */
int moe_fp8_prefill_set_timing_stages(moe_fp8_prefill* h, uint32_t stage_mask);
int moe_fp8_prefill_read_timing(moe_fp8_prefill* h, float* stage_ms, int32_t max_records,
                                int32_t* n_records);

/* ---- calibration (measurement only, not part of the method) ---------- */

/* Measured ceilings for rooflines, on the current device, asynchronous on
 * `stream`; *work (host) receives the launch's algorithmic work.
 *   MOE_CALIBRATE_MFMA: a persistent launch (two waves per SIMD) of eight
 *     independent chains of the 16x16x128 FP8 MFMA the GEMMs issue, n
 *     iterations per wave (1 <= n <= 2^30); *work = FLOPs.
 *   MOE_CALIBRATE_STREAM: a streaming read of buf (at most its first
 *     buf_bytes - 64 KiB bytes, under 4 GiB, in whole 32 KiB chunks) with the
 *     16-byte buffer loads and cache policy of the GEMMs' weight stream;
 *     *work = bytes read.
 * buf: device memory owned by the caller, 16-byte aligned, at least 64 KiB;
 * its last 64 KiB receive results.  Time the launch with events on
 * `stream`.  Errors: MOE_ERR_INVALID_ARG (kind, n, buf), MOE_ERR_DEVICE. */
enum { MOE_CALIBRATE_MFMA = 0, MOE_CALIBRATE_STREAM = 1 };
int moe_fp8_prefill_calibrate(int32_t kind, int64_t n, void* buf, int64_t buf_bytes, void* stream,
                              double* work);

/* Test hook for the fail-closed rule ("ktransformers #2244", Design): force
 * the next run to behave as if a HIP call failed (host-side flag only; no GPU
 * fault is produced). */
int moe_fp8_prefill_debug_inject_failure(moe_fp8_prefill* h);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_PREFILL_H_ */
