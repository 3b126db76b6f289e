// Driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of the
// library's host code (fp8_blockwise_routed_amd/csrc/moe_api.cpp; the kernels
// are compiled in but never launched).  It exercises every path that needs no
// GPU: description validation (valid and each kind of invalid field, older
// struct sizes), the workspace and weight size queries, the error strings,
// create() where no device is usable, and every entry point with a null
// handle or null pointers.  Exit status 0 means no sanitizer report (reports
// abort the program) and every call returned its expected code.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "moe_fp8_prefill.h"

static int failures = 0;
#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

static const uint8_t kCodes[64] = {0};
static const float kScales[64] = {0};

static moe_fp8_prefill_desc base() {
  moe_fp8_prefill_desc d;
  std::memset(&d, 0, sizeof(d));
  d.struct_size = (int32_t)sizeof(d);
  d.num_experts = 8;
  d.top_k = 2;
  d.hidden = 256;
  d.inter = 192;
  d.max_rows = 64;
  d.out_dtype = MOE_DTYPE_BF16;
  d.activation = MOE_ACT_SILU_UNCLAMPED;
  d.block = 128;
  d.routed_scale = 2.5f;
  d.gate = d.up = d.down = kCodes;
  d.gate_scale = d.up_scale = d.down_scale = kScales;
  return d;
}

int main() {
  moe_fp8_prefill_desc d = base();
  CHECK(moe_fp8_prefill_validate(&d) == MOE_OK);
  CHECK(moe_fp8_prefill_workspace_bytes(&d) > 0);
  CHECK(moe_fp8_prefill_weight_bytes(&d) > 0);
  // one h group per row: the exact-tie quantiser's buffers are counted
  moe_fp8_prefill_desc one = base();
  one.inter = 128;
  CHECK(moe_fp8_prefill_workspace_bytes(&one) > 0);
  CHECK(moe_fp8_prefill_weight_bytes(&one) > 0);

  struct Bad {
    void (*edit)(moe_fp8_prefill_desc*);
    int expect;
  };
  const Bad bad[] = {
      {[](moe_fp8_prefill_desc* p) { p->struct_size = 12; }, MOE_ERR_INVALID_ARG},
      {[](moe_fp8_prefill_desc* p) { p->num_experts = 0; }, MOE_ERR_INVALID_ARG},
      {[](moe_fp8_prefill_desc* p) { p->top_k = 9; }, MOE_ERR_UNSUPPORTED},
      {[](moe_fp8_prefill_desc* p) { p->hidden = 200; }, MOE_ERR_UNSUPPORTED},
      {[](moe_fp8_prefill_desc* p) { p->hidden = 128 * 129; }, MOE_ERR_UNSUPPORTED},
      {[](moe_fp8_prefill_desc* p) { p->inter = 0; }, MOE_ERR_INVALID_ARG},
      {[](moe_fp8_prefill_desc* p) { p->max_rows = 0; }, MOE_ERR_INVALID_ARG},
      {[](moe_fp8_prefill_desc* p) { p->block = 64; }, MOE_ERR_UNSUPPORTED},
      {[](moe_fp8_prefill_desc* p) { p->out_dtype = 7; }, MOE_ERR_UNSUPPORTED},
      {[](moe_fp8_prefill_desc* p) { p->activation = 5; }, MOE_ERR_UNSUPPORTED},
      {[](moe_fp8_prefill_desc* p) { p->activation = MOE_ACT_SILU_CLAMPED; }, MOE_ERR_INVALID_ARG},
      {[](moe_fp8_prefill_desc* p) { p->activation_limit = 3.0f; }, MOE_ERR_INVALID_ARG},
      {[](moe_fp8_prefill_desc* p) { p->routed_scale = 1.0f / 0.0f; }, MOE_ERR_INVALID_ARG},
      {[](moe_fp8_prefill_desc* p) { p->gate = nullptr; }, MOE_ERR_INVALID_ARG},
      {[](moe_fp8_prefill_desc* p) { p->shared_experts = 2; }, MOE_ERR_UNSUPPORTED},
      {[](moe_fp8_prefill_desc* p) { p->num_experts = 1025; p->top_k = 2; }, MOE_ERR_UNSUPPORTED},
      {[](moe_fp8_prefill_desc* p) { p->inter_full = 100; p->inter_offset = 50; }, MOE_ERR_INVALID_ARG},
      {[](moe_fp8_prefill_desc* p) { p->inter_offset = 3; }, MOE_ERR_INVALID_ARG},
      {[](moe_fp8_prefill_desc* p) { p->max_rows = 1 << 30; }, MOE_ERR_UNSUPPORTED},
  };
  for (const Bad& b : bad) {
    moe_fp8_prefill_desc x = base();
    b.edit(&x);
    CHECK(moe_fp8_prefill_validate(&x) == b.expect);
    CHECK(moe_fp8_prefill_workspace_bytes(&x) < 0);
  }
  CHECK(moe_fp8_prefill_validate(nullptr) == MOE_ERR_INVALID_ARG);
  // callers built before the later fields
  moe_fp8_prefill_desc old = base();
  old.struct_size = (int32_t)offsetof(moe_fp8_prefill_desc, shared_experts);
  CHECK(moe_fp8_prefill_validate(&old) == MOE_OK);
  // a valid clamped share
  moe_fp8_prefill_desc share = base();
  share.activation = MOE_ACT_SILU_CLAMPED;
  share.activation_limit = 10.0f;
  share.inter_full = 1536;
  share.inter_offset = 192;
  CHECK(moe_fp8_prefill_validate(&share) == MOE_OK);

  for (int code = -1; code <= 8; ++code) CHECK(moe_fp8_prefill_strerror(code) != nullptr);

  // no usable device here: create refuses and leaves the handle null
  moe_fp8_prefill* h = reinterpret_cast<moe_fp8_prefill*>(0x1);
  const int rc = moe_fp8_prefill_create(&d, &h);
  CHECK(rc != MOE_OK && h == nullptr);
  moe_fp8_prefill* hs = reinterpret_cast<moe_fp8_prefill*>(0x1);
  CHECK(moe_fp8_prefill_create_streamed(&d, 3, &hs) == MOE_ERR_INVALID_ARG && hs == nullptr);
  CHECK(moe_fp8_prefill_create(nullptr, &h) != MOE_OK);
  CHECK(moe_fp8_prefill_create(&d, nullptr) == MOE_ERR_INVALID_ARG);

  // null handles
  float f[16] = {0};
  int32_t n = 0;
  int64_t rows = 0;
  CHECK(moe_fp8_prefill_run(nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_run_static(nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_run_decode(nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_run_logits(nullptr, nullptr, nullptr, 0, 1, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_route(nullptr, nullptr, 0, 1, nullptr, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_status(nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_stage(nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_select_slot(nullptr, 0) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_debug_plan(nullptr, nullptr, nullptr, nullptr, nullptr, 0) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_debug_activations(nullptr, nullptr, nullptr, 0) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_debug_intermediates(nullptr, nullptr, nullptr, nullptr, 0, &rows) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_debug_gate_up(nullptr, f, 1, &rows) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_debug_unpack(nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_set_timing(nullptr, 1) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_set_timing_stages(nullptr, 1u) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_read_timing(nullptr, f, 1, &n) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_debug_inject_failure(nullptr) == MOE_ERR_INVALID_ARG);
  double work = 0.0;
  CHECK(moe_fp8_prefill_calibrate(0, 1, nullptr, 1 << 20, nullptr, &work) == MOE_ERR_INVALID_ARG);
  CHECK(moe_fp8_prefill_calibrate(9, 1, f, 1 << 20, nullptr, &work) == MOE_ERR_INVALID_ARG);
  moe_fp8_prefill_destroy(nullptr);

  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("sanitized host API: ok\n");
  return 0;
}
