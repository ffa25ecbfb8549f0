// Host half of libkda under AddressSanitizer and UndefinedBehaviorSanitizer:
// the argument checks, the workspace query and the status strings, called
// with every kind of bad argument.  Every call here is rejected before any
// HIP call, so the fake device pointers are never dereferenced and no GPU is
// needed.  Exits 0 when every status is the documented one.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

static int failures = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}
#define FAKE ((void*)(uintptr_t)0x1000)
#define FAKEF ((const float*)(uintptr_t)0x1000)
#define FAKEI ((const int32_t*)(uintptr_t)0x1000)

static int dense_call(int64_t T, int32_t H, int32_t N, size_t wsb, float lb, const void* q,
                      const int32_t* cu) {
  return kda_chunk_prefill_fwd(q, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKEF, lb, 0.088f, NULL, cu,
                               FAKE, FAKE, FAKE, NULL, T, H, N, KDA_STATE_FP32, wsb);
}
static int dense(int64_t T, int32_t H, int32_t N, size_t wsb) {
  return dense_call(T, H, N, wsb, -5.f, FAKE, FAKEI);
}
static int dense_lb(float lb, size_t wsb) { return dense_call(16384, 16, 8, wsb, lb, FAKE, FAKEI); }

int main(void) {
  // workspace query: pure, zero for bad sizes, monotone
  expect(kda_get_workspace_size(-1, 16, 8) == 0, 1, "workspace size of negative tokens");
  expect(kda_get_workspace_size(10, 0, 8) == 0, 1, "workspace size of zero heads");
  size_t prev = 0;
  for (int32_t n = 1; n <= 4096; n *= 4) {
    const size_t w = kda_get_workspace_size(1 << 20, 64, n);
    expect(w >= prev, 1, "workspace size monotone in sequences");
    prev = w;
  }
  const size_t wsb = kda_get_workspace_size(16384, 16, 8);

  // the dense entry
  expect(dense_call(16384, 16, 8, wsb, -5.f, NULL, FAKEI), KDA_ERR_INVALID_ARG, "null q");
  expect(dense_call(16384, 16, 8, wsb, -5.f, FAKE, NULL), KDA_ERR_INVALID_ARG, "null cu_seqlens");
  expect(dense(-1, 16, 8, wsb), KDA_ERR_INVALID_ARG, "negative tokens");
  expect(dense((int64_t)1 << 40, 16, 8, wsb), KDA_ERR_INVALID_ARG, "too many tokens");
  expect(dense(16384, 0, 8, wsb), KDA_ERR_INVALID_ARG, "zero heads");
  expect(dense(16384, 16, 0, wsb), KDA_ERR_INVALID_ARG, "zero sequences");
  expect(dense(16384, 16, INT32_MAX, wsb), KDA_ERR_INVALID_ARG, "grid overflow");
  expect(dense_lb(-7.f, wsb), KDA_ERR_UNSUPPORTED, "lower_bound below the minimum");
  expect(dense_lb(0.5f, wsb), KDA_ERR_UNSUPPORTED, "positive lower_bound");
  expect(dense_lb(nanf(""), wsb), KDA_ERR_INVALID_ARG, "NaN lower_bound");
  expect(dense(16384, 16, 8, 0), KDA_ERR_WORKSPACE_TOO_SMALL, "short workspace");
  expect(dense(1 << 20, 16, 8, wsb), KDA_ERR_INVALID_ARG, "rows past 32-bit offsets");

  /* an int outside the enumerators, as a C caller may pass it */
  expect(kda_chunk_prefill_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKEF, -5.f, 0.088f, NULL,
                               FAKEI, FAKE, FAKE, FAKE, NULL, 16384, 16, 8, (kda_state_dtype_t)7, wsb),
         KDA_ERR_INVALID_ARG, "state dtype outside the enumerators");

  // the strided entry: strides whose products would wrap 64 bits
  const int64_t row = 16 * 128;
  const int64_t bad[] = {(int64_t)1 << 55, (int64_t)1 << 62, INT64_MAX - 7, -8};
  for (int field = 0; field < 12; ++field)
    for (int bi = 0; bi < 4; ++bi) {
      kda_strides_t st = {row, 128, row, 128, row, 128, row, 128, 16, 1, row, 128};
      ((int64_t*)&st)[field] = bad[bi];
      expect(kda_chunk_prefill_fwd_strided(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKEF, -5.f, 0.088f,
                                           NULL, FAKEI, FAKE, FAKE, FAKE, NULL, 16384, 16, 8,
                                           KDA_STATE_FP32, wsb, &st),
             KDA_ERR_INVALID_ARG, "huge or negative stride");
    }

  // checkpoints: bad interval, short capacity
  expect(kda_chunk_prefill_fwd_checkpoints(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKEF, -5.f, 0.088f,
                                           NULL, FAKEI, FAKE, FAKE, FAKE, NULL, 16384, 16, 8,
                                           KDA_STATE_FP32, wsb, NULL, FAKE, 24, 1024),
         KDA_ERR_INVALID_ARG, "checkpoint interval not a multiple of 16");
  expect(kda_chunk_prefill_fwd_checkpoints(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKEF, -5.f, 0.088f,
                                           NULL, FAKEI, FAKE, FAKE, FAKE, NULL, 16384, 16, 8,
                                           KDA_STATE_FP32, wsb, NULL, FAKE, 64, 10),
         KDA_ERR_INVALID_ARG, "checkpoint capacity too small");

  // the speculative-decode step
  const size_t wss = kda_get_workspace_size(8, 2, 2);
  expect(kda_spec_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKEF, -5.f, 0.088f, NULL, 16,
                              FAKEI, FAKEI, 4, FAKEI, FAKE, FAKE, NULL, 8, 2, 2, KDA_STATE_FP32, wss),
         KDA_ERR_INVALID_ARG, "null state pool");
  expect(kda_spec_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKEF, -5.f, 0.088f, FAKE,
                              (int64_t)1 << 62, FAKEI, FAKEI, 4, FAKEI, FAKE, FAKE, NULL, 8, 2, 2,
                              KDA_STATE_FP32, wss),
         KDA_ERR_INVALID_ARG, "pool too large to address");
  expect(kda_spec_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKEF, -5.f, 0.088f, FAKE, 16,
                              FAKEI, FAKEI, 0, FAKEI, FAKE, FAKE, NULL, 8, 2, 2, KDA_STATE_FP32, wss),
         KDA_ERR_INVALID_ARG, "zero index stride");

  // the gate / beta projections
  const size_t wsp = kda_gate_proj_workspace_size(8, 7168, 144);
  expect(wsp > 0, 1, "projection workspace size");
  expect(kda_gate_proj_workspace_size(-1, 7168, 144) == 0, 1, "projection workspace, negative tokens");
  expect(kda_gate_proj(NULL, FAKE, FAKE, FAKE, FAKE, FAKE, wsp, NULL, 8, 7168, 144, 1536),
         KDA_ERR_INVALID_ARG, "projection, null hidden");
  expect(kda_gate_proj(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wsp, NULL, 65537, 7168, 144, 1536),
         KDA_ERR_INVALID_ARG, "projection, too many tokens");
  expect(kda_gate_proj(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wsp, NULL, 8, 7170, 144, 1536),
         KDA_ERR_INVALID_ARG, "projection, hidden_dim not a multiple of 8");
  expect(kda_gate_proj(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wsp, NULL, 8, 7168, 120, 1536),
         KDA_ERR_INVALID_ARG, "projection, n_ab below the rank");
  expect(kda_gate_proj(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wsp, NULL, 8, 7168, 144, 1544),
         KDA_ERR_INVALID_ARG, "projection, n_b not a multiple of 16");
  expect(kda_gate_proj(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wsp - 1, NULL, 8, 7168, 144, 1536),
         KDA_ERR_WORKSPACE_TOO_SMALL, "projection, short workspace");
  expect(kda_gate_proj(NULL, FAKE, FAKE, NULL, NULL, NULL, 0, NULL, 0, 7168, 144, 1536), KDA_OK,
         "projection of zero tokens");

  // status strings and the test hooks
  for (int c = -1; c <= 6; ++c) /* also values outside the enumerators */
    if (!kda_status_string((kda_status_t)c) || !strlen(kda_status_string((kda_status_t)c))) ++failures;
  expect(kda_debug_set_kernel(7), -1, "invalid kernel selector");
  expect(kda_debug_set_vsplit(3), -1, "invalid split");
  expect(strlen(kda_last_hip_error()) == 0, 1, "no HIP error recorded");

  printf("host checks: %d failures\n", failures);
  return failures ? 1 : 0;
}
