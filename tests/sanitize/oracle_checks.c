/* The fp64 oracle (oracle/kda_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: a small ragged batch (an empty sequence, a
 * one-token one, zero q / k rows, infinite beta logits) with each initial
 * state kind and several thread counts; checks that the outputs are finite,
 * that the thread count does not change them, and that the empty sequence
 * keeps its state.  Exits 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                   const uint16_t *beta_logits, const float *A_log, const float *dt_bias,
                   double lower_bound, double scale, const void *initial_state, int state_kind,
                   const int32_t *cu_seqlens, int heads, int num_seqs, double *out,
                   double *final_state, int threads);

#define D 128

static uint16_t bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  return (uint16_t)((u + 0x7FFF + ((u >> 16) & 1)) >> 16);
}

static uint32_t rng = 12345u;
static float unif(void) {
  rng = rng * 1664525u + 1013904223u;
  return (float)((rng >> 8) * (1.0 / 16777216.0)) * 2.f - 1.f;
}

int main(void) {
  const int H = 2, N = 4;
  const int32_t cu[5] = {0, 9, 9, 10, 24}; /* lengths 9, 0, 1, 14 */
  const int T = 24;
  uint16_t *q = malloc(sizeof(uint16_t) * T * H * D), *k = malloc(sizeof(uint16_t) * T * H * D);
  uint16_t *v = malloc(sizeof(uint16_t) * T * H * D), *g = malloc(sizeof(uint16_t) * T * H * D);
  uint16_t *b = malloc(sizeof(uint16_t) * T * H);
  float A_log[2] = {0.5f, 2.0f};
  float *dt = malloc(sizeof(float) * H * D);
  for (int i = 0; i < T * H * D; ++i) {
    q[i] = bf16(unif());
    k[i] = bf16(unif());
    v[i] = bf16(unif());
    g[i] = bf16(3.f * unif());
  }
  for (int i = 0; i < T * H; ++i) b[i] = bf16(unif());
  for (int i = 0; i < H * D; ++i) dt[i] = 0.1f * unif();
  memset(q + 3 * H * D, 0, sizeof(uint16_t) * H * D); /* token 3: zero q */
  memset(k + 5 * H * D, 0, sizeof(uint16_t) * H * D); /* token 5: zero k */
  b[2 * H] = 0x7F80;                                   /* +inf */
  b[12 * H + 1] = 0xFF80;                              /* -inf */

  const size_t SS = (size_t)N * H * D * D;
  float *s32 = malloc(sizeof(float) * SS);
  uint16_t *s16 = malloc(sizeof(uint16_t) * SS);
  double *s64 = malloc(sizeof(double) * SS);
  for (size_t i = 0; i < SS; ++i) {
    s32[i] = 0.02f * unif();
    s16[i] = bf16(s32[i]);
    s64[i] = s32[i];
  }
  double *out = malloc(sizeof(double) * T * H * D), *fin = malloc(sizeof(double) * SS);
  double *out1 = malloc(sizeof(double) * T * H * D), *fin1 = malloc(sizeof(double) * SS);
  int failures = 0;
  const void *states[4] = {NULL, s32, s16, s64};
  const int kinds[4] = {0, 0, 1, 2};
  for (int s = 0; s < 4; ++s) {
    if (kda_oracle_fwd(q, k, v, g, b, A_log, dt, -5.0, 0.0883883, states[s], kinds[s], cu, H, N,
                       out1, fin1, 1)) {
      ++failures;
      continue;
    }
    for (int threads = 2; threads <= 8; threads *= 2) {
      if (kda_oracle_fwd(q, k, v, g, b, A_log, dt, -5.0, 0.0883883, states[s], kinds[s], cu, H, N,
                         out, fin, threads))
        ++failures;
      if (memcmp(out, out1, sizeof(double) * T * H * D) || memcmp(fin, fin1, sizeof(double) * SS))
        ++failures;
    }
    for (int i = 0; i < T * H * D; ++i)
      if (!isfinite(out1[i])) ++failures;
    for (size_t i = 0; i < SS; ++i)
      if (!isfinite(fin1[i])) ++failures;
    /* sequence 1 is empty: its final state is its initial state */
    for (size_t i = (size_t)1 * H * D * D; i < (size_t)2 * H * D * D; ++i) {
      double want = 0.0;
      if (s == 1) want = s32[i];
      if (s == 2) { uint32_t u = (uint32_t)s16[i] << 16; float f; memcpy(&f, &u, 4); want = f; }
      if (s == 3) want = s64[i];
      if (fin1[i] != want) { ++failures; break; }
    }
  }
  /* bad arguments are rejected */
  if (kda_oracle_fwd(NULL, k, v, g, b, A_log, dt, -5.0, 0.088, NULL, 0, cu, H, N, out, fin, 1) == 0) ++failures;
  if (kda_oracle_fwd(q, k, v, g, b, A_log, dt, -5.0, 0.088, NULL, 7, cu, H, N, out, fin, 1) == 0) ++failures;
  printf("oracle checks: %d failures\n", failures);
  free(q); free(k); free(v); free(g); free(b); free(dt); free(s32); free(s16); free(s64);
  free(out); free(fin); free(out1); free(fin1);
  return failures ? 1 : 0;
}
