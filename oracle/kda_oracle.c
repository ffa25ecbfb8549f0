/*
 * kda_oracle.c -- plain fp64 CPU oracle for the Kimi Delta Attention (KDA)
 * chunked-prefill forward.  TEST INFRASTRUCTURE ONLY: this file is the
 * correctness reference that the GPU path is checked against.  It shares no
 * code, header, table or helper with the GPU library, and the GPU library
 * never calls it.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.
 *
 * What it computes (the plain definition, token by token, in double):
 *
 *   The recurrence is named in vLLM PR #55737's report ("Use FlashKDA for KDA
 *   chunked prefill", section "Features and motivation" and the wrapper
 *   listing in "Key source snippets"): a bounded gate
 *       log a_t[c] = lower_bound * sigmoid(exp(A_log[h]) * (g_t[c] + dt_bias[h][c])),
 *   q and k L2-normalised inside the kernel, raw beta logits (sigmoid applied
 *   inside), and the softmax-style scale head_dim^-1/2 applied to q.  A_log is
 *   one value per head and dt_bias one row of head_dim values per head (the
 *   same listing passes A_log.view(-1) and dt_bias.view(-1, head_dim)).
 *   The state is head_dim x head_dim per (sequence, head) and is carried in
 *   and out as initial/final state (same listing; the checkpoint dtypes fp32
 *   and bf16 come from PR #56485's report, "Implementation breakdown").
 *
 *   The full update the pages name but do not print is read as the gated
 *   delta rule, with S[c][j] indexed by key channel c (row) and value
 *   channel j (column):
 *       S_t = (I - beta_t k_t k_t^T) Diag(a_t) S_{t-1} + beta_t k_t v_t^T
 *       o_t = scale * S_t^T q_t
 *   where k_t and q_t are the L2-normalised vectors
 *       x / sqrt(sum_c x[c]^2 + 1e-6)
 *   and beta_t = 1 / (1 + exp(-beta_logit_t)).  o_t sees token t's own write.
 *
 *   (I - b k k^T) X is evaluated as X - b k (k^T X), which is the same matrix
 *   product with the parentheses moved; a dense brute-force check in the test
 *   suite builds the explicit matrices instead.
 *
 * Inputs are the raw storage the GPU path receives: bf16 values as their 16-bit
 * patterns, fp32 tensors as float.  bf16 and fp32 values widen to double
 * exactly.  Outputs are double and unrounded.
 *
 * Threads run over independent (sequence, head) pairs only; each pair is a
 * straight token loop.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KDA_ORACLE_D 128
#define KDA_ORACLE_EPS 1e-6

/* Exact widening of a bf16 bit pattern: bf16 is the top half of an IEEE fp32. */
static double bf16_bits_to_double(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

struct oracle_job {
  const uint16_t *q, *k, *v, *g, *beta_logits;
  const float *A_log, *dt_bias;
  double lower_bound, scale;
  const void *initial_state; /* NULL means zeros */
  int state_kind;            /* 0 fp32, 1 bf16 bit patterns, 2 double */
  const int32_t *cu_seqlens;
  int heads, num_seqs;
  double *out, *final_state;
  int next_task; /* shared work counter, accessed atomically */
};

static void oracle_pair(const struct oracle_job *J, int n, int h, double *S) {
  const int D = KDA_ORACLE_D;
  const int H = J->heads;
  double q[KDA_ORACLE_D], k[KDA_ORACLE_D], v[KDA_ORACLE_D], a[KDA_ORACLE_D];
  double p[KDA_ORACLE_D];

  /* initial state: exact widening, or zeros */
  size_t soff = ((size_t)n * H + h) * D * D;
  for (int i = 0; i < D * D; ++i) {
    if (!J->initial_state) {
      S[i] = 0.0;
    } else if (J->state_kind == 1) {
      S[i] = bf16_bits_to_double(((const uint16_t *)J->initial_state)[soff + i]);
    } else if (J->state_kind == 2) {
      S[i] = ((const double *)J->initial_state)[soff + i];
    } else {
      S[i] = (double)((const float *)J->initial_state)[soff + i];
    }
  }

  const double eA = exp((double)J->A_log[h]);
  const float *dtb = J->dt_bias + (size_t)h * D;

  for (int64_t t = J->cu_seqlens[n]; t < J->cu_seqlens[n + 1]; ++t) {
    size_t row = ((size_t)t * H + h) * D;
    double qq = 0.0, kk = 0.0;
    for (int c = 0; c < D; ++c) {
      q[c] = bf16_bits_to_double(J->q[row + c]);
      k[c] = bf16_bits_to_double(J->k[row + c]);
      v[c] = bf16_bits_to_double(J->v[row + c]);
      qq += q[c] * q[c];
      kk += k[c] * k[c];
    }
    /* in-kernel L2 normalisation of q and k */
    const double rq = 1.0 / sqrt(qq + KDA_ORACLE_EPS);
    const double rk = 1.0 / sqrt(kk + KDA_ORACLE_EPS);
    for (int c = 0; c < D; ++c) {
      q[c] *= rq;
      k[c] *= rk;
    }
    /* beta from its raw logit */
    const double b = 1.0 / (1.0 + exp(-bf16_bits_to_double(J->beta_logits[(size_t)t * H + h])));
    /* bounded per-channel gate: a = exp(lower_bound * sigmoid(exp(A_log) * (g + dt_bias))) */
    for (int c = 0; c < D; ++c) {
      const double x = eA * (bf16_bits_to_double(J->g[row + c]) + (double)dtb[c]);
      const double lam = J->lower_bound / (1.0 + exp(-x));
      a[c] = exp(lam);
    }
    /* S <- Diag(a) S   (decay acts on the key index, i.e. the rows) */
    for (int c = 0; c < D; ++c)
      for (int j = 0; j < D; ++j) S[c * D + j] *= a[c];
    /* p = S^T k  (what the decayed state currently stores under key k) */
    for (int j = 0; j < D; ++j) p[j] = 0.0;
    for (int c = 0; c < D; ++c)
      for (int j = 0; j < D; ++j) p[j] += S[c * D + j] * k[c];
    /* S <- S - b k p^T + b k v^T   ==  (I - b k k^T) S + b k v^T */
    for (int c = 0; c < D; ++c)
      for (int j = 0; j < D; ++j) S[c * D + j] += b * k[c] * (v[j] - p[j]);
    /* o = scale * S^T q with the updated state */
    double *o = J->out + row;
    for (int j = 0; j < D; ++j) o[j] = 0.0;
    for (int c = 0; c < D; ++c)
      for (int j = 0; j < D; ++j) o[j] += S[c * D + j] * q[c];
    for (int j = 0; j < D; ++j) o[j] *= J->scale;
  }

  if (J->final_state) memcpy(J->final_state + soff, S, sizeof(double) * D * D);
}

static void *oracle_worker(void *arg) {
  struct oracle_job *J = (struct oracle_job *)arg;
  double *S = (double *)malloc(sizeof(double) * KDA_ORACLE_D * KDA_ORACLE_D);
  if (!S) return (void *)1;
  const int tasks = J->num_seqs * J->heads;
  for (;;) {
    int task = __atomic_fetch_add(&J->next_task, 1, __ATOMIC_RELAXED);
    if (task >= tasks) break;
    oracle_pair(J, task / J->heads, task % J->heads, S);
  }
  free(S);
  return NULL;
}

/*
 * kda_oracle_fwd: run the recurrence for every (sequence, head).
 *   q, k, v, g    : bf16 bit patterns, [T, heads, 128] dense
 *   beta_logits   : bf16 bit patterns, [T, heads] dense
 *   A_log         : fp32 [heads];  dt_bias: fp32 [heads, 128]
 *   initial_state : [num_seqs, heads, 128, 128]: fp32 (state_kind 0), bf16 bit
 *                   patterns (1) or double (2); NULL = zeros
 *   cu_seqlens    : int32 [num_seqs + 1], cu[0] = 0, non-decreasing
 *   out           : double [T, heads, 128]; rows of tokens outside every
 *                   sequence are left untouched
 *   final_state   : double [num_seqs, heads, 128, 128] (may be NULL)
 *   threads       : worker threads (<= 0 means 1)
 * Returns 0 on success, -1 on bad arguments, -2 on allocation/thread failure.
 */
int kda_oracle_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                   const uint16_t *beta_logits, const float *A_log, const float *dt_bias,
                   double lower_bound, double scale, const void *initial_state, int state_kind,
                   const int32_t *cu_seqlens, int heads, int num_seqs, double *out,
                   double *final_state, int threads) {
  if (!q || !k || !v || !g || !beta_logits || !A_log || !dt_bias || !cu_seqlens || !out)
    return -1;
  if (heads <= 0 || num_seqs < 0 || state_kind < 0 || state_kind > 2) return -1;
  struct oracle_job J;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta_logits = beta_logits;
  J.A_log = A_log; J.dt_bias = dt_bias;
  J.lower_bound = lower_bound; J.scale = scale;
  J.initial_state = initial_state; J.state_kind = state_kind;
  J.cu_seqlens = cu_seqlens; J.heads = heads; J.num_seqs = num_seqs;
  J.out = out; J.final_state = final_state;
  J.next_task = 0;

  int tasks = num_seqs * heads;
  if (threads <= 0) threads = 1;
  if (threads > tasks) threads = tasks > 0 ? tasks : 1;
  if (threads == 1) return oracle_worker(&J) == NULL ? 0 : -2;

  pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)threads);
  if (!tid) return -2;
  int started = 0;
  for (; started < threads; ++started)
    if (pthread_create(&tid[started], NULL, oracle_worker, &J) != 0) break;
  for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
  free(tid);
  /* a claimed task always completes, so every task ran iff all were claimed */
  return J.next_task >= tasks ? 0 : -2;
}
