/*
 * KDA forward oracle: the gated delta rule evaluated one token at a time.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct CPU
 * definition that the HIP kernels are checked against.  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header or table with the GPU library.
 *
 * What it computes (page "feat(kda): integrate KDA attention with tokamax
 * backend and CP support", Implementation Details, "Delta Rule formulation"),
 * for every batch row b and head h independently, token by token:
 *     S'       = diag(exp(g_t)) S            decay, one factor per key channel
 *     residual = v_t - k_t^T S'              (a V-vector)
 *     S        = S' + beta_t k_t residual^T  rank-one delta-rule write
 *     o_t      = scale * q_t^T S             read-out after the write
 * S is K x V, so "S * exp(g_t)" scales the rows (key axis) of S: the residual
 * contracts k_t against the key axis of the decayed state.  The output uses
 * the state after token t's own write, because the read-out follows the
 * update in the formulation.
 *
 * Options taken from the chunk_kda signature on the same page (Public API):
 *   - scale (the caller passes 1/sqrt(K) when none is given);
 *   - use_qk_l2norm_in_kernel: q and k are divided by sqrt(sum x^2 + 1e-6)
 *     before use (the page gives no epsilon; 1e-6 is this oracle's choice);
 *   - segment_ids [B,T], 1-based, 0 = padding (KimiDeltaAttention.__call__):
 *     a new segment starts at every token whose id is non-zero and differs
 *     from the previous token's id (padding in between also ends a segment);
 *     each segment restarts the recurrence from its own initial state (or
 *     zero); padding tokens leave the state alone and get o = 0;
 *   - initial_state / output_final_state: one K x V state per (b, h), or per
 *     (b, segment, h) when segment_ids are given, segments numbered in order
 *     of appearance within the row, at most n_max of them;
 *   - use_gate_in_kernel with A_log, dt_bias (kda_oracle_fwd_gate): g holds
 *     raw gate values that are activated here before use.  The pages name
 *     the parameters and a sigmoid (layer pipeline, "Gate generation": the
 *     activation is a sigmoid from A_log and dt_bias; page 2 follow-ups: the
 *     safe gate has sigmoid lower-bound semantics with lower_bound in
 *     [-5, 0)).  Reading taken here, per head h and key channel c:
 *         z = exp(A_log_h) * (g_raw + dt_bias_{h,c})
 *         safe gate:  g = lower_bound * sigmoid(z)    (in (lower_bound, 0))
 *         otherwise:  g = log(sigmoid(z))             (decay exp(g) = sigmoid(z))
 *     with A_log absent meaning exp(A_log) = 1 and dt_bias absent meaning 0.
 *
 * Arithmetic is in REAL (double by default; float in the fp32 build), sums
 * run over the channel index in ascending order, exp/sqrt from libm.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef REAL
#define REAL double
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS 1
#define ORACLE_TOO_MANY_SEGMENTS 2
#define ORACLE_NO_MEMORY 3

static REAL rexp(REAL x) { return (REAL)exp((double)x); }
static REAL rsqrt_(REAL x) { return (REAL)sqrt((double)x); }

typedef struct {
  int64_t B, T, H, K, V;
  const float *q, *k, *v, *g, *beta;
  double scale;
  int l2norm;
  int gate_mode;                /* 0: g is the log decay; 1: log sigmoid; 2: lower_bound * sigmoid */
  double lower_bound;
  const float *a_log;           /* [H] or NULL */
  const float *dt_bias;         /* [H,K] or NULL */
  const float *initial_state;   /* may be NULL */
  const int32_t *segment_ids;   /* may be NULL */
  int64_t n_max;
  double *o;
  double *final_state;          /* may be NULL */
} job_t;

typedef struct {
  const job_t *job;
  int64_t first, stride;        /* items first, first+stride, ... over B*H */
  int status;
} worker_t;

/* The log decay of key channel c of head h for the stored gate value x. */
static REAL gate_log_decay(const job_t *j, int64_t h, int64_t c, REAL x) {
  if (j->gate_mode == 0) return x;
  const REAL a = j->a_log ? rexp((REAL)j->a_log[h]) : (REAL)1;
  const REAL z = a * (x + (j->dt_bias ? (REAL)j->dt_bias[h * j->K + c] : (REAL)0));
  const REAL sig = (REAL)1 / ((REAL)1 + rexp(-z));
  if (j->gate_mode == 2) return (REAL)j->lower_bound * sig;
  return (REAL)log((double)sig);
}

/* Index of the state slot for (b, seg, h) in [B,H,K,V] or [B,N_max,H,K,V]. */
static int64_t state_offset(const job_t *j, int64_t b, int64_t seg, int64_t h) {
  if (j->segment_ids == NULL) return ((b * j->H) + h) * j->K * j->V;
  return (((b * j->n_max) + seg) * j->H + h) * j->K * j->V;
}

static void load_state(const job_t *j, int64_t b, int64_t seg, int64_t h, REAL *S) {
  const int64_t n = j->K * j->V;
  if (j->initial_state == NULL) {
    for (int64_t i = 0; i < n; ++i) S[i] = 0;
    return;
  }
  const float *src = j->initial_state + state_offset(j, b, seg, h);
  for (int64_t i = 0; i < n; ++i) S[i] = (REAL)src[i];
}

static void store_state(const job_t *j, int64_t b, int64_t seg, int64_t h, const REAL *S) {
  if (j->final_state == NULL) return;
  double *dst = j->final_state + state_offset(j, b, seg, h);
  const int64_t n = j->K * j->V;
  for (int64_t i = 0; i < n; ++i) dst[i] = (double)S[i];
}

/* One (b, h) recurrence over all T tokens of the row. */
static int run_row_head(const job_t *j, int64_t b, int64_t h, REAL *S, REAL *qq, REAL *kk, REAL *r) {
  const int64_t T = j->T, H = j->H, K = j->K, V = j->V;
  const int have_seg = j->segment_ids != NULL;
  int32_t prev = 0;
  int64_t seg = -1;
  int live = 0;                 /* a segment is open and its state is in S */

  for (int64_t t = 0; t < T; ++t) {
    const int32_t s = have_seg ? j->segment_ids[b * T + t] : 1;
    double *orow = j->o + ((b * T + t) * H + h) * V;
    if (s == 0) {               /* padding: output zero, state untouched */
      for (int64_t x = 0; x < V; ++x) orow[x] = 0.0;
      prev = 0;
      continue;
    }
    if (t == 0 || s != prev) {  /* a new segment begins here */
      if (live) store_state(j, b, seg, h, S);
      seg += 1;
      if (have_seg && seg >= j->n_max && (j->initial_state || j->final_state)) {
        return ORACLE_TOO_MANY_SEGMENTS;
      }
      load_state(j, b, seg, h, S);
      live = 1;
    }
    prev = s;

    const int64_t qk_off = ((b * T + t) * H + h) * K;
    const int64_t v_off = ((b * T + t) * H + h) * V;
    for (int64_t c = 0; c < K; ++c) {
      qq[c] = (REAL)j->q[qk_off + c];
      kk[c] = (REAL)j->k[qk_off + c];
    }
    if (j->l2norm) {
      REAL sq = 0, sk = 0;
      for (int64_t c = 0; c < K; ++c) { sq += qq[c] * qq[c]; sk += kk[c] * kk[c]; }
      const REAL nq = rsqrt_(sq + (REAL)1e-6), nk = rsqrt_(sk + (REAL)1e-6);
      for (int64_t c = 0; c < K; ++c) { qq[c] /= nq; kk[c] /= nk; }
    }
    const REAL bt = (REAL)j->beta[(b * T + t) * H + h];

    /* S' = diag(exp(g_t)) S : row c of S (key channel c) scaled by exp(g_tc) */
    for (int64_t c = 0; c < K; ++c) {
      const REAL d = rexp(gate_log_decay(j, h, c, (REAL)j->g[qk_off + c]));
      REAL *row = S + c * V;
      for (int64_t x = 0; x < V; ++x) row[x] *= d;
    }
    /* residual = v_t - k_t^T S' */
    for (int64_t x = 0; x < V; ++x) {
      REAL acc = 0;
      for (int64_t c = 0; c < K; ++c) acc += kk[c] * S[c * V + x];
      r[x] = (REAL)j->v[v_off + x] - acc;
    }
    /* S = S' + beta_t k_t residual^T */
    for (int64_t c = 0; c < K; ++c) {
      const REAL w = bt * kk[c];
      REAL *row = S + c * V;
      for (int64_t x = 0; x < V; ++x) row[x] += w * r[x];
    }
    /* o_t = scale q_t^T S */
    for (int64_t x = 0; x < V; ++x) {
      REAL acc = 0;
      for (int64_t c = 0; c < K; ++c) acc += qq[c] * S[c * V + x];
      orow[x] = (double)((REAL)j->scale * acc);
    }
  }
  if (live) store_state(j, b, seg, h, S);
  return ORACLE_OK;
}

static void *worker_main(void *arg) {
  worker_t *w = (worker_t *)arg;
  const job_t *j = w->job;
  const int64_t K = j->K, V = j->V;
  REAL *S = (REAL *)malloc(sizeof(REAL) * (size_t)(K * V));
  REAL *qq = (REAL *)malloc(sizeof(REAL) * (size_t)K);
  REAL *kk = (REAL *)malloc(sizeof(REAL) * (size_t)K);
  REAL *r = (REAL *)malloc(sizeof(REAL) * (size_t)V);
  w->status = ORACLE_OK;
  if (!S || !qq || !kk || !r) {
    w->status = ORACLE_NO_MEMORY;
  } else {
    for (int64_t item = w->first; item < j->B * j->H; item += w->stride) {
      const int rc = run_row_head(j, item / j->H, item % j->H, S, qq, kk, r);
      if (rc != ORACLE_OK) w->status = rc;
    }
  }
  free(S); free(qq); free(kk); free(r);
  return NULL;
}

/*
 * Inputs are fp32 arrays holding the exact values the GPU receives (bf16
 * inputs widened exactly).  o [B,T,H,V] and final_state are written in
 * double.  Returns 0, or a nonzero ORACLE_* code.
 */
int kda_oracle_fwd_gate(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                        const float *q, const float *k, const float *v,
                        const float *g, const float *beta, double scale, int l2norm,
                        int gate_mode, double lower_bound, const float *a_log, const float *dt_bias,
                        const float *initial_state, const int32_t *segment_ids,
                        int64_t n_max, double *o, double *final_state, int num_threads) {
  if (B < 0 || T < 0 || H < 0 || K < 1 || V < 1 || !q || !k || !v || !g || !beta || !o)
    return ORACLE_BAD_ARGS;
  if (gate_mode < 0 || gate_mode > 2) return ORACLE_BAD_ARGS;
  if (segment_ids && (initial_state || final_state) && n_max < 1) return ORACLE_BAD_ARGS;
  job_t job = {B, T, H, K, V, q, k, v, g, beta, scale, l2norm, gate_mode, lower_bound, a_log, dt_bias,
               initial_state, segment_ids, n_max, o, final_state};
  if (final_state) {
    /* Slots no segment reaches stay zero. */
    const int64_t n = (segment_ids ? B * n_max : B) * H * K * V;
    memset(final_state, 0, sizeof(double) * (size_t)n);
  }
  const int64_t items = B * H;
  if (items == 0) return ORACLE_OK;
  if (num_threads < 1) num_threads = 1;
  if (num_threads > items) num_threads = (int)items;
  worker_t *ws = (worker_t *)calloc((size_t)num_threads, sizeof(worker_t));
  pthread_t *th = (pthread_t *)calloc((size_t)num_threads, sizeof(pthread_t));
  if (!ws || !th) { free(ws); free(th); return ORACLE_NO_MEMORY; }
  for (int i = 0; i < num_threads; ++i) {
    ws[i].job = &job; ws[i].first = i; ws[i].stride = num_threads;
  }
  for (int i = 1; i < num_threads; ++i) pthread_create(&th[i], NULL, worker_main, &ws[i]);
  worker_main(&ws[0]);
  for (int i = 1; i < num_threads; ++i) pthread_join(th[i], NULL);
  int status = ORACLE_OK;
  for (int i = 0; i < num_threads; ++i) if (ws[i].status != ORACLE_OK) status = ws[i].status;
  free(ws); free(th);
  return status;
}

/* The forward with g already the log decay. */
int kda_oracle_fwd(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                   const float *q, const float *k, const float *v,
                   const float *g, const float *beta, double scale, int l2norm,
                   const float *initial_state, const int32_t *segment_ids,
                   int64_t n_max, double *o, double *final_state, int num_threads) {
  return kda_oracle_fwd_gate(B, T, H, K, V, q, k, v, g, beta, scale, l2norm, 0, 0.0, NULL, NULL,
                             initial_state, segment_ids, n_max, o, final_state, num_threads);
}

/* Size in bytes of REAL in this build (8 for the fp64 build, 4 for fp32). */
int kda_oracle_real_bytes(void) { return (int)sizeof(REAL); }
