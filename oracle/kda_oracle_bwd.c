/*
 * KDA backward oracle: reverse mode of the gated delta rule, one token at a
 * time.
 *
 * TEST INFRASTRUCTURE ONLY.  The slow, plainly written CPU definition of the
 * gradients the HIP backward is checked against; only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header or table with the GPU library (nor with the forward oracle: the
 * forward states it needs are recomputed here by its own token loop).
 *
 * The forward (page "feat(kda): integrate KDA attention with tokamax backend
 * and CP support", Implementation Details, "Delta Rule formulation"; the
 * backward pass is the separate kernel work that page's follow-ups refer
 * to), per (row b, head h, segment), token by token, with q^, k^ the inputs
 * after the optional L2 norm:
 *     S_a = diag(exp(g_t)) S_{t-1}
 *     r   = v_t - S_a^T k^
 *     S_t = S_a + beta_t k^ r^T
 *     o_t = scale S_t^T q^
 * Given dL/do_t for every token and dL/dS for each segment's final state,
 * the chain rule taken through one token backwards, with dS = dL/dS_t:
 *     dS  += scale q^ do_t^T          dq^ = scale S_t do_t
 *     dbeta = k^T dS r                 dk^ = beta dS r
 *     dr   = beta dS^T k^              dv  = dr
 *     dS_a = dS - k^ dr^T              dk^ -= S_a dr
 *     dg_c = sum_j dS_a[c,j] S_a[c,j]  (S_a[c,.] = exp(g_c) S_{t-1}[c,.])
 *     dL/dS_{t-1} = diag(exp(g_t)) dS_a
 * and through the L2 norm x^ = x / n, n = sqrt(sum x^2 + 1e-6):
 *     dx = dx^ / n - x (x . dx^) / n^3.
 * The gradient of a segment's initial state is dL/dS before its first token.
 * Padding tokens (and segments past n_max, which the forward rejects) carry
 * no gradient.
 *
 * States are recomputed from a checkpoint every kBlock tokens (the forward
 * run once, keeping the state at each block start; each block replayed in
 * full before its tokens are taken backwards), which changes no arithmetic.
 * REAL is double (float in the fp32 build); sums run over the channel index
 * in ascending order.
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

enum { kBlock = 64 };

typedef struct {
  int64_t B, T, H, K, V;
  const float *q, *k, *v, *g, *beta;
  double scale;
  int l2norm;
  const float *initial_state;   /* NULL or [B,H,K,V] / [B,n_max,H,K,V] */
  const int32_t *segment_ids;   /* NULL or [B,T] */
  int64_t n_max;
  const double *d_o;            /* [B,T,H,V] */
  const double *d_final;        /* NULL or the state shape */
  double *dq, *dk, *dv, *dg, *dbeta;   /* same shapes as q, k, v, g, beta; zeroed by the caller */
  double *d_initial;            /* NULL or the state shape */
} bjob_t;

typedef struct {
  const bjob_t *j;
  int64_t next;
  int err;
  pthread_mutex_t mu;
} pool_t;

static int64_t slot(const bjob_t *j, int64_t b, int64_t seg, int64_t h) {
  return j->segment_ids ? ((b * j->n_max + seg) * j->H + h) * j->K * j->V : (b * j->H + h) * j->K * j->V;
}

/* q^ or k^ of token t (normalised when asked); returns the norm used (1 without). */
static REAL unit_vec(const bjob_t *j, const float *x, int64_t off, REAL *out) {
  REAL ss = 0;
  for (int64_t c = 0; c < j->K; ++c) ss += (REAL)x[off + c] * (REAL)x[off + c];
  const REAL n = j->l2norm ? (REAL)sqrt((double)(ss + (REAL)1e-6)) : (REAL)1;
  for (int64_t c = 0; c < j->K; ++c) out[c] = (REAL)x[off + c] / n;
  return n;
}

/* One forward step on S (K x V) for token (b, t, h); leaves S_a in Sa. */
static void step_forward(const bjob_t *j, int64_t b, int64_t t, int64_t h, REAL *S, REAL *Sa, REAL *kk, REAL *r) {
  const int64_t K = j->K, V = j->V, qk = ((b * j->T + t) * j->H + h) * K, vo = ((b * j->T + t) * j->H + h) * V;
  const REAL bt = (REAL)j->beta[(b * j->T + t) * j->H + h];
  unit_vec(j, j->k, qk, kk);
  for (int64_t c = 0; c < K; ++c) {
    const REAL d = (REAL)exp((double)j->g[qk + c]);
    for (int64_t x = 0; x < V; ++x) Sa[c * V + x] = d * S[c * V + x];
  }
  for (int64_t x = 0; x < V; ++x) {
    REAL acc = 0;
    for (int64_t c = 0; c < K; ++c) acc += kk[c] * Sa[c * V + x];
    r[x] = (REAL)j->v[vo + x] - acc;
  }
  for (int64_t c = 0; c < K; ++c)
    for (int64_t x = 0; x < V; ++x) S[c * V + x] = Sa[c * V + x] + bt * kk[c] * r[x];
}

/* Gradients of one segment [t0, t1) of row b, head h, state slot seg. */
static int segment_backward(const bjob_t *j, int64_t b, int64_t h, int64_t seg, int64_t t0, int64_t t1) {
  const int64_t K = j->K, V = j->V, KV = K * V, n = t1 - t0, nb = (n + kBlock - 1) / kBlock;
  REAL *ck = malloc(sizeof(REAL) * (size_t)(nb * KV));           /* state at each block start */
  REAL *blk = malloc(sizeof(REAL) * (size_t)((kBlock + 1) * KV)); /* states S_{t-1}..S_t of one block */
  REAL *Sa = malloc(sizeof(REAL) * (size_t)KV), *dS = malloc(sizeof(REAL) * (size_t)KV);
  REAL *work = malloc(sizeof(REAL) * (size_t)(6 * K + 2 * V));
  if (!ck || !blk || !Sa || !dS || !work) {
    free(ck); free(blk); free(Sa); free(dS); free(work);
    return ORACLE_NO_MEMORY;
  }
  REAL *qq = work, *kk = work + K, *dqq = work + 2 * K, *dkk = work + 3 * K, *tmp = work + 4 * K;
  REAL *r = work + 6 * K, *dr = work + 6 * K + V;

  /* forward once, keeping the block-start states */
  REAL *S = blk;
  for (int64_t i = 0; i < KV; ++i)
    S[i] = j->initial_state ? (REAL)j->initial_state[slot(j, b, seg, h) + i] : (REAL)0;
  for (int64_t t = t0; t < t1; ++t) {
    if ((t - t0) % kBlock == 0) memcpy(ck + ((t - t0) / kBlock) * KV, S, sizeof(REAL) * (size_t)KV);
    step_forward(j, b, t, h, S, Sa, kk, r);
  }

  for (int64_t i = 0; i < KV; ++i) dS[i] = j->d_final ? (REAL)j->d_final[slot(j, b, seg, h) + i] : (REAL)0;
  for (int64_t bi = nb - 1; bi >= 0; --bi) {
    const int64_t s0 = t0 + bi * kBlock, s1 = s0 + kBlock < t1 ? s0 + kBlock : t1;
    /* replay the block: blk[i] = state before token s0 + i, blk[s1 - s0] = after the last */
    memcpy(blk, ck + bi * KV, sizeof(REAL) * (size_t)KV);
    for (int64_t t = s0; t < s1; ++t) {
      memcpy(blk + (t - s0 + 1) * KV, blk + (t - s0) * KV, sizeof(REAL) * (size_t)KV);
      step_forward(j, b, t, h, blk + (t - s0 + 1) * KV, Sa, kk, r);
    }
    for (int64_t t = s1 - 1; t >= s0; --t) {
      const REAL *Sprev = blk + (t - s0) * KV, *St = blk + (t - s0 + 1) * KV;
      const int64_t tok = (b * j->T + t) * j->H + h, qk = tok * K, vo = tok * V;
      const REAL bt = (REAL)j->beta[tok], sc = (REAL)j->scale;
      const REAL nq = unit_vec(j, j->q, qk, qq), nk = unit_vec(j, j->k, qk, kk);
      const double *dot = j->d_o + vo;
      /* recompute S_a and r of this token */
      for (int64_t c = 0; c < K; ++c) {
        const REAL d = (REAL)exp((double)j->g[qk + c]);
        for (int64_t x = 0; x < V; ++x) Sa[c * V + x] = d * Sprev[c * V + x];
      }
      for (int64_t x = 0; x < V; ++x) {
        REAL acc = 0;
        for (int64_t c = 0; c < K; ++c) acc += kk[c] * Sa[c * V + x];
        r[x] = (REAL)j->v[vo + x] - acc;
      }
      /* read-out: o_t = scale S_t^T q^ */
      for (int64_t c = 0; c < K; ++c) {
        REAL acc = 0;
        for (int64_t x = 0; x < V; ++x) {
          dS[c * V + x] += sc * qq[c] * (REAL)dot[x];
          acc += St[c * V + x] * (REAL)dot[x];
        }
        dqq[c] = sc * acc;
      }
      /* write: S_t = S_a + beta k^ r^T */
      REAL db = 0;
      for (int64_t c = 0; c < K; ++c) {
        REAL acc = 0;
        for (int64_t x = 0; x < V; ++x) acc += dS[c * V + x] * r[x];
        db += kk[c] * acc;
        dkk[c] = bt * acc;
      }
      for (int64_t x = 0; x < V; ++x) {
        REAL acc = 0;
        for (int64_t c = 0; c < K; ++c) acc += dS[c * V + x] * kk[c];
        dr[x] = bt * acc;
        j->dv[vo + x] = (double)dr[x];
      }
      j->dbeta[tok] = (double)db;
      /* residual: r = v - S_a^T k^ */
      for (int64_t c = 0; c < K; ++c) {
        REAL acc = 0;
        for (int64_t x = 0; x < V; ++x) {
          dS[c * V + x] -= kk[c] * dr[x];
          acc += Sa[c * V + x] * dr[x];
        }
        dkk[c] -= acc;
      }
      /* decay: S_a = diag(exp(g)) S_{t-1}; dS becomes dL/dS_{t-1} */
      for (int64_t c = 0; c < K; ++c) {
        const REAL d = (REAL)exp((double)j->g[qk + c]);
        REAL acc = 0;
        for (int64_t x = 0; x < V; ++x) {
          acc += dS[c * V + x] * Sa[c * V + x];
          dS[c * V + x] *= d;
        }
        j->dg[qk + c] = (double)acc;
      }
      /* L2 norm */
      for (int pass = 0; pass < 2; ++pass) {
        const float *x = pass == 0 ? j->q : j->k;
        REAL *dx = pass == 0 ? dqq : dkk;
        double *out = pass == 0 ? j->dq : j->dk;
        const REAL nn = pass == 0 ? nq : nk;
        if (!j->l2norm) {
          for (int64_t c = 0; c < K; ++c) out[qk + c] = (double)dx[c];
          continue;
        }
        REAL xd = 0;
        for (int64_t c = 0; c < K; ++c) xd += (REAL)x[qk + c] * dx[c];
        for (int64_t c = 0; c < K; ++c) tmp[c] = dx[c] / nn - (REAL)x[qk + c] * xd / (nn * nn * nn);
        for (int64_t c = 0; c < K; ++c) out[qk + c] = (double)tmp[c];
      }
    }
  }
  if (j->d_initial)
    for (int64_t i = 0; i < KV; ++i) j->d_initial[slot(j, b, seg, h) + i] = (double)dS[i];
  free(ck); free(blk); free(Sa); free(dS); free(work);
  return ORACLE_OK;
}

static int row_head(const bjob_t *j, int64_t b, int64_t h) {
  if (!j->segment_ids) return segment_backward(j, b, h, 0, 0, j->T);
  const int32_t *ids = j->segment_ids + b * j->T;
  int64_t seg = 0;
  for (int64_t t = 0; t < j->T;) {
    if (ids[t] == 0) { ++t; continue; }
    int64_t e = t + 1;
    while (e < j->T && ids[e] == ids[t]) ++e;
    if (seg >= j->n_max) return ORACLE_TOO_MANY_SEGMENTS;
    const int rc = segment_backward(j, b, h, seg, t, e);
    if (rc != ORACLE_OK) return rc;
    ++seg;
    t = e;
  }
  return ORACLE_OK;
}

static void *worker(void *arg) {
  pool_t *p = arg;
  const bjob_t *j = p->j;
  for (;;) {
    pthread_mutex_lock(&p->mu);
    const int64_t item = p->next++;
    const int stop = p->err != ORACLE_OK;
    pthread_mutex_unlock(&p->mu);
    if (stop || item >= j->B * j->H) break;
    const int rc = row_head(j, item / j->H, item % j->H);
    if (rc != ORACLE_OK) {
      pthread_mutex_lock(&p->mu);
      if (p->err == ORACLE_OK) p->err = rc;
      pthread_mutex_unlock(&p->mu);
    }
  }
  return NULL;
}

int kda_oracle_bwd(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, const float *q, const float *k,
                   const float *v, const float *g, const float *beta, double scale, int l2norm,
                   const float *initial_state, const int32_t *segment_ids, int64_t n_max, const double *d_o,
                   const double *d_final, double *dq, double *dk, double *dv, double *dg, double *dbeta,
                   double *d_initial, int num_threads) {
  if (B < 0 || T < 0 || H < 0 || K < 1 || V < 1 || !q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv ||
      !dg || !dbeta)
    return ORACLE_BAD_ARGS;
  if (segment_ids && (initial_state || d_final || d_initial) && n_max < 1) return ORACLE_BAD_ARGS;
  bjob_t j = {B, T, H, K, V, q, k, v, g, beta, scale, l2norm, initial_state, segment_ids, n_max > 0 ? n_max : T,
              d_o, d_final, dq, dk, dv, dg, dbeta, d_initial};
  if (d_initial) {
    const int64_t n = (segment_ids ? B * j.n_max : B) * H * K * V;
    memset(d_initial, 0, sizeof(double) * (size_t)n);
  }
  pool_t p = {&j, 0, ORACLE_OK, PTHREAD_MUTEX_INITIALIZER};
  if (num_threads < 1) num_threads = 1;
  if (num_threads > 256) num_threads = 256;
  pthread_t th[256];
  int started = 0;
  for (int i = 0; i < num_threads; ++i)
    if (pthread_create(&th[i], NULL, worker, &p) == 0) ++started;
  if (started == 0) worker(&p);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  return p.err;
}

int kda_oracle_bwd_real_bytes(void) { return (int)sizeof(REAL); }
