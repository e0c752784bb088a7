/*
 * Runs the forward and backward oracles over small inputs that reach every
 * branch of their loops (fixed rows, packed segments with padding and a
 * segment-count overflow, initial and final states, the in-kernel L2 norm,
 * both in-kernel gate forms, several threads, empty inputs).  Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py;
 * any out-of-bounds access, use of freed memory or undefined arithmetic
 * aborts the run.  Prints "ok" on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int kda_oracle_fwd_gate(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, const float *q, const float *k,
                        const float *v, const float *g, const float *beta, double scale, int l2norm, int gate_mode,
                        double lower_bound, const float *a_log, const float *dt_bias, const float *initial_state,
                        const int32_t *segment_ids, int64_t n_max, double *o, double *final_state, int num_threads);
int kda_oracle_bwd(int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, const float *q, const float *k,
                   const float *v, const float *g, const float *beta, double scale, int l2norm,
                   const float *initial_state, const int32_t *segment_ids, int64_t n_max, const double *d_o,
                   const double *d_final, double *dq, double *dk, double *dv, double *dg, double *dbeta,
                   double *d_initial, int num_threads);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {   /* splitmix64 -> [0, 1) */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) / 9007199254740992.0;
}
static float *randf(int64_t n, double lo, double hi) {
  float *x = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) x[i] = (float)(lo + (hi - lo) * uniform());
  return x;
}
static double *zerod(int64_t n) { return (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double)); }

static int fails = 0;
static void expect(int got, int want, const char *what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    ++fails;
  }
}

/* One forward and one backward call; seg may be NULL. */
static void run_case(const char *name, int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, const int32_t *seg,
                     int64_t n_max, int with_init, int with_fin, int l2norm, int gate_mode, int threads,
                     int want_fwd) {
  const int64_t tok = B * T * H;
  const int64_t states = (seg ? B * n_max : B) * H * K * V;
  float *q = randf(tok * K, -1, 1), *k = randf(tok * K, -1, 1), *v = randf(tok * V, -1, 1);
  float *g = randf(tok * K, -2, 0), *beta = randf(tok, 0, 1);
  float *init = with_init ? randf(states, -0.1, 0.1) : NULL;
  float *a_log = randf(H, -0.5, 0.5), *dt_bias = randf(H * K, -1, 1);
  double *o = zerod(tok * V), *fin = with_fin ? zerod(states) : NULL;
  char what[128];
  snprintf(what, sizeof what, "%s forward", name);
  expect(kda_oracle_fwd_gate(B, T, H, K, V, q, k, v, g, beta, 0.125, l2norm, gate_mode, -3.0,
                             gate_mode ? a_log : NULL, gate_mode ? dt_bias : NULL, init, seg, n_max, o, fin,
                             threads),
         want_fwd, what);
  if (gate_mode == 0 && want_fwd == 0) {
    double *d_o = zerod(tok * V), *d_fin = with_fin ? zerod(states) : NULL;
    for (int64_t i = 0; i < tok * V; ++i) d_o[i] = uniform() - 0.5;
    if (d_fin)
      for (int64_t i = 0; i < states; ++i) d_fin[i] = uniform() - 0.5;
    double *dq = zerod(tok * K), *dk = zerod(tok * K), *dv = zerod(tok * V), *dg = zerod(tok * K);
    double *db = zerod(tok), *dinit = (with_init || !seg) ? zerod(states) : NULL;
    snprintf(what, sizeof what, "%s backward", name);
    expect(kda_oracle_bwd(B, T, H, K, V, q, k, v, g, beta, 0.125, l2norm, init, seg, n_max, d_o, d_fin, dq, dk, dv,
                          dg, db, dinit, threads),
           0, what);
    free(d_o); free(d_fin); free(dq); free(dk); free(dv); free(dg); free(db); free(dinit);
  }
  free(q); free(k); free(v); free(g); free(beta); free(init); free(a_log); free(dt_bias); free(o); free(fin);
}

int main(void) {
  /* fixed rows, ragged last chunk */
  run_case("fixed", 2, 70, 3, 8, 4, NULL, 0, 1, 1, 0, 0, 4, 0);
  run_case("fixed_l2", 1, 33, 2, 4, 8, NULL, 0, 0, 1, 1, 0, 1, 0);
  run_case("gate_plain", 1, 20, 2, 4, 4, NULL, 0, 1, 1, 0, 1, 2, 0);
  run_case("gate_safe", 1, 20, 2, 4, 4, NULL, 0, 1, 1, 1, 2, 3, 0);
  run_case("empty", 1, 0, 2, 4, 4, NULL, 0, 1, 1, 0, 0, 2, 0);
  /* packed: two rows, padding inside and after, a length-1 segment */
  {
    const int64_t B = 2, T = 24;
    int32_t seg[2 * 24];
    for (int t = 0; t < T; ++t) {
      seg[t] = t < 5 ? 1 : t < 6 ? 2 : t < 9 ? 0 : t < 20 ? 3 : 0;
      seg[T + t] = t < 12 ? 7 : 4;
    }
    run_case("packed", B, T, 2, 4, 4, seg, 4, 1, 1, 0, 0, 3, 0);
    run_case("packed_l2_gate", B, T, 2, 4, 4, seg, 3, 1, 1, 1, 2, 2, 0);
    run_case("packed_no_states", B, T, 2, 4, 4, seg, 0, 0, 0, 0, 0, 1, 0);
    /* more segments in a row than n_max: the oracle reports it */
    run_case("packed_overflow", B, T, 2, 4, 4, seg, 2, 1, 1, 0, 0, 2, 2);
  }
  if (fails) return 1;
  printf("ok\n");
  return 0;
}
