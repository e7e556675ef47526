/* Host driver for the sanitizer builds of the oracle (test infrastructure).
 * Runs oracle_gate, oracle_kda_fwd and oracle_kda_bwd on small random problems, with and
 * without dt_bias and an initial state, every gate kind, several thread
 * counts, empty and rejected shapes, and checks what the four-step update of
 * the "K3 notes" (section "KDA 递归核心") fixes exactly: the result does not
 * depend on the thread count, and with g = 0, beta = 1 and a unit key the
 * state reproduces v on that key.  Exit status 0 means every check held. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gate(const double* g_raw, const double* A_log, const double* dt_bias, int kind,
                double lower_bound, long B, long T, long HV, long K, double* g_out);
int oracle_kda_fwd(const double* q, const double* k, const double* v, const double* g_raw,
                   const double* beta, const double* A_log, const double* dt_bias, int kind,
                   double lower_bound, const double* S0, long B, long T, long H, long HV,
                   long K, long V, double* o, double* S_out, int nthreads);

int oracle_kda_bwd(const double* q, const double* k, const double* v, const double* g_raw,
                   const double* beta, const double* A_log, const double* dt_bias, int kind,
                   double lower_bound, const double* S0, const double* dout, const double* dST,
                   long B, long T, long H, long HV, long K, long V, double* dq, double* dk,
                   double* dv, double* dbeta, double* dg_raw, double* dA_log, double* ddt_bias,
                   double* dS0, int nthreads);

static double urand(void) { return (double)rand() / RAND_MAX * 2.0 - 1.0; }

static double* fill(long n, double scale) {
  double* x = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
  for (long i = 0; i < n; ++i) x[i] = scale * urand();
  return x;
}

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); ++fails; } } while (0)

/* The gradient oracle on the same kind of problem, with one and with three
 * threads: the results must be equal element for element. */
static void run_bwd_case(long B, long T, long H, long HV, long K, long V, int kind, int bias,
                         int s0, int dst) {
  double *q = fill(B * T * H * K, 0.3), *k = fill(B * T * H * K, 0.3), *v = fill(B * T * HV * V, 1.0);
  double *g = fill(B * T * HV * K, 1.0), *beta = fill(B * T * HV, 0.5), *A = fill(HV, 0.5);
  double *dt = bias ? fill(HV * K, 1.0) : NULL, *S0 = s0 ? fill(B * HV * K * V, 0.1) : NULL;
  double *dout = fill(B * T * HV * V, 1.0), *dST = dst ? fill(B * HV * K * V, 1.0) : NULL;
  if (kind == 2)
    for (long i = 0; i < B * T * HV * K; ++i) g[i] = -0.2 * fabs(g[i]);
  const long n[8] = {B * T * H * K, B * T * H * K, B * T * HV * V, B * T * HV, B * T * HV * K, HV,
                     HV * K, B * HV * K * V};
  double* out[2][8];
  for (int r = 0; r < 2; ++r) {
    for (int j = 0; j < 8; ++j) out[r][j] = fill(n[j], 0);
    CHECK(oracle_kda_bwd(q, k, v, g, beta, A, dt, kind, -5.0, S0, dout, dST, B, T, H, HV, K, V,
                         out[r][0], out[r][1], out[r][2], out[r][3], out[r][4], out[r][5],
                         bias ? out[r][6] : NULL, out[r][7], r ? 3 : 1) == 0,
          "kda_bwd rejected a valid case");
  }
  for (int j = 0; j < 8; ++j)
    for (long i = 0; i < n[j]; ++i)
      if ((j != 6 || bias) && out[0][j][i] != out[1][j][i]) {
        CHECK(0, "bwd output %d differs with the thread count", j);
        break;
      }
  for (int r = 0; r < 2; ++r)
    for (int j = 0; j < 8; ++j) free(out[r][j]);
  free(q); free(k); free(v); free(g); free(beta); free(A); free(dt); free(S0); free(dout); free(dST);
}

static void run_case(long B, long T, long H, long HV, long K, long V, int kind, int bias, int s0) {
  double *q = fill(B * T * H * K, 0.3), *k = fill(B * T * H * K, 0.3), *v = fill(B * T * HV * V, 1.0);
  double *g = fill(B * T * HV * K, 1.0), *beta = fill(B * T * HV, 0.5), *A = fill(HV, 0.5);
  double *dt = bias ? fill(HV * K, 1.0) : NULL, *S0 = s0 ? fill(B * HV * K * V, 0.1) : NULL;
  for (long i = 0; i < B * T * HV; ++i) beta[i] = 0.5 + 0.5 * beta[i];
  double *o1 = fill(B * T * HV * V, 0), *o3 = fill(B * T * HV * V, 0);
  double *S1 = fill(B * HV * K * V, 0), *S3 = fill(B * HV * K * V, 0);
  CHECK(oracle_kda_fwd(q, k, v, g, beta, A, dt, kind, -5.0, S0, B, T, H, HV, K, V, o1, S1, 1) == 0,
        "kda_fwd rejected a valid case");
  CHECK(oracle_kda_fwd(q, k, v, g, beta, A, dt, kind, -5.0, S0, B, T, H, HV, K, V, o3, S3, 3) == 0,
        "kda_fwd rejected a valid case (3 threads)");
  CHECK(memcmp(o1, o3, sizeof(double) * B * T * HV * V) == 0, "o depends on the thread count");
  CHECK(memcmp(S1, S3, sizeof(double) * B * HV * K * V) == 0, "S depends on the thread count");
  double* gg = fill(B * T * HV * K, 0);
  CHECK(oracle_gate(g, A, dt, kind, -5.0, B, T, HV, K, gg) == 0, "gate rejected a valid case");
  for (long i = 0; i < B * T * HV * K; ++i)
    CHECK(kind == 2 ? gg[i] == g[i] : (gg[i] <= 0.0 && (kind != 1 || gg[i] >= -5.0)),
          "gate value %g out of range (kind %d)", gg[i], kind);
  free(q); free(k); free(v); free(g); free(beta); free(A); free(dt); free(S0);
  free(o1); free(o3); free(S1); free(S3); free(gg);
}

/* g = 0 (gate none), beta = 1, a unit key: k_t . S_t = v_t after token t. */
static void reconstruction(void) {
  const long T = 5, K = 8, V = 6;
  double q[5 * 8], k[5 * 8], v[5 * 6], g[5 * 8], beta[5], A = 0.0, o[5 * 6], S[8 * 6];
  for (long t = 0; t < T; ++t) {
    double n = 0.0;
    for (long c = 0; c < K; ++c) { k[t * K + c] = urand(); n += k[t * K + c] * k[t * K + c]; }
    for (long c = 0; c < K; ++c) { k[t * K + c] /= sqrt(n); q[t * K + c] = k[t * K + c]; g[t * K + c] = 0.0; }
    for (long j = 0; j < V; ++j) v[t * V + j] = urand();
    beta[t] = 1.0;
  }
  CHECK(oracle_kda_fwd(q, k, v, g, beta, &A, NULL, 2, -5.0, NULL, 1, T, 1, 1, K, V, o, S, 1) == 0,
        "reconstruction case rejected");
  /* q = k, so o_T = s k_T . S_T = s v_T */
  for (long j = 0; j < V; ++j)
    CHECK(fabs(o[(T - 1) * V + j] - v[(T - 1) * V + j] / sqrt((double)K)) < 1e-12,
          "reconstruction: %g vs %g", o[(T - 1) * V + j], v[(T - 1) * V + j] / sqrt((double)K));
  for (long j = 0; j < V; ++j) {
    double p = 0.0;
    for (long c = 0; c < K; ++c) p += k[(T - 1) * K + c] * S[c * V + j];
    CHECK(fabs(p - v[(T - 1) * V + j]) < 1e-12, "k.S = %g, v = %g", p, v[(T - 1) * V + j]);
  }
}

int main(void) {
  srand(1);
  for (int kind = 0; kind < 3; ++kind)
    for (int bias = 0; bias < 2; ++bias)
      for (int s0 = 0; s0 < 2; ++s0) run_case(2, 37, 2, 4, 8, 6, kind, bias, s0);
  run_case(1, 1, 1, 3, 16, 16, 1, 1, 1);
  run_case(3, 0, 1, 1, 4, 4, 0, 0, 1);   /* T = 0: the state passes through */
  run_case(0, 5, 1, 2, 4, 4, 1, 0, 0);   /* B = 0: nothing to do */
  reconstruction();
  for (int kind = 0; kind < 3; ++kind) run_bwd_case(2, 21, 1, 2, 6, 5, kind, kind != 2, 1, 1);
  run_bwd_case(1, 9, 2, 2, 4, 4, 1, 0, 0, 0);
  run_bwd_case(2, 0, 1, 1, 4, 4, 0, 1, 1, 1);  /* T = 0: dS0 = dST */
  double x = 0.0, y = 0.0;
  CHECK(oracle_kda_bwd(&x, &x, &x, &x, &x, &x, NULL, 1, -5.0, NULL, &x, NULL, 1, 1, 2, 3, 1, 1,
                       &y, &y, &y, &y, &y, &y, NULL, NULL, 1) == -1, "bwd: HV %% H != 0 accepted");
  CHECK(oracle_kda_fwd(&x, &x, &x, &x, &x, &x, NULL, 1, -5.0, NULL, 1, 1, 2, 3, 1, 1, &y, NULL, 1) == -1,
        "HV %% H != 0 accepted");
  CHECK(oracle_kda_fwd(NULL, &x, &x, &x, &x, &x, NULL, 1, -5.0, NULL, 1, 1, 1, 1, 1, 1, &y, NULL, 1) == -1,
        "null q accepted");
  CHECK(oracle_gate(&x, &x, NULL, 7, -5.0, 1, 1, 1, 1, &y) == -1, "bad gate kind accepted");
  if (fails) { fprintf(stderr, "%d check(s) failed\n", fails); return 1; }
  printf("oracle driver: all checks passed\n");
  return 0;
}
