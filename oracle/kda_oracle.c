/*
 * CPU oracle for the Kimi Delta Attention (KDA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library; the two are built
 * separately and neither includes the other.
 *
 * Arithmetic is IEEE binary64 throughout.  Inputs arrive as doubles holding
 * exactly the values the GPU path reads (bf16/fp32 values widen exactly).
 *
 * What is computed, and where the pages define it:
 *
 *  - Gate activation ("K3 notes", section "Gate 激活", two-gate table and the
 *    kda_gate_reference code panel; "Gate 在 API 中的位置" for the in-op gate):
 *        input = g_raw + dt_bias[hv, kappa]   (dt_bias may be absent)
 *        rate  = exp(A_log[hv])
 *        safe      : g = L * sigmoid(rate * input)        in [L, 0]
 *        standard  : g = -rate * softplus(input)          in (-inf, 0]
 *        none      : g = g_raw   (caller supplies the log-decay itself)
 *
 *  - The recurrence ("K3 notes", section "KDA 递归核心", subsection
 *    "逐步公式": the four-step update), state S[kappa][v] (key rows, value
 *    columns), for every token t in order:
 *        1. decay   S_dec = exp(g_t) (.) S_{t-1}       (row kappa scaled)
 *        2. predict p_t   = k_t . S_dec ; residual r_t = v_t - p_t
 *        3. write   S_t   = S_dec + (beta_t k_t) outer r_t
 *        4. read    o_t   = (1/sqrt(K)) q_t . S_t
 *    The 1/sqrt(K) read scale is the one printed in that subsection's step 4
 *    and in the ledger's derivation DER1 step 4; the code panel on the same
 *    page leaves it out, and this oracle follows the formula.
 *
 *  - GVA ("K3 notes" input table: q and k already repeat_interleave'd to HV):
 *    value head hv reads query/key head h = hv / (HV / H).
 *
 * Layouts (row-major, contiguous):
 *    q, k   [B, T, H, K]      v      [B, T, HV, V]
 *    g_raw  [B, T, HV, K]     beta   [B, T, HV]
 *    A_log  [HV]              dt_bias[HV, K] or NULL
 *    S0     [B, HV, K, V] or NULL (zeros)
 *    o      [B, T, HV, V]     S_out  [B, HV, K, V] or NULL
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_GATE_STANDARD 0
#define ORACLE_GATE_SAFE 1
#define ORACLE_GATE_NONE 2

/* softplus(x) = log(1 + e^x), written so that neither branch overflows. */
static double softplus(double x) {
  if (isnan(x)) return x;
  return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* sigmoid(z) = 1 / (1 + e^-z); e^-z overflowing to +inf gives the exact
 * limit 0, and NaN stays NaN. */
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* One gate value.  "Gate 激活", two-gate table / kda_gate_reference. */
static double gate_one(double graw, double rate, double bias, int kind, double L) {
  double input = graw + bias;
  if (kind == ORACLE_GATE_SAFE) return L * sigmoid(rate * input);
  if (kind == ORACLE_GATE_STANDARD) return -rate * softplus(input);
  return graw; /* ORACLE_GATE_NONE */
}

/* g = gate(g_raw) elementwise over [B, T, HV, K].  Returns 0, or -1 on a bad
 * argument. */
int oracle_gate(const double* g_raw, const double* A_log, const double* dt_bias, int kind,
                double lower_bound, long B, long T, long HV, long K, double* g_out) {
  if (!g_raw || !A_log || !g_out || B < 0 || T < 0 || HV <= 0 || K <= 0) return -1;
  if (kind < 0 || kind > 2) return -1;
  for (long b = 0; b < B; ++b)
    for (long t = 0; t < T; ++t)
      for (long hv = 0; hv < HV; ++hv) {
        double rate = exp(A_log[hv]);
        long base = ((b * T + t) * HV + hv) * K;
        for (long c = 0; c < K; ++c) {
          double bias = dt_bias ? dt_bias[hv * K + c] : 0.0;
          g_out[base + c] = gate_one(g_raw[base + c], rate, bias, kind, lower_bound);
        }
      }
  return 0;
}

typedef struct {
  const double *q, *k, *v, *g_raw, *beta, *A_log, *dt_bias, *S0;
  int kind;
  double L;
  long B, T, H, HV, K, V;
  double *o, *S_out;
  long next;            /* next (b, hv) pair to take */
  pthread_mutex_t lock;
} job_t;

/* The recurrence for one (b, hv) pair, token by token. */
static void run_pair(const job_t* J, long b, long hv, double* S, double* alpha, double* p) {
  const long T = J->T, H = J->H, HV = J->HV, K = J->K, V = J->V;
  const long h = hv / (HV / H);
  const double rate = exp(J->A_log[hv]);
  const double scale = 1.0 / sqrt((double)K);

  if (J->S0)
    memcpy(S, J->S0 + (b * HV + hv) * K * V, sizeof(double) * K * V);
  else
    memset(S, 0, sizeof(double) * K * V);

  for (long t = 0; t < T; ++t) {
    const double* qt = J->q + ((b * T + t) * H + h) * K;
    const double* kt = J->k + ((b * T + t) * H + h) * K;
    const double* vt = J->v + ((b * T + t) * HV + hv) * V;
    const double* gt = J->g_raw + ((b * T + t) * HV + hv) * K;
    const double bt = J->beta[(b * T + t) * HV + hv];
    double* ot = J->o + ((b * T + t) * HV + hv) * V;

    /* gate -> per-key-channel retain factor exp(g) */
    for (long c = 0; c < K; ++c) {
      double bias = J->dt_bias ? J->dt_bias[hv * K + c] : 0.0;
      alpha[c] = exp(gate_one(gt[c], rate, bias, J->kind, J->L));
    }
    /* 1. decay: row c of S scaled by exp(g_t[c]) */
    for (long c = 0; c < K; ++c)
      for (long j = 0; j < V; ++j) S[c * V + j] *= alpha[c];
    /* 2. predict with the key, then the residual */
    for (long j = 0; j < V; ++j) p[j] = 0.0;
    for (long c = 0; c < K; ++c)
      for (long j = 0; j < V; ++j) p[j] += kt[c] * S[c * V + j];
    for (long j = 0; j < V; ++j) p[j] = vt[j] - p[j]; /* p now holds r_t */
    /* 3. rank-1 write of beta_t k_t against the residual */
    for (long c = 0; c < K; ++c) {
      double a = bt * kt[c];
      for (long j = 0; j < V; ++j) S[c * V + j] += a * p[j];
    }
    /* 4. read with the query, scaled by 1/sqrt(K) */
    for (long j = 0; j < V; ++j) {
      double acc = 0.0;
      for (long c = 0; c < K; ++c) acc += qt[c] * S[c * V + j];
      ot[j] = scale * acc;
    }
  }
  if (J->S_out) memcpy(J->S_out + (b * HV + hv) * K * V, S, sizeof(double) * K * V);
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  double* S = (double*)malloc(sizeof(double) * J->K * J->V);
  double* alpha = (double*)malloc(sizeof(double) * J->K);
  double* p = (double*)malloc(sizeof(double) * J->V);
  for (;;) {
    pthread_mutex_lock(&J->lock);
    long pair = J->next++;
    pthread_mutex_unlock(&J->lock);
    if (pair >= J->B * J->HV) break;
    run_pair(J, pair / J->HV, pair % J->HV, S, alpha, p);
  }
  free(S);
  free(alpha);
  free(p);
  return NULL;
}

/* The KDA forward pass over all (b, hv) pairs, spread over `nthreads` host
 * threads (pairs are independent).  Returns 0, or -1 on a bad argument. */
int oracle_kda_fwd(const double* q, const double* k, const double* v, const double* g_raw,
                   const double* beta, const double* A_log, const double* dt_bias, int kind,
                   double lower_bound, const double* S0, long B, long T, long H, long HV,
                   long K, long V, double* o, double* S_out, int nthreads) {
  if (!q || !k || !v || !g_raw || !beta || !A_log || !o) return -1;
  if (B < 0 || T < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || HV % H != 0) return -1;
  if (kind < 0 || kind > 2) return -1;
  job_t J = {q, k, v, g_raw, beta, A_log, dt_bias, S0, kind, lower_bound,
             B, T, H, HV, K, V, o, S_out, 0};
  pthread_mutex_init(&J.lock, NULL);
  long pairs = B * HV;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > pairs) nthreads = (int)(pairs > 0 ? pairs : 1);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &J);
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.lock);
  return 0;
}
