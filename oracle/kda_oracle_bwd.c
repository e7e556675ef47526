/*
 * CPU oracle for the gradients of the Kimi Delta Attention forward pass
 * (binary64).
 *
 * TEST INFRASTRUCTURE ONLY: built and called by the tests (and the benchmark's
 * CPU-baseline leg), never by the library.  It shares no code with the HIP
 * library, nor with kda_oracle.c beyond restating the same gate formulas.
 *
 * The pages print no derivation of the backward pass (the "K3 notes" ledger
 * only lists one).  What is differentiated is the four-step update of "K3
 * notes", section "KDA 递归核心", for one (sequence b, value head hv) with the
 * state S[K][V]:
 *
 *     Sd_t = diag(alpha_t) S_{t-1},      alpha_t = exp(g_t)
 *     r_t  = v_t - Sd_t^T k_t
 *     S_t  = Sd_t + beta_t k_t r_t^T
 *     o_t  = s S_t^T q_t,                s = 1/sqrt(K)
 *
 * and the gate of section "Gate 激活" (x = g_raw + dt_bias, rate = exp(A_log)):
 * safe g = L sigmoid(rate x), standard g = -rate softplus(x), none g = g_raw.
 * Given dL/do (and optionally dL/dS_T), reverse-mode differentiation of those
 * lines, token by token from the last, gives (dS the running dL/dS_t):
 *
 *     dS   += s q_t do_t^T                    dq_t  = s S_t do_t
 *     dbeta_t = k_t^T dS r_t                  dr_t  = beta_t dS^T k_t
 *     dv_t  = dr_t                            dk_t  = beta_t dS r_t - Sd_t dr_t
 *     dSd   = dS - k_t dr_t^T                 dg_t  = rowsum(dSd (.) Sd_t)
 *     dS_{t-1} = diag(alpha_t) dSd
 *
 * then the gate's chain rule into g_raw, dt_bias and A_log.  Under GVA the
 * gradients of q and k sum over the value heads that share them.  Nothing is
 * fused or reordered beyond that: every state S_t of a pair is kept.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

enum { BWD_GATE_STANDARD = 0, BWD_GATE_SAFE = 1, BWD_GATE_NONE = 2 };

static double bwd_sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

static double bwd_softplus(double x) {
  return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* g and its derivatives: dg/dx, and dg/dA_log (= dg/drate * rate). */
static void gate_grad(double graw, double rate, double bias, int kind, double L, double* g,
                      double* dg_dx, double* dg_dalog) {
  const double x = graw + bias;
  if (kind == BWD_GATE_SAFE) {
    const double z = rate * x, sg = bwd_sigmoid(z);
    *g = L * sg;
    *dg_dx = L * sg * (1.0 - sg) * rate;
    *dg_dalog = L * sg * (1.0 - sg) * z;
  } else if (kind == BWD_GATE_STANDARD) {
    *g = -rate * bwd_softplus(x);
    *dg_dx = -rate * bwd_sigmoid(x);
    *dg_dalog = *g;
  } else {
    *g = graw;
    *dg_dx = 1.0;
    *dg_dalog = 0.0;
  }
}

typedef struct {
  const double *q, *k, *v, *g_raw, *beta, *A_log, *dt_bias, *S0, *dout, *dST;
  int kind;
  double L;
  long B, T, H, HV, K, V;
  double *dq, *dk, *dv, *dbeta, *dg_raw, *dS0;
  double *dalog_part, *dbias_part; /* per (b, hv): [B, HV] and [B, HV, K] */
  long next;                       /* next (b, h) group to take */
  pthread_mutex_t lock;
} bwd_job_t;

/* Forward then backward for one (b, hv) pair; dq, dk of the pair's q/k head
 * are accumulated (the caller owns every value head of that head). */
static void bwd_pair(const bwd_job_t* J, long b, long hv, double* S, double* alpha, double* dgx,
                     double* dga, double* dS, double* dSd, double* r, double* dr) {
  const long T = J->T, H = J->H, HV = J->HV, K = J->K, V = J->V, KV = K * V;
  const long h = hv / (HV / H);
  const double rate = exp(J->A_log[hv]);
  const double s = 1.0 / sqrt((double)K);

  /* forward, keeping S_{-1} .. S_{T-1} (S + (t + 1) KV) and the gate */
  if (J->S0) memcpy(S, J->S0 + (b * HV + hv) * KV, sizeof(double) * KV);
  else memset(S, 0, sizeof(double) * KV);
  for (long t = 0; t < T; ++t) {
    const long bt = b * T + t;
    const double* kt = J->k + (bt * H + h) * K;
    const double* vt = J->v + (bt * HV + hv) * V;
    const double* gt = J->g_raw + (bt * HV + hv) * K;
    const double be = J->beta[bt * HV + hv];
    const double* Sp = S + t * KV;
    double* Sn = S + (t + 1) * KV;
    for (long c = 0; c < K; ++c) {
      double g;
      gate_grad(gt[c], rate, J->dt_bias ? J->dt_bias[hv * K + c] : 0.0, J->kind, J->L, &g,
                dgx + t * K + c, dga + t * K + c);
      alpha[t * K + c] = exp(g);
    }
    for (long j = 0; j < V; ++j) {
      double p = 0.0;
      for (long c = 0; c < K; ++c) p += kt[c] * alpha[t * K + c] * Sp[c * V + j];
      r[j] = vt[j] - p;
    }
    for (long c = 0; c < K; ++c)
      for (long j = 0; j < V; ++j)
        Sn[c * V + j] = alpha[t * K + c] * Sp[c * V + j] + be * kt[c] * r[j];
  }

  /* backward */
  if (J->dST) memcpy(dS, J->dST + (b * HV + hv) * KV, sizeof(double) * KV);
  else memset(dS, 0, sizeof(double) * KV);
  double dalog = 0.0;
  double* dbias = J->dbias_part + (b * HV + hv) * K;
  for (long t = T - 1; t >= 0; --t) {
    const long bt = b * T + t;
    const double* qt = J->q + (bt * H + h) * K;
    const double* kt = J->k + (bt * H + h) * K;
    const double* vt = J->v + (bt * HV + hv) * V;
    const double* dot = J->dout + (bt * HV + hv) * V;
    const double be = J->beta[bt * HV + hv];
    const double* Sp = S + t * KV;      /* S_{t-1} */
    const double* St = S + (t + 1) * KV; /* S_t */
    double* dqt = J->dq + (bt * H + h) * K;
    double* dkt = J->dk + (bt * H + h) * K;
    /* read: o_t = s S_t^T q_t */
    for (long c = 0; c < K; ++c) {
      double acc = 0.0;
      for (long j = 0; j < V; ++j) {
        dS[c * V + j] += s * qt[c] * dot[j];
        acc += St[c * V + j] * dot[j];
      }
      dqt[c] += s * acc;
    }
    /* write and residual: S_t = Sd + beta k r^T, r = v - Sd^T k */
    for (long j = 0; j < V; ++j) {
      double p = 0.0;
      for (long c = 0; c < K; ++c) p += kt[c] * alpha[t * K + c] * Sp[c * V + j];
      r[j] = vt[j] - p;
    }
    double db = 0.0;
    for (long j = 0; j < V; ++j) {
      double a = 0.0;
      for (long c = 0; c < K; ++c) a += dS[c * V + j] * kt[c];
      dr[j] = be * a;
      db += a * r[j];
      J->dv[(bt * HV + hv) * V + j] = dr[j];
    }
    J->dbeta[bt * HV + hv] = db;
    for (long c = 0; c < K; ++c) {
      double a = 0.0, pr = 0.0;
      for (long j = 0; j < V; ++j) {
        a += dS[c * V + j] * r[j];
        pr += alpha[t * K + c] * Sp[c * V + j] * dr[j];
      }
      dkt[c] += be * a - pr;
    }
    /* decay: Sd = diag(alpha) S_{t-1} */
    for (long c = 0; c < K; ++c) {
      const double al = alpha[t * K + c];
      double dg = 0.0;
      for (long j = 0; j < V; ++j) {
        dSd[c * V + j] = dS[c * V + j] - kt[c] * dr[j];
        dg += dSd[c * V + j] * al * Sp[c * V + j];
      }
      for (long j = 0; j < V; ++j) dS[c * V + j] = al * dSd[c * V + j];
      /* gate */
      J->dg_raw[(bt * HV + hv) * K + c] = dg * dgx[t * K + c];
      if (J->kind != BWD_GATE_NONE) dbias[c] += dg * dgx[t * K + c]; /* none: no bias */
      dalog += dg * dga[t * K + c];
    }
  }
  J->dalog_part[b * HV + hv] = dalog;
  if (J->dS0) memcpy(J->dS0 + (b * HV + hv) * KV, dS, sizeof(double) * KV);
}

static void* bwd_worker(void* arg) {
  bwd_job_t* J = (bwd_job_t*)arg;
  const long KV = J->K * J->V, G = J->HV / J->H;
  double* S = (double*)malloc(sizeof(double) * (J->T + 1) * KV);
  double* alpha = (double*)malloc(sizeof(double) * (J->T > 0 ? J->T : 1) * J->K);
  double* dgx = (double*)malloc(sizeof(double) * (J->T > 0 ? J->T : 1) * J->K);
  double* dga = (double*)malloc(sizeof(double) * (J->T > 0 ? J->T : 1) * J->K);
  double* dS = (double*)malloc(sizeof(double) * KV);
  double* dSd = (double*)malloc(sizeof(double) * KV);
  double* r = (double*)malloc(sizeof(double) * J->V);
  double* dr = (double*)malloc(sizeof(double) * J->V);
  for (;;) {
    pthread_mutex_lock(&J->lock);
    long grp = J->next++;
    pthread_mutex_unlock(&J->lock);
    if (grp >= J->B * J->H) break;
    const long b = grp / J->H, h = grp % J->H;
    for (long j = 0; j < G; ++j) bwd_pair(J, b, h * G + j, S, alpha, dgx, dga, dS, dSd, r, dr);
  }
  free(S); free(alpha); free(dgx); free(dga); free(dS); free(dSd); free(r); free(dr);
  return NULL;
}

/* Gradients of L = sum(o * dout) + sum(S_T * dST) (dST may be NULL) with
 * respect to every input, over all (b, hv) pairs on `nthreads` host threads
 * (one (b, q/k head) group per thread at a time).  Shapes as the forward
 * oracle; outputs dq, dk [B,T,H,K], dv [B,T,HV,V], dbeta [B,T,HV], dg_raw
 * [B,T,HV,K], dA_log [HV], ddt_bias [HV,K] (may be NULL), dS0 [B,HV,K,V] (may
 * be NULL).  Returns 0, or -1 on a bad argument. */
int oracle_kda_bwd(const double* q, const double* k, const double* v, const double* g_raw,
                   const double* beta, const double* A_log, const double* dt_bias, int kind,
                   double lower_bound, const double* S0, const double* dout, const double* dST,
                   long B, long T, long H, long HV, long K, long V, double* dq, double* dk,
                   double* dv, double* dbeta, double* dg_raw, double* dA_log, double* ddt_bias,
                   double* dS0, int nthreads) {
  if (!q || !k || !v || !g_raw || !beta || !A_log || !dout) return -1;
  if (!dq || !dk || !dv || !dbeta || !dg_raw || !dA_log) return -1;
  if (B < 0 || T < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || HV % H != 0) return -1;
  if (kind < 0 || kind > 2) return -1;
  memset(dq, 0, sizeof(double) * B * T * H * K);
  memset(dk, 0, sizeof(double) * B * T * H * K);
  double* dalog_part = (double*)calloc((size_t)(B * HV > 0 ? B * HV : 1), sizeof(double));
  double* dbias_part = (double*)calloc((size_t)(B * HV * K > 0 ? B * HV * K : 1), sizeof(double));
  bwd_job_t J = {q, k, v, g_raw, beta, A_log, dt_bias, S0, dout, dST, kind, lower_bound,
                 B, T, H, HV, K, V, dq, dk, dv, dbeta, dg_raw, dS0, dalog_part, dbias_part, 0};
  pthread_mutex_init(&J.lock, NULL);
  long groups = B * H;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > groups) nthreads = (int)(groups > 0 ? groups : 1);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, bwd_worker, &J);
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.lock);
  /* sums over the sequences, in a fixed order */
  for (long hv = 0; hv < HV; ++hv) {
    double a = 0.0;
    for (long b = 0; b < B; ++b) a += dalog_part[b * HV + hv];
    dA_log[hv] = a;
    if (ddt_bias)
      for (long c = 0; c < K; ++c) {
        double d = 0.0;
        for (long b = 0; b < B; ++b) d += dbias_part[(b * HV + hv) * K + c];
        ddt_bias[hv * K + c] = d;
      }
  }
  free(dalog_part);
  free(dbias_part);
  return 0;
}
