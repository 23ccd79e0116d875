/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the Gated DeltaNet (GDN) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP library under gated_deltanet_chunkwise_amd/.
 *
 * What it computes (token by token, in the order the method defines it):
 *
 *   Gate.  The KDA gate guide (MindSpeed-Ops issue page, "core computation
 *   logic": formula + numerically stable softplus) defines the gate activation
 *   y = -exp(A_log[h]) * softplus(x + dt_bias), softplus(x) = x for x > 20 and
 *   log(1 + exp(x)) otherwise.  GDN uses the per-value-head scalar case:
 *   g[t,hv] = -exp(A_log[hv]) * softplus(g_raw[t,hv] + dt_bias[hv]).
 *   log1p(exp(x)) is used for log(1+exp(x)); it is the same function.
 *
 *   Recurrence.  The Ascend GDN blog (hwcomputing.csdn.net, section "GDN
 *   sequence structure and Triton introduction") describes GDN as linear
 *   attention + gating + the delta rule, with one fixed-size state matrix per
 *   head updated as each token arrives.  That update is the gated delta rule
 *       S_t = exp(g_t) * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *       o_t = scale * S_t q_t,
 *   with S_t of shape V x K.  The oracle keeps H = S^T (K x V, row-major, V
 *   contiguous) and expands the product:
 *       p   = H^T k_t                      (= S_{t-1} k_t, a V-vector)
 *       H  <- a H + beta_t k_t (v_t - a p)^T,   a = exp(g_t)
 *       o_t = scale * H^T q_t
 *   which is the same matrix identity written for the transpose.
 *
 *   Heads.  H query/key heads, HV value heads, HV a multiple of H; value head
 *   hv reads key/query head hv / (HV/H) (consecutive groups).
 *
 *   Sequences.  Either B fixed-length sequences of T tokens, or one packed
 *   batch of N sequences given by int64 offsets cu_seqlens[0..N] (the G_T_CONTIG
 *   page, "varlen checklist": offsets are int64, token positions are absolute
 *   packed indices).  The state starts from h0[n,hv] (or zero) at every
 *   sequence start.
 *
 * Layouts (all fp64, row-major, contiguous):
 *   q, k    [Ttot][H][K]      Ttot = B*T, or the packed total
 *   v       [Ttot][HV][V]
 *   g, beta [Ttot][HV]        g is the log-decay (already gated)
 *   h0, fin [N][HV][K][V]     element [n][hv][i][j] = S[j][i]
 *   o       [Ttot][HV][V]
 *
 * Work units are (sequence n, value head hv) pairs, unit id = n*HV + hv; they
 * are independent and are spread over a pthread pool.  A unit list restricts
 * the computation to some units (only their o rows and final states are
 * written).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Return codes. */
#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/* softplus as the KDA gate guide states it: identity above 20. */
static double oracle_softplus(double x) { return x > 20.0 ? x : log1p(exp(x)); }

void gdn_oracle_gate(const double *g_raw, const double *A_log, const double *dt_bias,
                     int64_t ntok, int HV, double *g_out) {
  for (int64_t t = 0; t < ntok; ++t)
    for (int hv = 0; hv < HV; ++hv) {
      double x = g_raw[t * HV + hv] + (dt_bias ? dt_bias[hv] : 0.0);
      g_out[t * HV + hv] = -exp(A_log[hv]) * oracle_softplus(x);
    }
}

/* KDA gate, per channel (the KDA gate guide, "core computation logic": the
 * formula, the stable softplus, fp32 inside the operator -- here fp64):
 *   yg[t,h,d] = -exp(A_log[h]) * softplus(g[t,h,d] + dt_bias[h*D + d]).
 * Layouts: g, yg [T][H][D] contiguous; A_log [H]; dt_bias [H*D] or NULL (no
 * bias).  T is the number of rows after flattening the leading dimensions. */
void gdn_oracle_kda_gate(const double *g, const double *A_log, const double *dt_bias,
                         int64_t T, int H, int D, double *yg) {
  for (int64_t t = 0; t < T; ++t)
    for (int h = 0; h < H; ++h) {
      const double head_scale = -exp(A_log[h]);
      const int64_t row = (t * H + h) * (int64_t)D;
      for (int d = 0; d < D; ++d) {
        const double biased = g[row + d] + (dt_bias ? dt_bias[(int64_t)h * D + d] : 0.0);
        yg[row + d] = head_scale * oracle_softplus(biased);
      }
    }
}

typedef struct {
  int HV, H, K, V, N;
  const int64_t *bos; /* [N+1] sequence offsets */
  const double *q, *k, *v, *g, *beta, *h0;
  double scale;
  const int32_t *units;
  int n_units;
  double *o, *fin;
  int next; /* shared work counter (guarded by mu) */
  int status;
  pthread_mutex_t mu;
} oracle_job;

static int oracle_take(oracle_job *J) {
  pthread_mutex_lock(&J->mu);
  int u = J->next < J->n_units ? J->next++ : -1;
  pthread_mutex_unlock(&J->mu);
  return u;
}

static void oracle_run_unit(const oracle_job *J, int unit, double *Hs, double *p) {
  const int HV = J->HV, H = J->H, K = J->K, V = J->V;
  const int n = unit / HV, hv = unit % HV;
  const int h = hv / (HV / H);
  if (J->h0)
    memcpy(Hs, J->h0 + ((int64_t)n * HV + hv) * K * V, sizeof(double) * K * V);
  else
    memset(Hs, 0, sizeof(double) * K * V);
  for (int64_t t = J->bos[n]; t < J->bos[n + 1]; ++t) {
    const double *kt = J->k + (t * H + h) * K;
    const double *qt = J->q + (t * H + h) * K;
    const double *vt = J->v + (t * HV + hv) * V;
    const double a = exp(J->g[t * HV + hv]);
    const double b = J->beta[t * HV + hv];
    /* p = S_{t-1} k_t = H^T k_t */
    for (int j = 0; j < V; ++j) p[j] = 0.0;
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < V; ++j) p[j] += Hs[i * V + j] * kt[i];
    /* H <- a H + b k (v - a p)^T */
    for (int j = 0; j < V; ++j) p[j] = vt[j] - a * p[j];
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < V; ++j) Hs[i * V + j] = a * Hs[i * V + j] + b * kt[i] * p[j];
    /* o_t = scale * H^T q_t */
    double *ot = J->o + (t * HV + hv) * V;
    for (int j = 0; j < V; ++j) ot[j] = 0.0;
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < V; ++j) ot[j] += Hs[i * V + j] * qt[i];
    for (int j = 0; j < V; ++j) ot[j] *= J->scale;
  }
  if (J->fin) memcpy(J->fin + ((int64_t)n * HV + hv) * K * V, Hs, sizeof(double) * K * V);
}

static void *oracle_worker(void *arg) {
  oracle_job *J = (oracle_job *)arg;
  double *Hs = (double *)malloc(sizeof(double) * J->K * J->V);
  double *p = (double *)malloc(sizeof(double) * J->V);
  if (!Hs || !p) {
    pthread_mutex_lock(&J->mu);
    J->status = ORACLE_ENOMEM;
    pthread_mutex_unlock(&J->mu);
  } else {
    for (int i; (i = oracle_take(J)) >= 0;)
      oracle_run_unit(J, J->units ? J->units[i] : i, Hs, p);
  }
  free(Hs);
  free(p);
  return NULL;
}

/*
 * Recurrence from a given log-decay g.  cu_seqlens (host, N+1 entries) may be
 * NULL: then N = B sequences of T tokens each.  Returns ORACLE_* codes.
 */
int gdn_oracle_recurrence(int B, int T, int H, int HV, int K, int V,
                          const int64_t *cu_seqlens, int N,
                          const double *q, const double *k, const double *v,
                          const double *g, const double *beta, const double *h0,
                          double scale, const int32_t *units, int n_units,
                          double *o, double *final_state, int nthreads) {
  if (H <= 0 || HV <= 0 || HV % H || K <= 0 || V <= 0 || T < 0 || B < 0) return ORACLE_EINVAL;
  int64_t *bos;
  if (cu_seqlens) {
    if (N < 0 || B != 1) return ORACLE_EINVAL;
    if (cu_seqlens[0] != 0 || cu_seqlens[N] != T) return ORACLE_EINVAL;
    for (int n = 0; n < N; ++n)
      if (cu_seqlens[n + 1] < cu_seqlens[n]) return ORACLE_EINVAL;
    bos = (int64_t *)malloc(sizeof(int64_t) * (N + 1));
    if (!bos) return ORACLE_ENOMEM;
    memcpy(bos, cu_seqlens, sizeof(int64_t) * (N + 1));
  } else {
    N = B;
    bos = (int64_t *)malloc(sizeof(int64_t) * (N + 1));
    if (!bos) return ORACLE_ENOMEM;
    for (int n = 0; n <= N; ++n) bos[n] = (int64_t)n * T;
  }
  int total = N * HV;
  if (units) {
    for (int i = 0; i < n_units; ++i)
      if (units[i] < 0 || units[i] >= total) {
        free(bos);
        return ORACLE_EINVAL;
      }
  } else {
    n_units = total;
  }
  oracle_job J;
  memset(&J, 0, sizeof J);
  J.HV = HV; J.H = H; J.K = K; J.V = V; J.N = N;
  J.bos = bos; J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0;
  J.scale = scale; J.units = units; J.n_units = n_units;
  J.o = o; J.fin = final_state;
  pthread_mutex_init(&J.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n_units) nthreads = n_units > 0 ? n_units : 1;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
  int started = 0;
  if (th)
    for (; started < nthreads - 1; ++started)
      if (pthread_create(&th[started], NULL, oracle_worker, &J)) break;
  oracle_worker(&J); /* the calling thread works too */
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  free(bos);
  return J.status;
}

/* Full forward pass: gate, then the recurrence. */
int gdn_oracle_fwd(int B, int T, int H, int HV, int K, int V,
                   const int64_t *cu_seqlens, int N,
                   const double *q, const double *k, const double *v,
                   const double *g_raw, const double *beta,
                   const double *A_log, const double *dt_bias, const double *h0,
                   double scale, const int32_t *units, int n_units,
                   double *o, double *final_state, int nthreads) {
  int64_t ntok = cu_seqlens ? (int64_t)T : (int64_t)B * T;
  double *g = (double *)malloc(sizeof(double) * (ntok > 0 ? ntok : 1) * HV);
  if (!g) return ORACLE_ENOMEM;
  gdn_oracle_gate(g_raw, A_log, dt_bias, ntok, HV, g);
  int rc = gdn_oracle_recurrence(B, T, H, HV, K, V, cu_seqlens, N, q, k, v, g, beta, h0,
                                 scale, units, n_units, o, final_state, nthreads);
  free(g);
  return rc;
}
