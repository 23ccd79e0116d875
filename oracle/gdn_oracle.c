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
 *
 * Backward (gdn_oracle_bwd).  The pages name the backward kernels (dv_local,
 * dq/dk/dw/dg, dg, the WY backward, dh/du of the state recurrence; the Ascend
 * GDN blog, "Ascend-affine tiling", and the G_T_CONTIG page, "fix" and
 * "correctness gates", whose dq/dk/dw/dg test takes automatic differentiation
 * as its oracle) but do not write their formulas.  The oracle is therefore the
 * plain reverse-mode derivative of the token recurrence above: for the scalar
 *     L = sum_t <do_t, o_t> + <dht, H_final>
 * it returns dL/dq, dL/dk, dL/dv, dL/dbeta, dL/dg_raw, dL/dA_log, dL/ddt_bias
 * and dL/dh0, walking each sequence's tokens backwards with the states H_{t-1}
 * kept from a forward sweep.  Per token (a = exp(g_t), p = H_{t-1}^T k_t,
 * u = v_t - a p, H_t = a H_{t-1} + beta k_t u^T, dH the running dL/dH_t):
 *     dH   += scale q_t do_t^T                   (o_t = scale H_t^T q_t)
 *     dq_t  = scale H_t do_t
 *     du    = beta dH^T k_t,   dv_t = du,   dp = -a du
 *     dbeta = k_t^T dH u
 *     dk_t  = beta dH u + H_{t-1} dp
 *     da    = <dH, H_{t-1}> - p . du,   dg_t = a da
 *     dH   <- a dH + k_t dp^T                    (now dL/dH_{t-1})
 * and through the gate g = -exp(A_log) softplus(x), x = g_raw + dt_bias:
 *     dg_raw = dg (-exp(A_log)) softplus'(x),  softplus'(x) = 1 (x > 20) else
 *     1 / (1 + exp(-x));  dA_log += dg g;  ddt_bias += dg_raw.
 * dq and dk of key head h sum the value heads that read it.
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

/*
 * Host twin of the library's gdn_fwd, with its argument order: the sizes
 * (B, T, H, HV, K, V, num_seqs, scale standing in for its parameter struct),
 * then q, k, v, g_raw, beta, A_log, dt_bias, cu_seqlens, initial_state, o,
 * final_state, all fp64 host arrays in the library's layouts; the workspace
 * and stream have no counterpart, nthreads takes their place.  cu_seqlens
 * NULL: B sequences of T tokens; otherwise num_seqs packed sequences (B = 1).
 * dt_bias and initial_state may be NULL (zero); final_state may be NULL (not
 * written).  Returns ORACLE_* codes.
 */
int gdn_ref_fwd(int B, int T, int H, int HV, int K, int V, int num_seqs, double scale,
                const double *q, const double *k, const double *v, const double *g_raw,
                const double *beta, const double *A_log, const double *dt_bias,
                const int64_t *cu_seqlens, const double *initial_state, double *o,
                double *final_state, int nthreads) {
  int N = cu_seqlens ? num_seqs : B;
  double *fin = final_state;
  if (!fin && N > 0 && HV > 0 && K > 0 && V > 0) {
    fin = (double *)malloc(sizeof(double) * (size_t)N * HV * K * V);
    if (!fin) return ORACLE_ENOMEM;
  }
  int rc = gdn_oracle_fwd(B, T, H, HV, K, V, cu_seqlens, N, q, k, v, g_raw, beta, A_log,
                          dt_bias, initial_state, scale, NULL, 0, o, fin, nthreads);
  if (fin != final_state) free(fin);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Backward: reverse-mode derivative of the token recurrence (see the top).  */

static double oracle_softplus_slope(double x) { return x > 20.0 ? 1.0 : 1.0 / (1.0 + exp(-x)); }

typedef struct {
  int HV, H, K, V, N;
  const int64_t *bos;
  const double *q, *k, *v, *g_raw, *beta, *A_log, *dt_bias, *h0, *dout, *dht;
  double scale;
  const int32_t *units;
  int n_units;
  double *dqh, *dkh;       /* [Ttot][HV][K], per value head (summed after) */
  double *dv, *dg_raw, *dbeta, *dh0;
  double *dA_part, *db_part; /* [N][HV] per-sequence sums */
  int next;
  int status;
  pthread_mutex_t mu;
} oracle_bwd_job;

static int oracle_bwd_take(oracle_bwd_job *J) {
  pthread_mutex_lock(&J->mu);
  int u = J->next < J->n_units ? J->next++ : -1;
  pthread_mutex_unlock(&J->mu);
  return u;
}

static int oracle_bwd_unit(const oracle_bwd_job *J, int unit) {
  const int HV = J->HV, H = J->H, K = J->K, V = J->V;
  const int n = unit / HV, hv = unit % HV, h = hv / (HV / H);
  const int64_t t0 = J->bos[n], L = J->bos[n + 1] - t0;
  const int64_t KV = (int64_t)K * V;
  double *hist = (double *)malloc(sizeof(double) * KV * (L > 0 ? L : 1));
  double *Hs = (double *)malloc(sizeof(double) * KV);
  double *dH = (double *)malloc(sizeof(double) * KV);
  double *p = (double *)malloc(sizeof(double) * V);
  double *u = (double *)malloc(sizeof(double) * V);
  double *du = (double *)malloc(sizeof(double) * V);
  double *gl = (double *)malloc(sizeof(double) * (L > 0 ? L : 1));
  int rc = ORACLE_OK;
  if (!hist || !Hs || !dH || !p || !u || !du || !gl) {
    rc = ORACLE_ENOMEM;
    goto out;
  }
  const double ea = exp(J->A_log[hv]);
  const double bias = J->dt_bias ? J->dt_bias[hv] : 0.0;
  /* Forward sweep, keeping H_{t-1} of every token. */
  if (J->h0)
    memcpy(Hs, J->h0 + ((int64_t)n * HV + hv) * KV, sizeof(double) * KV);
  else
    memset(Hs, 0, sizeof(double) * KV);
  for (int64_t s = 0; s < L; ++s) {
    const int64_t t = t0 + s;
    const double *kt = J->k + (t * H + h) * K;
    const double *vt = J->v + (t * HV + hv) * V;
    gl[s] = -ea * oracle_softplus(J->g_raw[t * HV + hv] + bias);
    const double a = exp(gl[s]), b = J->beta[t * HV + hv];
    memcpy(hist + s * KV, Hs, sizeof(double) * KV);
    for (int j = 0; j < V; ++j) p[j] = 0.0;
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < V; ++j) p[j] += Hs[i * V + j] * kt[i];
    for (int j = 0; j < V; ++j) u[j] = vt[j] - a * p[j];
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < V; ++j) Hs[i * V + j] = a * Hs[i * V + j] + b * kt[i] * u[j];
  }
  /* Backward sweep. */
  if (J->dht)
    memcpy(dH, J->dht + ((int64_t)n * HV + hv) * KV, sizeof(double) * KV);
  else
    memset(dH, 0, sizeof(double) * KV);
  double dA_sum = 0.0, db_sum = 0.0;
  for (int64_t s = L - 1; s >= 0; --s) {
    const int64_t t = t0 + s;
    const double *kt = J->k + (t * H + h) * K;
    const double *qt = J->q + (t * H + h) * K;
    const double *vt = J->v + (t * HV + hv) * V;
    const double *dot = J->dout + (t * HV + hv) * V;
    const double *Hp = hist + s * KV;
    const double a = exp(gl[s]), b = J->beta[t * HV + hv];
    /* recompute p, u and H_t from H_{t-1} */
    for (int j = 0; j < V; ++j) p[j] = 0.0;
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < V; ++j) p[j] += Hp[i * V + j] * kt[i];
    for (int j = 0; j < V; ++j) u[j] = vt[j] - a * p[j];
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < V; ++j) Hs[i * V + j] = a * Hp[i * V + j] + b * kt[i] * u[j];
    /* o_t = scale H_t^T q_t */
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < V; ++j) dH[i * V + j] += J->scale * qt[i] * dot[j];
    double *dq = J->dqh + (t * HV + hv) * K;
    for (int i = 0; i < K; ++i) {
      double acc = 0.0;
      for (int j = 0; j < V; ++j) acc += Hs[i * V + j] * dot[j];
      dq[i] = J->scale * acc;
    }
    /* H_t = a H_{t-1} + b k u^T,  u = v - a H_{t-1}^T k */
    for (int j = 0; j < V; ++j) {
      double acc = 0.0;
      for (int i = 0; i < K; ++i) acc += dH[i * V + j] * kt[i];
      du[j] = b * acc;
    }
    double dbeta = 0.0;
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < V; ++j) dbeta += dH[i * V + j] * kt[i] * u[j];
    double *dk = J->dkh + (t * HV + hv) * K;
    for (int i = 0; i < K; ++i) {
      double acc_u = 0.0, acc_p = 0.0;
      for (int j = 0; j < V; ++j) {
        acc_u += dH[i * V + j] * u[j];
        acc_p += Hp[i * V + j] * (-a * du[j]);
      }
      dk[i] = b * acc_u + acc_p;
    }
    double *dv = J->dv + (t * HV + hv) * V;
    for (int j = 0; j < V; ++j) dv[j] = du[j];
    double da = 0.0;
    for (int64_t e = 0; e < KV; ++e) da += dH[e] * Hp[e];
    for (int j = 0; j < V; ++j) da -= p[j] * du[j];
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < V; ++j) dH[i * V + j] = a * dH[i * V + j] + kt[i] * (-a * du[j]);
    const double dg = a * da;
    const double x = J->g_raw[t * HV + hv] + bias;
    const double dgr = dg * (-ea) * oracle_softplus_slope(x);
    J->dbeta[t * HV + hv] = dbeta;
    J->dg_raw[t * HV + hv] = dgr;
    dA_sum += dg * gl[s];
    db_sum += dgr;
  }
  J->dA_part[(int64_t)n * HV + hv] = dA_sum;
  J->db_part[(int64_t)n * HV + hv] = db_sum;
  if (J->dh0) memcpy(J->dh0 + ((int64_t)n * HV + hv) * KV, dH, sizeof(double) * KV);
out:
  free(hist); free(Hs); free(dH); free(p); free(u); free(du); free(gl);
  return rc;
}

static void *oracle_bwd_worker(void *arg) {
  oracle_bwd_job *J = (oracle_bwd_job *)arg;
  for (int i; (i = oracle_bwd_take(J)) >= 0;) {
    int rc = oracle_bwd_unit(J, J->units ? J->units[i] : i);
    if (rc) {
      pthread_mutex_lock(&J->mu);
      J->status = rc;
      pthread_mutex_unlock(&J->mu);
    }
  }
  return NULL;
}

/*
 * Backward of gdn_oracle_fwd for L = sum <dout, o> + <dht, final state>.
 * Inputs as gdn_oracle_fwd, plus dout [Ttot][HV][V] and dht [N][HV][K][V]
 * (NULL = 0).  Outputs: dq, dk [Ttot][H][K]; dv [Ttot][HV][V]; dg_raw, dbeta
 * [Ttot][HV]; dA_log, ddt_bias [HV]; dh0 [N][HV][K][V] (NULL = not wanted).
 * With a unit list only those (n, hv) units contribute: dv, dg_raw, dbeta and
 * dh0 of other units are left as they are, dq/dk/dA_log/ddt_bias sum the
 * listed units only.  Memory: one unit holds its sequence length x K x V
 * doubles of states.
 */
int gdn_oracle_bwd(int B, int T, int H, int HV, int K, int V,
                   const int64_t *cu_seqlens, int N,
                   const double *q, const double *k, const double *v,
                   const double *g_raw, const double *beta,
                   const double *A_log, const double *dt_bias, const double *h0,
                   double scale, const double *dout, const double *dht,
                   const int32_t *units, int n_units,
                   double *dq, double *dk, double *dv, double *dg_raw, double *dbeta,
                   double *dA_log, double *ddt_bias, double *dh0, int nthreads) {
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
  const int total = N * HV;
  if (units) {
    for (int i = 0; i < n_units; ++i)
      if (units[i] < 0 || units[i] >= total) {
        free(bos);
        return ORACLE_EINVAL;
      }
  } else {
    n_units = total;
  }
  const int64_t ntok = bos[N];
  oracle_bwd_job J;
  memset(&J, 0, sizeof J);
  J.HV = HV; J.H = H; J.K = K; J.V = V; J.N = N; J.bos = bos;
  J.q = q; J.k = k; J.v = v; J.g_raw = g_raw; J.beta = beta; J.A_log = A_log;
  J.dt_bias = dt_bias; J.h0 = h0; J.dout = dout; J.dht = dht; J.scale = scale;
  J.units = units; J.n_units = n_units;
  J.dqh = (double *)calloc((size_t)(ntok > 0 ? ntok : 1) * HV * K, sizeof(double));
  J.dkh = (double *)calloc((size_t)(ntok > 0 ? ntok : 1) * HV * K, sizeof(double));
  J.dA_part = (double *)calloc((size_t)(total > 0 ? total : 1), sizeof(double));
  J.db_part = (double *)calloc((size_t)(total > 0 ? total : 1), sizeof(double));
  J.dv = dv; J.dg_raw = dg_raw; J.dbeta = dbeta; J.dh0 = dh0;
  if (!J.dqh || !J.dkh || !J.dA_part || !J.db_part) {
    free(J.dqh); free(J.dkh); free(J.dA_part); free(J.db_part); free(bos);
    return ORACLE_ENOMEM;
  }
  pthread_mutex_init(&J.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n_units) nthreads = n_units > 0 ? n_units : 1;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
  int started = 0;
  if (th)
    for (; started < nthreads - 1; ++started)
      if (pthread_create(&th[started], NULL, oracle_bwd_worker, &J)) break;
  oracle_bwd_worker(&J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  /* Key-head gradients: sum the value heads of each group, in head order. */
  const int G = HV / H;
  for (int64_t t = 0; t < ntok; ++t)
    for (int h = 0; h < H; ++h)
      for (int i = 0; i < K; ++i) {
        double sq = 0.0, sk = 0.0;
        for (int r = 0; r < G; ++r) {
          sq += J.dqh[(t * HV + h * G + r) * K + i];
          sk += J.dkh[(t * HV + h * G + r) * K + i];
        }
        dq[(t * H + h) * K + i] = sq;
        dk[(t * H + h) * K + i] = sk;
      }
  /* Per-head parameter gradients: sum over sequences, in sequence order. */
  for (int hv = 0; hv < HV; ++hv) {
    double sa = 0.0, sb = 0.0;
    for (int n = 0; n < N; ++n) {
      sa += J.dA_part[(int64_t)n * HV + hv];
      sb += J.db_part[(int64_t)n * HV + hv];
    }
    dA_log[hv] = sa;
    if (ddt_bias) ddt_bias[hv] = sb;
  }
  free(J.dqh); free(J.dkh); free(J.dA_part); free(J.db_part); free(bos);
  return J.status;
}
