/*
 * KDA oracle: a plain, slow, FP64 CPU implementation of the Kimi Delta
 * Attention operator (forward and its reverse-mode gradient).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or helper with the GPU path.
 *
 * What it computes (per packed sequence, per head; all arithmetic in double):
 *
 *   Prologue ("KDA Memory with Recompute: FLA vs cuDNN Frontend FROST",
 *   section "Sources and measurement configuration": Q/K L2 normalisation
 *   inside the operator, beta through a sigmoid, a safe gate bounded below
 *   by -5 that is driven by FP32 A_log and dt_bias):
 *     qh = scale * q / sqrt(|q|^2 + eps)        kh = k / sqrt(|k|^2 + eps)
 *     beta = sigmoid(raw_beta)
 *     gate mode 0 (default reading; the formula is not printed):
 *       z = exp(A_log[h]) * (raw_g + dt_bias[h,:]),  g = L * sigmoid(z)
 *     gate mode 1 (alternative reading):
 *       g = max(L, -exp(A_log[h]) * softplus(raw_g + dt_bias[h,:]))
 *
 *   Token recurrence (the gated delta rule with a per-channel decay, as the
 *   pieces in "KDA at the production shape..." section 1.1 and the per-chunk
 *   operation table of section 2.1 describe it; the state restarts at every
 *   packed-sequence boundary per the measurement configuration of the FROST
 *   page, from zero there, which measures no initial and no final state):
 *     St = Diag(exp(g_t)) S_{t-1}           (channel-wise decay of the state)
 *     u_t = v_t - St^T kh_t                 (delta-rule prediction error)
 *     S_t = St + beta_t kh_t u_t^T          (rank-one write)
 *     o_t = S_t^T qh_t
 *   which is S_t = (I - beta k k^T) Diag(e^g) S_{t-1} + beta k v^T.
 *
 *   Optional state input and output (kda_oracle_ex): each sequence n may
 *   start from a given S_{-1} = h0[n] instead of zero, and its last state
 *   S_{L-1} is returned as ht[n] (an empty sequence passes h0 through). The
 *   backward then takes a gradient dht[n] of the loss with respect to ht[n]
 *   (the reverse sweep starts from it instead of zero) and returns dh0[n],
 *   the gradient with respect to h0[n] (the sweep's dS once it has passed
 *   the first token). Both are [N, H, K, V].
 *
 *   Backward: reverse-mode differentiation of exactly the steps above, token
 *   by token in reverse order, then of the prologue. All seven inputs
 *   (q, k, v, raw_g, raw_beta, A_log, dt_bias) are differentiated, matching
 *   "All seven tensor inputs differentiated" on the FROST page.
 *
 * The reverse sweep needs S_{t-1} in reverse order; the forward stores the
 * state every CKPT tokens and each block is recomputed from its checkpoint.
 * That is an order of evaluation, not a change of arithmetic.
 *
 * Layout: token-major [T, H, D] arrays, D contiguous, double precision.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define CKPT 256

typedef struct {
  int H, K, V;
  double scale, lower_bound, eps;
  int gate_mode;
  const double *q, *k, *v, *raw_g, *raw_beta, *A_log, *dt_bias, *dO;
  double *o, *dq, *dk, *dv, *draw_g, *draw_beta;
  const double *h0, *dht; /* [N,H,K,V] or NULL (zero) */
  double *ht, *dh0;       /* [N,H,K,V] or NULL (not written) */
} prob_t;

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double softplus(double x) { return x > 30.0 ? x : log1p(exp(x)); }

/* Per-token prologue values for one head. */
typedef struct {
  double rq, rk, beta;
  double *qh, *kh, *qbar, *g, *z; /* length K */
} tok_t;

static void prologue(const prob_t *p, int64_t t, int h, tok_t *w) {
  const int K = p->K;
  const double *q = p->q + ((size_t)t * p->H + h) * K;
  const double *k = p->k + ((size_t)t * p->H + h) * K;
  const double *x = p->raw_g + ((size_t)t * p->H + h) * K;
  double sq = 0, sk = 0;
  for (int i = 0; i < K; ++i) { sq += q[i] * q[i]; sk += k[i] * k[i]; }
  w->rq = 1.0 / sqrt(sq + p->eps);
  w->rk = 1.0 / sqrt(sk + p->eps);
  for (int i = 0; i < K; ++i) {
    w->qbar[i] = q[i] * w->rq;
    w->qh[i] = p->scale * w->qbar[i];
    w->kh[i] = k[i] * w->rk;
  }
  w->beta = sigmoid(p->raw_beta[(size_t)t * p->H + h]);
  const double ea = exp(p->A_log[h]);
  for (int i = 0; i < K; ++i) {
    const double xb = x[i] + p->dt_bias[(size_t)h * K + i];
    if (p->gate_mode == 0) {
      w->z[i] = ea * xb;
      w->g[i] = p->lower_bound * sigmoid(w->z[i]);
    } else {
      w->z[i] = xb;
      const double c = -ea * softplus(xb);
      w->g[i] = c > p->lower_bound ? c : p->lower_bound;
    }
  }
}

/* One forward token step: S (K x V, row-major) is updated in place.
   St_out (optional) receives the decayed state, u_out the prediction error. */
static void step(const prob_t *p, const tok_t *w, const double *v, double *S,
                 double *St_out, double *u_out, double *o_out) {
  const int K = p->K, V = p->V;
  for (int i = 0; i < K; ++i) {
    const double d = exp(w->g[i]);
    for (int j = 0; j < V; ++j) S[(size_t)i * V + j] *= d;
  }
  if (St_out) memcpy(St_out, S, sizeof(double) * K * V);
  for (int j = 0; j < V; ++j) u_out[j] = v[j];
  for (int i = 0; i < K; ++i)
    for (int j = 0; j < V; ++j) u_out[j] -= S[(size_t)i * V + j] * w->kh[i];
  for (int i = 0; i < K; ++i) {
    const double c = w->beta * w->kh[i];
    for (int j = 0; j < V; ++j) S[(size_t)i * V + j] += c * u_out[j];
  }
  if (o_out) {
    for (int j = 0; j < V; ++j) o_out[j] = 0;
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < V; ++j) o_out[j] += S[(size_t)i * V + j] * w->qh[i];
  }
}

typedef struct {
  double *S, *St, *u, *dS, *dSt, *du, *dqh, *dkh, *dg, *tmp;
  double *qh, *kh, *qbar, *g, *z;
  double *ckpt, *blk; /* checkpoints and per-block S_{t-1} states */
} scratch_t;

/* Forward and (if dO) backward for one (sequence, head) task.
   dA_log_out / ddt_out receive this task's contribution. */
static int run_task(const prob_t *p, int n, int64_t t0, int64_t t1, int h,
                    double *dA_log_out, double *ddt_out) {
  const int K = p->K, V = p->V, H = p->H;
  const size_t KV = (size_t)K * V;
  const size_t soff = ((size_t)n * H + h) * KV; /* this task's [K,V] state slot */
  const int64_t L = t1 - t0;
  int err = 0;
  scratch_t s;
  memset(&s, 0, sizeof s);
  const int64_t nck = (L + CKPT - 1) / CKPT;
  s.S = calloc(KV, sizeof(double));
  s.St = calloc(KV, sizeof(double));
  s.dS = calloc(KV, sizeof(double));
  s.dSt = calloc(KV, sizeof(double));
  s.u = calloc(V, sizeof(double));
  s.du = calloc(V, sizeof(double));
  s.tmp = calloc(V > K ? V : K, sizeof(double));
  s.dqh = calloc(K, sizeof(double));
  s.dkh = calloc(K, sizeof(double));
  s.dg = calloc(K, sizeof(double));
  s.qh = calloc(K, sizeof(double));
  s.kh = calloc(K, sizeof(double));
  s.qbar = calloc(K, sizeof(double));
  s.g = calloc(K, sizeof(double));
  s.z = calloc(K, sizeof(double));
  s.ckpt = p->dO ? calloc((size_t)(nck > 0 ? nck : 1) * KV, sizeof(double)) : NULL;
  s.blk = p->dO ? calloc((size_t)CKPT * KV, sizeof(double)) : NULL;
  if (!s.S || !s.St || !s.dS || !s.dSt || !s.u || !s.du || !s.tmp || !s.dqh ||
      !s.dkh || !s.dg || !s.qh || !s.kh || !s.qbar || !s.g || !s.z ||
      (p->dO && (!s.ckpt || !s.blk))) {
    err = 1;
    goto done;
  }
  tok_t w = {0, 0, 0, s.qh, s.kh, s.qbar, s.g, s.z};

  /* ---- forward: token recurrence from S = h0 (or 0) at the sequence start ---- */
  if (p->h0) memcpy(s.S, p->h0 + soff, sizeof(double) * KV);
  for (int64_t t = t0; t < t1; ++t) {
    if (s.ckpt && (t - t0) % CKPT == 0)
      memcpy(s.ckpt + (size_t)((t - t0) / CKPT) * KV, s.S, sizeof(double) * KV);
    prologue(p, t, h, &w);
    step(p, &w, p->v + ((size_t)t * H + h) * V, s.S, NULL, s.u,
         p->o ? p->o + ((size_t)t * H + h) * V : s.tmp);
  }
  if (p->ht) memcpy(p->ht + soff, s.S, sizeof(double) * KV);
  if (!p->dO) goto done;

  /* ---- backward: reverse sweep from dS = dht (or 0) after the sequence end ---- */
  if (p->dht)
    memcpy(s.dS, p->dht + soff, sizeof(double) * KV);
  else
    memset(s.dS, 0, sizeof(double) * KV);
  *dA_log_out = 0;
  for (int i = 0; i < K; ++i) ddt_out[i] = 0;
  const double ea = exp(p->A_log[h]);
  for (int64_t b = nck - 1; b >= 0; --b) {
    const int64_t bs = t0 + b * CKPT;
    const int64_t be = bs + CKPT < t1 ? bs + CKPT : t1;
    /* recompute the block: blk[j] = S_{t-1} for t = bs + j */
    memcpy(s.S, s.ckpt + (size_t)b * KV, sizeof(double) * KV);
    for (int64_t t = bs; t < be; ++t) {
      memcpy(s.blk + (size_t)(t - bs) * KV, s.S, sizeof(double) * KV);
      prologue(p, t, h, &w);
      step(p, &w, p->v + ((size_t)t * H + h) * V, s.S, NULL, s.u, s.tmp);
    }
    for (int64_t t = be - 1; t >= bs; --t) {
      const size_t th = (size_t)t * H + h;
      const double *dOt = p->dO + th * V;
      const double *vt = p->v + th * V;
      prologue(p, t, h, &w);
      /* redo the step from S_{t-1} to get St, u and S_t */
      memcpy(s.S, s.blk + (size_t)(t - bs) * KV, sizeof(double) * KV);
      step(p, &w, vt, s.S, s.St, s.u, NULL);
      /* o_t = S_t^T qh:  dqh = S_t dO,  dS += qh dO^T */
      for (int i = 0; i < K; ++i) {
        double a = 0;
        for (int j = 0; j < V; ++j) a += s.S[(size_t)i * V + j] * dOt[j];
        s.dqh[i] = a;
        for (int j = 0; j < V; ++j) s.dS[(size_t)i * V + j] += w.qh[i] * dOt[j];
      }
      /* S_t = St + beta kh u^T */
      double dbeta = 0;
      for (int j = 0; j < V; ++j) s.du[j] = 0;
      for (int i = 0; i < K; ++i) {
        double a = 0; /* (dS u)_i */
        for (int j = 0; j < V; ++j) {
          a += s.dS[(size_t)i * V + j] * s.u[j];
          s.du[j] += s.dS[(size_t)i * V + j] * w.kh[i];
        }
        dbeta += w.kh[i] * a;
        s.dkh[i] = w.beta * a;
      }
      for (int j = 0; j < V; ++j) s.du[j] *= w.beta;
      /* u = v - St^T kh:  dv = du, dSt = dS - kh du^T, dkh -= St du */
      double *dvt = p->dv + th * V;
      for (int j = 0; j < V; ++j) dvt[j] = s.du[j];
      for (int i = 0; i < K; ++i) {
        double a = 0;
        for (int j = 0; j < V; ++j) {
          s.dSt[(size_t)i * V + j] = s.dS[(size_t)i * V + j] - w.kh[i] * s.du[j];
          a += s.St[(size_t)i * V + j] * s.du[j];
        }
        s.dkh[i] -= a;
      }
      /* St = Diag(e^g) S_{t-1}: dg_i = sum_j dSt_ij St_ij, dS_{t-1} = Diag(e^g) dSt */
      for (int i = 0; i < K; ++i) {
        double a = 0;
        const double d = exp(w.g[i]);
        for (int j = 0; j < V; ++j) {
          a += s.dSt[(size_t)i * V + j] * s.St[(size_t)i * V + j];
          s.dS[(size_t)i * V + j] = d * s.dSt[(size_t)i * V + j];
        }
        s.dg[i] = a;
      }
      /* prologue VJP */
      double qd = 0, kd = 0;
      for (int i = 0; i < K; ++i) {
        qd += w.qbar[i] * s.dqh[i];
        kd += w.kh[i] * s.dkh[i];
      }
      double *dqt = p->dq + th * K, *dkt = p->dk + th * K, *dxt = p->draw_g + th * K;
      for (int i = 0; i < K; ++i) {
        /* qh = scale * qbar, qbar = q * rq */
        dqt[i] = p->scale * w.rq * (s.dqh[i] - w.qbar[i] * qd);
        dkt[i] = w.rk * (s.dkh[i] - w.kh[i] * kd);
      }
      p->draw_beta[th] = dbeta * w.beta * (1.0 - w.beta);
      for (int i = 0; i < K; ++i) {
        const double xb = p->raw_g[th * K + i] + p->dt_bias[(size_t)h * K + i];
        double dx, dA;
        if (p->gate_mode == 0) {
          const double sz = sigmoid(w.z[i]);
          const double dz = s.dg[i] * p->lower_bound * sz * (1.0 - sz);
          dx = dz * ea;
          dA = dz * w.z[i];
        } else {
          const double c = -ea * softplus(xb);
          if (c > p->lower_bound) {
            dx = -s.dg[i] * ea * sigmoid(xb);
            dA = s.dg[i] * c;
          } else {
            dx = 0;
            dA = 0;
          }
        }
        dxt[i] = dx;
        ddt_out[i] += dx;
        *dA_log_out += dA;
      }
    }
  }
  /* dS now holds the gradient with respect to the state entering the first token */
  if (p->dh0) memcpy(p->dh0 + soff, s.dS, sizeof(double) * KV);
done:
  free(s.S); free(s.St); free(s.dS); free(s.dSt); free(s.u); free(s.du);
  free(s.tmp); free(s.dqh); free(s.dkh); free(s.dg); free(s.qh); free(s.kh);
  free(s.qbar); free(s.g); free(s.z); free(s.ckpt); free(s.blk);
  return err;
}

/* Entry point. cu_seqlens: [n_seqs+1], non-decreasing from 0. dO == NULL runs
   the forward only (gradient pointers, dht and dh0 are then ignored). h0, ht,
   dht, dh0: [n_seqs, H, K, V] or NULL (h0, dht NULL = zero; ht, dh0 NULL =
   not written). o may be NULL when
   only gradients are wanted. Returns 0 on success, 1 on bad arguments or
   allocation failure. n_threads <= 0 uses the OpenMP default. */
int kda_oracle_ex(int n_seqs, const int64_t *cu_seqlens, int H, int K, int V,
                  double scale, double lower_bound, double eps, int gate_mode,
                  const double *q, const double *k, const double *v,
                  const double *raw_g, const double *raw_beta,
                  const double *A_log, const double *dt_bias, const double *dO,
                  double *o, double *dq, double *dk, double *dv, double *draw_g,
                  double *draw_beta, double *dA_log, double *ddt_bias,
                  const double *h0, double *ht, const double *dht, double *dh0,
                  int n_threads) {
  if (n_seqs < 0 || H <= 0 || K <= 0 || V <= 0 || !cu_seqlens) return 1;
  if (gate_mode != 0 && gate_mode != 1) return 1;
  if (cu_seqlens[0] != 0) return 1;
  for (int n = 0; n < n_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return 1;
  prob_t p = {H, K, V, scale, lower_bound, eps, gate_mode, q, k, v, raw_g,
              raw_beta, A_log, dt_bias, dO, o, dq, dk, dv, draw_g, draw_beta,
              h0, dO ? dht : NULL, ht, dO ? dh0 : NULL};
  const int ntask = n_seqs * H;
  double *pa = NULL, *pb = NULL;
  if (dO) {
    pa = calloc((size_t)(ntask > 0 ? ntask : 1), sizeof(double));
    pb = calloc((size_t)(ntask > 0 ? ntask : 1) * K, sizeof(double));
    if (!pa || !pb) { free(pa); free(pb); return 1; }
  }
  int err = 0;
#ifdef _OPENMP
  const int nth = n_threads > 0 ? n_threads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nth) reduction(|| : err)
#endif
  for (int task = 0; task < ntask; ++task) {
    const int n = task / H, h = task % H;
    if (run_task(&p, n, cu_seqlens[n], cu_seqlens[n + 1], h,
                 dO ? pa + task : NULL, dO ? pb + (size_t)task * K : NULL))
      err = 1;
  }
  if (dO && !err) {
    /* fixed-order combination of per-task gate-parameter partials */
    for (int h = 0; h < H; ++h) {
      double a = 0;
      for (int n = 0; n < n_seqs; ++n) a += pa[n * H + h];
      dA_log[h] = a;
      for (int i = 0; i < K; ++i) {
        double b = 0;
        for (int n = 0; n < n_seqs; ++n) b += pb[(size_t)(n * H + h) * K + i];
        ddt_bias[(size_t)h * K + i] = b;
      }
    }
  }
  free(pa);
  free(pb);
  return err;
}

/* The operator without state input or output (every sequence starts from zero). */
int kda_oracle(int n_seqs, const int64_t *cu_seqlens, int H, int K, int V,
               double scale, double lower_bound, double eps, int gate_mode,
               const double *q, const double *k, const double *v,
               const double *raw_g, const double *raw_beta,
               const double *A_log, const double *dt_bias, const double *dO,
               double *o, double *dq, double *dk, double *dv, double *draw_g,
               double *draw_beta, double *dA_log, double *ddt_bias,
               int n_threads) {
  return kda_oracle_ex(n_seqs, cu_seqlens, H, K, V, scale, lower_bound, eps,
                       gate_mode, q, k, v, raw_g, raw_beta, A_log, dt_bias, dO,
                       o, dq, dk, dv, draw_g, draw_beta, dA_log, ddt_bias, NULL,
                       NULL, NULL, NULL, n_threads);
}

/* Prologue alone, for checking the prologue step: qh, kh [T,H,K], beta [T,H]
   and gcum [T,H,K], the cumulative sum of g restarted every `chunk` tokens
   from each sequence start. Returns 0, or 1 on bad arguments. */
int kda_oracle_prologue(int n_seqs, const int64_t *cu_seqlens, int H, int K,
                        double scale, double lower_bound, double eps,
                        int gate_mode, int chunk, const double *q,
                        const double *k, const double *raw_g,
                        const double *raw_beta, const double *A_log,
                        const double *dt_bias, double *qh, double *kh,
                        double *beta, double *gcum) {
  if (n_seqs < 0 || H <= 0 || K <= 0 || chunk <= 0 || !cu_seqlens) return 1;
  prob_t p = {H, K, 1, scale, lower_bound, eps, gate_mode, q, k, NULL, raw_g,
              raw_beta, A_log, dt_bias, NULL, NULL, NULL, NULL, NULL, NULL,
              NULL, NULL, NULL, NULL, NULL};
  double *buf = calloc((size_t)5 * K, sizeof(double));
  if (!buf) return 1;
  tok_t w = {0, 0, 0, buf, buf + K, buf + 2 * K, buf + 3 * K, buf + 4 * K};
  for (int n = 0; n < n_seqs; ++n) {
    for (int h = 0; h < H; ++h) {
      for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
        const size_t th = (size_t)t * H + h;
        const int64_t j = (t - cu_seqlens[n]) % chunk;
        prologue(&p, t, h, &w);
        beta[th] = w.beta;
        for (int i = 0; i < K; ++i) {
          qh[th * K + i] = w.qh[i];
          kh[th * K + i] = w.kh[i];
          gcum[th * K + i] = (j == 0 ? 0.0 : gcum[(th - H) * K + i]) + w.g[i];
        }
      }
    }
  }
  free(buf);
  return 0;
}
