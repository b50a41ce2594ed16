/*
 * GDN-2 oracle: a plain, slow, FP64 CPU implementation of the gated delta
 * rule with a per-channel erase gate and a per-channel write gate (forward
 * and its reverse-mode gradient).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite may load this code. It
 * shares no code, header, table or helper with the GPU path, nor with the
 * KDA oracle in kda_oracle.c (the tests compare the two).
 *
 * Reading ("KDA at the production shape...", section 1.6, and the per-chunk
 * operation table of section 2.1): GDN-2 replaces the scalar beta of the
 * delta rule by a channel-wise erase gate b_t (one value per key channel)
 * and a channel-wise write gate w_t (one value per value channel); KDA is
 * the special case b_t = w_t = beta_t in every channel. The table's rows
 * akk = (b k Gamma)(k / Gamma)^T, w = M^-1 (b k Gamma) and u = M^-1 (w v)
 * are the chunk form of the token recurrence below. Per packed sequence and
 * head, all arithmetic in double:
 *
 *   Prologue, as for KDA (Q/K L2 normalisation inside the operator, the
 *   bounded gate driven by FP32 A_log / dt_bias; gate modes as in
 *   kda_oracle.c), and the two gates through a sigmoid:
 *     qh = scale * q / sqrt(|q|^2 + eps)        kh = k / sqrt(|k|^2 + eps)
 *     b = sigmoid(raw_b)  [K]                   w = sigmoid(raw_w)  [V]
 *     mode 0: z = exp(A_log[h]) (raw_g + dt_bias[h,:]), g = L sigmoid(z)
 *     mode 1: g = max(L, -exp(A_log[h]) softplus(raw_g + dt_bias[h,:]))
 *   Token recurrence (state K x V, zero at every sequence start):
 *     Sd  = Diag(exp(g_t)) S_{t-1}        decay
 *     e   = b_t * kh_t                     erase key  [K]
 *     c   = w_t * v_t                      written value  [V]
 *     u   = c - Sd^T e                     [V]
 *     S_t = Sd + kh_t u^T
 *     o_t = S_t^T qh_t
 *   i.e. S_t = (I - kh (b kh)^T) Diag(e^g) S_{t-1} + kh (w v)^T.
 *
 *   Backward: the reverse sweep of exactly these steps, then the prologue.
 *   Outputs: dq, dk, dv, draw_g [T,H,K], draw_b [T,H,K], draw_w [T,H,V],
 *   dA_log [H], ddt_bias [H,K].
 *
 * The sweep needs S_{t-1} in reverse order: states are kept every BLOCK
 * tokens and each block is recomputed from its kept state (an order of
 * evaluation, not a change of arithmetic).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BLOCK 128

typedef struct {
  int H, K, V, gate_mode;
  double scale, lb, eps;
  const double *q, *k, *v, *rg, *rb, *rw, *A_log, *dt_bias, *dO;
  double *o, *dq, *dk, *dv, *drg, *drb, *drw;
} g2_t;

static double g2_sig(double x) { return 1.0 / (1.0 + exp(-x)); }
static double g2_softplus(double x) { return x > 30.0 ? x : log1p(exp(x)); }

/* per-token values of one head */
typedef struct {
  double rq, rk;
  double *qb, *qh, *kh, *b, *w, *g, *z;
} g2_tok;

static void g2_prologue(const g2_t *p, int64_t t, int h, g2_tok *x) {
  const int K = p->K, V = p->V;
  const size_t tk = ((size_t)t * p->H + h) * K, tv = ((size_t)t * p->H + h) * V;
  double a = 0, c = 0;
  for (int i = 0; i < K; ++i) {
    a += p->q[tk + i] * p->q[tk + i];
    c += p->k[tk + i] * p->k[tk + i];
  }
  x->rq = 1.0 / sqrt(a + p->eps);
  x->rk = 1.0 / sqrt(c + p->eps);
  const double ea = exp(p->A_log[h]);
  for (int i = 0; i < K; ++i) {
    x->qb[i] = p->q[tk + i] * x->rq;
    x->qh[i] = p->scale * x->qb[i];
    x->kh[i] = p->k[tk + i] * x->rk;
    x->b[i] = g2_sig(p->rb[tk + i]);
    const double xb = p->rg[tk + i] + p->dt_bias[(size_t)h * K + i];
    if (p->gate_mode == 0) {
      x->z[i] = ea * xb;
      x->g[i] = p->lb * g2_sig(x->z[i]);
    } else {
      x->z[i] = xb;
      const double d = -ea * g2_softplus(xb);
      x->g[i] = d > p->lb ? d : p->lb;
    }
  }
  for (int j = 0; j < V; ++j) x->w[j] = g2_sig(p->rw[tv + j]);
}

/* S (K x V) advanced by one token in place; Sd (optional) gets the decayed
   state, u the written row, o (optional) the output. */
static void g2_step(const g2_t *p, const g2_tok *x, const double *vt, double *S, double *Sd,
                    double *u, double *o) {
  const int K = p->K, V = p->V;
  for (int i = 0; i < K; ++i) {
    const double d = exp(x->g[i]);
    for (int j = 0; j < V; ++j) S[(size_t)i * V + j] *= d;
  }
  if (Sd) memcpy(Sd, S, sizeof(double) * K * V);
  for (int j = 0; j < V; ++j) {
    double acc = x->w[j] * vt[j];
    for (int i = 0; i < K; ++i) acc -= S[(size_t)i * V + j] * (x->b[i] * x->kh[i]);
    u[j] = acc;
  }
  for (int i = 0; i < K; ++i)
    for (int j = 0; j < V; ++j) S[(size_t)i * V + j] += x->kh[i] * u[j];
  if (o) {
    for (int j = 0; j < V; ++j) {
      double acc = 0;
      for (int i = 0; i < K; ++i) acc += S[(size_t)i * V + j] * x->qh[i];
      o[j] = acc;
    }
  }
}

static int g2_task(const g2_t *p, int64_t t0, int64_t t1, int h, double *dA_out, double *ddt_out) {
  const int K = p->K, V = p->V, H = p->H;
  const size_t KV = (size_t)K * V;
  const int64_t L = t1 - t0, nb = (L + BLOCK - 1) / BLOCK;
  double *mem = calloc((size_t)(4 + (p->dO ? (nb > 0 ? nb : 1) + BLOCK : 0)) * KV +
                           (size_t)12 * (K > V ? K : V), sizeof(double));
  if (!mem) return 1;
  double *S = mem, *Sd = S + KV, *dS = Sd + KV, *dSd = dS + KV, *kept = dSd + KV;
  double *blk = kept + (p->dO ? (size_t)(nb > 0 ? nb : 1) * KV : 0);
  double *vec = blk + (p->dO ? (size_t)BLOCK * KV : 0);
  const int M = K > V ? K : V;
  double *u = vec, *du = vec + M, *dqh = vec + 2 * M, *dkh = vec + 3 * M, *dg = vec + 4 * M,
         *db = vec + 5 * M;
  double *tmp = vec + 6 * M;
  g2_tok x = {0, 0, vec + 7 * M, vec + 8 * M, vec + 9 * M, vec + 10 * M, vec + 11 * M, NULL, NULL};
  double *gz = malloc(sizeof(double) * 2 * K);
  if (!gz) { free(mem); return 1; }
  x.g = gz;
  x.z = gz + K;

  for (int64_t t = t0; t < t1; ++t) {
    if (p->dO && (t - t0) % BLOCK == 0) memcpy(kept + (size_t)((t - t0) / BLOCK) * KV, S, sizeof(double) * KV);
    g2_prologue(p, t, h, &x);
    g2_step(p, &x, p->v + ((size_t)t * H + h) * V, S, NULL, u,
            p->o ? p->o + ((size_t)t * H + h) * V : tmp);
  }
  if (!p->dO) goto out;

  memset(dS, 0, sizeof(double) * KV);
  *dA_out = 0;
  for (int i = 0; i < K; ++i) ddt_out[i] = 0;
  const double ea = exp(p->A_log[h]);
  for (int64_t bk = nb - 1; bk >= 0; --bk) {
    const int64_t bs = t0 + bk * BLOCK, be = bs + BLOCK < t1 ? bs + BLOCK : t1;
    memcpy(S, kept + (size_t)bk * KV, sizeof(double) * KV);
    for (int64_t t = bs; t < be; ++t) {
      memcpy(blk + (size_t)(t - bs) * KV, S, sizeof(double) * KV);
      g2_prologue(p, t, h, &x);
      g2_step(p, &x, p->v + ((size_t)t * H + h) * V, S, NULL, u, NULL);
    }
    for (int64_t t = be - 1; t >= bs; --t) {
      const size_t thk = ((size_t)t * H + h) * K, thv = ((size_t)t * H + h) * V;
      const double *dOt = p->dO + thv, *vt = p->v + thv;
      g2_prologue(p, t, h, &x);
      memcpy(S, blk + (size_t)(t - bs) * KV, sizeof(double) * KV);
      g2_step(p, &x, vt, S, Sd, u, NULL);  /* S = S_t, Sd = decayed S_{t-1} */
      /* o = S^T qh */
      for (int i = 0; i < K; ++i) {
        double acc = 0;
        for (int j = 0; j < V; ++j) {
          acc += S[(size_t)i * V + j] * dOt[j];
          dS[(size_t)i * V + j] += x.qh[i] * dOt[j];
        }
        dqh[i] = acc;
      }
      /* S = Sd + kh u^T: dkh = dS u, du = dS^T kh, dSd = dS */
      for (int j = 0; j < V; ++j) du[j] = 0;
      for (int i = 0; i < K; ++i) {
        double acc = 0;
        for (int j = 0; j < V; ++j) {
          acc += dS[(size_t)i * V + j] * u[j];
          du[j] += dS[(size_t)i * V + j] * x.kh[i];
        }
        dkh[i] = acc;
      }
      /* u = c - Sd^T e, e = b kh, c = w v:
         dc = du; dSd = dS - e du^T; de = -Sd du */
      double *dvt = p->dv + thv, *drw = p->drw + thv;
      for (int j = 0; j < V; ++j) {
        dvt[j] = du[j] * x.w[j];
        drw[j] = du[j] * vt[j] * x.w[j] * (1.0 - x.w[j]);
      }
      for (int i = 0; i < K; ++i) {
        const double e = x.b[i] * x.kh[i];
        double de = 0;
        for (int j = 0; j < V; ++j) {
          de -= Sd[(size_t)i * V + j] * du[j];
          dSd[(size_t)i * V + j] = dS[(size_t)i * V + j] - e * du[j];
        }
        db[i] = de * x.kh[i];
        dkh[i] += de * x.b[i];
      }
      /* Sd = Diag(e^g) S_{t-1}: dg = rowsum(dSd * Sd), dS_{t-1} = Diag(e^g) dSd */
      for (int i = 0; i < K; ++i) {
        const double d = exp(x.g[i]);
        double acc = 0;
        for (int j = 0; j < V; ++j) {
          acc += dSd[(size_t)i * V + j] * Sd[(size_t)i * V + j];
          dS[(size_t)i * V + j] = d * dSd[(size_t)i * V + j];
        }
        dg[i] = acc;
      }
      /* prologue */
      double qd = 0, kd = 0;
      for (int i = 0; i < K; ++i) {
        qd += x.qb[i] * dqh[i];
        kd += x.kh[i] * dkh[i];
      }
      for (int i = 0; i < K; ++i) {
        p->dq[thk + i] = p->scale * x.rq * (dqh[i] - x.qb[i] * qd);
        p->dk[thk + i] = x.rk * (dkh[i] - x.kh[i] * kd);
        p->drb[thk + i] = db[i] * x.b[i] * (1.0 - x.b[i]);
        double dx, dA;
        if (p->gate_mode == 0) {
          const double s = g2_sig(x.z[i]), dz = dg[i] * p->lb * s * (1.0 - s);
          dx = dz * ea;
          dA = dz * x.z[i];
        } else {
          const double d = -ea * g2_softplus(x.z[i]);
          dx = d > p->lb ? -dg[i] * ea * g2_sig(x.z[i]) : 0.0;
          dA = d > p->lb ? dg[i] * d : 0.0;
        }
        p->drg[thk + i] = dx;
        ddt_out[i] += dx;
        *dA_out += dA;
      }
    }
  }
out:
  free(gz);
  free(mem);
  return 0;
}

/* Entry point. cu_seqlens [n_seqs+1] non-decreasing from 0; dO == NULL runs
   the forward only. Arrays are token-major [T,H,D], double. Returns 0, or 1
   on bad arguments or allocation failure. */
int gdn2_oracle(int n_seqs, const int64_t *cu_seqlens, int H, int K, int V, double scale,
                double lower_bound, double eps, int gate_mode, const double *q,
                const double *k, const double *v, const double *raw_g, const double *raw_b,
                const double *raw_w, const double *A_log, const double *dt_bias,
                const double *dO, double *o, double *dq, double *dk, double *dv,
                double *draw_g, double *draw_b, double *draw_w, double *dA_log,
                double *ddt_bias, int n_threads) {
  if (n_seqs < 0 || H <= 0 || K <= 0 || V <= 0 || !cu_seqlens || cu_seqlens[0] != 0) return 1;
  if (gate_mode != 0 && gate_mode != 1) return 1;
  for (int n = 0; n < n_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return 1;
  g2_t p = {H, K, V, gate_mode, scale, lower_bound, eps, q, k, v, raw_g, raw_b, raw_w,
            A_log, dt_bias, dO, o, dq, dk, dv, draw_g, draw_b, draw_w};
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
    if (g2_task(&p, cu_seqlens[n], cu_seqlens[n + 1], h, dO ? pa + task : NULL,
                dO ? pb + (size_t)task * K : NULL))
      err = 1;
  }
  if (dO && !err) {
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
