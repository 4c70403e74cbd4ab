/*
 * Plain fp64 CPU oracle for gated delta-rule attention over packed
 * variable-length sequences (KDA: per-channel log-gate; GDN: scalar log-decay
 * with grouped Q/K heads).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or constant with the HIP path.
 *
 * What it computes (the token recurrence, evaluated one token at a time):
 *   The pages (FlashInfer PR #8218, description: "Cake KDA ... chunked
 *   training for packed variable-length sequences at head dim 128", workload
 *   paragraph) describe KDA training on a packed batch where g is a
 *   pre-activated fp32 log-gate [T,H,128] and beta a BF16 [T,H] write
 *   strength; PR #7723 (description) describes the GDN form with a scalar
 *   log-decay per value head and Q/K heads shared by groups of value heads,
 *   dq/dk being reduced over each group.  The recurrence itself is not
 *   printed on the pages; this file takes the plainest reading:
 *
 *     S_0  = h0[doc, j]           (K x V, zero when no initial state)
 *     S'_t = Diag(exp(g_t)) S_{t-1}          (scalar exp(g_t) for GDN)
 *     r_t  = v_t - S'_t^T k_t
 *     S_t  = S'_t + beta_t k_t r_t^T
 *     o_t  = scale * S_t^T q_t
 *     ht[doc, j] = S at the document's last token
 *
 *   The state restarts at every document boundary of cu_seqlens.  Value head
 *   j reads Q/K head j / (Hv / Hqk) (contiguous groups).
 *
 * The backward is the reverse-mode derivative of that loop, derived by hand
 * for the loss  sum(o * dout) + sum(ht * dht):
 *
 *     dS    = dht (or 0)
 *     for t = last .. first:
 *        dS   += scale q_t dout_t^T
 *        dq_t += scale S_t dout_t
 *        u     = dS^T k_t ;   dr = beta_t u
 *        dbeta_t = r_t . u ;  dv_t = dr
 *        dk_t += beta_t dS r_t - S'_t dr
 *        dS'   = dS - k_t dr^T
 *        dg_t  = sum_v dS'[:,v] * S'_t[:,v]    (GDN: also summed over channels)
 *        dS    = Diag(exp(g_t)) dS'
 *     dh0 = dS
 *
 *   dq and dk of a Q/K head are the sums over its group's value heads.
 *   The forward state is checkpointed every 64 tokens and each 64-token block
 *   is replayed before its reverse sweep, to bound memory.
 *
 * Work is split over independent units (document, Q/K head) with OpenMP; a
 * unit owns its group's value heads, so the dq/dk sums need no locking.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BLOCK 64

typedef struct {
  int T, N, Hqk, Hv, K, V, per_channel;
  const double *q, *k, *v, *g, *beta, *h0;
  const int32_t *cu;
  double scale;
} oproblem;

/* element accessors for the [T, heads, dim] layouts */
static inline const double *row_qk(const double *x, const oproblem *p, int t, int i) {
  return x + ((size_t)t * p->Hqk + i) * p->K;
}
static inline const double *row_v(const double *x, const oproblem *p, int t, int j) {
  return x + ((size_t)t * p->Hv + j) * p->V;
}

/* decay factor of channel c at token t for value head j */
static inline double decay(const oproblem *p, int t, int j, int c) {
  if (p->per_channel) return exp(p->g[((size_t)t * p->Hv + j) * p->K + c]);
  return exp(p->g[(size_t)t * p->Hv + j]);
}

/* One recurrence step in place: S <- S'_t + beta k r^T.  Writes r (V) and,
 * if Sp is not NULL, the decayed state S'_t (K x V). */
static void step(const oproblem *p, double *S, int t, int j, double *r, double *Sp) {
  const int K = p->K, V = p->V;
  const int i = j / (p->Hv / p->Hqk);
  const double *kt = row_qk(p->k, p, t, i);
  const double *vt = row_v(p->v, p, t, j);
  const double b = p->beta[(size_t)t * p->Hv + j];
  for (int c = 0; c < K; ++c) {
    const double a = decay(p, t, j, c);
    double *Sr = S + (size_t)c * V;
    for (int e = 0; e < V; ++e) Sr[e] *= a;
  }
  if (Sp) memcpy(Sp, S, sizeof(double) * (size_t)K * V);
  for (int e = 0; e < V; ++e) r[e] = vt[e];
  for (int c = 0; c < K; ++c) {
    const double *Sr = S + (size_t)c * V;
    for (int e = 0; e < V; ++e) r[e] -= Sr[e] * kt[c];
  }
  for (int c = 0; c < K; ++c) {
    double *Sr = S + (size_t)c * V;
    const double bk = b * kt[c];
    for (int e = 0; e < V; ++e) Sr[e] += bk * r[e];
  }
}

static void init_state(const oproblem *p, double *S, int n, int j) {
  const size_t KV = (size_t)p->K * p->V;
  if (p->h0)
    memcpy(S, p->h0 + ((size_t)n * p->Hv + j) * KV, sizeof(double) * KV);
  else
    memset(S, 0, sizeof(double) * KV);
}

/* Forward of one (document, value head). */
static void forward_unit(const oproblem *p, int n, int j, double *o, double *ht,
                         double *S, double *r) {
  const int K = p->K, V = p->V;
  const int i = j / (p->Hv / p->Hqk);
  init_state(p, S, n, j);
  for (int t = p->cu[n]; t < p->cu[n + 1]; ++t) {
    step(p, S, t, j, r, NULL);
    const double *qt = row_qk(p->q, p, t, i);
    double *ot = o + ((size_t)t * p->Hv + j) * V;
    for (int e = 0; e < V; ++e) ot[e] = 0.0;
    for (int c = 0; c < K; ++c) {
      const double *Sr = S + (size_t)c * V;
      for (int e = 0; e < V; ++e) ot[e] += Sr[e] * qt[c];
    }
    for (int e = 0; e < V; ++e) ot[e] *= p->scale;
  }
  if (ht) memcpy(ht + ((size_t)n * p->Hv + j) * (size_t)K * V, S, sizeof(double) * (size_t)K * V);
}

static int valid(const oproblem *p) {
  if (p->T < 0 || p->N < 0 || p->Hqk <= 0 || p->Hv <= 0 || p->K <= 0 || p->V <= 0) return 0;
  if (p->Hv % p->Hqk) return 0;
  if (p->cu[0] != 0 || p->cu[p->N] != p->T) return 0;
  for (int n = 0; n < p->N; ++n)
    if (p->cu[n + 1] < p->cu[n]) return 0;
  return 1;
}

int gdr_oracle_forward(int T, int N, int Hqk, int Hv, int K, int V, int per_channel,
                       const double *q, const double *k, const double *v, const double *g,
                       const double *beta, const int32_t *cu_seqlens, const double *h0,
                       double scale, double *o, double *ht, int nthreads) {
  oproblem p = {T, N, Hqk, Hv, K, V, per_channel, q, k, v, g, beta, h0, cu_seqlens, scale};
  if (!valid(&p)) return 1;
  const int units = N * Hv;
  int failed = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double *S = (double *)malloc(sizeof(double) * (size_t)K * V);
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    if (!S || !r) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int u = 0; u < units; ++u) forward_unit(&p, u / Hv, u % Hv, o, ht, S, r);
    }
    free(S);
    free(r);
  }
  return failed ? 2 : 0;
}

/* Backward of one (document, value head); adds into dq/dk (the caller's unit
 * owns the group's Q/K rows of this document) and writes dv, dg, dbeta, dh0. */
static int backward_unit(const oproblem *p, int n, int j, const double *dout, const double *dht,
                         double *dq, double *dk, double *dv, double *dg, double *dbeta,
                         double *dh0) {
  const int K = p->K, V = p->V;
  const size_t KV = (size_t)K * V;
  const int i = j / (p->Hv / p->Hqk);
  const int t_begin = p->cu[n], t_end = p->cu[n + 1];
  const int L = t_end - t_begin;
  const int nb = (L + ORACLE_BLOCK - 1) / ORACLE_BLOCK;

  double *ckpt = (double *)malloc(sizeof(double) * KV * (size_t)(nb > 0 ? nb : 1));
  double *prev = (double *)malloc(sizeof(double) * KV * ORACLE_BLOCK); /* S_{t-1} per token */
  double *S = (double *)malloc(sizeof(double) * KV);
  double *Sp = (double *)malloc(sizeof(double) * KV);
  double *dS = (double *)malloc(sizeof(double) * KV);
  double *r = (double *)malloc(sizeof(double) * V);
  double *u = (double *)malloc(sizeof(double) * V);
  double *dr = (double *)malloc(sizeof(double) * V);
  if (!ckpt || !prev || !S || !Sp || !dS || !r || !u || !dr) {
    free(ckpt); free(prev); free(S); free(Sp); free(dS); free(r); free(u); free(dr);
    return 1;
  }

  /* forward sweep, keeping the state at every block start */
  init_state(p, S, n, j);
  for (int b = 0; b < nb; ++b) {
    memcpy(ckpt + (size_t)b * KV, S, sizeof(double) * KV);
    const int t0 = t_begin + b * ORACLE_BLOCK;
    const int t1 = t0 + ORACLE_BLOCK < t_end ? t0 + ORACLE_BLOCK : t_end;
    for (int t = t0; t < t1; ++t) step(p, S, t, j, r, NULL);
  }

  if (dht)
    memcpy(dS, dht + ((size_t)n * p->Hv + j) * KV, sizeof(double) * KV);
  else
    memset(dS, 0, sizeof(double) * KV);

  for (int b = nb - 1; b >= 0; --b) {
    const int t0 = t_begin + b * ORACLE_BLOCK;
    const int t1 = t0 + ORACLE_BLOCK < t_end ? t0 + ORACLE_BLOCK : t_end;
    /* replay the block, keeping S_{t-1} of each token */
    memcpy(S, ckpt + (size_t)b * KV, sizeof(double) * KV);
    for (int t = t0; t < t1; ++t) {
      memcpy(prev + (size_t)(t - t0) * KV, S, sizeof(double) * KV);
      step(p, S, t, j, r, NULL);
    }
    for (int t = t1 - 1; t >= t0; --t) {
      /* rebuild S'_t, r_t and S_t from S_{t-1} */
      memcpy(S, prev + (size_t)(t - t0) * KV, sizeof(double) * KV);
      step(p, S, t, j, r, Sp);
      const double *qt = row_qk(p->q, p, t, i);
      const double *kt = row_qk(p->k, p, t, i);
      const double *dot = row_v(dout, p, t, j);
      const double b_t = p->beta[(size_t)t * p->Hv + j];
      double *dqt = dq + ((size_t)t * p->Hqk + i) * K;
      double *dkt = dk + ((size_t)t * p->Hqk + i) * K;
      double *dvt = dv + ((size_t)t * p->Hv + j) * V;

      /* o_t = scale S_t^T q_t */
      for (int c = 0; c < K; ++c) {
        double *dSr = dS + (size_t)c * V;
        const double *Sr = S + (size_t)c * V;
        const double sq = p->scale * qt[c];
        double acc = 0.0;
        for (int e = 0; e < V; ++e) {
          dSr[e] += sq * dot[e];
          acc += Sr[e] * dot[e];
        }
        dqt[c] += p->scale * acc;
      }
      /* S_t = S'_t + beta k r^T,  r = v - S'^T k */
      for (int e = 0; e < V; ++e) u[e] = 0.0;
      for (int c = 0; c < K; ++c) {
        const double *dSr = dS + (size_t)c * V;
        for (int e = 0; e < V; ++e) u[e] += dSr[e] * kt[c];
      }
      double db = 0.0;
      for (int e = 0; e < V; ++e) {
        dr[e] = b_t * u[e];
        db += r[e] * u[e];
        dvt[e] = dr[e];
      }
      dbeta[(size_t)t * p->Hv + j] = db;
      for (int c = 0; c < K; ++c) {
        const double *dSr = dS + (size_t)c * V;
        const double *Spr = Sp + (size_t)c * V;
        double acc = 0.0;
        for (int e = 0; e < V; ++e) acc += b_t * dSr[e] * r[e] - Spr[e] * dr[e];
        dkt[c] += acc;
      }
      /* dS' = dS - k dr^T ; dg from S'_t = Diag(a) S_{t-1} ; dS_{t-1} = Diag(a) dS' */
      double dg_total = 0.0;
      for (int c = 0; c < K; ++c) {
        double *dSr = dS + (size_t)c * V;
        const double *Spr = Sp + (size_t)c * V;
        double acc = 0.0;
        for (int e = 0; e < V; ++e) {
          dSr[e] -= kt[c] * dr[e];
          acc += dSr[e] * Spr[e];
        }
        if (p->per_channel)
          dg[((size_t)t * p->Hv + j) * K + c] = acc;
        else
          dg_total += acc;
        const double a = decay(p, t, j, c);
        for (int e = 0; e < V; ++e) dSr[e] *= a;
      }
      if (!p->per_channel) dg[(size_t)t * p->Hv + j] = dg_total;
    }
  }
  if (dh0) memcpy(dh0 + ((size_t)n * p->Hv + j) * KV, dS, sizeof(double) * KV);

  free(ckpt); free(prev); free(S); free(Sp); free(dS); free(r); free(u); free(dr);
  return 0;
}

int gdr_oracle_backward(int T, int N, int Hqk, int Hv, int K, int V, int per_channel,
                        const double *q, const double *k, const double *v, const double *g,
                        const double *beta, const int32_t *cu_seqlens, const double *h0,
                        double scale, const double *dout, const double *dht, double *dq,
                        double *dk, double *dv, double *dg, double *dbeta, double *dh0,
                        int nthreads) {
  oproblem p = {T, N, Hqk, Hv, K, V, per_channel, q, k, v, g, beta, h0, cu_seqlens, scale};
  if (!valid(&p)) return 1;
  const int group = Hv / Hqk;
  const int units = N * Hqk;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
  for (int uix = 0; uix < units; ++uix) {
    const int n = uix / Hqk, i = uix % Hqk;
    for (int t = p.cu[n]; t < p.cu[n + 1]; ++t) {
      memset(dq + ((size_t)t * Hqk + i) * K, 0, sizeof(double) * K);
      memset(dk + ((size_t)t * Hqk + i) * K, 0, sizeof(double) * K);
    }
    for (int j = i * group; j < (i + 1) * group; ++j)
      if (backward_unit(&p, n, j, dout, dht, dq, dk, dv, dg, dbeta, dh0)) {
#pragma omp atomic write
        failed = 1;
      }
  }
  return failed ? 2 : 0;
}
