/* Drives the fp64 oracle over ragged packs (empty, single-token and partial
 * documents, h0 and dht present or not, both gate forms, grouped heads) so that
 * an AddressSanitizer build of oracle/gdr_oracle.c checks every access it makes.
 * Exit status 0 when every call returned 0 and every output is finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gdr_oracle_forward(int T, int N, int Hqk, int Hv, int K, int V, int per_channel, const double *q,
                       const double *k, const double *v, const double *g, const double *beta,
                       const int32_t *cu_seqlens, const double *h0, double scale, double *o, double *ht,
                       int nthreads);
int gdr_oracle_backward(int T, int N, int Hqk, int Hv, int K, int V, int per_channel, const double *q,
                        const double *k, const double *v, const double *g, const double *beta,
                        const int32_t *cu_seqlens, const double *h0, double scale, const double *dout,
                        const double *dht, double *dq, double *dk, double *dv, double *dg, double *dbeta,
                        double *dh0, int nthreads);

static uint64_t state = 88172645463325252ull;
static double urand(void) { /* xorshift64 */
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (double)(state >> 11) / 9007199254740992.0;
}
static double *fill(size_t n, double lo, double hi) {
  double *x = (double *)malloc((n ? n : 1) * sizeof(double));
  for (size_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * urand();
  return x;
}
static int finite_all(const double *x, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return 0;
  return 1;
}

int main(void) {
  int bad = 0;
  for (int trial = 0; trial < 40; ++trial) {
    const int N = 1 + (int)(urand() * 4), grp = 1 + (int)(urand() * 3), Hqk = 1 + (int)(urand() * 2);
    const int Hv = Hqk * grp, K = 3 + (int)(urand() * 6), V = 2 + (int)(urand() * 6);
    const int pc = trial & 1, with_h0 = (trial >> 1) & 1, with_dht = (trial >> 2) & 1;
    int32_t *cu = (int32_t *)malloc((N + 1) * sizeof(int32_t));
    cu[0] = 0;
    for (int n = 0; n < N; ++n) {
      const double r = urand();
      const int len = r < 0.2 ? 0 : (r < 0.35 ? 1 : (int)(urand() * 150));
      cu[n + 1] = cu[n] + len;
    }
    const int T = cu[N];
    const size_t nq = (size_t)T * Hqk * K, nv = (size_t)T * Hv * V, ng = (size_t)T * Hv * (pc ? K : 1);
    const size_t ns = (size_t)N * Hv * K * V;
    double *q = fill(nq, -1, 1), *k = fill(nq, -0.3, 0.3), *v = fill(nv, -1, 1), *g = fill(ng, -5, 0);
    double *beta = fill((size_t)T * Hv, 0, 1), *dout = fill(nv, -1, 1);
    double *h0 = with_h0 ? fill(ns, -0.1, 0.1) : NULL, *dht = with_dht ? fill(ns, -0.1, 0.1) : NULL;
    double *o = fill(nv, 0, 0), *ht = fill(ns, 0, 0), *dq = fill(nq, 0, 0), *dk = fill(nq, 0, 0);
    double *dv = fill(nv, 0, 0), *dg = fill(ng, 0, 0), *db = fill((size_t)T * Hv, 0, 0), *dh0 = fill(ns, 0, 0);
    const double scale = 1.0 / sqrt((double)K);
    const int threads = 1 + (trial % 3);
    if (gdr_oracle_forward(T, N, Hqk, Hv, K, V, pc, q, k, v, g, beta, cu, h0, scale, o, ht, threads)) ++bad;
    if (gdr_oracle_backward(T, N, Hqk, Hv, K, V, pc, q, k, v, g, beta, cu, h0, scale, dout, dht, dq, dk, dv, dg,
                            db, dh0, threads))
      ++bad;
    if (!finite_all(o, nv) || !finite_all(ht, ns) || !finite_all(dq, nq) || !finite_all(dk, nq) ||
        !finite_all(dv, nv) || !finite_all(dg, ng) || !finite_all(db, (size_t)T * Hv) || !finite_all(dh0, ns))
      ++bad;
    free(cu); free(q); free(k); free(v); free(g); free(beta); free(dout); free(h0); free(dht);
    free(o); free(ht); free(dq); free(dk); free(dv); free(dg); free(db); free(dh0);
  }
  /* a problem the oracle must refuse: cu_seqlens that do not end at T */
  {
    int32_t cu[2] = {0, 5};
    double x[64] = {0};
    if (gdr_oracle_forward(4, 1, 1, 1, 2, 2, 1, x, x, x, x, x, cu, NULL, 1.0, x, x, 1) == 0) ++bad;
  }
  printf("oracle driver: %d failures\n", bad);
  return bad != 0;
}
