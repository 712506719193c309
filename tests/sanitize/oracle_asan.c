/*
 * The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
 * code only).  Drives every oracle entry point on small seeded inputs, with
 * empty sequences, several units and two OpenMP threads, and checks pins that
 * a broken index would fail:
 *   - T chained decode steps equal one forward over T tokens;
 *   - gates at +inf (alpha = 1, nothing written) from zero states give o = 0;
 *   - GLA with alpha = 1 equals causal linear attention o_t = sum_{j<=t} (q_t.k_j) v_j;
 *   - the backward's dq equals a central difference of the forward.
 * Exit status 0 when every check passes.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gsa_fwd_nl(const double *q, const double *k, const double *v, const double *g,
                      const double *k0, const double *v0, double *o, double *kf, double *vf,
                      double *s_out, double *z_out, long B, long H, long T, long dk, long dv,
                      long m, double tau, int act, int nthreads);
int oracle_gla_fwd_gm(const double *q, const double *k, const double *v, const double *g,
                      const double *s0, double *o, double *sf, long B, long H, long T, long dk,
                      long dv, double tau, int gate_mode, int nthreads);
int oracle_gsa_decode_step_nl(const double *q, const double *k, const double *v, const double *g,
                              double *kstate, double *vstate, double *o, long N, long H, long dk,
                              long dv, long m, double tau, int act, int nthreads);
int oracle_gsa_bwd_nl(const double *q, const double *k, const double *v, const double *g,
                      const double *dO, const double *k0, const double *v0, const double *dkf,
                      const double *dvf, double *dq, double *dk, double *dv, double *dg,
                      double *dk0, double *dv0, long B, long H, long T, long d_k, long d_v,
                      long m, double tau, int act, int nthreads);

static unsigned long long rs = 88172645463325252ULL;
static double rnd(void) { /* xorshift64, uniform in [-1, 1) */
  rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17;
  return (double)(rs >> 11) / 4503599627370496.0 - 1.0;
}
static double *arr(long n, double scale) {
  double *p = malloc((n > 0 ? n : 1) * sizeof(double));
  for (long i = 0; i < n; i++) p[i] = rnd() * scale;
  return p;
}
static int fails = 0;
static void check(int ok, const char *what, double err) {
  printf("%-58s %s (%.3g)\n", what, ok ? "ok" : "FAIL", err);
  if (!ok) fails++;
}
static double maxdiff(const double *a, const double *b, long n) {
  double e = 0;
  for (long i = 0; i < n; i++) e = fmax(e, fabs(a[i] - b[i]));
  return e;
}

int main(void) {
  const long B = 2, H = 3, T = 37, d = 5, m = 4;
  const long U = B * H, nq = U * T * d, ng = U * T * m, ns = U * m * d;
  double *q = arr(nq, 0.5), *k = arr(nq, 0.5), *v = arr(nq, 0.5), *g = arr(ng, 2.0);
  double *k0 = arr(ns, 0.3), *v0 = arr(ns, 0.3);
  double *o = arr(nq, 0), *kf = arr(ns, 0), *vf = arr(ns, 0), *s = arr(ng, 0), *z = arr(ng, 0);
  int act;
  for (act = 0; act <= 4; act++) {
    /* forward, then the same tokens as T decode steps */
    int rc = oracle_gsa_fwd_nl(q, k, v, g, k0, v0, o, kf, vf, s, z, B, H, T, d, d, m, 8.0, act, 2);
    double *ks = malloc(ns * sizeof(double)), *vs = malloc(ns * sizeof(double));
    double *qt = malloc(U * d * sizeof(double)), *kt = malloc(U * d * sizeof(double));
    double *vt = malloc(U * d * sizeof(double)), *gt = malloc(U * m * sizeof(double));
    double *ot = malloc(U * d * sizeof(double));
    memcpy(ks, k0, ns * sizeof(double));
    memcpy(vs, v0, ns * sizeof(double));
    double err = 0;
    for (long t = 0; t < T && rc == 0; t++) {
      for (long u = 0; u < U; u++) {
        memcpy(qt + u * d, q + (u * T + t) * d, d * sizeof(double));
        memcpy(kt + u * d, k + (u * T + t) * d, d * sizeof(double));
        memcpy(vt + u * d, v + (u * T + t) * d, d * sizeof(double));
        memcpy(gt + u * m, g + (u * T + t) * m, m * sizeof(double));
      }
      rc |= oracle_gsa_decode_step_nl(qt, kt, vt, gt, ks, vs, ot, B, H, d, d, m, 8.0, act, 2);
      for (long u = 0; u < U; u++)
        err = fmax(err, maxdiff(ot + u * d, o + (u * T + t) * d, d));
    }
    err = fmax(err, fmax(maxdiff(ks, kf, ns), maxdiff(vs, vf, ns)));
    char what[96];
    snprintf(what, sizeof what, "read %d: chained decode == forward", act);
    check(rc == 0 && err < 1e-12, what, err);
    free(ks); free(vs); free(qt); free(kt); free(vt); free(gt); free(ot);
  }
  /* alpha = 1 everywhere from zero states: nothing is ever written */
  {
    double *gi = arr(ng, 0);
    for (long i = 0; i < ng; i++) gi[i] = INFINITY;
    int rc = oracle_gsa_fwd_nl(q, k, v, gi, NULL, NULL, o, NULL, NULL, NULL, NULL, B, H, T, d, d,
                               m, 8.0, 0, 1);
    double e = 0;
    for (long i = 0; i < nq; i++) e = fmax(e, fabs(o[i]));
    check(rc == 0 && e == 0.0, "alpha = 1 from zero states: o == 0", e);
    free(gi);
  }
  /* GLA, alpha = 1: causal linear attention */
  {
    double *gi = arr(nq, 0), *ref = arr(nq, 0);
    for (long i = 0; i < nq; i++) gi[i] = INFINITY;
    int rc = oracle_gla_fwd_gm(q, k, v, gi, NULL, o, NULL, B, H, T, d, d, 16.0, 0, 2);
    for (long u = 0; u < U; u++)
      for (long t = 0; t < T; t++)
        for (long j = 0; j <= t; j++) {
          double a = 0;
          for (long c = 0; c < d; c++) a += q[(u * T + t) * d + c] * k[(u * T + j) * d + c];
          for (long c = 0; c < d; c++) ref[(u * T + t) * d + c] += a * v[(u * T + j) * d + c];
        }
    double e = maxdiff(o, ref, nq);
    check(rc == 0 && e < 1e-12, "GLA alpha = 1 == causal linear attention", e);
    rc = oracle_gla_fwd_gm(q, k, v, g, NULL, o, NULL, B, H, 0, d, d, 16.0, 1, 2);
    check(rc == 0, "GLA T = 0 (log-decay gates)", 0);
    free(gi); free(ref);
  }
  /* backward: dq against a central difference of L = <W, o> + <A, Kf> + <Bv, Vf> */
  {
    double *W = arr(nq, 1.0), *A = arr(ns, 1.0), *Bv = arr(ns, 1.0);
    double *dq = arr(nq, 0), *dk = arr(nq, 0), *dv = arr(nq, 0), *dg = arr(ng, 0);
    double *dk0 = arr(ns, 0), *dv0 = arr(ns, 0);
    int rc = oracle_gsa_bwd_nl(q, k, v, g, W, k0, v0, A, Bv, dq, dk, dv, dg, dk0, dv0, B, H, T, d,
                               d, m, 8.0, 0, 2);
    double worst = 0;
    const long idx[] = {0, 7, nq / 2 + 3, nq - 1};
    for (int n = 0; n < 4; n++) {
      double L[2];
      for (int sgn = 0; sgn < 2; sgn++) {
        const double h = 1e-6, keep = q[idx[n]];
        q[idx[n]] = keep + (sgn ? -h : h);
        rc |= oracle_gsa_fwd_nl(q, k, v, g, k0, v0, o, kf, vf, NULL, NULL, B, H, T, d, d, m, 8.0,
                                0, 1);
        q[idx[n]] = keep;
        double acc = 0;
        for (long i = 0; i < nq; i++) acc += W[i] * o[i];
        for (long i = 0; i < ns; i++) acc += A[i] * kf[i] + Bv[i] * vf[i];
        L[sgn] = acc;
      }
      worst = fmax(worst, fabs((L[0] - L[1]) / 2e-6 - dq[idx[n]]));
    }
    check(rc == 0 && worst < 1e-6, "backward dq == central difference", worst);
    rc = oracle_gsa_bwd_nl(q, k, v, g, W, NULL, NULL, NULL, NULL, dq, dk, dv, dg, dk0, dv0, B, H,
                           0, d, d, m, 8.0, 3, 1);
    check(rc == 0, "backward T = 0", 0);
    free(W); free(A); free(Bv); free(dq); free(dk); free(dv); free(dg); free(dk0); free(dv0);
  }
  free(q); free(k); free(v); free(g); free(k0); free(v0); free(o); free(kf); free(vf); free(s);
  free(z);
  printf("%s\n", fails ? "FAILED" : "all ok");
  return fails ? 1 : 0;
}
