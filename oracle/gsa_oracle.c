/*
 * Plain fp64 CPU oracle for Gated Slot Attention (GSA) and gated linear
 * attention (GLA): the token-by-token recurrences, nothing else.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The HIP product path
 * never links, calls or falls back to it; the two share no code.
 *
 * Source: "Gated Slot Attention for Efficient Linear-Time Sequence Modeling"
 * (arXiv 2409.07146).
 *   - Forget gate (Sec. 3.3 and its footnote 2): alpha_t = sigmoid(g_t)^(1/tau),
 *     i.e. log alpha_t = log sigmoid(g_t) / tau, one value per slot.
 *   - Per-slot gated RNN (Sec. 3.2, Eq. 6 -- the display is lost in the text we
 *     have; restated from the surrounding prose and App. A/B): the write
 *     intensity is coupled to the forget gate, 1 - alpha_t (HGRN2-style
 *     coupling, Sec. 2.3 and App. A Eq. 13), so per slot c
 *         Kt[c,:] <- alpha_t[c] * Kt[c,:] + (1 - alpha_t[c]) * k_t
 *         Vt[c,:] <- alpha_t[c] * Vt[c,:] + (1 - alpha_t[c]) * v_t
 *   - Read (Sec. 3.2, Eq. 7, two-pass GLA linked by softmax; App. B): the
 *     slot scores o'_t = Kt q_t are normalised by a softmax over the m slots,
 *     s_t = softmax(o'_t), and the output is o_t = Vt^T s_t.  The state is
 *     updated with token t before it is read (inclusive read).
 *   - No normaliser term and no temperature (Sec. 2.2 footnote 1; App. A
 *     footnote 8).
 *   - Non-linearity ablations (Sec. 4.1.3, Table 2): the softmax may be
 *     replaced by an element-wise function of each slot score z, s_t[c] =
 *     f(z[c]): 1 = none (f(z) = z), 2 = Swish (z * sigmoid(z)), 3 = ReLU
 *     (max(z, 0)), 4 = ReLU^2 (max(z, 0)^2); 0 is the softmax.
 *   - GLA (Sec. 2.3, with beta = 1): S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T,
 *     o_t = S_t^T q_t, alpha_t per key dimension.  The gate is given either as
 *     logits (alpha = sigmoid(g)^(1/tau), gate_mode 0) or as per-token
 *     log-decays (alpha = exp(min(g, 0)), gate_mode 1): a gate vector computed
 *     elsewhere, such as the rank-one gate of Lattice's simplified chunk
 *     recurrence.
 *
 * All arithmetic is fp64.  log sigmoid uses the textbook stable split
 * min(x,0) - log1p(exp(-|x|)); 1 - alpha is formed as -expm1(log alpha) so
 * that it stays accurate when alpha is close to 1.  Infinite logits give the
 * exact limits (g = +inf: alpha = 1; g = -inf: alpha = 0).
 *
 * Layouts (row-major, contiguous):
 *   q, k [B,H,T,dk]; v, o [B,H,T,dv]; g [B,H,T,m] (GSA) or [B,H,T,dk] (GLA)
 *   GSA states [B,H,m,dk] / [B,H,m,dv]; GLA state [B,H,dk,dv]
 * Units (b,h) are independent; OpenMP runs them in parallel when nthreads > 1.
 * Return value: 0 on success, 1 on a bad argument, 2 on allocation failure.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double log_sigmoid(double x)
{
    return (x < 0.0 ? x : 0.0) - log1p(exp(-fabs(x)));
}

/* Element-wise slot read functions of the ablation study (Table 2). */
static double slot_fn(double x, int act)
{
    switch (act) {
    case 1:
        return x;
    case 2:
        return x / (1.0 + exp(-x));
    case 3:
        return x > 0.0 ? x : 0.0;
    default:
        return x > 0.0 ? x * x : 0.0;
    }
}

/* One GSA token step on one unit's slot states (Sec. 3.2). */
static void gsa_token(const double *qt, const double *kt, const double *vt,
                      const double *gt, double *K, double *V, double *ot,
                      double *st, double *zt, double *z, double *s,
                      long dk, long dv, long m, double tau, int act)
{
    long c, x;
    double zmax = -INFINITY, sum = 0.0;
    for (c = 0; c < m; c++) {
        double la = log_sigmoid(gt[c]) / tau;
        double a = exp(la);
        double w = -expm1(la);
        double acc = 0.0;
        double *Kc = K + c * dk, *Vc = V + c * dv;
        for (x = 0; x < dk; x++) {
            Kc[x] = a * Kc[x] + w * kt[x];
            acc += Kc[x] * qt[x];
        }
        for (x = 0; x < dv; x++)
            Vc[x] = a * Vc[x] + w * vt[x];
        z[c] = acc;
        if (acc > zmax)
            zmax = acc;
    }
    if (act == 0) {
        for (c = 0; c < m; c++) {
            s[c] = exp(z[c] - zmax);
            sum += s[c];
        }
        for (c = 0; c < m; c++)
            s[c] /= sum;
    } else {
        for (c = 0; c < m; c++)
            s[c] = slot_fn(z[c], act);
    }
    for (x = 0; x < dv; x++) {
        double acc = 0.0;
        for (c = 0; c < m; c++)
            acc += V[c * dv + x] * s[c];
        ot[x] = acc;
    }
    if (st)
        memcpy(st, s, (size_t)m * sizeof(double));
    if (zt)
        memcpy(zt, z, (size_t)m * sizeof(double));
}

/*
 * GSA forward over whole sequences.  k0/v0 nullable (zero initial state);
 * kf/vf nullable; s_out/z_out nullable [B,H,T,m] (slot read weights / raw
 * scores).  act: 0 softmax, 1..4 the element-wise ablations above.
 */
int oracle_gsa_fwd_nl(const double *q, const double *k, const double *v,
                      const double *g, const double *k0, const double *v0,
                      double *o, double *kf, double *vf, double *s_out,
                      double *z_out, long B, long H, long T, long dk, long dv,
                      long m, double tau, int act, int nthreads)
{
    long units = B * H, u;
    int err = 0;
    if (!q || !k || !v || !g || !o || B < 0 || H < 0 || T < 0 || dk < 1 ||
        dv < 1 || m < 1 || !(tau > 0.0) || act < 0 || act > 4)
        return 1;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : err)
#endif
    for (u = 0; u < units; u++) {
        double *K = calloc((size_t)(m * dk), sizeof(double));
        double *V = calloc((size_t)(m * dv), sizeof(double));
        double *z = malloc((size_t)m * sizeof(double));
        double *s = malloc((size_t)m * sizeof(double));
        long t;
        if (!K || !V || !z || !s) {
            err |= 2;
        } else {
            if (k0)
                memcpy(K, k0 + u * m * dk, (size_t)(m * dk) * sizeof(double));
            if (v0)
                memcpy(V, v0 + u * m * dv, (size_t)(m * dv) * sizeof(double));
            for (t = 0; t < T; t++) {
                long row = u * T + t;
                gsa_token(q + row * dk, k + row * dk, v + row * dv, g + row * m,
                          K, V, o + row * dv, s_out ? s_out + row * m : NULL,
                          z_out ? z_out + row * m : NULL, z, s, dk, dv, m, tau, act);
            }
            if (kf)
                memcpy(kf + u * m * dk, K, (size_t)(m * dk) * sizeof(double));
            if (vf)
                memcpy(vf + u * m * dv, V, (size_t)(m * dv) * sizeof(double));
        }
        free(K);
        free(V);
        free(z);
        free(s);
    }
    return err;
}

/* The method as published: the softmax read. */
int oracle_gsa_fwd(const double *q, const double *k, const double *v,
                   const double *g, const double *k0, const double *v0,
                   double *o, double *kf, double *vf, double *s_out,
                   double *z_out, long B, long H, long T, long dk, long dv,
                   long m, double tau, int nthreads)
{
    return oracle_gsa_fwd_nl(q, k, v, g, k0, v0, o, kf, vf, s_out, z_out, B, H,
                             T, dk, dv, m, tau, 0, nthreads);
}

/* GLA forward (Sec. 2.3, beta = 1): per key dimension decay, S in R^{dk x dv}. */
int oracle_gla_fwd_gm(const double *q, const double *k, const double *v,
                      const double *g, const double *s0, double *o, double *sf,
                      long B, long H, long T, long dk, long dv, double tau,
                      int gate_mode, int nthreads)
{
    long units = B * H, u;
    int err = 0;
    if (!q || !k || !v || !g || !o || B < 0 || H < 0 || T < 0 || dk < 1 ||
        dv < 1 || !(tau > 0.0) || gate_mode < 0 || gate_mode > 1)
        return 1;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : err)
#endif
    for (u = 0; u < units; u++) {
        double *S = calloc((size_t)(dk * dv), sizeof(double));
        long t, x, y;
        if (!S) {
            err |= 2;
            continue;
        }
        if (s0)
            memcpy(S, s0 + u * dk * dv, (size_t)(dk * dv) * sizeof(double));
        for (t = 0; t < T; t++) {
            long row = u * T + t;
            const double *qt = q + row * dk, *kt = k + row * dk;
            const double *vt = v + row * dv, *gt = g + row * dk;
            double *ot = o + row * dv;
            for (x = 0; x < dk; x++) {
                double a = gate_mode == 0 ? exp(log_sigmoid(gt[x]) / tau)
                                          : exp(gt[x] < 0.0 ? gt[x] : 0.0);
                double *Sx = S + x * dv;
                for (y = 0; y < dv; y++)
                    Sx[y] = a * Sx[y] + kt[x] * vt[y];
            }
            for (y = 0; y < dv; y++) {
                double acc = 0.0;
                for (x = 0; x < dk; x++)
                    acc += S[x * dv + y] * qt[x];
                ot[y] = acc;
            }
        }
        if (sf)
            memcpy(sf + u * dk * dv, S, (size_t)(dk * dv) * sizeof(double));
        free(S);
    }
    return err;
}

int oracle_gla_fwd(const double *q, const double *k, const double *v,
                   const double *g, const double *s0, double *o, double *sf,
                   long B, long H, long T, long dk, long dv, double tau,
                   int nthreads)
{
    return oracle_gla_fwd_gm(q, k, v, g, s0, o, sf, B, H, T, dk, dv, tau, 0,
                             nthreads);
}

/*
 * One recurrent GSA step for N independent sequences x H heads; the slot states
 * [N,H,m,dk] / [N,H,m,dv] are advanced in place and o [N,H,dv] is written.
 */
int oracle_gsa_decode_step_nl(const double *q, const double *k, const double *v,
                              const double *g, double *kstate, double *vstate,
                              double *o, long N, long H, long dk, long dv, long m,
                              double tau, int act, int nthreads)
{
    long units = N * H, u;
    int err = 0;
    if (!q || !k || !v || !g || !kstate || !vstate || !o || N < 0 || H < 0 ||
        dk < 1 || dv < 1 || m < 1 || !(tau > 0.0) || act < 0 || act > 4)
        return 1;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads) reduction(| : err)
#endif
    for (u = 0; u < units; u++) {
        double *z = malloc((size_t)m * sizeof(double));
        double *s = malloc((size_t)m * sizeof(double));
        if (!z || !s) {
            err |= 2;
        } else {
            gsa_token(q + u * dk, k + u * dk, v + u * dv, g + u * m,
                      kstate + u * m * dk, vstate + u * m * dv, o + u * dv,
                      NULL, NULL, z, s, dk, dv, m, tau, act);
        }
        free(z);
        free(s);
    }
    return err;
}

int oracle_gsa_decode_step(const double *q, const double *k, const double *v,
                           const double *g, double *kstate, double *vstate,
                           double *o, long N, long H, long dk, long dv, long m,
                           double tau, int nthreads)
{
    return oracle_gsa_decode_step_nl(q, k, v, g, kstate, vstate, o, N, H, dk,
                                     dv, m, tau, 0, nthreads);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
