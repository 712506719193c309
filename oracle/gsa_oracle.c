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
 *   - Backward (App. B trains the model; the gradient itself is that of the
 *     recurrence above): oracle_gsa_bwd differentiates the token recurrence in
 *     reverse mode, keeping every state of the forward sweep.
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

/* Derivatives of the element-wise slot reads (act 1..4). */
static double slot_grad(double x, int act)
{
    switch (act) {
    case 1:
        return 1.0;
    case 2: {
        double sg = 1.0 / (1.0 + exp(-x));
        return sg * (1.0 + x * (1.0 - sg));
    }
    case 3:
        return x > 0.0 ? 1.0 : 0.0;
    default:
        return x > 0.0 ? 2.0 * x : 0.0;
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

/*
 * Gradients of the GSA forward with respect to q, k, v, the
 * gate logits g and the initial states, given the gradient dO of the outputs
 * and (nullable) the gradients dkf / dvf of the final states.  This is the
 * plain definition: reverse-mode differentiation of the token recurrence
 * (Sec. 3.2-3.3), with every state of the forward sweep kept.  (App. B trains
 * the same function; how its kernels save and recompute states is a matter of
 * memory, not of the result.)
 *
 * Reverse sweep, per unit, t = T-1 .. 0, with dK, dV the adjoints of the
 * states after token t (starting from dkf, dvf):
 *   ds[c] = Vt[c,:] . dO_t              (o_t = Vt^T s_t)
 *   dV[c,:] += s_t[c] dO_t
 *   dz = s_t * (ds - s_t . ds)          (softmax Jacobian; for an element-wise
 *                                        read s = f(z): dz = f'(z) * ds)
 *   dq_t = Kt^T dz,   dK[c,:] += dz[c] q_t
 *   dk_t = dK^T w_t,  dv_t = dV^T w_t    (w_t = 1 - alpha_t)
 *   dalpha[c] = dK[c,:] . (K_{t-1}[c,:] - k_t) + dV[c,:] . (V_{t-1}[c,:] - v_t)
 *   dg_t[c] = dalpha[c] * alpha_t[c] * sigmoid(-g_t[c]) / tau
 *   dK[c,:] *= alpha_t[c], dV[c,:] *= alpha_t[c]   (adjoints of K_{t-1}, V_{t-1})
 * dk0 / dv0 (nullable) receive the adjoints left after t = 0.
 * Layouts as for oracle_gsa_fwd; dO and dv [B,H,T,dv], dg [B,H,T,m].
 */
int oracle_gsa_bwd_nl(const double *q, const double *k, const double *v,
                      const double *g, const double *dO, const double *k0,
                      const double *v0, const double *dkf, const double *dvf,
                      double *dq, double *dk, double *dv, double *dg,
                      double *dk0, double *dv0, long B, long H, long T,
                      long d_k, long d_v, long m, double tau, int act,
                      int nthreads)
{
    long units = B * H, u;
    int err = 0;
    if (!q || !k || !v || !g || !dO || !dq || !dk || !dv || !dg || B < 0 ||
        H < 0 || T < 0 || d_k < 1 || d_v < 1 || m < 1 || !(tau > 0.0) ||
        act < 0 || act > 4)
        return 1;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : err)
#endif
    for (u = 0; u < units; u++) {
        /* Ks[t] / Vs[t]: the states before token t (t = 0 .. T) */
        double *Ks = malloc((size_t)((T + 1) * m * d_k) * sizeof(double));
        double *Vs = malloc((size_t)((T + 1) * m * d_v) * sizeof(double));
        double *S = malloc((size_t)((T > 0 ? T : 1) * m) * sizeof(double));
        double *Z = malloc((size_t)((T > 0 ? T : 1) * m) * sizeof(double));
        double *dK = calloc((size_t)(m * d_k), sizeof(double));
        double *dV = calloc((size_t)(m * d_v), sizeof(double));
        double *ds = malloc((size_t)m * sizeof(double));
        double *dz = malloc((size_t)m * sizeof(double));
        long t, c, x;
        if (!Ks || !Vs || !S || !Z || !dK || !dV || !ds || !dz) {
            err |= 2;
        } else {
            /* forward sweep: the states and the slot read weights */
            for (c = 0; c < m * d_k; c++)
                Ks[c] = k0 ? k0[u * m * d_k + c] : 0.0;
            for (c = 0; c < m * d_v; c++)
                Vs[c] = v0 ? v0[u * m * d_v + c] : 0.0;
            for (t = 0; t < T; t++) {
                long row = u * T + t;
                const double *qt = q + row * d_k, *kt = k + row * d_k;
                const double *vt = v + row * d_v, *gt = g + row * m;
                const double *Kp = Ks + t * m * d_k, *Vp = Vs + t * m * d_v;
                double *Kn = Ks + (t + 1) * m * d_k, *Vn = Vs + (t + 1) * m * d_v;
                double *st = S + t * m, zmax = -INFINITY, sum = 0.0;
                for (c = 0; c < m; c++) {
                    double la = log_sigmoid(gt[c]) / tau;
                    double a = exp(la), w = -expm1(la), acc = 0.0;
                    for (x = 0; x < d_k; x++) {
                        Kn[c * d_k + x] = a * Kp[c * d_k + x] + w * kt[x];
                        acc += Kn[c * d_k + x] * qt[x];
                    }
                    for (x = 0; x < d_v; x++)
                        Vn[c * d_v + x] = a * Vp[c * d_v + x] + w * vt[x];
                    Z[t * m + c] = acc;
                    if (acc > zmax)
                        zmax = acc;
                }
                if (act == 0) {
                    for (c = 0; c < m; c++) {
                        st[c] = exp(Z[t * m + c] - zmax);
                        sum += st[c];
                    }
                    for (c = 0; c < m; c++)
                        st[c] /= sum;
                } else {
                    for (c = 0; c < m; c++)
                        st[c] = slot_fn(Z[t * m + c], act);
                }
            }
            /* reverse sweep */
            if (dkf)
                memcpy(dK, dkf + u * m * d_k, (size_t)(m * d_k) * sizeof(double));
            if (dvf)
                memcpy(dV, dvf + u * m * d_v, (size_t)(m * d_v) * sizeof(double));
            for (t = T - 1; t >= 0; t--) {
                long row = u * T + t;
                const double *qt = q + row * d_k, *kt = k + row * d_k;
                const double *vt = v + row * d_v, *gt = g + row * m;
                const double *dOt = dO + row * d_v, *st = S + t * m;
                const double *Kp = Ks + t * m * d_k, *Vp = Vs + t * m * d_v;
                const double *Kn = Ks + (t + 1) * m * d_k, *Vn = Vs + (t + 1) * m * d_v;
                double sds = 0.0;
                for (c = 0; c < m; c++) {
                    double acc = 0.0;
                    for (x = 0; x < d_v; x++)
                        acc += Vn[c * d_v + x] * dOt[x];
                    ds[c] = acc;
                    sds += st[c] * acc;
                    for (x = 0; x < d_v; x++)
                        dV[c * d_v + x] += st[c] * dOt[x];
                }
                for (c = 0; c < m; c++)
                    dz[c] = act == 0 ? st[c] * (ds[c] - sds)
                                     : slot_grad(Z[t * m + c], act) * ds[c];
                for (x = 0; x < d_k; x++) {
                    double acc = 0.0;
                    for (c = 0; c < m; c++)
                        acc += Kn[c * d_k + x] * dz[c];
                    dq[row * d_k + x] = acc;
                }
                for (c = 0; c < m; c++)
                    for (x = 0; x < d_k; x++)
                        dK[c * d_k + x] += dz[c] * qt[x];
                for (x = 0; x < d_k; x++)
                    dk[row * d_k + x] = 0.0;
                for (x = 0; x < d_v; x++)
                    dv[row * d_v + x] = 0.0;
                for (c = 0; c < m; c++) {
                    double la = log_sigmoid(gt[c]) / tau;
                    double a = exp(la), w = -expm1(la), da = 0.0;
                    double sig_neg = exp(log_sigmoid(-gt[c]));
                    for (x = 0; x < d_k; x++) {
                        dk[row * d_k + x] += w * dK[c * d_k + x];
                        da += dK[c * d_k + x] * (Kp[c * d_k + x] - kt[x]);
                        dK[c * d_k + x] *= a;
                    }
                    for (x = 0; x < d_v; x++) {
                        dv[row * d_v + x] += w * dV[c * d_v + x];
                        da += dV[c * d_v + x] * (Vp[c * d_v + x] - vt[x]);
                        dV[c * d_v + x] *= a;
                    }
                    dg[row * m + c] = da * a * sig_neg / tau;
                }
            }
            if (dk0)
                memcpy(dk0 + u * m * d_k, dK, (size_t)(m * d_k) * sizeof(double));
            if (dv0)
                memcpy(dv0 + u * m * d_v, dV, (size_t)(m * d_v) * sizeof(double));
        }
        free(Ks);
        free(Vs);
        free(S);
        free(Z);
        free(dK);
        free(dV);
        free(ds);
        free(dz);
    }
    return err;
}

/* The method as published: the softmax read. */
int oracle_gsa_bwd(const double *q, const double *k, const double *v,
                   const double *g, const double *dO, const double *k0,
                   const double *v0, const double *dkf, const double *dvf,
                   double *dq, double *dk, double *dv, double *dg, double *dk0,
                   double *dv0, long B, long H, long T, long d_k, long d_v,
                   long m, double tau, int nthreads)
{
    return oracle_gsa_bwd_nl(q, k, v, g, dO, k0, v0, dkf, dvf, dq, dk, dv, dg,
                             dk0, dv0, B, H, T, d_k, d_v, m, tau, 0, nthreads);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
