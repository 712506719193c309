"""Chunkwise-parallel GSA / GLA in float64 numpy -- a second, independent
implementation used only to pin the recurrent oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: "Gated Slot Attention for Efficient Linear-Time Sequence Modeling".
* App. A.1 (chunkwise form, Eq. 14-16): the sequence is cut into N = ceil(T/C)
  chunks; within a chunk the output is an inter-chunk term read from the state
  at the chunk start plus an intra-chunk causal term, and the state is carried
  to the next chunk.  Element-wise gating keeps this rearrangement exact.
* App. A.1 (the secondary chunking it points to; App. B runs it on 16-token
  sub-chunks): see gla_*_secondary below.
* App. B: GSA is two such GLA passes.  The first pass takes the queries and
  keys with the slot write intensities I = 1 - A as its values; a softmax over
  the slots of its output gives the queries of the second pass, whose keys are
  I and values are V.  The per-slot decay sits on the value (slot) dimension in
  the first pass and on the key (slot) dimension in the second, as in the
  paper's listing.  The preprocessing step is the chunk-local cumulative sum
  of log alpha.

Every decay factor exp(G_j - G_r) is formed as the exponential of an explicit
sum of log alpha over tokens r+1..j (never as a difference of two cumulative
sums), so alpha = 0 (log alpha = -inf) is handled exactly.
"""
from __future__ import annotations

import numpy as np


def log_sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def _pair_logdecay(la):
    """D[j, r, :] = sum of la[i] for r < i <= j (0 when r == j); -inf for r > j."""
    L, d = la.shape
    D = np.full((L, L, d), -np.inf)
    for r in range(L):
        D[r, r] = 0.0
        if r + 1 < L:
            D[r + 1:, r] = np.cumsum(la[r + 1:], axis=0)
    return D


def gla_key_decay(q, k, v, la, S0=None, C=64):
    """One unit of GLA with decay on the key (row) dimension of S [dk, dv].
    q, k, la: [T, dk]; v: [T, dv].  Returns (o [T, dv], S_final)."""
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for n0 in range(0, T, C):
        sl = slice(n0, min(n0 + C, T))
        qc, kc, vc, lc = q[sl], k[sl], v[sl], la[sl]
        D = _pair_logdecay(lc)
        Gf = np.cumsum(lc, axis=0)            # decay from the chunk start to j
        inter = (qc * np.exp(Gf)) @ S
        A = np.einsum("jc,rc,jrc->jr", qc, kc, np.exp(D))
        o[sl] = inter + A @ vc
        S = np.exp(Gf[-1])[:, None] * S + (kc * np.exp(D[-1])).T @ vc
    return o, S


def gla_value_decay(q, k, w, la, P0=None, C=64):
    """One unit of GLA with decay on the value (column) dimension of P [dk, m].
    q, k: [T, dk]; w, la: [T, m].  Returns (o [T, m], P_final)."""
    T, dk = q.shape
    m = w.shape[1]
    P = np.zeros((dk, m)) if P0 is None else np.array(P0, dtype=np.float64)
    o = np.zeros((T, m))
    for n0 in range(0, T, C):
        sl = slice(n0, min(n0 + C, T))
        qc, kc, wc, lc = q[sl], k[sl], w[sl], la[sl]
        D = _pair_logdecay(lc)
        Gf = np.cumsum(lc, axis=0)
        inter = np.exp(Gf) * (qc @ P)
        A = qc @ kc.T
        intra = np.einsum("jr,rc,jrc->jc", A, wc, np.exp(D))
        o[sl] = inter + intra
        P = P * np.exp(Gf[-1])[None, :] + kc.T @ (wc * np.exp(D[-1]))
    return o, P


# --------------------------------------------------- secondary chunking
# App. A.1 points to a secondary chunking of each chunk (sub-chunks of Cs
# tokens; App. B runs it with Cs = 16).  A query row j of sub-chunk J meets a
# key row r of an earlier sub-chunk R through a matrix product whose two
# factors are decays to and from a reference point, the first token of J:
# exp(sum of log alpha over (ref, j]) <= 1 on the query side and
# exp(sum over (r, ref]) <= 1 on the key side, so nothing is divided; rows of
# the same sub-chunk meet through their pairwise decays directly.  The state
# read and the carry are the chunk form's.

def _span_logsum(lc, a, b):
    """Sum of lc over rows (a, b] (0 when b <= a), per column, as an explicit
    sum (so that log alpha = -inf never meets another -inf)."""
    if b <= a:
        return np.zeros(lc.shape[1])
    return lc[a + 1:b + 1].sum(axis=0)


def _sub_chunks(L, Cs):
    return [(s0, min(s0 + Cs, L)) for s0 in range(0, L, Cs)]


def gla_value_decay_secondary(q, k, w, la, P0=None, C=64, Cs=16):
    """gla_value_decay with the intra-chunk term by secondary chunking."""
    T, dk = q.shape
    m = w.shape[1]
    P = np.zeros((dk, m)) if P0 is None else np.array(P0, dtype=np.float64)
    o = np.zeros((T, m))
    for n0 in range(0, T, C):
        n1 = min(n0 + C, T)
        qc, kc, wc, lc = q[n0:n1], k[n0:n1], w[n0:n1], la[n0:n1]
        L = n1 - n0
        A = qc @ kc.T
        for (j0, j1) in _sub_chunks(L, Cs):
            ref = j0
            # earlier sub-chunks: one product through the reference point
            if j0 > 0:
                kside = np.stack([wc[r] * np.exp(_span_logsum(lc, r, ref)) for r in range(j0)])
                inner = A[j0:j1, :j0] @ kside                       # [rows, m]
                qside = np.stack([np.exp(_span_logsum(lc, ref, j)) for j in range(j0, j1)])
                o[n0 + j0:n0 + j1] += qside * inner
            # the same sub-chunk: pairwise decays
            for j in range(j0, j1):
                for r in range(j0, j + 1):
                    o[n0 + j] += A[j, r] * wc[r] * np.exp(_span_logsum(lc, r, j))
        # the state read and the carry (chunk form)
        Gf = np.stack([_span_logsum(lc, -1, j) for j in range(L)])
        o[n0:n1] += np.exp(Gf) * (qc @ P)
        P = P * np.exp(Gf[-1])[None, :] + kc.T @ (wc * np.exp(np.stack([_span_logsum(lc, r, L - 1) for r in range(L)])))
    return o, P


def gla_key_decay_secondary(q, k, v, la, S0=None, C=64, Cs=16):
    """gla_key_decay with the intra-chunk term by secondary chunking."""
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for n0 in range(0, T, C):
        n1 = min(n0 + C, T)
        qc, kc, vc, lc = q[n0:n1], k[n0:n1], v[n0:n1], la[n0:n1]
        L = n1 - n0
        Acc = np.zeros((L, L))
        for (j0, j1) in _sub_chunks(L, Cs):
            ref = j0
            if j0 > 0:
                qside = np.stack([qc[j] * np.exp(_span_logsum(lc, ref, j)) for j in range(j0, j1)])
                kside = np.stack([kc[r] * np.exp(_span_logsum(lc, r, ref)) for r in range(j0)])
                Acc[j0:j1, :j0] = qside @ kside.T
            for j in range(j0, j1):
                for r in range(j0, j + 1):
                    Acc[j, r] = np.sum(qc[j] * kc[r] * np.exp(_span_logsum(lc, r, j)))
        Gf = np.stack([_span_logsum(lc, -1, j) for j in range(L)])
        o[n0:n1] = (qc * np.exp(Gf)) @ S + Acc @ vc
        S = np.exp(Gf[-1])[:, None] * S + (kc * np.exp(np.stack([_span_logsum(lc, r, L - 1) for r in range(L)]))).T @ vc
    return o, S


def gsa_fwd_secondary(q, k, v, g, k0=None, v0=None, tau=8.0, C=64, Cs=16, nonlinearity="softmax"):
    """GSA (two passes) with both intra-chunk terms by secondary chunking."""
    B, H, T, dk = q.shape
    m = g.shape[-1]
    o = np.zeros(v.shape)
    kf = np.zeros((B, H, m, dk))
    vf = np.zeros((B, H, m, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            la = log_sigmoid(g[b, h]) / tau
            w = -np.expm1(la)
            P0 = None if k0 is None else np.asarray(k0[b, h], dtype=np.float64).T
            ok, P = gla_value_decay_secondary(q[b, h], k[b, h], w, la, P0, C, Cs)
            s = slot_read(ok, nonlinearity)
            o[b, h], vf[b, h] = gla_key_decay_secondary(s, w, v[b, h], la,
                                                        None if v0 is None else v0[b, h], C, Cs)
            kf[b, h] = P.T
    return o, kf, vf


def softmax_slots(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def slot_read(x, nonlinearity="softmax"):
    """The link between the two passes: the softmax over the slots (Sec. 3.2),
    or an element-wise replacement from the ablation study (Table 2)."""
    x = np.asarray(x, dtype=np.float64)
    if nonlinearity == "softmax":
        return softmax_slots(x)
    if nonlinearity == "identity":
        return x.copy()
    if nonlinearity == "swish":
        return x * (0.5 * (1.0 + np.tanh(0.5 * x)))   # sigmoid via tanh
    if nonlinearity == "relu":
        return np.where(x > 0.0, x, 0.0)
    if nonlinearity == "relu2":
        return np.where(x > 0.0, x * x, 0.0)
    raise ValueError(nonlinearity)


def gsa_unit(q, k, v, g, k0=None, v0=None, tau=8.0, C=64, nonlinearity="softmax"):
    """One (b,h) unit of GSA as two chunked GLA passes.  Returns
    (o, Kt_final [m,dk], Vt_final [m,dv], s [T,m])."""
    la = log_sigmoid(g) / tau
    w = -np.expm1(la)
    P0 = None if k0 is None else np.asarray(k0, dtype=np.float64).T
    ok, P = gla_value_decay(q, k, w, la, P0, C)
    s = slot_read(ok, nonlinearity)
    o, Vf = gla_key_decay(s, w, v, la, v0, C)
    return o, P.T, Vf, s


def gsa_fwd(q, k, v, g, k0=None, v0=None, tau=8.0, C=64, nonlinearity="softmax"):
    B, H, T, dk = q.shape
    m = g.shape[-1]
    o = np.zeros(v.shape)
    kf = np.zeros((B, H, m, dk))
    vf = np.zeros((B, H, m, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            o[b, h], kf[b, h], vf[b, h], _ = gsa_unit(
                q[b, h], k[b, h], v[b, h], g[b, h],
                None if k0 is None else k0[b, h], None if v0 is None else v0[b, h], tau, C,
                nonlinearity)
    return o, kf, vf


def gla_fwd(q, k, v, g, s0=None, tau=16.0, C=64):
    B, H, T, dk = q.shape
    o = np.zeros(v.shape)
    sf = np.zeros((B, H, dk, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            la = log_sigmoid(g[b, h]) / tau
            o[b, h], sf[b, h] = gla_key_decay(q[b, h], k[b, h], v[b, h], la,
                                              None if s0 is None else s0[b, h], C)
    return o, sf


# ----------------------------------------------------------------- backward
# App. B's training scheme in chunk form: the two GLA passes are differentiated
# in reverse order (pass 2 first), the write intensity I = 1 - alpha collects
# the gradient of both passes, and the forget-gate gradient is the reversed
# cumulative sum over tokens of each pass's "scaled-by-e^G" products minus its
# "scaled-by-e^-G" products (pass 2: Q.dQ - K.dK with its query s and key I;
# pass 1: O.dO - V.dV with its output o' and value I), plus the final-state
# terms.  Chunk start states come from the forward recurrence, chunk-end
# adjoints from the reverse one; within a chunk every decay is exp of an
# explicit sum of log alpha, as in the forward.

def _chunks(T, C):
    return [slice(n0, min(n0 + C, T)) for n0 in range(0, T, C)]


def gla_key_decay_bwd(q, k, v, la, S0, do, dSf, C=64):
    """Backward of gla_key_decay (S [dk, dv], decay on rows).  Returns
    (dq, dk, dv, dG, dS0) with dG[t, c] = dL/dG_t[c], G the running sum of la."""
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    starts = []
    for sl in _chunks(T, C):          # forward: chunk start states
        starts.append(S.copy())
        lc, kc, vc = la[sl], k[sl], v[sl]
        D = _pair_logdecay(lc)
        S = np.exp(np.cumsum(lc, axis=0)[-1])[:, None] * S + (kc * np.exp(D[-1])).T @ vc
    dq, dkk, dvv, dG = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros((T, dk))
    U = np.zeros((dk, dv)) if dSf is None else np.array(dSf, dtype=np.float64)
    if dSf is not None and T > 0:
        dG[T - 1] += np.sum(U * S, axis=1)        # the final state carries e^{G_T}
    for i in reversed(range(len(starts))):
        sl = _chunks(T, C)[i]
        qc, kc, vc, lc, dc = q[sl], k[sl], v[sl], la[sl], do[sl]
        D = np.exp(_pair_logdecay(lc))                # D[j, r] = decay from r to j
        Gf = np.exp(np.cumsum(lc, axis=0))
        A = dc @ vc.T                                 # dO_j . v_r
        dq[sl] = Gf * (dc @ starts[i].T) + np.einsum("jr,rc,jrc->jc", A, kc, D)
        dkk[sl] = np.einsum("tj,tc,tjc->jc", A, qc, D) + D[-1] * (vc @ U.T)
        Bm = np.einsum("tc,jc,tjc->tj", qc, kc, D)
        dvv[sl] = Bm.T @ dc + (kc * D[-1]) @ U
        dG[sl] += qc * dq[sl] - kc * dkk[sl]
        U = Gf[-1][:, None] * U + (qc * Gf).T @ dc
    return dq, dkk, dvv, dG, U


def gla_value_decay_bwd(q, k, w, la, P0, do, dPf, C=64):
    """Backward of gla_value_decay (P [dk, m], decay on columns).  Returns
    (dq, dk, dw, dG, dP0)."""
    T, dk = q.shape
    m = w.shape[1]
    P = np.zeros((dk, m)) if P0 is None else np.array(P0, dtype=np.float64)
    starts, outs = [], np.zeros((T, m))
    for sl in _chunks(T, C):
        starts.append(P.copy())
        qc, kc, wc, lc = q[sl], k[sl], w[sl], la[sl]
        D = np.exp(_pair_logdecay(lc))
        Gf = np.exp(np.cumsum(lc, axis=0))
        outs[sl] = Gf * (qc @ P) + np.einsum("jr,rc,jrc->jc", qc @ kc.T, wc, D)
        P = P * Gf[-1][None, :] + kc.T @ (wc * D[-1])
    dq, dkk, dw, dG = np.zeros_like(q), np.zeros_like(k), np.zeros_like(w), np.zeros((T, m))
    U = np.zeros((dk, m)) if dPf is None else np.array(dPf, dtype=np.float64)
    if dPf is not None and T > 0:
        dG[T - 1] += np.sum(U * P, axis=0)
    for i in reversed(range(len(starts))):
        sl = _chunks(T, C)[i]
        qc, kc, wc, lc, dc = q[sl], k[sl], w[sl], la[sl], do[sl]
        D = np.exp(_pair_logdecay(lc))
        Gf = np.exp(np.cumsum(lc, axis=0))
        dq[sl] = (dc * Gf) @ starts[i].T + np.einsum("jc,rc,jrc->jr", dc, wc, D) @ kc
        E = np.einsum("tc,jc,tjc->tj", dc, wc, D)
        dkk[sl] = E.T @ qc + (wc * D[-1]) @ U.T
        dw[sl] = np.einsum("tj,tc,tjc->jc", qc @ kc.T, dc, D) + D[-1] * (kc @ U)
        dG[sl] += outs[sl] * dc - wc * dw[sl]
        U = U * Gf[-1][None, :] + qc.T @ (dc * Gf)
    return dq, dkk, dw, dG, U


def gsa_bwd_unit(q, k, v, g, do, k0=None, v0=None, dkf=None, dvf=None, tau=8.0, C=64):
    """Gradients of one (b,h) unit of GSA (softmax read) through the two chunked
    GLA passes.  Returns (dq, dk, dv, dg, dk0, dv0)."""
    la = log_sigmoid(g) / tau
    w = -np.expm1(la)
    P0 = None if k0 is None else np.asarray(k0, dtype=np.float64).T
    z, _ = gla_value_decay(q, k, w, la, P0, C)
    s = softmax_slots(z)
    ds, dw2, dv, dG2, dv0 = gla_key_decay_bwd(s, w, v, la, v0, do, dvf, C)      # pass 2
    dz = s * (ds - np.sum(s * ds, axis=-1, keepdims=True))                       # softmax
    dPf = None if dkf is None else np.asarray(dkf, dtype=np.float64).T
    dq, dk, dw1, dG1, dP0 = gla_value_decay_bwd(q, k, w, la, P0, dz, dPf, C)    # pass 1
    dI = dw1 + dw2
    dG = dG1 + dG2
    dla = np.cumsum(dG[::-1], axis=0)[::-1] - np.exp(la) * dI                   # reversed cumsum
    dg = dla * np.exp(log_sigmoid(-np.asarray(g, dtype=np.float64))) / tau
    return dq, dk, dv, dg, dP0.T, dv0


def gsa_bwd(q, k, v, g, do, k0=None, v0=None, dkf=None, dvf=None, tau=8.0, C=64):
    """[B,H,...] wrapper of gsa_bwd_unit; returns a dict like oracle.gsa_bwd."""
    B, H = q.shape[:2]
    out = {n: [] for n in ("dq", "dk", "dv", "dg", "dk0", "dv0")}
    opt = lambda x, b, h: None if x is None else x[b, h]
    res = [[gsa_bwd_unit(q[b, h], k[b, h], v[b, h], g[b, h], do[b, h], opt(k0, b, h), opt(v0, b, h),
                         opt(dkf, b, h), opt(dvf, b, h), tau, C) for h in range(H)] for b in range(B)]
    for i, n in enumerate(("dq", "dk", "dv", "dg", "dk0", "dv0")):
        out[n] = np.array([[res[b][h][i] for h in range(H)] for b in range(B)])
    return out
