"""fp64 numpy model of the chunked (UT / WY) form of the gated delta rule.

Test infrastructure.  It is NOT the oracle and not the GPU path: it restates
in numpy the chunk-level algebra that the GPU kernels evaluate, so that a test
can pin the derivation itself against the token-by-token oracle (they must
agree to rounding in fp64 for every chunk length and ragged tail).

Derivation (from the token recurrence M_t = a_t M_{t-1} + k_t u_t^T with
u_t = b_t (v_t - a_t M_{t-1}^T k_t), state M = S^T of shape [dk, dv]).
Within one chunk of length C with incoming state M0, local index r = 1..C:
  g_r = sum_{s<=r} ln a_s,  gam_r = exp(g_r),  G_rs = exp(g_r - g_s) (r >= s)
  M_r = gam_r M0 + sum_{s<=r} G_rs k_s u_s^T
  (I + diag(b) A) U = diag(b) (V - diag(gam) K M0),  A = strict_tril(K K^T * G)
  => U = Ut - W M0 with T = (I + diag(b) A)^-1 diag(b), Ut = T V,
                        W = T diag(gam) K
  O   = diag(gam) Q M0 + tril(Q K^T * G) U          (diagonal included)
  M_C = gam_C M0 + (diag(exp(g_C - g)) K)^T U
Only exponents g_r - g_s with r >= s (and g_C - g_s) are formed: all <= 0.

`rnd` (optional) is applied to every operand that a matrix-core product would
consume in reduced precision; the default keeps fp64 throughout.
"""
from __future__ import annotations

import numpy as np


def _ident(x):
    return x


def chunked_fwd_head(q, k, v, alpha, beta, M0, C, *, eps=1e-6, scale=1.0,
                     qk_l2norm=True, rnd=None):
    """One head. q,k [T,dk], v [T,dv], alpha/beta [T], M0 [dk,dv] or None."""
    rnd = rnd or _ident
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    alpha = np.asarray(alpha, np.float64)
    beta = np.asarray(beta, np.float64)
    T, dk = q.shape
    dv = v.shape[1]
    M = np.zeros((dk, dv)) if M0 is None else np.array(M0, np.float64)
    if qk_l2norm:
        rq = scale / np.sqrt((q * q).sum(1) + eps)
        rk = 1.0 / np.sqrt((k * k).sum(1) + eps)
    else:
        rq = np.full(T, scale)
        rk = np.ones(T)
    out = np.zeros((T, dv))
    for t0 in range(0, T, C):
        t1 = min(T, t0 + C)
        n = t1 - t0
        Q, K, V = q[t0:t1], k[t0:t1], v[t0:t1]
        a, b = alpha[t0:t1], beta[t0:t1]
        cq, ck = rq[t0:t1], rk[t0:t1]
        g = np.cumsum(np.log(a))
        low = np.tril(np.ones((n, n), dtype=bool))
        diff = np.where(low, g[:, None] - g[None, :], -np.inf)
        G = np.exp(diff)                                   # zero above the diagonal
        gam = np.exp(g)
        # Gram products on raw operands, scalings applied afterwards
        KK = rnd(K) @ rnd(K).T * np.outer(ck, ck)
        QK = rnd(Q) @ rnd(K).T * np.outer(cq, ck)
        A = np.tril(KK * G, -1)
        L = np.eye(n) + b[:, None] * A
        Tm = np.linalg.solve(L, np.diag(b))                # (I + diag(b) A)^-1 diag(b)
        W = rnd(Tm * (gam * ck)[None, :]) @ rnd(K)         # T diag(gam r_k) K
        Ut = rnd(Tm) @ rnd(V)
        U = Ut - rnd(W) @ rnd(M)
        P = QK * G                                          # tril incl. diagonal
        O = (gam * cq)[:, None] * (rnd(Q) @ rnd(M)) + rnd(P) @ rnd(U)
        wlast = np.exp(g[-1] - g) * ck
        M = np.exp(g[-1]) * M + rnd(K).T @ rnd(wlast[:, None] * U)
        out[t0:t1] = O
    return out, M


def chunked_fwd(q, k, v, alpha, beta, state_in, C, **kw):
    """All heads. Shapes as the oracle: q,k [B,H,T,dk] ... state [B,H,dk,dv]."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, H, T, dv))
    st = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            o, m = chunked_fwd_head(q[b, h], k[b, h], v[b, h], alpha[b, h], beta[b, h],
                                    None if state_in is None else state_in[b, h], C, **kw)
            out[b, h] = o
            st[b, h] = m
    return out, st
