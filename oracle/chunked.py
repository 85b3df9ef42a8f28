"""Chunk-parallel fp64 evaluation of KDA, used to pin the token-by-token oracle.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).

"Kimi K3 Technical Report: Open Frontier Intelligence", §2.1.1, "chunkwise
parallel form": within chunk t, eq. (3) defines the per-channel cumulative
decay Gamma (rows gamma^1..gamma^C); the UT transform yields U and W with
pseudo-values V~ = U - W S; eq. (4) gives A = Tril[(Q*Gamma)(K/Gamma)^T] and
O = (Gamma*Q) S + A V~.  The page leaves U, W and the state hand-off between
chunks to the Kimi Linear paper; they follow from eq. (1) by unrolling it over
one chunk (worked out in the module's own comments below), which is the plain
reading this file takes:

  with delta_r = beta_r (v_r - (Diag(alpha_r) S_{r-1})^T k_r), eq. (1) reads
  S_r = Diag(alpha_r) S_{r-1} + k_r delta_r^T, so inside a chunk entered with S
      S_r   = Diag(Gamma_r) S + sum_{i<=r} Diag(Gamma_r / Gamma_i) k_i delta_i^T
      (I + L) Delta = Diag(beta) (V - (K*Gamma) S),
          L_ri = beta_r sum_j k_rj k_ij Gamma_rj / Gamma_ij   (i < r only)
      U = (I + L)^-1 Diag(beta) V,  W = (I + L)^-1 Diag(beta) (K*Gamma),
      V~ = Delta = U - W S
      S_next = Diag(Gamma_C) S + (K * Gamma_C / Gamma)^T V~.

Everything is dense numpy in fp64 with an explicit matrix inverse; nothing is
blocked or fused.  1/Gamma is formed directly, which is exact in fp64 while
C * |g_min| stays below ~700 (C <= 128 at g_min = -5).
"""
from __future__ import annotations

import numpy as np


def chunked_sequence(q, k, v, g, beta, S0, C: int, scale: float = 1.0):
    """One sequence of one head.  q,k,g: [T, Dk]; v: [T, Dv]; beta: [T];
    S0: [Dk, Dv].  Returns (o [T, Dv], S_final [Dk, Dv])."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    S = np.array(S0, dtype=np.float64, copy=True)
    T = k.shape[0]
    o = np.zeros((T, v.shape[1]))
    for s in range(0, T, C):
        e = min(s + C, T)
        Q, K, V, G, b = q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e]
        n = e - s
        lam = np.cumsum(G, axis=0)           # log of eq. (3): log gamma^r
        Gam = np.exp(lam)
        Kp, Km, Qp = K * Gam, K / Gam, scale * Q * Gam
        L = np.tril(b[:, None] * (Kp @ Km.T), k=-1)
        Tinv = np.linalg.inv(np.eye(n) + L)  # UT transform, explicit inverse
        U = Tinv @ (b[:, None] * V)
        W = Tinv @ (b[:, None] * Kp)
        Vt = U - W @ S                       # pseudo-values
        A = np.tril(Qp @ Km.T)               # eq. (4), diagonal kept
        o[s:e] = Qp @ S + A @ Vt             # eq. (4)
        S = np.exp(lam[-1])[:, None] * S + (K * np.exp(lam[-1] - lam)).T @ Vt
    return o, S
