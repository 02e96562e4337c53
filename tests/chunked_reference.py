"""Independent fp64 NumPy implementation of KDA in chunked form (test helper).

This is the chunk-parallel formulation that the primer attributes to FlashKDA
(bayesiansapien wiki page, section 2 "FlashKDA's complexity": per-chunk
cumulative decay, decayed Q/K, the inverse (I+L)^-1 by a Neumann factorisation,
a causal mask, then a chunk-level recurrence).  It is written from the
derivation below, not from the oracle, and is used to pin the oracle: both must
agree to rounding for every chunk size.

Within one chunk with rows r = 1..C, start state S0, and G_r = sum_{i<=r} g_i
(per key channel):

    S_r = Diag(e^{G_r}) S0 + sum_{j<=r} Diag(e^{G_r - G_j}) k_j u_j^T
    u_r = beta_r (v_r - S'_r^T k_r)
=>  (I + A) U = Diag(beta) (V - Ktil S0),  A_rj = beta_r Ktil_r . Khat_j  (j < r)
    with Ktil = k * e^{G}, Khat = k * e^{-G}, Qtil = q * e^{G}
    U  = T V - T Ktil S0,                   T = (I + A)^{-1} Diag(beta)
    O  = Qtil S0 + tril(Qtil Khat^T) U      (diagonal included)
    S_C = Diag(e^{G_C}) S0 + Kend^T U,      Kend = k * e^{G_C - G}

A is strictly lower triangular, hence nilpotent, so (I + A)^{-1} is also the
finite Neumann series sum_n (-A)^n = prod_i (I + (-A)^{2^i}).
"""
from __future__ import annotations

import numpy as np


def inverse_unit_lower(A: np.ndarray, method: str) -> np.ndarray:
    """(I + A)^{-1} for strictly lower-triangular A."""
    n = A.shape[0]
    eye = np.eye(n)
    if method == "solve":
        return np.linalg.solve(eye + A, eye)
    if method == "neumann":
        # prod_{i} (I + (-A)^{2^i}) until the power vanishes (2^i >= n).
        result = eye.copy()
        P = -A
        span = 1
        while span < n:
            result = result @ (eye + P)
            P = P @ P
            span *= 2
        return result
    raise ValueError(method)


def chunked_prefill(q, k, v, g, beta, S0=None, C=64, method="solve"):
    """Chunked KDA over [B,T,H,.] fp64 inputs; returns (o, S_T)."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for r0 in range(0, T, C):
                r1 = min(T, r0 + C)
                qc, kc, vc, gc = q[b, r0:r1, h], k[b, r0:r1, h], v[b, r0:r1, h], g[b, r0:r1, h]
                bc = beta[b, r0:r1, h]
                G = np.cumsum(gc, axis=0)
                Qt, Kt, Kh = qc * np.exp(G), kc * np.exp(G), kc * np.exp(-G)
                Kend = kc * np.exp(G[-1][None, :] - G)
                A = np.tril(bc[:, None] * (Kt @ Kh.T), -1)
                Tm = inverse_unit_lower(A, method) @ np.diag(bc)
                U = Tm @ vc - (Tm @ Kt) @ S
                o[b, r0:r1, h] = Qt @ S + np.tril(Qt @ Kh.T) @ U
                S = np.exp(G[-1])[:, None] * S + Kend.T @ U
            S_T[b, h] = S
    return o, S_T
