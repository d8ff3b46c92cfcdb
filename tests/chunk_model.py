"""Chunkwise WY/UT-form model of the delta rule in numpy fp64 (test-only).

This is neither the oracle nor the GPU path: it writes out, in plain numpy,
the chunk algebra that the HIP kernels implement, so that a test can show that
the algebra itself equals the token-by-token oracle for any chunk size before
any kernel is trusted.

Chunk form (Parallelizing Linear Transformers with the Delta Rule over
Sequence Length: products of Householder-like transitions written in WY form,
page 3 abstract; the UT transform T = (I + A)^-1 diag(beta) named in the
Gated DeltaNet review thread, review 2 "Strengths"; gating inside a chunk by
cumulative decay products, page 1 answer W2).  With h = S^T (d_k x d_v), a
chunk of rows r = 1..L, b = cumsum(g) inside the chunk, gamma = exp(b),
Gamma_rj = exp(b_r - b_j) for j <= r:

    A   = strictLower(diag(beta) (K K^T) * Gamma)
    R   = (I + A)^-1,   T = R diag(beta)
    X   = V - diag(gamma) K h
    V'  = T X                                   (the per-token deltas)
    O   = diag(gamma) Q h + ((Q K^T) * Gamma) V'
    h+  = gamma_L h + Khat^T V',   Khat_r = exp(b_L - b_r) k_r
"""
from __future__ import annotations

import numpy as np


def _gates(g, L):
    b = np.cumsum(g) if g is not None else np.zeros(L)
    gam = np.exp(b)
    low = np.tril(np.ones((L, L)))
    Gam = np.exp((b[:, None] - b[None, :]) * low) * low
    return b, gam, Gam


def forward_substitution(A):
    """R = (I + A)^-1 for strictly lower-triangular A, row by row:
    R_r = e_r - sum_{j<r} A_rj R_j."""
    L = A.shape[0]
    R = np.zeros_like(A)
    for r in range(L):
        R[r] = -A[r, :r] @ R[:r]
        R[r, r] += 1.0
    return R


def chunk_prep(K, beta, g):
    L = K.shape[0]
    b, gam, Gam = _gates(g, L)
    A = np.tril(beta[:, None] * (K @ K.T) * Gam, -1)
    R = forward_substitution(A)
    return b, gam, Gam, A, R


def fwd_seq(q, k, v, beta, g, h0, C):
    """One sequence of one head.  q,k [T,Dk], v [T,Dv], beta,g [T], h0 [Dk,Dv].
    Returns o [T,Dv], hT [Dk,Dv] and the chunk-start states."""
    T, Dk = k.shape
    Dv = v.shape[1]
    h = np.zeros((Dk, Dv)) if h0 is None else np.array(h0, dtype=np.float64)
    o = np.zeros((T, Dv))
    states = []
    for s in range(0, T, C):
        e = min(s + C, T)
        Q, K, V, bt = q[s:e], k[s:e], v[s:e], beta[s:e]
        gg = None if g is None else g[s:e]
        b, gam, Gam, A, R = chunk_prep(K, bt, gg)
        states.append(h.copy())
        Tm = R * bt[None, :]
        X = V - gam[:, None] * (K @ h)
        Vp = Tm @ X
        P = (Q @ K.T) * Gam
        o[s:e] = gam[:, None] * (Q @ h) + P @ Vp
        Khat = np.exp(b[-1] - b)[:, None] * K
        h = gam[-1] * h + Khat.T @ Vp
    return o, h, states


def bwd_seq(q, k, v, beta, g, h0, dO, dhT, C):
    """Gradients of <dO, o> + <dhT, hT> for one sequence of one head, by the
    chunk algebra in reverse.  Returns dq, dk, dv, dbeta, dg (None if
    ungated), dh0."""
    T, Dk = k.shape
    Dv = v.shape[1]
    _, _, states = fwd_seq(q, k, v, beta, g, h0, C)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dbeta = np.zeros(T)
    dg = np.zeros(T)
    dh = np.zeros((Dk, Dv)) if dhT is None else np.array(dhT, dtype=np.float64)
    starts = list(range(0, T, C))
    for ci in reversed(range(len(starts))):
        s = starts[ci]
        e = min(s + C, T)
        L = e - s
        h = states[ci]
        Q, K, V, bt, dOc = q[s:e], k[s:e], v[s:e], beta[s:e], dO[s:e]
        gg = None if g is None else g[s:e]
        b, gam, Gam, A, R = chunk_prep(K, bt, gg)
        Tm = R * bt[None, :]
        KK = K @ K.T
        QK = Q @ K.T
        X = V - gam[:, None] * (K @ h)
        Vp = Tm @ X
        P = QK * Gam
        wC = np.exp(b[-1] - b)
        Khat = wC[:, None] * K
        # O = diag(gam) Q h + P V' ;  h+ = gam_L h + Khat^T V'
        dVp = P.T @ dOc + Khat @ dh
        dX = Tm.T @ dVp
        dP = (dOc @ Vp.T) * np.tril(np.ones((L, L)))
        dT = dVp @ X.T
        dR = dT * bt[None, :]
        dA = np.tril(-(R.T @ dR @ R.T), -1)
        dKhat = Vp @ dh.T
        dQc = gam[:, None] * (dOc @ h.T) + (dP * Gam) @ K
        F = dA * Gam * bt[:, None]
        dKc = ((dP * Gam).T @ Q - gam[:, None] * (dX @ h.T) + wC[:, None] * dKhat
               + F @ K + F.T @ K)
        dbc = (R * dT).sum(0) + (dA * Gam * KK).sum(1)
        # gate: b enters through gam (O, X), Gamma (P, A), Khat, gam_L (h+)
        db = gam * (dOc * (Q @ h)).sum(1) - gam * (dX * (K @ h)).sum(1)
        E = dP * QK * Gam + dA * bt[:, None] * KK * Gam
        db += E.sum(1) - E.sum(0)
        w = (dKhat * Khat).sum(1)
        db -= w
        db[-1] += w.sum() + gam[-1] * (dh * h).sum()
        dq[s:e] = dQc
        dk[s:e] = dKc
        dv[s:e] = dX
        dbeta[s:e] = dbc
        dg[s:e] = np.cumsum(db[::-1])[::-1]
        dh = gam[-1] * dh + Q.T @ (gam[:, None] * dOc) - K.T @ (gam[:, None] * dX)
    return dq, dk, dv, dbeta, (dg if g is not None else None), dh
