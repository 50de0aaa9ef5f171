"""NumPy model of the chunked algorithms the HIP kernels implement (test aid only).

The kernels do not run token by token: they process 64-token chunks with
matrix products.  This module states those chunk formulas in plain numpy so the
tests can check the algebra against the oracle on the CPU, independently of
any GPU.  It is not imported by the library and the library is not imported
here.

Delta rule (GDN / DeltaNet), one chunk of C tokens with keys K [C, dk], values
V [C, dv], write weights b, log gates a, within-chunk inclusive prefix
G_t = sum_{s<=t} a_s, start state S0 and start transition U0:
    M0    = strict_lower(diag(b) K K^T)
    N     = (I + M0)^-1                        (unit lower triangular)
    A0    = N diag(b)
    Abar  = Gamma o A0,  Gamma_ts = exp(G_t - G_s)  (t >= s)
    U1    = U0 - K^T (A0 (K U0))
    Z     = Abar (V - diag(exp(G)) K S0)
    S1    = exp(G_C) S0 + K^T diag(exp(G_C - G)) Z
    O     = diag(exp(G)) Q S0 + (tril(Q K^T) o Gamma) Z      (seam outputs)
KDA (delta rule with one gate per key channel), one chunk with per-channel
inclusive prefixes G [C, dk], the per-token largest gate summed, mu_t =
sum_{s<=t} max_c lg_sc, and the shifted prefixes H = G - mu (per channel
non-increasing in t, <= 0); H_C, mu_C, G_C are the chunk's last rows:
    M[i,j]  = b_i sum_c k_ic k_jc exp(H_ic - H_jc)   (i > j, every term <= |k_i k_j|)
              block pairs of 32, 16, 8, 4 tokens through keys decayed against
              the token between them (both factors <= |k|), the 4 x 4 diagonal
              blocks term by term
    X       = (I + M)^-1 diag(b)
    Kb      = K o exp(H),  Kd = (K o exp(H_C - H))^T            (both <= |k|)
    U1      = diag(exp(G_C - mu_C)) U0 - Kd X (Kb U0),  g += mu_C   (T = exp(g) U)
    S1      = diag(exp(G_C)) S0 + Kd X (diag(exp(mu_C - mu)) V - exp(mu_C) Kb S0)
Every factor is at most 1 whatever the gates; in the frame diag(exp(-mu)) the
Gram is that of the scalar-gated delta rule with the channel spread left over.
Scalar / diagonal families, per chunk:
    S1    = diag(exp(G_C)) S0 + (K o exp(G_C - G))^T V
"""
from __future__ import annotations

import numpy as np


def blocked_unit_lower_inverse(M, bs=16):
    """(I + M)^-1 for strictly lower M, by 16x16 diagonal blocks (forward
    substitution) and off-diagonal blocks N_ij = -N_ii sum_{k=j}^{i-1} M_ik N_kj."""
    C = M.shape[0]
    nb = C // bs
    N = np.zeros_like(M)
    blk = lambda i: slice(i * bs, (i + 1) * bs)
    for i in range(nb):
        Mi = M[blk(i), blk(i)]
        Ni = np.zeros((bs, bs))
        for r in range(bs):
            Ni[r, r] = 1.0
            for c in range(r):
                Ni[r, c] = -Mi[r, c:r] @ Ni[c:r, c]
        N[blk(i), blk(i)] = Ni
    for i in range(1, nb):
        for j in range(i):
            T = sum(M[blk(i), blk(kk)] @ N[blk(kk), blk(j)] for kk in range(j, i))
            N[blk(i), blk(j)] = -N[blk(i), blk(i)] @ T
    return N


def blocked_inverse_in_place(M, bs=16):
    """The same inverse computed in place in one array, in the order the GPU
    kernels use: diagonal blocks first, then block rows i = 1, 2, ... where all
    T_ij of row i are formed from row i's M blocks before N_ij overwrite them."""
    W = np.array(M, dtype=np.float64)
    nb = W.shape[0] // bs
    blk = lambda i: slice(i * bs, (i + 1) * bs)
    for i in range(nb):
        Mi = W[blk(i), blk(i)].copy()
        Ni = np.zeros((bs, bs))
        for r in range(bs):
            Ni[r, r] = 1.0
            for c in range(r):
                Ni[r, c] = -Mi[r, c:r] @ Ni[c:r, c]
        W[blk(i), blk(i)] = Ni
    for i in range(1, nb):
        T = [sum(W[blk(i), blk(k)] @ W[blk(k), blk(j)] for k in range(j, i)) for j in range(i)]
        for j in range(i):
            W[blk(i), blk(j)] = -W[blk(i), blk(i)] @ T[j]
    return np.tril(W)


def delta_chunk(K, V, b, a, S0, U0, Q=None, blocked=True):
    C = K.shape[0]
    G = np.cumsum(a)
    M0 = np.tril(b[:, None] * (K @ K.T), -1)
    N = blocked_unit_lower_inverse(M0) if (blocked and C % 16 == 0) else np.linalg.inv(np.eye(C) + M0)
    A0 = N * b[None, :]
    Gam = np.tril(np.exp(G[:, None] - G[None, :]))
    Abar = Gam * A0
    U1 = U0 - K.T @ (A0 @ (K @ U0))
    Z = Abar @ (V - np.exp(G)[:, None] * (K @ S0))
    S1 = np.exp(G[-1]) * S0 + K.T @ (np.exp(G[-1] - G)[:, None] * Z)
    O = None
    if Q is not None:
        O = np.exp(G)[:, None] * (Q @ S0) + (np.tril(Q @ K.T) * Gam) @ Z
    return S1, U1, G[-1], O


def delta_build(k, v, b, a, C=64):
    """Chunked build of one unit: k [L, dk], v [L, dv]; tail chunk zero-padded."""
    L, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv))
    U = np.eye(dk)
    g = 0.0
    for c0 in range(0, L, C):
        n = min(C, L - c0)
        K = np.zeros((C, dk)); K[:n] = k[c0:c0 + n]
        V = np.zeros((C, dv)); V[:n] = v[c0:c0 + n]
        bb = np.zeros(C); bb[:n] = b[c0:c0 + n]
        aa = np.zeros(C)
        if a is not None:
            aa[:n] = a[c0:c0 + n]
        S, U, gc, _ = delta_chunk(K, V, bb, aa, S, U)
        g += gc
    return g, U, S


def scalar_diag_build(k, v, lg, C=64):
    """Chunked build for scalar (lg [L]) or diagonal (lg [L, dk]) gates, or naive (lg None)."""
    L, dk = k.shape
    S = np.zeros((dk, v.shape[1]))
    g = np.zeros(dk) if (lg is not None and lg.ndim == 2) else 0.0
    for c0 in range(0, L, C):
        K = k[c0:c0 + C]
        V = v[c0:c0 + C]
        if lg is None:
            S = S + K.T @ V
            continue
        A = lg[c0:c0 + C]
        G = np.cumsum(A, axis=0)
        GC = G[-1]
        W = np.exp(GC - G)
        Kt = K * (W if W.ndim == 2 else W[:, None])
        S = (np.exp(GC)[:, None] if np.ndim(GC) == 1 else np.exp(GC)) * S + Kt.T @ V
        g = g + GC
    return g, S


def kda_gram(K, b, H):
    """Strictly lower M[i,j] = b_i sum_c k_ic k_jc exp(H_ic - H_jc) as the kernels form it:
    hierarchically, block pairs of size s = 32, 16, 8, 4 (rows s..2s-1 against columns
    0..s-1 of every 2s-token block) through keys decayed against the reference token
    2s*a + s - 1 between them (both factors <= |k|), and the sixteen 4 x 4 diagonal
    blocks term by term."""
    C = K.shape[0]
    M = np.zeros((C, C))
    for s in (32, 16, 8, 4):
        for a0 in range(0, C, 2 * s):
            r = a0 + s - 1
            rows = slice(a0 + s, a0 + 2 * s)
            cols = slice(a0, a0 + s)
            Kb = K[rows] * np.exp(H[rows] - H[r])
            Ka = K[cols] * np.exp(H[r] - H[cols])
            M[rows, cols] = b[rows, None] * (Kb @ Ka.T)
    for b0 in range(0, C, 4):
        for i in range(b0, b0 + 4):
            for j in range(b0, i):
                M[i, j] = b[i] * np.sum(K[i] * K[j] * np.exp(H[i] - H[j]))
    return M


def kda_chunk(K, V, b, LG, S0, U0):
    G = np.cumsum(LG, axis=0)
    mu = np.cumsum(LG.max(axis=1))
    H = G - mu[:, None]
    GC, HC, muC = G[-1], H[-1], mu[-1]
    X = blocked_unit_lower_inverse(kda_gram(K, b, H)) * b[None, :]
    Kb = K * np.exp(H)
    Kd = (K * np.exp(HC - H)).T
    U1 = np.exp(GC - muC)[:, None] * U0 - Kd @ (X @ (Kb @ U0))
    S1 = np.exp(GC)[:, None] * S0 + Kd @ (X @ (np.exp(muC - mu)[:, None] * V - np.exp(muC) * (Kb @ S0)))
    return S1, U1, muC


def kda_build(k, v, b, lg, C=64):
    """Chunked KDA build of one unit: k [L, dk], v [L, dv], b [L], lg [L, dk]; tail zero-padded."""
    L, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv))
    U = np.eye(dk)
    g = 0.0
    for c0 in range(0, L, C):
        n = min(C, L - c0)
        K = np.zeros((C, dk)); K[:n] = k[c0:c0 + n]
        V = np.zeros((C, dv)); V[:n] = v[c0:c0 + n]
        bb = np.zeros(C); bb[:n] = b[c0:c0 + n]
        LG = np.zeros((C, dk)); LG[:n] = lg[c0:c0 + n]
        S, U, m = kda_chunk(K, V, bb, LG, S, U)
        g += m
    return g, U, S
