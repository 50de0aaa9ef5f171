"""Brute-force matrix products on tiny inputs, written independently of the oracle.

The oracle applies each token as an operator to a running state.  This module
instead forms every per-token transition A_t as an explicit d_k x d_k matrix and
evaluates the closed sums

    T_C    = A_L A_{L-1} ... A_1
    S(C|0) = sum_t (A_L ... A_{t+1}) b_t k_t v_t^T

with numpy matrix products, which is the definition of the segment pair on the
youleyou.com page "小红书联合北大上交提出HYPIC，位置无关缓存降低首token延迟3.25倍"
(linear-layer paragraph: T_C is the product of all per-token transition
matrices; S(C|0) is the final state from a zero start).  Only for tiny shapes.
"""
from __future__ import annotations

import numpy as np

NAIVE, SCALAR, DIAG, DELTA, KDA = 0, 1, 2, 3, 4


def token_matrix(fam, k, beta=None, lg=None, lgv=None):
    """Explicit A_t and write weight b_t for one token (k: [dk])."""
    dk = k.shape[0]
    eye = np.eye(dk)
    if fam == NAIVE:
        return eye, 1.0
    if fam == SCALAR:
        return np.exp(lg) * eye, 1.0
    if fam == DIAG:
        return np.diag(np.exp(lgv)), 1.0
    if fam == KDA:  # erase after the per-channel decay
        return (eye - beta * np.outer(k, k)) @ np.diag(np.exp(lgv)), beta
    a = 1.0 if lg is None else np.exp(lg)
    return a * (eye - beta * np.outer(k, k)), beta


def unit_matrices(fam, k, beta, log_gate, gate_per_chain, t0, t1, h):
    mats = []
    for t in range(t0, t1):
        kt = k[t, h]
        if fam == SCALAR:
            lg = log_gate[h] if gate_per_chain else log_gate[t, h]
            mats.append(token_matrix(fam, kt, lg=lg))
        elif fam == DIAG:
            mats.append(token_matrix(fam, kt, lgv=log_gate[t, h]))
        elif fam == DELTA:
            lg = None if log_gate is None else log_gate[t, h]
            mats.append(token_matrix(fam, kt, beta=beta[t, h], lg=lg))
        elif fam == KDA:
            mats.append(token_matrix(fam, kt, beta=beta[t, h], lgv=log_gate[t, h]))
        else:
            mats.append(token_matrix(fam, kt))
    return mats


def brute_pair(fam, k, v, beta, log_gate, gate_per_chain, t0, t1, h):
    """(T_C dense, S(C|0)) of tokens t0..t1-1 of chain h by explicit products."""
    mats = unit_matrices(fam, k, beta, log_gate, gate_per_chain, t0, t1, h)
    dk = k.shape[2]
    n = len(mats)
    # suffix[t] = A_{n-1} ... A_{t+1}  (product of the matrices after token t)
    suffix = [None] * n
    acc = np.eye(dk)
    for t in range(n - 1, -1, -1):
        suffix[t] = acc.copy()
        acc = acc @ mats[t][0]
    T = acc
    S = np.zeros((dk, v.shape[2]))
    for t in range(n):
        A_after = suffix[t]
        b = mats[t][1]
        S += A_after @ (b * np.outer(k[t0 + t, h], v[t0 + t, h]))
    return T, S


def brute_build(fam, offsets, k, v, beta=None, log_gate=None, gate_per_chain=False):
    n_seg = len(offsets) - 1
    n_chain = k.shape[1]
    dk, dv = k.shape[2], v.shape[2]
    T = np.zeros((n_seg, n_chain, dk, dk))
    S = np.zeros((n_seg, n_chain, dk, dv))
    for s in range(n_seg):
        for h in range(n_chain):
            T[s, h], S[s, h] = brute_pair(fam, k, v, beta, log_gate, gate_per_chain,
                                          int(offsets[s]), int(offsets[s + 1]), h)
    return T, S


def brute_outputs(fam, q, k, v, beta, log_gate, gate_per_chain, h, S0):
    """o_t = S_t^T q_t with S_t = (A_t..A_1) S0 + S(1..t | 0), each by explicit products."""
    n = k.shape[0]
    outs = []
    for t in range(1, n + 1):
        T, S = brute_pair(fam, k, v, beta, log_gate, gate_per_chain, 0, t, h)
        St = T @ S0 + S
        outs.append(St.T @ q[t - 1, h])
    return np.stack(outs)
