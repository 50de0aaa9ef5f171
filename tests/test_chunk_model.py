"""The chunk formulas the kernels use, checked against the oracle in fp64 (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle import SCALAR, DIAG, DELTA, NAIVE, KDA
from segment_scan_amd import synth
from tests import chunk_model


def rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300)


def test_blocked_inverse():
    r = np.random.default_rng(0)
    M = np.tril(r.standard_normal((64, 64)) * 0.1, -1)
    N = chunk_model.blocked_unit_lower_inverse(M)
    np.testing.assert_allclose(N @ (np.eye(64) + M), np.eye(64), atol=1e-12)


def test_in_place_inverse_order():
    """The in-place block order of the kernels (block rows, T before N) gives the inverse."""
    r = np.random.default_rng(1)
    M = np.tril(r.standard_normal((64, 64)) * 0.1, -1)
    N = chunk_model.blocked_inverse_in_place(M)
    np.testing.assert_allclose(N @ (np.eye(64) + M), np.eye(64), atol=1e-12)


def test_two_level_block_inverse():
    """The factor passes' order: each 32 x 32 diagonal block from its two 16 x 16
    diagonal inverses and N_10 = -N_11 (M_10 N_00) at 16, then the same formula
    for the 32 x 32 off-diagonal block."""
    r = np.random.default_rng(2)
    M = np.tril(r.standard_normal((64, 64)) * 0.1, -1)

    def two_by_two(M, h, inv_diag):
        A, C, D = M[:h, :h], M[h:, :h], M[h:, h:]
        N00, N11 = inv_diag(A), inv_diag(D)
        N = np.zeros_like(M)
        N[:h, :h], N[h:, h:] = N00, N11
        N[h:, :h] = -N11 @ (C @ N00)
        return N

    def sub16(A):  # forward substitution, column by column
        n = A.shape[0]
        N = np.zeros((n, n))
        for c in range(n):
            x = np.zeros(n)
            for rr in range(n):
                x[rr] = 0.0 if rr < c else (1.0 if rr == c else -A[rr, :rr] @ x[:rr])
            N[:, c] = x
        return N

    N = two_by_two(M, 32, lambda B: two_by_two(B, 16, sub16))
    np.testing.assert_allclose(N @ (np.eye(64) + M), np.eye(64), atol=1e-12)


def test_weights_on_columns_then_rows():
    """A0 = (I + diag(b) L)^-1 diag(b) equals diag(b) (I + L diag(b))^-1 (L the
    strictly lower Gram), the form the factor passes compute; zero weights
    (tokens past a segment's end) included."""
    r = np.random.default_rng(3)
    K = r.standard_normal((64, 128))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    b = 1.0 / (1.0 + np.exp(-r.standard_normal(64)))
    b[50:] = 0.0
    L = np.tril(K @ K.T, -1)
    B = np.diag(b)
    lhs = np.linalg.inv(np.eye(64) + B @ L) @ B
    rhs = B @ np.linalg.inv(np.eye(64) + L @ B)
    np.testing.assert_allclose(rhs, lhs, atol=1e-12)


@pytest.mark.parametrize("gate_scale", [1.0, 1.0 / 64, 0.0])
@pytest.mark.parametrize("L", [256, 200, 64, 5])
def test_delta_chunked_build_matches_oracle(gate_scale, L):
    tk = synth.gdn_tiny(n_seg=1, L=L, gate_scale=gate_scale)
    g, U, S = oracle.build_pairs(DELTA, tk.offsets, tk.k, tk.v, tk.beta, tk.log_gate)
    gm, Um, Sm = chunk_model.delta_build(tk.k[:, 0], tk.v[:, 0], tk.beta[:, 0],
                                          None if tk.log_gate is None else tk.log_gate[:, 0])
    assert rel(Sm, S[0, 0]) < 1e-11
    assert rel(Um, U[0, 0]) < 1e-11
    assert abs(gm - g[0, 0]) < 1e-10 * max(1, abs(g[0, 0]))


def test_delta_chunk_outputs_match_oracle_seam():
    r = np.random.default_rng(3)
    w, dk = 8, 16
    tk = synth.gdn_tiny(n_seg=1, L=w)
    k = tk.k[:, :, :dk] / np.linalg.norm(tk.k[:, :, :dk], axis=-1, keepdims=True)
    q = r.standard_normal((w, 1, dk))
    v = tk.v[:, :, :dk]
    S0 = r.standard_normal((1, dk, dk))
    res = oracle.seam(DELTA, 1, w, q, k, v, tk.beta, tk.log_gate, S_run=S0)
    S1, _, _, O = chunk_model.delta_chunk(k[:, 0], v[:, 0], tk.beta[:, 0], tk.log_gate[:, 0], S0[0],
                                          np.eye(dk), Q=q[:, 0], blocked=False)
    assert rel(S1, res["S_run"][0]) < 1e-12
    assert rel(O, res["o"][:, 0]) < 1e-12


@pytest.mark.parametrize("fam", [NAIVE, SCALAR, DIAG])
def test_scalar_diag_chunked_build_matches_oracle(fam):
    if fam == DIAG:
        tk = synth.gla(n_seg=1, L=200, n_chain=1, d=32)
        lg = tk.log_gate[:, 0]
    elif fam == SCALAR:
        tk = synth.mamba2_like(n_seg=1, L=200, n_chain=1, d=32)
        lg = tk.log_gate[:, 0]
    else:
        tk = synth.naive(n_seg=1, L=200, n_chain=1, d=32)
        lg = None
    g, _, S = oracle.build_pairs(fam, tk.offsets, tk.k, tk.v, tk.beta, tk.log_gate)
    gm, Sm = chunk_model.scalar_diag_build(tk.k[:, 0], tk.v[:, 0], lg)
    assert rel(Sm, S[0, 0]) < 1e-12
    np.testing.assert_allclose(gm, g[0, 0], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("gate_scale", [1.0, 1.0 / 8, 0.0])
@pytest.mark.parametrize("L", [192, 150, 64, 7])
def test_kda_chunked_build_matches_oracle(gate_scale, L):
    """The KDA chunk form (per-token largest gate as the frame, sub-block Gram
    with reference tokens, decayed key copies) equals the token loop, including
    the split of T into exp(g) U."""
    r = np.random.default_rng(1000 + L)
    dk = dv = 16
    k = r.standard_normal((L, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((L, dv))
    b = 1.0 / (1.0 + np.exp(-r.standard_normal(L)))
    lg = -np.log1p(np.exp(r.standard_normal((L, dk)))) * gate_scale
    g, U, S = oracle.build_pairs(KDA, np.array([0, L], np.int32), k[:, None], v[:, None], b[:, None], lg[:, None])
    gm, Um, Sm = chunk_model.kda_build(k, v, b, lg)
    assert rel(Sm, S[0, 0]) < 1e-11
    assert rel(Um, U[0, 0]) < 1e-11
    assert abs(gm - g[0, 0]) < 1e-12 * max(1.0, abs(g[0, 0]))


@pytest.mark.parametrize("pattern", ["half", "all"])
def test_kda_strong_gates_stay_finite(pattern):
    """Channel gates of -30 per token (on a random half of the entries, or on
    every entry): every factor of the chunk form stays within [0, 1] and the
    chunked build equals the token loop (U of magnitude e^-1000 stays in range
    because the decay is carried by g)."""
    r = np.random.default_rng(5)
    L, dk = 150, 8
    k = r.standard_normal((L, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((L, dk))
    b = np.full(L, 0.5)
    lg = np.full((L, dk), -30.0)
    if pattern == "half":
        lg = lg * (r.random((L, dk)) < 0.5)
    with np.errstate(over="raise", invalid="raise"):
        gm, Um, Sm = chunk_model.kda_build(k, v, b, lg)
    g, U, S = oracle.build_pairs(KDA, np.array([0, L], np.int32), k[:, None], v[:, None], b[:, None], lg[:, None])
    assert np.isfinite(Um).all() and np.isfinite(Sm).all()
    assert rel(Um, U[0, 0]) < 1e-11 and rel(Sm, S[0, 0]) < 1e-11
    assert abs(gm - g[0, 0]) < 1e-12 * abs(g[0, 0]) + 1e-12
