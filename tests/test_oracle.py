"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these tests retypes the oracle's formula: each compares it with a
different computation (explicit matrix products, a closed form, a straight
recurrence over the concatenation, an algebraic invariant) or with a number
the pages print.  Pages: youleyou.com "小红书联合北大上交提出HYPIC，位置无关缓存降低首token延迟3.25倍"
(linear-layer and full-attention paragraphs) and llm-wiki.hwlabs.dev
"HYPIC: 하이브리드 어텐션 LLM 서빙에서 ..." (section 세그먼트 누적 전이 연산자).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import NAIVE, SCALAR, DIAG, DELTA, KDA, DENSE
from tests import brute

FAMS = [NAIVE, SCALAR, DIAG, DELTA, KDA]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 1e-300 else 1.0)


def rand_tokens(fam, n_tok, n_chain, dk, dv, seed, gate_scale=1.0, delta_gate=True, unit_keys=True):
    r = np.random.default_rng(seed)
    k = r.standard_normal((n_tok, n_chain, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((n_tok, n_chain, dv))
    q = r.standard_normal((n_tok, n_chain, dk))
    beta = None
    lg = None
    if fam == SCALAR:
        lg = -np.abs(r.standard_normal((n_tok, n_chain))) * 0.3 * gate_scale
    elif fam == DIAG:
        lg = -np.abs(r.standard_normal((n_tok, n_chain, dk))) * 0.3 * gate_scale
    elif fam == DELTA:
        beta = 1.0 / (1.0 + np.exp(-r.standard_normal((n_tok, n_chain))))
        if delta_gate:
            lg = -np.abs(r.standard_normal((n_tok, n_chain))) * 0.3 * gate_scale
    elif fam == KDA:
        beta = 1.0 / (1.0 + np.exp(-r.standard_normal((n_tok, n_chain))))
        lg = -np.abs(r.standard_normal((n_tok, n_chain, dk))) * 0.3 * gate_scale
    return dict(q=q, k=k, v=v, beta=beta, log_gate=lg)


# ---------------------------------------------------------------- brute force


@pytest.mark.parametrize("fam", FAMS)
@pytest.mark.parametrize("dk,dv", [(2, 3), (4, 4), (8, 5)])
def test_build_matches_brute_force_products(fam, dk, dv):
    offsets = np.array([0, 5, 6, 16], np.int32)  # ragged, includes a 1-token segment
    x = rand_tokens(fam, 16, 2, dk, dv, seed=100 + 10 * fam + dk)
    g, U, S = oracle.build_pairs(fam, offsets, x["k"], x["v"], x["beta"], x["log_gate"])
    Tb, Sb = brute.brute_build(fam, offsets, x["k"], x["v"], x["beta"], x["log_gate"])
    T = oracle.transition_dense(fam, g, U, dk)
    assert rel(T, Tb) < 1e-13
    assert rel(S, Sb) < 1e-13


def test_build_matches_brute_force_retnet_per_chain_gate():
    r = np.random.default_rng(7)
    k = r.standard_normal((12, 3, 4))
    v = r.standard_normal((12, 3, 4))
    lg = np.log(np.array([0.5, 0.9, 0.999]))
    offsets = np.array([0, 4, 12], np.int32)
    g, U, S = oracle.build_pairs(SCALAR, offsets, k, v, None, lg, gate_per_chain=True)
    Tb, Sb = brute.brute_build(SCALAR, offsets, k, v, None, lg, gate_per_chain=True)
    assert rel(oracle.transition_dense(SCALAR, g, U, 4), Tb) < 1e-13
    assert rel(S, Sb) < 1e-13
    # g is L * log(gamma) per chain
    np.testing.assert_allclose(g, np.array([[4], [8]]) * lg[None, :], rtol=1e-14)


@pytest.mark.parametrize("fam", FAMS)
def test_seam_outputs_match_brute_force(fam):
    dk = dv = 4
    n_seg, w = 3, 2
    x = rand_tokens(fam, n_seg * w, 2, dk, dv, seed=300 + fam)
    S0 = np.random.default_rng(5).standard_normal((2, dk, dv))
    res = oracle.seam(fam, n_seg, w, x["q"], x["k"], x["v"], x["beta"], x["log_gate"], S_run=S0)
    for h in range(2):
        ob = brute.brute_outputs(fam, x["q"], x["k"], x["v"], x["beta"], x["log_gate"], False, h, S0[h])
        assert rel(res["o"][:, h], ob) < 1e-13


# ------------------------------------------------------- composition law


@pytest.mark.parametrize("fam", FAMS)
@pytest.mark.parametrize("with_init", [False, True])
def test_composition_equals_sequential_recurrence(fam, with_init):
    """Build + ordered compose over any split = straight recurrence over the concatenation."""
    dk, dv, n_chain = 6, 5, 3
    offsets = np.array([0, 7, 8, 20, 33, 40], np.int32)
    x = rand_tokens(fam, 40, n_chain, dk, dv, seed=11 + fam)
    S0 = np.random.default_rng(3).standard_normal((n_chain, dk, dv)) if with_init else None
    g, U, S = oracle.build_pairs(fam, offsets, x["k"], x["v"], x["beta"], x["log_gate"])
    c = oracle.compose(fam, g, U, S, S_init=S0, want_prefix=True, want_total=True)
    Sseq, _ = oracle.sequential(fam, x["k"], x["v"], x["beta"], x["log_gate"], S_init=S0)
    assert rel(c["S_out"], Sseq) < 1e-12
    # prefix state i = recurrence over tokens [0, offsets[i])
    for i in range(1, len(offsets) - 1):
        sl = slice(0, offsets[i])
        Sp, _ = oracle.sequential(fam, x["k"][sl], x["v"][sl],
                                  None if x["beta"] is None else x["beta"][sl],
                                  None if x["log_gate"] is None else x["log_gate"][sl], S_init=S0)
        assert rel(c["prefix"][i], Sp) < 1e-12
    # total transition = pair built over the whole concatenation
    gw, Uw, Sw = oracle.build_pairs(fam, np.array([0, 40], np.int32), x["k"], x["v"], x["beta"], x["log_gate"])
    T_tot = oracle.transition_dense(fam, c["g_tot"], c["U_tot"], dk)
    assert rel(T_tot, oracle.transition_dense(fam, gw[0], None if Uw is None else Uw[0], dk)) < 1e-12


def test_three_segment_expansion():
    """e_ABC = T_C (T_B e_A + e_B) + e_C and T_ABC = T_C T_B T_A, evaluated by hand."""
    dk = dv = 5
    x = rand_tokens(DELTA, 30, 1, dk, dv, seed=21)
    offsets = np.array([0, 9, 20, 30], np.int32)
    g, U, S = oracle.build_pairs(DELTA, offsets, x["k"], x["v"], x["beta"], x["log_gate"])
    T = oracle.transition_dense(DELTA, g, U, dk)[:, 0]
    e = S[:, 0]
    e_abc = T[2] @ (T[1] @ e[0] + e[1]) + e[2]
    T_abc = T[2] @ T[1] @ T[0]
    c = oracle.compose(DELTA, g, U, S, want_total=True)
    assert rel(c["S_out"][0], e_abc) < 1e-13
    assert rel(oracle.transition_dense(DELTA, c["g_tot"], c["U_tot"], dk)[0], T_abc) < 1e-13


@pytest.mark.parametrize("fam", FAMS)
def test_associativity_and_identity(fam):
    dk = dv = 4
    x = rand_tokens(fam, 24, 2, dk, dv, seed=31 + fam)
    offsets = np.array([0, 5, 14, 24], np.int32)
    g, U, S = oracle.build_pairs(fam, offsets, x["k"], x["v"], x["beta"], x["log_gate"])
    sel = lambda a, i: None if a is None else a[i]
    # (p0 p1) p2
    c01 = oracle.compose(fam, g[:2], sel(U, slice(0, 2)), S[:2], want_total=True)
    left = oracle.compose(fam, np.stack([c01["g_tot"], g[2]]),
                          None if U is None else np.stack([c01["U_tot"], U[2]]),
                          np.stack([c01["S_out"], S[2]]), want_total=True)
    # p0 (p1 p2)
    c12 = oracle.compose(fam, g[1:], sel(U, slice(1, 3)), S[1:], want_total=True)
    right = oracle.compose(fam, np.stack([g[0], c12["g_tot"]]),
                           None if U is None else np.stack([U[0], c12["U_tot"]]),
                           np.stack([S[0], c12["S_out"]]), want_total=True)
    assert rel(left["S_out"], right["S_out"]) < 1e-13
    if fam in DENSE:
        assert rel(left["U_tot"], right["U_tot"]) < 1e-13
    np.testing.assert_allclose(left["g_tot"], right["g_tot"], rtol=1e-14, atol=1e-15)
    # identity pair (T = I, S = 0) leaves the state unchanged
    gl = oracle.gate_len(fam, dk)
    gi = np.zeros((1, 2) + ((dk,) if gl > 1 else ()))
    Ui = np.broadcast_to(np.eye(dk), (1, 2, dk, dk)).copy() if fam in DENSE else None
    Si = np.zeros((1, 2, dk, dv))
    St = np.random.default_rng(1).standard_normal((2, dk, dv))
    out = oracle.compose(fam, gi, Ui, Si, S_init=St)
    np.testing.assert_array_equal(out["S_out"], St)


@pytest.mark.parametrize("fam", FAMS)
def test_superposition_in_initial_state(fam):
    """S(C | S0) = T_C S0 + S(C | 0): the pair does not depend on the prefix."""
    dk, dv = 5, 4
    x = rand_tokens(fam, 17, 2, dk, dv, seed=41 + fam)
    S0 = np.random.default_rng(9).standard_normal((2, dk, dv))
    g, U, S = oracle.build_pairs(fam, np.array([0, 17], np.int32), x["k"], x["v"], x["beta"], x["log_gate"])
    T = oracle.transition_dense(fam, g, U, dk)[0]
    Sseq, _ = oracle.sequential(fam, x["k"], x["v"], x["beta"], x["log_gate"], S_init=S0)
    assert rel(Sseq, np.einsum("hij,hjk->hik", T, S0) + S[0]) < 1e-13


# ----------------------------------------------------------- special cases


def test_naive_plain_addition_is_exact():
    """With T = I, composing is plain addition -- bit for bit in the oracle."""
    dk = dv = 6
    x = rand_tokens(NAIVE, 20, 2, dk, dv, seed=51)
    g, U, S = oracle.build_pairs(NAIVE, np.array([0, 8, 20], np.int32), x["k"], x["v"])
    np.testing.assert_array_equal(g, 0.0)
    c = oracle.compose(NAIVE, g, U, S)
    np.testing.assert_array_equal(c["S_out"], S[0] + S[1])
    Sseq, _ = oracle.sequential(NAIVE, x["k"], x["v"])
    assert rel(Sseq, S[0] + S[1]) < 1e-14


def test_scalar_closed_form():
    """T_C = gamma^L, S = sum_t gamma^(L-t) k_t v_t^T."""
    r = np.random.default_rng(61)
    L, dk, dv = 37, 5, 3
    k = r.standard_normal((L, 2, dk))
    v = r.standard_normal((L, 2, dv))
    gam = np.array([0.9, 0.999])
    g, U, S = oracle.build_pairs(SCALAR, np.array([0, L], np.int32), k, v, None, np.log(gam), gate_per_chain=True)
    w = gam[None, :] ** (L - 1 - np.arange(L))[:, None]  # [L, chain]
    S_cf = np.einsum("th,thi,thj->hij", w, k, v)
    assert rel(S[0], S_cf) < 1e-13
    np.testing.assert_allclose(np.exp(g[0]), gam ** L, rtol=1e-12)


def test_diag_closed_form():
    """Row i of S = sum_t exp(sum_{s>t} log a_s[i]) k_t[i] v_t^T; T_C = diag(exp(sum log a))."""
    r = np.random.default_rng(71)
    L, dk, dv = 23, 6, 4
    k = r.standard_normal((L, 1, dk))
    v = r.standard_normal((L, 1, dv))
    lg = -np.abs(r.standard_normal((L, 1, dk))) * 0.2
    g, U, S = oracle.build_pairs(DIAG, np.array([0, L], np.int32), k, v, None, lg)
    suff = np.concatenate([np.cumsum(lg[::-1, 0], axis=0)[::-1][1:], np.zeros((1, dk))])  # sum_{s>t}
    S_cf = np.einsum("ti,ti,tj->ij", np.exp(suff), k[:, 0], v[:, 0])
    assert rel(S[0, 0], S_cf) < 1e-13
    np.testing.assert_allclose(g[0, 0], lg[:, 0].sum(axis=0), rtol=1e-13)


def test_delta_one_token():
    """One token: T = alpha (I - beta k k^T), S = beta k v^T."""
    r = np.random.default_rng(81)
    dk, dv = 7, 5
    k = r.standard_normal((1, 1, dk))
    v = r.standard_normal((1, 1, dv))
    beta = np.array([[0.37]])
    lg = np.array([[-0.25]])
    g, U, S = oracle.build_pairs(DELTA, np.array([0, 1], np.int32), k, v, beta, lg)
    T = oracle.transition_dense(DELTA, g, U, dk)[0, 0]
    kk = k[0, 0]
    np.testing.assert_allclose(T, np.exp(-0.25) * (np.eye(dk) - 0.37 * np.outer(kk, kk)), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S[0, 0], 0.37 * np.outer(kk, v[0, 0]), rtol=1e-14, atol=1e-15)


def test_delta_overwrite_retrieval():
    """alpha = 1, beta = 1, unit key written twice: reading the key returns the last value."""
    r = np.random.default_rng(91)
    dk, dv = 8, 6
    key = r.standard_normal(dk)
    key /= np.linalg.norm(key)
    v1, v2 = r.standard_normal(dv), r.standard_normal(dv)
    k = np.stack([key, key])[:, None]
    v = np.stack([v1, v2])[:, None]
    beta = np.ones((2, 1))
    g, U, S = oracle.build_pairs(DELTA, np.array([0, 2], np.int32), k, v, beta, None)
    np.testing.assert_allclose(S[0, 0].T @ key, v2, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(g, 0.0)


def test_householder_limit_is_orthogonal():
    """beta = 2 with unit keys makes every factor a reflection, so U is orthogonal."""
    r = np.random.default_rng(101)
    dk = 9
    L = 25
    k = r.standard_normal((L, 1, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((L, 1, dk))
    beta = np.full((L, 1), 2.0)
    g, U, S = oracle.build_pairs(DELTA, np.array([0, L], np.int32), k, v, beta, None)
    Uu = U[0, 0]
    np.testing.assert_allclose(Uu.T @ Uu, np.eye(dk), atol=1e-13)
    # beta in [0, 2] keeps the spectral norm at most 1
    beta2 = r.uniform(0, 2, (L, 1))
    _, U2, _ = oracle.build_pairs(DELTA, np.array([0, L], np.int32), k, v, beta2, None)
    assert np.linalg.norm(U2[0, 0], 2) <= 1.0 + 1e-13


# ------------------------------------------------ naive-addition error size


def test_naive_addition_error_closed_form():
    """Scalar family: ||(S1 + S2) - (T2 S1 + S2)|| = (1 - gamma^L2) ||S1||, exactly."""
    r = np.random.default_rng(111)
    L1, L2, dk = 40, 25, 4
    k = r.standard_normal((L1 + L2, 1, dk))
    v = r.standard_normal((L1 + L2, 1, dk))
    gam = 0.97
    g, U, S = oracle.build_pairs(SCALAR, np.array([0, L1, L1 + L2], np.int32), k, v, None,
                                 np.log([gam]), gate_per_chain=True)
    true = oracle.compose(SCALAR, g, U, S)["S_out"][0]
    naive_sum = S[0, 0] + S[1, 0]
    err = np.linalg.norm(naive_sum - true)
    np.testing.assert_allclose(err, (1 - gam ** L2) * np.linalg.norm(S[0, 0]), rtol=1e-12)


def test_naive_addition_error_matches_pages_22_percent():
    """The pages: dropping T(C2) on a slow-decay RetNet head costs 22 % of the state
    norm at 256 tokens [youleyou, linear-layer paragraph].  Reconstruction: the
    slowest decay RetNet's schedule uses, gamma = 1 - 2^-10 (see the fixture)."""
    with open(os.path.join(GOLDEN, "naive_addition_retnet.json")) as f:
        fx = json.load(f)
    gam = fx["gamma"]
    L1, L2 = fx["L1"], fx["L2"]
    r = np.random.default_rng(fx["seed"])
    dk = fx["d"]
    k = r.standard_normal((L1 + L2, 1, dk)) / np.sqrt(dk)
    v = r.standard_normal((L1 + L2, 1, dk)) / np.sqrt(dk)
    g, U, S = oracle.build_pairs(SCALAR, np.array([0, L1, L1 + L2], np.int32), k, v, None,
                                 np.log([gam]), gate_per_chain=True)
    true = oracle.compose(SCALAR, g, U, S)["S_out"][0]
    frac = np.linalg.norm(S[0, 0] + S[1, 0] - true) / np.linalg.norm(S[0, 0])
    assert abs(frac - fx["pages_fraction"]) <= fx["tolerance"], frac


def test_kda_with_equal_channel_gates_is_gdn():
    """KDA whose gate is the same on every channel is the gated delta rule: the
    scalar gate commutes with the erase factor."""
    dk, dv = 6, 5
    x = rand_tokens(DELTA, 19, 2, dk, dv, seed=4300)
    lgv = np.repeat(x["log_gate"][:, :, None], dk, axis=2)
    off = np.array([0, 7, 19], np.int32)
    gd, Ud, Sd = oracle.build_pairs(DELTA, off, x["k"], x["v"], x["beta"], x["log_gate"])
    gk, Uk, Sk = oracle.build_pairs(KDA, off, x["k"], x["v"], x["beta"], lgv)
    assert rel(Sk, Sd) < 1e-13
    assert rel(oracle.transition_dense(KDA, gk, Uk, dk), oracle.transition_dense(DELTA, gd, Ud, dk)) < 1e-13
    np.testing.assert_allclose(gk, gd, rtol=1e-13)  # the largest channel gate is the gate


def test_kda_without_erase_is_gla():
    """beta -> 0 removes the erase and the write: T is the diagonal family's diag(exp(sum lg));
    with keys orthogonal to each other the erase of one token does not touch the others'
    writes, so S is the diagonal family's state with values scaled by beta."""
    dk, dv = 4, 3
    x = rand_tokens(KDA, 4, 1, dk, dv, seed=4301)
    off = np.array([0, 4], np.int32)
    beta0 = np.zeros_like(x["beta"])
    g, U, S = oracle.build_pairs(KDA, off, x["k"], x["v"], beta0, x["log_gate"])
    gd, _, _ = oracle.build_pairs(DIAG, off, x["k"], x["v"], None, x["log_gate"])
    assert rel(oracle.transition_dense(KDA, g, U, dk), oracle.transition_dense(DIAG, gd, None, dk)) < 1e-14
    assert np.abs(S).max() == 0.0
    # orthonormal keys (one basis vector per token): the erase of token t only
    # touches channel t, which holds no earlier write
    k = np.eye(dk)[:, None, :]
    b = np.full((dk, 1), 0.7)
    _, _, Sk = oracle.build_pairs(KDA, off, k, x["v"], b, x["log_gate"])
    _, _, Sg = oracle.build_pairs(DIAG, off, k, 0.7 * x["v"], None, x["log_gate"])
    assert rel(Sk, Sg) < 1e-14


def test_kda_decay_applies_before_the_erase():
    """One token from a nonzero state: S' = (I - b k k^T) diag(a) S + b k v^T, written
    out by hand (the order of decay and erase matters when the gates differ)."""
    dk, dv = 3, 2
    k = np.array([[[0.6, 0.8, 0.0]]])
    v = np.array([[[1.0, -2.0]]])
    b = np.array([[0.5]])
    lg = np.log(np.array([[[0.5, 0.9, 0.2]]]))
    S0 = np.array([[[1.0, 2.0], [3.0, -1.0], [0.5, 0.5]]])
    S1, _ = oracle.sequential(KDA, k, v, b, lg, S_init=S0)
    D = np.diag([0.5, 0.9, 0.2])
    kk = k[0, 0]
    want = (np.eye(3) - 0.5 * np.outer(kk, kk)) @ D @ S0[0] + 0.5 * np.outer(kk, v[0, 0])
    assert rel(S1[0], want) < 1e-15
    wrong = D @ ((np.eye(3) - 0.5 * np.outer(kk, kk)) @ S0[0]) + 0.5 * np.outer(kk, v[0, 0])
    assert rel(want, wrong) > 1e-2  # the test tells the two orders apart


# ---------------------------------------------------------------- seam step


@pytest.mark.parametrize("fam", FAMS)
def test_seam_step_equals_sequential_over_windows_and_bodies(fam):
    """Windows run token by token on the running state, bodies compose by their
    cached pair: the result equals straight recurrence over
    [window_0, body_0, window_1, body_1, ...] [youleyou, full-attention paragraph]."""
    dk, dv, n_chain, n_seg, w = 5, 4, 2, 4, 3
    body_len = [6, 1, 9, 4]
    n_body = sum(body_len)
    xw = rand_tokens(fam, n_seg * w, n_chain, dk, dv, seed=121 + fam)
    xb = rand_tokens(fam, n_body, n_chain, dk, dv, seed=131 + fam)
    off = np.concatenate([[0], np.cumsum(body_len)]).astype(np.int32)
    body = oracle.build_pairs(fam, off, xb["k"], xb["v"], xb["beta"], xb["log_gate"])
    S0 = np.random.default_rng(4).standard_normal((n_chain, dk, dv))
    res = oracle.seam(fam, n_seg, w, xw["q"], xw["k"], xw["v"], xw["beta"], xw["log_gate"],
                      body=body, S_run=S0, want_window_pairs=True)
    # interleave windows and bodies into one token stream
    order = []
    for s in range(n_seg):
        order += [("w", s * w + j) for j in range(w)]
        order += [("b", t) for t in range(off[s], off[s + 1])]
    cat = lambda key: None if xw[key] is None else np.stack(
        [(xw if src == "w" else xb)[key][i] for src, i in order])
    Sseq, oseq = oracle.sequential(fam, cat("k"), cat("v"), cat("beta"), cat("log_gate"), S_init=S0, q=cat("q"))
    assert rel(res["S_run"], Sseq) < 1e-12
    wpos = [p for p, (src, _) in enumerate(order) if src == "w"]
    assert rel(res["o"], oseq[wpos]) < 1e-12
    # each window's own pair is the pair of its tokens
    for s in range(n_seg):
        sl = slice(s * w, (s + 1) * w)
        gw, Uw, Sw = oracle.build_pairs(fam, np.array([0, w], np.int32), xw["k"][sl], xw["v"][sl],
                                        None if xw["beta"] is None else xw["beta"][sl],
                                        None if xw["log_gate"] is None else xw["log_gate"][sl])
        assert rel(res["wS"][s], Sw[0]) < 1e-13
        np.testing.assert_allclose(res["wg"][s], gw[0], rtol=1e-13, atol=1e-15)
        if fam in DENSE:
            assert rel(res["wU"][s], Uw[0]) < 1e-13


# -------------------------------------------------------- the tiny GDN workload


def test_gdn_tiny_workload_compose_vs_sequential():
    """1 head, d = 64, 4 x 256 tokens, fp32 inputs: build per segment, compose in
    order, compare to the straight recurrence (fp64 on both sides)."""
    from segment_scan_amd import synth
    for scale in (1.0, 1.0 / 64, 0.0):
        tk = synth.gdn_tiny(gate_scale=scale)
        g, U, S = oracle.build_pairs(DELTA, tk.offsets, tk.k, tk.v, tk.beta, tk.log_gate)
        c = oracle.compose(DELTA, g, U, S)
        Sseq, _ = oracle.sequential(DELTA, tk.k, tk.v, tk.beta, tk.log_gate)
        assert rel(c["S_out"], Sseq) < 1e-11, scale


# ------------------------------------------------------- rotary re-rotation


def rope_keys(k, pos, base):
    """Rotary encoding of keys at positions pos (RoFormer, pairs (2i, 2i+1) turned
    by pos * base^(-2i/d)), written with complex numbers rather than matrices."""
    dk = k.shape[-1]
    theta = base ** (-np.arange(dk // 2) * 2.0 / dk)
    z = (k[..., 0::2] + 1j * k[..., 1::2]) * np.exp(1j * np.asarray(pos, np.float64)[:, None, None] * theta)
    out = np.empty_like(k)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


@pytest.mark.parametrize("fam", [NAIVE, SCALAR, DELTA])
@pytest.mark.parametrize("base", [10000.0, 500.0])
def test_rerotation_equals_building_at_the_new_offset(fam, base):
    # A pair built from keys rotated at positions 0..L-1 of its segment, then
    # re-rotated to offset p, must equal the pair built from the keys rotated at
    # p .. p+L-1 [youleyou, linear-layer paragraph: re-rotation aligns a cached
    # segment exactly].
    dk, dv = 8, 5
    offsets = np.array([0, 5, 6, 16, 23], np.int32)
    x = rand_tokens(fam, 23, 3, dk, dv, seed=4100 + fam)
    local = np.concatenate([np.arange(offsets[s + 1] - offsets[s]) for s in range(4)])
    p = np.array([7, 0, -3, 40961], np.int32)
    absolute = local + np.repeat(p, np.diff(offsets))
    g0, U0, S0 = oracle.build_pairs(fam, offsets, rope_keys(x["k"], local, base), x["v"], x["beta"], x["log_gate"])
    g1, U1, S1 = oracle.build_pairs(fam, offsets, rope_keys(x["k"], absolute, base), x["v"], x["beta"],
                                    x["log_gate"])
    Ur, Sr = oracle.rerotate(fam, U0, S0, p, base)
    assert rel(Sr, S1) < 1e-11
    if fam == DELTA:
        assert rel(Ur, U1) < 1e-11
    assert np.array_equal(g0, g1)


def test_rerotation_closed_form_two_dims():
    # d_k = 2: R(p) is the plane rotation by angle p (theta_0 = 1).
    S = np.array([[[[1.0, 2.0, -1.0], [0.5, -3.0, 4.0]]]])
    U = np.array([[[[2.0, 1.0], [-1.0, 0.25]]]])
    p = 3
    c, s = np.cos(p), np.sin(p)
    R = np.array([[c, -s], [s, c]])
    Ur, Sr = oracle.rerotate(DELTA, U, S, [p])
    np.testing.assert_allclose(Sr[0, 0], R @ S[0, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(Ur[0, 0], R @ U[0, 0] @ R.T, rtol=0, atol=1e-14)


def test_rerotation_group_law_and_composition():
    # R(0) = I, R(p) R(q) = R(p + q), and re-rotating every pair of a chain by
    # one offset re-rotates the composed state and transition by that offset.
    dk, dv = 8, 8
    x = rand_tokens(DELTA, 20, 2, dk, dv, seed=4200)
    offsets = np.array([0, 4, 11, 20], np.int32)
    g, U, S = oracle.build_pairs(DELTA, offsets, x["k"], x["v"], x["beta"], x["log_gate"])
    U0, S0 = oracle.rerotate(DELTA, U, S, [0, 0, 0])
    assert np.array_equal(U0, U) and np.array_equal(S0, S)
    Ua, Sa = oracle.rerotate(DELTA, *oracle.rerotate(DELTA, U, S, [5, -2, 100]), [-12, 9, 3])
    Ub, Sb = oracle.rerotate(DELTA, U, S, [-7, 7, 103])
    assert rel(Sa, Sb) < 1e-12 and rel(Ua, Ub) < 1e-12
    Ur, Sr = oracle.rerotate(DELTA, U, S, [31, 31, 31])
    a = oracle.compose(DELTA, g, U, S, want_total=True)
    b = oracle.compose(DELTA, g, Ur, Sr, want_total=True)
    Ut_r, Sc_r = oracle.rerotate(DELTA, a["U_tot"][None], a["S_out"][None], [31])
    assert rel(b["S_out"], Sc_r[0]) < 1e-12 and rel(b["U_tot"], Ut_r[0]) < 1e-12
    assert np.array_equal(a["g_tot"], b["g_tot"])


def test_rerotation_refuses_diagonal_family():
    S = np.zeros((1, 1, 4, 4))
    with pytest.raises(ValueError):
        oracle.rerotate(DIAG, None, S, [3])
