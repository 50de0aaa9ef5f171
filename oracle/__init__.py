"""fp64 CPU oracle for the linear-attention hot path of position-independent caching.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``segment_scan_amd``) never imports, links or calls it, and this package never
imports the product path.  It shares no code with the HIP library: the
arithmetic lives in ``hypic_ref.c`` (plain C, fp64, token by token), and this
module only marshals numpy arrays into it.

Every function takes fp64 numpy arrays holding the exact values the GPU path
sees (bf16/fp32 inputs widened exactly), in the layouts documented in
``hypic_ref.c``, and returns fp64 arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

NAIVE, SCALAR, DIAG, DELTA, KDA = 0, 1, 2, 3, 4
DENSE = (DELTA, KDA)  # families whose transition is a dense exp(g) U

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hypic_ref.c")
_LIB = os.path.join(_HERE, "libhypic_ref.so")
# The mutation test points this at a deliberately broken build of the oracle
# to check that the pins catch it.
_LIB_OVERRIDE = os.environ.get("HYPIC_REF_LIB")
_lib = None


def compile_to(src: str, out: str) -> None:
    cmd = ["gcc", "-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O3 -fopenmp, fp64, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        compile_to(_SRC, tmp)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.hypic_ref_build.argtypes = [I, I, P, I, I, I, P, P, P, P, I, P, P, P, I]
        lib.hypic_ref_compose.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, I]
        lib.hypic_ref_seam.argtypes = [I, I, I, I, I, I, P, P, P, P, P, I, P, P, P, P, P, P, P, P, I]
        lib.hypic_ref_sequential.argtypes = [I, I, I, I, I, P, P, P, P, P, I, P, P, P, I]
        lib.hypic_ref_rerotate.argtypes = [I, I, I, I, I, P, ctypes.c_double, P, P, I]
        for f in (lib.hypic_ref_build, lib.hypic_ref_compose, lib.hypic_ref_seam,
                  lib.hypic_ref_sequential, lib.hypic_ref_rerotate):
            f.restype = I
        lib.hypic_ref_max_threads.restype = I
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().hypic_ref_max_threads())


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _threads(n):
    return max_threads() if n is None else int(n)


def _check(rc, name):
    if rc != 0:
        raise ValueError("%s failed with status %d" % (name, rc))


def gate_len(fam: int, dk: int) -> int:
    return dk if fam == DIAG else 1


def build_pairs(fam, offsets, k, v, beta=None, log_gate=None, gate_per_chain=False,
                want_U=True, n_threads=None):
    """Per-(segment, chain) factored transition and zero-start state.

    k: [n_tok, n_chain, dk]; v: [n_tok, n_chain, dv]; offsets: n_seg + 1 ints.
    Returns (g, U, S): g [n_seg, n_chain] (diag: [.., dk]), U [n_seg, n_chain, dk, dk]
    for the delta family (else None), S [n_seg, n_chain, dk, dv].
    """
    k, v, beta, log_gate = _f64(k), _f64(v), _f64(beta), _f64(log_gate)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    n_seg = off.size - 1
    n_tok, n_chain, dk = k.shape
    dv = v.shape[2]
    gl = gate_len(fam, dk)
    g = np.zeros((n_seg, n_chain) + ((dk,) if gl > 1 else ()), np.float64)
    U = np.zeros((n_seg, n_chain, dk, dk), np.float64) if (fam in DENSE and want_U) else None
    S = np.zeros((n_seg, n_chain, dk, dv), np.float64)
    rc = _load().hypic_ref_build(fam, n_seg, _p(off), n_chain, dk, dv, _p(k), _p(v), _p(beta),
                                 _p(log_gate), int(bool(gate_per_chain)), _p(g), _p(U), _p(S),
                                 _threads(n_threads))
    _check(rc, "hypic_ref_build")
    return g, U, S


def compose(fam, g, U, S, S_init=None, want_prefix=False, want_total=False, n_threads=None):
    """Ordered composition along each chain; returns dict with S_out and optional extras."""
    g, U, S, S_init = _f64(g), _f64(U), _f64(S), _f64(S_init)
    n_seg, n_chain, dk, dv = S.shape
    gl = gate_len(fam, dk)
    S_out = np.zeros((n_chain, dk, dv), np.float64)
    prefix = np.zeros((n_seg, n_chain, dk, dv), np.float64) if want_prefix else None
    g_tot = np.zeros((n_chain,) + ((dk,) if gl > 1 else ()), np.float64) if want_total else None
    U_tot = np.zeros((n_chain, dk, dk), np.float64) if (want_total and fam in DENSE) else None
    rc = _load().hypic_ref_compose(fam, n_seg, n_chain, dk, dv, _p(g), _p(U), _p(S), _p(S_init),
                                   _p(S_out), _p(prefix), _p(g_tot), _p(U_tot),
                                   _threads(n_threads))
    _check(rc, "hypic_ref_compose")
    return {"S_out": S_out, "prefix": prefix, "g_tot": g_tot, "U_tot": U_tot}


def seam(fam, n_seg, w, q, k, v, beta=None, log_gate=None, gate_per_chain=False,
         body=None, S_run=None, want_window_pairs=False, n_threads=None):
    """Seam-window step: returns dict with S_run (final), o, and optional window pairs.

    body: None or (g, U, S) cached body pairs, composed after each window.
    """
    q, k, v, beta, log_gate = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(log_gate)
    n_tok, n_chain, dk = k.shape
    dv = v.shape[2]
    assert n_tok == n_seg * w
    gl = gate_len(fam, dk)
    S = np.zeros((n_chain, dk, dv), np.float64) if S_run is None else _f64(S_run).copy()
    o = np.zeros((n_tok, n_chain, dv), np.float64)
    bg = bU = bS = None
    if body is not None:
        bg, bU, bS = (_f64(x) for x in body)
    wg = wU = wS = None
    if want_window_pairs:
        wg = np.zeros((n_seg, n_chain) + ((dk,) if gl > 1 else ()), np.float64)
        wU = np.zeros((n_seg, n_chain, dk, dk), np.float64) if fam in DENSE else None
        wS = np.zeros((n_seg, n_chain, dk, dv), np.float64)
    rc = _load().hypic_ref_seam(fam, n_seg, w, n_chain, dk, dv, _p(q), _p(k), _p(v), _p(beta),
                                _p(log_gate), int(bool(gate_per_chain)), _p(bg), _p(bU), _p(bS),
                                _p(S), _p(o), _p(wg), _p(wU), _p(wS), _threads(n_threads))
    _check(rc, "hypic_ref_seam")
    return {"S_run": S, "o": o, "wg": wg, "wU": wU, "wS": wS}


def sequential(fam, k, v, beta=None, log_gate=None, gate_per_chain=False, S_init=None, q=None,
               n_threads=None):
    """Straight token-by-token recurrence over all tokens; returns (S_final, o or None)."""
    q, k, v, beta, log_gate, S_init = (_f64(x) for x in (q, k, v, beta, log_gate, S_init))
    n_tok, n_chain, dk = k.shape
    dv = v.shape[2]
    S = np.zeros((n_chain, dk, dv), np.float64)
    o = np.zeros((n_tok, n_chain, dv), np.float64) if q is not None else None
    rc = _load().hypic_ref_sequential(fam, n_tok, n_chain, dk, dv, _p(q), _p(k), _p(v), _p(beta),
                                      _p(log_gate), int(bool(gate_per_chain)), _p(S_init), _p(S),
                                      _p(o), _threads(n_threads))
    _check(rc, "hypic_ref_sequential")
    return S, o


def rerotate(fam, U, S, delta, base=10000.0, n_threads=None):
    """State re-rotation of cached pairs to offsets delta[s] (see hypic_ref.c):
    returns (U', S') = (R U R^T, R S) per (segment, chain); U' None unless delta family."""
    S = _f64(S).copy()
    U = None if U is None else _f64(U).copy()
    n_seg, n_chain, dk, dv = S.shape
    d = np.ascontiguousarray(delta, dtype=np.int32)
    assert d.shape == (n_seg,)
    rc = _load().hypic_ref_rerotate(fam, n_seg, n_chain, dk, dv, _p(d), float(base), _p(U), _p(S),
                                    _threads(n_threads))
    _check(rc, "hypic_ref_rerotate")
    return U, S


def transition_dense(fam, g, U, dk):
    """Dense T = exp(g) U (delta), diag(exp(g)) (diag), exp(g) I (scalar), I (naive).

    g: [..] or [.., dk] (diag); U: [.., dk, dk] (delta).  Returns [.., dk, dk].
    """
    g = np.asarray(g, np.float64)
    eye = np.eye(dk)
    if fam == NAIVE:
        return np.broadcast_to(eye, g.shape + (dk, dk)).copy()
    if fam == SCALAR:
        return np.exp(g)[..., None, None] * eye
    if fam == DIAG:
        return np.exp(g)[..., :, None] * eye
    return np.exp(g)[..., None, None] * np.asarray(U, np.float64)
