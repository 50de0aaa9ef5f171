"""Helpers for the GPU parity tests: upload oracle-exact inputs, compare results."""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {"bf16": 2e-3, "f32": 1e-5}


def announce(*parts):
    """Name the case on stdout before any GPU work, so a failing run names it."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def dev(arr, dtype: str):
    """fp64 numpy array holding exact dtype values -> GPU tensor of that dtype (exact)."""
    if arr is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float64))
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    return t.to(tdt).cuda()


def dev_f32(arr):
    return None if arr is None else torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def host(t):
    return None if t is None else t.detach().double().cpu().numpy()


def upload_tokens(tk, with_q=False):
    d = {"k": dev(tk.k, tk.dtype), "v": dev(tk.v, tk.dtype),
         "beta": dev(tk.beta, tk.dtype) if tk.beta is not None else None}
    if tk.log_gate is not None:
        d["log_gate"] = dev_f32(tk.log_gate) if tk.gate_per_chain else dev(tk.log_gate, tk.dtype)
    else:
        d["log_gate"] = None
    if with_q:
        d["q"] = dev(tk.q, tk.dtype)
    return d


def rel_err_units(got, ref, unit_dims=2):
    """Relative Frobenius error per unit (leading `unit_dims` axes); guard on tiny references."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    lead = ref.shape[:unit_dims]
    g2 = got.reshape(lead + (-1,))
    r2 = ref.reshape(lead + (-1,))
    num = np.linalg.norm(g2 - r2, axis=-1)
    den = np.linalg.norm(r2, axis=-1)
    return np.where(den > 1e-30, num / np.maximum(den, 1e-300), num)


def assert_units_close(name, got, ref, tol, unit_dims=2):
    err = rel_err_units(got, ref, unit_dims)
    worst = float(err.max())
    assert np.isfinite(got).all(), "%s: non-finite output" % name
    assert worst <= tol, "%s: max relative Frobenius error %.3e > %.1e (unit %s)" % (
        name, worst, tol, np.unravel_index(int(err.argmax()), err.shape))
    return worst


def assert_g_close(name, got, ref, tol):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bound = tol * np.maximum(1.0, np.abs(ref))
    bad = np.abs(got - ref) > bound
    assert not bad.any(), "%s: %d g values off, worst |diff| %.3e" % (name, int(bad.sum()), float(np.abs(got - ref).max()))
