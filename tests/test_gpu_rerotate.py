"""GPU parity: rotary re-rotation of cached pairs (hypic_rerotate) vs the oracle.

Tolerance: the rotation is fp32 on exact fp32 inputs with cos/sin formed in
fp64 and rounded to fp32.  Each output element c*a - s*b carries at most about
3 * 2^-24 * (|a| + |b|) of rounding (cos/sin rounding, the product, the fma),
i.e. ~4.2e-7 of its row pair's norm; U is rotated on both sides, which at
most doubles that.  Per unit the relative Frobenius error is therefore below
1e-6.  Offsets up to 2^24 tokens add at most 2^24 * 2^-52 rad of angle
difference between the device's and the host's fp64 pow (below 1e-8 rad).
"""
import numpy as np
import pytest

import oracle
from oracle import NAIVE, SCALAR, DELTA
from segment_scan_amd import api, synth
from tests.gpu_util import announce, assert_units_close, dev_f32, host

pytestmark = pytest.mark.gpu

TOL = 1e-6


def _pairs(fam, n_seg, n_chain, d, seed):
    r = np.random.default_rng(seed)
    S = r.standard_normal((n_seg, n_chain, d, d)).astype(np.float32).astype(np.float64)
    U = None
    if fam == DELTA:
        U = (r.standard_normal((n_seg, n_chain, d, d)) * (0.5 / np.sqrt(d))).astype(np.float32).astype(np.float64)
    return U, S


def _run(fam, U, S, pos, base=10000.0):
    import torch
    Ug = dev_f32(U) if U is not None else None
    Sg = dev_f32(S)
    api.rerotate(fam, torch.tensor(pos, dtype=torch.int32, device="cuda"), Sg, Ug, rope_base=base)
    torch.cuda.synchronize()
    return host(Ug), host(Sg)


def _check(fam, U, S, pos, name, base=10000.0, tol=TOL):
    announce(name, "fam", fam, "segs", S.shape[0], "chains", S.shape[1], "d", S.shape[2])
    Ug, Sg = _run(fam, U, S, pos, base)
    Ur, Sr = oracle.rerotate(fam, U, S, pos, base)
    assert_units_close(name + ".S", Sg, Sr, tol)
    if fam == DELTA:
        assert_units_close(name + ".U", Ug, Ur, tol)


POS = [0, 1, -37, 512, 100_000, 1 << 24, -(1 << 24) + 3]


@pytest.mark.parametrize("d", [128, 64])
def test_rerotate_delta(d):
    U, S = _pairs(DELTA, len(POS), 6, d, seed=50 + d)
    _check(DELTA, U, S, POS, "delta_d%d" % d)


@pytest.mark.parametrize("fam", [NAIVE, SCALAR])
def test_rerotate_state_only_families(fam):
    U, S = _pairs(fam, len(POS), 5, 128, seed=60 + fam)
    _check(fam, U, S, POS, "fam%d" % fam)
    U, S = _pairs(fam, 3, 2, 64, seed=70 + fam)
    _check(fam, U, S, [9, -9, 4096], "fam%d_d64" % fam, base=500000.0)


def test_rerotate_single_unit_and_unit_base():
    U, S = _pairs(DELTA, 1, 1, 128, seed=80)
    _check(DELTA, U, S, [3], "one_unit")
    _check(DELTA, U, S, [3], "base_one", base=1.0)  # every pair turned by 3 rad


def test_rerotate_extreme_offsets():
    """int32 extremes: the angle p * theta_i is ill-conditioned in fp64 itself
    (one ulp of theta moves it by up to 2^31 * 2^-53 * 2 ~ 5e-7 rad between the
    device's and the host's pow), so the bound is 4e-6 here."""
    U, S = _pairs(DELTA, 2, 3, 128, seed=81)
    _check(DELTA, U, S, [2**31 - 1, -2**31], "int32_extremes", tol=4e-6)


def test_rerotate_round_trip_and_addition():
    """p then -p returns the pair; p then q equals p + q (device only)."""
    import torch
    U, S = _pairs(DELTA, 4, 3, 128, seed=82)
    announce("round_trip")
    Ug, Sg = dev_f32(U), dev_f32(S)
    p = torch.tensor([5, -700, 123456, 1], dtype=torch.int32, device="cuda")
    api.rerotate(DELTA, p, Sg, Ug)
    api.rerotate(DELTA, -p, Sg, Ug)
    torch.cuda.synchronize()
    assert_units_close("round_trip.S", host(Sg), S, 2 * TOL)
    assert_units_close("round_trip.U", host(Ug), U, 2 * TOL)
    q = torch.tensor([1, 2, -3, 40000], dtype=torch.int32, device="cuda")
    api.rerotate(DELTA, p, Sg, Ug)
    api.rerotate(DELTA, q, Sg, Ug)
    torch.cuda.synchronize()
    Ur, Sr = oracle.rerotate(DELTA, U, S, (p + q).cpu().numpy())
    assert_units_close("addition.S", host(Sg), Sr, 2 * TOL)
    assert_units_close("addition.U", host(Ug), Ur, 2 * TOL)


def test_rerotate_warm_request_full_size_sampled():
    """The warm 100k-token request's cached pairs at full size (196 segments x
    480 chains, d = 128, 12.3 GB of U and S), drawn on the GPU as the benchmark
    draws them, re-rotated in the launch the benchmark times; sampled units are
    checked against the oracle."""
    import torch
    n_seg, n, d = synth.WARM_SEGS, synth.WARM_LAYERS * synth.WARM_HEADS, synth.WARM_D
    announce("warm_full", n_seg, n, d)
    gen = torch.Generator(device="cuda").manual_seed(20260702)
    U = torch.randn((n_seg, n, d, d), device="cuda", generator=gen) * (0.5 / np.sqrt(d))
    S = torch.randn((n_seg, n, d, d), device="cuda", generator=gen)
    pos = torch.randint(-(1 << 20), 1 << 20, (n_seg,), device="cuda", generator=gen, dtype=torch.int32)
    samples = [(0, 0), (0, n - 1), (n_seg - 1, 0), (n_seg - 1, n - 1), (97, 251), (13, 479), (150, 3)]
    U0 = [host(U[s, h]) for s, h in samples]
    S0 = [host(S[s, h]) for s, h in samples]
    api.rerotate(DELTA, pos, S, U)
    torch.cuda.synchronize()
    pos_h = pos.cpu().numpy()
    for i, (s, h) in enumerate(samples):
        Ur, Sr = oracle.rerotate(DELTA, U0[i][None, None], S0[i][None, None], [pos_h[s]])
        assert_units_close("warm_full.S(%d,%d)" % (s, h), host(S[s, h])[None, None], Sr, TOL)
        assert_units_close("warm_full.U(%d,%d)" % (s, h), host(U[s, h])[None, None], Ur, TOL)
    del U, S
    torch.cuda.empty_cache()
