"""GPU parity: dense (delta-family) ordered composition vs the oracle."""
import numpy as np
import pytest

import oracle
from segment_scan_amd import api, synth
from segment_scan_amd.synth import DELTA
from tests.gpu_util import announce, assert_g_close, assert_units_close, dev_f32, host

pytestmark = pytest.mark.gpu


def _check(g, U, S, S_init, name, tol=1e-5, want_total=True):
    import torch
    announce(name, "segs", S.shape[0], "chains", S.shape[1], "d", S.shape[2])
    res = api.compose(DELTA, dev_f32(g), dev_f32(U), dev_f32(S),
                      S_init=None if S_init is None else dev_f32(S_init), want_prefix=True,
                      want_total=want_total)
    torch.cuda.synchronize()
    ref = oracle.compose(DELTA, g, U, S, S_init=S_init, want_prefix=True, want_total=want_total)
    assert_units_close(name + ".S_out", host(res["S_out"]), ref["S_out"], tol, unit_dims=1)
    assert_units_close(name + ".prefix", host(res["prefix"]), ref["prefix"], tol)
    if want_total:
        assert_g_close(name + ".g_tot", host(res["g_tot"]), ref["g_tot"], tol)
        assert_units_close(name + ".U_tot", host(res["U_tot"]), ref["U_tot"], tol, unit_dims=1)


def test_compose_dense_random_pairs_warm_layer():
    """Random cached pairs of the warm-reuse recipe (g = 0, U ~ N(0, 1/(4d)), S ~ N(0,1)):
    each step roughly halves ||S||, so every step is numerically non-trivial."""
    g, U, S = synth.warm_pairs_layer(0, n_seg=24, n_head=6)
    _check(g, U, S, None, "warm_pairs")


def test_compose_dense_gated_built_pairs_with_init():
    """Pairs from the oracle's build of slow-gated GDN tokens (T not negligible)."""
    tk = synth.gdn_cold(n_seg=6, L=64, n_chain=4, gate_scale=1.0 / 64)
    g, U, S = oracle.build_pairs(DELTA, tk.offsets, tk.k, tk.v, tk.beta, tk.log_gate)
    f32 = lambda x: x.astype(np.float32).astype(np.float64)
    S_init = f32(np.random.default_rng(2).standard_normal(S.shape[1:]))
    _check(f32(g), f32(U), f32(S), S_init, "gated_pairs")


def test_compose_dense_d64_one_segment():
    g, U, S = synth.warm_pairs_layer(1, n_seg=1, n_head=3, d=64)
    _check(g, U, S, None, "d64_one")
    g, U, S = synth.warm_pairs_layer(2, n_seg=5, n_head=3, d=64)
    _check(g, U, S, None, "d64_five", want_total=False)


def test_compose_dense_many_chains_in_place():
    """70 chains (one workgroup per chain; a count that is not a multiple of 8),
    S_out the same buffer as S_init, prefix states and totals."""
    import torch
    g, U, S = synth.warm_pairs_layer(4, n_seg=3, n_head=70)
    g = g - 0.01 * np.arange(g.size).reshape(g.shape) / g.size  # nonzero gates
    g = g.astype(np.float32).astype(np.float64)
    S_init = np.random.default_rng(4).standard_normal(S.shape[1:]).astype(np.float32).astype(np.float64)
    announce("many_chains_in_place", "chains", 70)
    st = dev_f32(S_init)
    res = api.compose(DELTA, dev_f32(g), dev_f32(U), dev_f32(S), S_init=st, S_out=st, want_prefix=True,
                      want_total=True)
    torch.cuda.synchronize()
    assert res["S_out"].data_ptr() == st.data_ptr()
    ref = oracle.compose(DELTA, g, U, S, S_init=S_init, want_prefix=True, want_total=True)
    assert_units_close("inplace.S_out", host(st), ref["S_out"], 1e-5, unit_dims=1)
    assert_units_close("inplace.prefix", host(res["prefix"]), ref["prefix"], 1e-5)
    assert_g_close("inplace.g_tot", host(res["g_tot"]), ref["g_tot"], 1e-5)
    assert_units_close("inplace.U_tot", host(res["U_tot"]), ref["U_tot"], 1e-5, unit_dims=1)


def test_compose_dense_two_level_schedule():
    """Few chains, no prefix states: with a workspace the composition runs in two
    levels (37 segments -> 8 blocks of up to 5, the last one ragged); S_out,
    g_total and U_total must match the oracle, and the single-pass schedule."""
    import torch
    g, U, S = synth.warm_pairs_layer(5, n_seg=37, n_head=5)
    g = (g - 0.02 * np.arange(g.size).reshape(g.shape) / g.size).astype(np.float32).astype(np.float64)
    S_init = np.random.default_rng(5).standard_normal(S.shape[1:]).astype(np.float32).astype(np.float64)
    need = api.compose_workspace_size(DELTA, 37, 5, 128)
    assert need > 0
    announce("two_level", "segs", 37, "chains", 5, "workspace", need)
    dg, dU, dS, dI = dev_f32(g), dev_f32(U), dev_f32(S), dev_f32(S_init)
    ws = torch.full((need,), 0x7F, device="cuda", dtype=torch.uint8)
    tree = api.compose(DELTA, dg, dU, dS, S_init=dI, want_total=True, workspace=ws)
    flat = api.compose(DELTA, dg, dU, dS, S_init=dI, want_total=True, workspace=None)
    torch.cuda.synchronize()
    ref = oracle.compose(DELTA, g, U, S, S_init=S_init, want_total=True)
    for name, res in (("tree", tree), ("flat", flat)):
        assert_units_close(name + ".S_out", host(res["S_out"]), ref["S_out"], 1e-5, unit_dims=1)
        assert_g_close(name + ".g_tot", host(res["g_tot"]), ref["g_tot"], 1e-5)
        assert_units_close(name + ".U_tot", host(res["U_tot"]), ref["U_tot"], 1e-5, unit_dims=1)


def test_compose_dense_scan_with_prefix_states():
    """Few chains with prefix states: the three-phase scan (37 segments -> 8 blocks,
    the last ragged; block pairs, block start states in order, then every block
    again from its start state) must match the oracle, as the single pass must,
    at the fp32-class bound on every prefix state and on U_total (a product of
    37 random factors, whose rounding accumulates with nothing added)."""
    import torch
    g, U, S = synth.warm_pairs_layer(6, n_seg=37, n_head=5)
    g = (g - 0.03 * np.arange(g.size).reshape(g.shape) / g.size).astype(np.float32).astype(np.float64)
    S_init = np.random.default_rng(6).standard_normal(S.shape[1:]).astype(np.float32).astype(np.float64)
    need = api.compose_workspace_size(DELTA, 37, 5, 128, want_prefix=True)
    assert need > 0 and api.compose_workspace_size(DELTA, 37, 5, 128) > 0  # both schedules take a workspace
    announce("scan_prefix", "segs", 37, "chains", 5, "workspace", need)
    dg, dU, dS, dI = dev_f32(g), dev_f32(U), dev_f32(S), dev_f32(S_init)
    ws = torch.full((need,), 0x7F, device="cuda", dtype=torch.uint8)
    scan = api.compose(DELTA, dg, dU, dS, S_init=dI, want_prefix=True, want_total=True, workspace=ws)
    flat = api.compose(DELTA, dg, dU, dS, S_init=dI, want_prefix=True, want_total=True, workspace=None)
    torch.cuda.synchronize()
    ref = oracle.compose(DELTA, g, U, S, S_init=S_init, want_prefix=True, want_total=True)
    for name, res, tol in (("scan", scan, 1e-5), ("flat", flat, 1e-5)):
        assert_units_close(name + ".S_out", host(res["S_out"]), ref["S_out"], tol, unit_dims=1)
        assert_units_close(name + ".prefix", host(res["prefix"]), ref["prefix"], tol)
        assert_g_close(name + ".g_tot", host(res["g_tot"]), ref["g_tot"], tol)
        assert_units_close(name + ".U_tot", host(res["U_tot"]), ref["U_tot"], tol, unit_dims=1)


def test_compose_dense_warm_layer_full_length():
    """One layer of the warm 100k-token request composed on its own: 196 random
    fp32 pairs x 16 heads (one workgroup per 32-column tile), prefix states,
    g_total and U_total, all at the fp32-class bound."""
    g, U, S = synth.warm_pairs_layer(0)
    _check(g, U, S, None, "warm_layer0_full")


def test_compose_dense_warm_request_layers_0_and_29():
    """The whole warm request's pairs (30 layers x 16 heads = 480 chains x 196
    segments, fp32) composed in one call, with prefix states and totals; layers
    0 and 29 (drawn by the seeded generator) are compared with the oracle at the
    fp32-class bound, the other layers carry pairs of the same recipe drawn on
    the GPU."""
    import torch
    H, d, n_seg = synth.WARM_HEADS, synth.WARM_D, synth.WARM_SEGS
    n_chain = synth.WARM_LAYERS * H
    announce("warm_request_compose", "chains", n_chain, "segs", n_seg)
    gen = torch.Generator(device="cuda").manual_seed(7)
    U = torch.randn((n_seg, n_chain, d, d), device="cuda", generator=gen) * (0.5 / np.sqrt(d))
    S = torch.randn((n_seg, n_chain, d, d), device="cuda", generator=gen)
    g = torch.zeros((n_seg, n_chain), device="cuda")
    layers = (0, 29)
    pairs = [synth.warm_pairs_layer(layer) for layer in layers]
    for li, layer in enumerate(layers):
        sl = slice(layer * H, (layer + 1) * H)
        U[:, sl] = dev_f32(pairs[li][1])
        S[:, sl] = dev_f32(pairs[li][2])
    res = api.compose(DELTA, g, U, S, want_prefix=True, want_total=True)
    torch.cuda.synchronize()
    del U, S
    for li, layer in enumerate(layers):
        sl = slice(layer * H, (layer + 1) * H)
        ref = oracle.compose(DELTA, *pairs[li], S_init=None, want_prefix=True, want_total=True)
        name = "warm_req.l%d" % layer
        assert_units_close(name + ".S_out", host(res["S_out"][sl]), ref["S_out"], 1e-5, unit_dims=1)
        assert_units_close(name + ".prefix", host(res["prefix"][:, sl]), ref["prefix"], 1e-5)
        assert_g_close(name + ".g_tot", host(res["g_tot"][sl]), ref["g_tot"], 1e-5)
        assert_units_close(name + ".U_tot", host(res["U_tot"][sl]), ref["U_tot"], 1e-5, unit_dims=1)
