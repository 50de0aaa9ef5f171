"""GPU parity: hypic_seg_build_compose against the oracle, in its three
schedules: sequential (build, then compose), pipelined (groups of segments
built on the caller's stream, each group composed on a second stream while the
next is built, the group pairs composed in order at the end) and fused (the
composition folded into the delta build's state pass as a tree whose last
arrival at each node composes it)."""
import numpy as np
import pytest

import oracle
from segment_scan_amd import api, synth
from segment_scan_amd.synth import DELTA, DIAG, KDA, NAIVE, SCALAR
from tests.gpu_util import TOL, announce, assert_g_close, assert_units_close, dev_f32, host, upload_tokens

pytestmark = pytest.mark.gpu


def _run(tk, offsets, S0=None, want_total=True, mode=api.BC_PIPELINED):
    import torch
    d = upload_tokens(tk)
    g, U, S, res = api.seg_build_compose(tk.fam, list(offsets), d["k"], d["v"], d["beta"], d["log_gate"],
                                         tk.gate_per_chain, S_init=None if S0 is None else dev_f32(S0),
                                         want_total=want_total, mode=mode)
    g2, U2, S2 = api.seg_build(tk.fam, list(offsets), d["k"], d["v"], d["beta"], d["log_gate"], tk.gate_per_chain)
    torch.cuda.synchronize()
    # the pairs are those of the plain build (same kernels, same inputs)
    assert torch.equal(S, S2) and torch.equal(g, g2), "pairs differ from hypic_seg_build"
    if U is not None:
        assert torch.equal(U, U2), "U differs from hypic_seg_build"
    return g, U, S, res


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_cold_request_full_size(mode):
    """The 32k-token cold request (32 heads x 64 segments x 512 tokens), in the
    sequential schedule, the pipelined one (four groups of 16 segments) and the
    fused one; S_out, g_total and U_total against the oracle's composition of
    its own pairs."""
    tk = synth.gdn_cold()
    announce("build_compose_cold", "mode", mode)
    g, U, S, res = _run(tk, tk.offsets, mode=mode)
    rg, rU, rS = oracle.build_pairs(DELTA, tk.offsets, tk.k, tk.v, tk.beta, tk.log_gate)
    ref = oracle.compose(DELTA, rg, rU, rS, want_total=True)
    assert_units_close("cold.S_out", host(res["S_out"]), ref["S_out"], TOL["bf16"], unit_dims=1)
    assert_g_close("cold.g_tot", host(res["g_tot"]), ref["g_tot"], TOL["bf16"])
    # U_total of 64 segments is e^-52-class small; compared as the transition exp(g) U
    assert_units_close("cold.U_tot", host(res["U_tot"]), ref["U_tot"], TOL["bf16"], unit_dims=1)


def _family_tokens(kind, n_seg, L, n_chain, gate_scale):
    if kind == "naive":
        return synth.naive(n_seg=n_seg, L=L, n_chain=n_chain)
    if kind == "scalar":
        return synth.mamba2_like(n_seg=n_seg, L=L, n_chain=n_chain, gate_scale=gate_scale)
    if kind == "gla":
        return synth.gla(n_seg=n_seg, L=L, n_chain=n_chain, gate_scale=gate_scale)
    if kind == "kda":
        return synth.kda(n_seg=n_seg, L=L, n_chain=n_chain, gate_scale=gate_scale)
    return synth.gdn_cold(n_seg=n_seg, L=L, n_chain=n_chain, gate_scale=gate_scale)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("kind", ["naive", "scalar", "gla", "gdn", "kda"])
def test_many_groups_equal_straight_recurrence(kind, mode):
    """600 segments of 24 tokens on 2 chains (three groups of 256 segments),
    slow gates so that every segment's transition matters, a nonzero start
    state: S_out against straight recurrence over all 14,400 tokens."""
    n_seg, L, H = 600, 24, 2
    tk = _family_tokens(kind, n_seg, L, H, 1.0 / 256)
    S0 = np.random.default_rng(21).standard_normal((H, 128, 128)).astype(np.float32).astype(np.float64)
    announce("build_compose_groups", kind, "segs", n_seg, "mode", mode)
    g, U, S, res = _run(tk, tk.offsets, S0=S0, mode=mode)
    Sseq, _ = oracle.sequential(tk.fam, tk.k, tk.v, tk.beta, tk.log_gate, tk.gate_per_chain, S_init=S0)
    assert_units_close(kind + ".S_out", host(res["S_out"]), Sseq, TOL["bf16"], unit_dims=1)


def test_one_group_and_ragged():
    """Few segments (one group: build then compose on the caller's stream),
    ragged lengths including a 1-token segment."""
    lengths = [1, 63, 64, 65, 200, 130, 7]
    tk = synth.gdn_cold(n_seg=1, L=sum(lengths), n_chain=3, gate_scale=1.0 / 64)
    offsets = synth.ragged_offsets(lengths)
    announce("build_compose_one_group")
    g, U, S, res = _run(tk, offsets)
    Sseq, _ = oracle.sequential(DELTA, tk.k, tk.v, tk.beta, tk.log_gate)
    assert_units_close("one_group.S_out", host(res["S_out"]), Sseq, TOL["bf16"], unit_dims=1)


@pytest.mark.parametrize("lengths", [[64, 64], [1, 63, 64, 65, 200, 130, 7], [24] * 600])
def test_fused_tree_shapes(lengths):
    """The fused schedule on trees of 2 leaves, of 7 ragged segments (a 1-token
    one; the tree's right edge has nodes with one child) and of 600 segments (3
    build launches whose workgroups meet at the upper nodes): S_out, g_total and
    U_total against the straight recurrence over all tokens, and a second call
    bit for bit equal to the first."""
    import torch
    n_chain = 2 if len(lengths) > 100 else 3
    tk = synth.gdn_cold(n_seg=1, L=sum(lengths), n_chain=n_chain, gate_scale=1.0 / 64)
    offsets = synth.ragged_offsets(lengths)
    announce("build_compose_fused", "segs", len(lengths), "chains", n_chain)
    g, U, S, res = _run(tk, offsets, mode=api.BC_FUSED)
    Sseq, _ = oracle.sequential(DELTA, tk.k, tk.v, tk.beta, tk.log_gate)
    assert_units_close("fused.S_out", host(res["S_out"]), Sseq, TOL["bf16"], unit_dims=1)
    # the composition alone: the oracle composing the pairs this call built
    # (fp32 pairs: the fp32 class for the composed state)
    ref = oracle.compose(DELTA, host(g), host(U), host(S), want_total=True)
    assert_units_close("fused.S_out_vs_own_pairs", host(res["S_out"]), ref["S_out"], TOL["f32"], unit_dims=1)
    assert_g_close("fused.g_tot", host(res["g_tot"]), ref["g_tot"], TOL["f32"])
    assert_units_close("fused.U_tot", host(res["U_tot"]), ref["U_tot"], TOL["bf16"], unit_dims=1)
    _, _, _, res2 = _run(tk, offsets, mode=api.BC_FUSED)
    torch.cuda.synchronize()
    for key in ("S_out", "g_tot", "U_tot"):
        assert torch.equal(res[key], res2[key]), key + " differs between two fused calls"


def test_fused_without_totals():
    """The fused schedule asked for S_out alone (no g_total, no U_total: the root
    writes neither), against the sequential schedule's S_out."""
    import torch
    lengths = [64] * 12
    tk = synth.gdn_cold(n_seg=1, L=sum(lengths), n_chain=4, gate_scale=1.0 / 64)
    offsets = synth.ragged_offsets(lengths)
    announce("build_compose_fused_no_totals")
    _, _, _, res = _run(tk, offsets, want_total=False, mode=api.BC_FUSED)
    _, _, _, ref = _run(tk, offsets, want_total=False, mode=api.BC_SEQUENTIAL)
    torch.cuda.synchronize()
    assert res.get("g_tot") is None and res.get("U_tot") is None
    assert_units_close("fused_no_totals.S_out", host(res["S_out"]), host(ref["S_out"]).astype(np.float64),
                       TOL["f32"], unit_dims=1)
