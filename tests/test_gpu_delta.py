"""GPU parity: delta-rule (DeltaNet / GDN) segment build vs the oracle."""
import numpy as np
import pytest

import oracle
from segment_scan_amd import api, synth
from segment_scan_amd.synth import DELTA
from tests.gpu_util import TOL, announce, assert_g_close, assert_units_close, host, upload_tokens

pytestmark = pytest.mark.gpu


def gpu_build(tk, offsets=None):
    import torch
    offsets = tk.offsets if offsets is None else offsets
    d = upload_tokens(tk)
    g, U, S = api.seg_build(DELTA, list(offsets), d["k"], d["v"], d["beta"], d["log_gate"])
    torch.cuda.synchronize()
    return g, U, S


def check_build(tk, name, offsets=None):
    offsets = tk.offsets if offsets is None else np.asarray(offsets, np.int32)
    announce(name, "dtype", tk.dtype, "chains", tk.n_chain, "segs", len(offsets) - 1, "d", tk.dk)
    g, U, S = gpu_build(tk, offsets)
    rg, rU, rS = oracle.build_pairs(DELTA, offsets, tk.k, tk.v, tk.beta, tk.log_gate)
    tol = TOL[tk.dtype]
    eS = assert_units_close(name + ".S", host(S), rS, tol)
    eU = assert_units_close(name + ".U", host(U), rU, tol)
    assert_g_close(name + ".g", host(g), rg, tol)
    print("  max rel err S %.2e U %.2e" % (eS, eU), flush=True)
    return g, U, S


@pytest.mark.parametrize("gate_scale", [1.0, 1.0 / 64, 0.0])
def test_gdn_tiny_fp32(gate_scale):
    """1 head, d = 64, 4 x 256 tokens, fp32 (fp32 tolerance); slow-gate variants keep T_C non-negligible."""
    tk = synth.gdn_tiny(gate_scale=gate_scale)
    check_build(tk, "gdn_tiny_%g" % gate_scale)


def test_gdn_tiny_fp32_compose_vs_sequential():
    import torch
    tk = synth.gdn_tiny(gate_scale=1.0 / 64)
    g, U, S = gpu_build(tk)
    res = api.compose(DELTA, g, U, S)
    torch.cuda.synchronize()
    Sseq, _ = oracle.sequential(DELTA, tk.k, tk.v, tk.beta, tk.log_gate)
    assert_units_close("gdn_tiny_e2e", host(res["S_out"]), Sseq, TOL["f32"], unit_dims=1)


def test_gdn_cold_bf16_reduced():
    """32 heads, d = 128, 4 of the 64 x 512-token segments, bf16."""
    tk = synth.gdn_cold(n_seg=4)
    check_build(tk, "gdn_cold_4seg")


@pytest.mark.parametrize("gate_scale", [1.0 / 64, 0.0])
def test_gdn_cold_slow_gates(gate_scale):
    tk = synth.gdn_cold(n_seg=2, n_chain=4, gate_scale=gate_scale)
    check_build(tk, "gdn_slow_%g" % gate_scale)


def test_gdn_ragged_segments():
    """Segment lengths that are not multiples of the 64-token chunk, incl. 1 token."""
    lengths = [1, 63, 64, 65, 200, 130]
    tk = synth.gdn_cold(n_seg=1, L=sum(lengths), n_chain=3, gate_scale=1.0 / 16)
    check_build(tk, "gdn_ragged", synth.ragged_offsets(lengths))


def test_gdn_d64_bf16_and_d128_fp32():
    tk = synth.gdn_cold(n_seg=3, L=100, n_chain=2, d=64)
    check_build(tk, "gdn_d64_bf16")
    tk = synth.gdn_cold(n_seg=2, L=100, n_chain=2, d=128, dtype="f32", gate_scale=1.0 / 16)
    check_build(tk, "gdn_d128_f32")


def test_gdn_cold_full_size_every_unit():
    """The 32k-token cold request at full size (32 heads x 64 segments x 512), in
    the launch the benchmark times; every one of the 2048 units against one
    oracle pass over the whole request."""
    tk = synth.gdn_cold()
    check_build(tk, "gdn_cold_full")


def test_gdn_build_then_compose_matches_sequential():
    """Cold path end to end on the GPU (build of every segment, ordered compose)
    against straight recurrence over the whole request, slow gates so that
    every segment's T_C matters."""
    import torch
    tk = synth.gdn_cold(n_seg=8, L=256, n_chain=4, gate_scale=1.0 / 64)
    g, U, S = gpu_build(tk)
    res = api.compose(DELTA, g, U, S)
    torch.cuda.synchronize()
    Sseq, _ = oracle.sequential(DELTA, tk.k, tk.v, tk.beta, tk.log_gate)
    assert_units_close("gdn_e2e", host(res["S_out"]), Sseq, TOL["bf16"], unit_dims=1)


def test_gdn_segment_length_limits():
    """A 2048-token segment (longest of the two-kernel fp16 path, where its
    rounding error accumulates most) and a 2049-token one (single-kernel path)."""
    for L in (2048, 2049):
        tk = synth.gdn_cold(n_seg=1, L=L, n_chain=2, gate_scale=1.0 / 64)
        check_build(tk, "gdn_long_%d" % L)


def test_gdn_many_ragged_segments_two_launches():
    """300 ragged segments (1..130 tokens): two launches that reuse one workspace."""
    rng = np.random.default_rng(5)
    lengths = [int(x) for x in rng.integers(1, 131, 300)]
    tk = synth.gdn_cold(n_seg=1, L=sum(lengths), n_chain=2, gate_scale=1.0 / 16)
    check_build(tk, "gdn_300seg", synth.ragged_offsets(lengths))


def test_gdn_longest_first_across_launches():
    """250 segments, the two longest (2100 and 2400 tokens, beyond the two-kernel
    path) at the end of the batch: sorted longest first over the whole batch, the
    first launch holds them (and takes the single-kernel path) with the 238 next
    longest, the second launch the 10 shortest (two-kernel path)."""
    rng = np.random.default_rng(6)
    lengths = [int(x) for x in rng.integers(1, 200, 248)] + [2100, 2400]
    tk = synth.gdn_cold(n_seg=1, L=sum(lengths), n_chain=2, gate_scale=1.0 / 32)
    check_build(tk, "gdn_lpt_2launch", synth.ragged_offsets(lengths))


def test_deltanet_ungated_d128():
    """DeltaNet (no gate, log_gate NULL) through the d = 128 bf16 path."""
    tk = synth.gdn_cold(n_seg=3, L=192, n_chain=2)
    tk.log_gate = None
    check_build(tk, "deltanet_d128")


def test_gdn_strong_and_zero_gates_d128():
    """Log gates of -30 or 0 per token through the d = 128 bf16 path: chunks whose
    total decay underflows fp32 (the state is forgotten) next to undecayed ones,
    tails of 2 tokens."""
    tk = synth.gdn_cold(n_seg=2, L=130, n_chain=2)
    r = np.random.default_rng(21)
    tk.log_gate = np.where(r.random(tk.log_gate.shape) < 0.5, -30.0, 0.0)
    check_build(tk, "gdn_strong_gates_d128")


def test_value_channels_of_very_different_scales():
    """Value channels scaled by powers of two from 2^-20 to 2^17 (the values stay bf16
    numbers).  Each state column depends on its own value channel only, so every
    column of S keeps the bf16 bound on its own: the state pass scales its fp16
    operands per column, and the scaled conversion paths all run here."""
    tk = synth.gdn_cold(n_seg=2, n_chain=2, gate_scale=1.0 / 16)
    e = np.array([-20, -9, -3, 0, 5, 11, 17])[np.arange(tk.dv) % 7]
    tk.v = tk.v * np.exp2(e)
    g, U, S = gpu_build(tk)
    rg, rU, rS = oracle.build_pairs(DELTA, tk.offsets, tk.k, tk.v, tk.beta, tk.log_gate)
    tol = TOL[tk.dtype]
    Sg = np.asarray(host(S), np.float64)
    col_err = np.linalg.norm(Sg - rS, axis=-2) / np.linalg.norm(rS, axis=-2)  # [seg, chain, column]
    assert np.isfinite(Sg).all()
    worst = float(col_err.max())
    print("  max per-column rel err S %.2e" % worst, flush=True)
    assert worst <= tol, "column %s: %.3e" % (np.unravel_index(int(col_err.argmax()), col_err.shape), worst)
    assert_units_close("scaled_v.U", host(U), rU, tol)
    assert_g_close("scaled_v.g", host(g), rg, tol)


def test_explicit_workspace_reused_across_calls():
    """A caller-owned workspace of the queried size serves two different batches;
    results equal those of calls with their own workspace."""
    import torch
    tk = synth.gdn_cold(n_seg=4, L=256, n_chain=2)
    announce("explicit_ws")
    d = upload_tokens(tk)
    off = list(tk.offsets)
    need = api.seg_build_workspace_size(DELTA, off, 2, 128, torch.bfloat16)
    assert need == 4 * 4 * 2 * 8704
    ws = torch.full((need,), 0xAB, device="cuda", dtype=torch.uint8)
    g1, U1, S1 = api.seg_build(DELTA, off, d["k"], d["v"], d["beta"], d["log_gate"], workspace=ws)
    g2, U2, S2 = api.seg_build(DELTA, off[:3], d["k"][:off[2]], d["v"][:off[2]], d["beta"][:off[2]],
                               d["log_gate"][:off[2]], workspace=ws)
    g0, U0, S0 = api.seg_build(DELTA, off, d["k"], d["v"], d["beta"], d["log_gate"])
    torch.cuda.synchronize()
    assert torch.equal(S1, S0) and torch.equal(U1, U0) and torch.equal(g1, g0)
    assert torch.equal(S2, S0[:2]) and torch.equal(U2, U0[:2])
    with pytest.raises(api.HypicError, match="workspace too small"):
        api.seg_build(DELTA, off, d["k"], d["v"], d["beta"], d["log_gate"], workspace=ws[:need - 16])


def test_gdn_ragged_request_longest_first():
    """The ragged 32k-token cold request (64 segments of 58 .. 2048 tokens, 32
    heads), built with the longest segments' workgroups first: every unit
    against the oracle."""
    tk = synth.gdn_ragged()
    lens = np.diff(tk.offsets)
    assert lens.min() < 100 and lens.max() == 2048
    check_build(tk, "gdn_ragged32k")
