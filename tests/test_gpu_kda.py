"""GPU parity: KDA (delta rule with per-channel gates) segment build vs the oracle.

The library and the oracle split T_C = exp(g) U the same way (g is the sum
over tokens of each token's largest channel gate), so g, U and S(C|0) are
compared directly; U is also compared as exp(g_gpu - g_ref) U_gpu, the
transition on the oracle's scale.  Tolerances as for the other families: 2e-3
for bf16 tokens, 1e-5 for fp32 tokens (relative Frobenius per unit).
"""
import numpy as np
import pytest

import oracle
from segment_scan_amd import api, synth
from segment_scan_amd.synth import KDA
from tests.gpu_util import TOL, announce, assert_g_close, assert_units_close, host, upload_tokens

pytestmark = pytest.mark.gpu


def gpu_build(tk, offsets):
    import torch
    d = upload_tokens(tk)
    g, U, S = api.seg_build(KDA, list(offsets), d["k"], d["v"], d["beta"], d["log_gate"])
    torch.cuda.synchronize()
    return host(g), host(U), host(S)


def compare(name, g, U, S, rg, rU, rS, tol):
    eS = assert_units_close(name + ".S", S, rS, tol)
    assert_g_close(name + ".g", g, rg, tol)
    assert_units_close(name + ".U", U, rU, tol)
    Ts = np.exp(g - rg)[..., None, None] * U
    eT = assert_units_close(name + ".T", Ts, rU, tol)
    print("  max rel err S %.2e T %.2e" % (eS, eT), flush=True)


def check_build(tk, name, offsets=None):
    offsets = tk.offsets if offsets is None else np.asarray(offsets, np.int32)
    announce(name, "dtype", tk.dtype, "chains", tk.n_chain, "segs", len(offsets) - 1, "d", tk.dk)
    g, U, S = gpu_build(tk, offsets)
    rg, rU, rS = oracle.build_pairs(KDA, offsets, tk.k, tk.v, tk.beta, tk.log_gate)
    compare(name, g, U, S, rg, rU, rS, TOL[tk.dtype])
    return g, U, S


def test_kda_bf16_d128():
    """The cold request's recipe, 4 segments x 512 tokens, 4 heads."""
    tk = synth.kda(n_seg=4, n_chain=4)
    check_build(tk, "kda_bf16_d128")


@pytest.mark.parametrize("gate_scale", [1.0, 1.0 / 8, 1.0 / 64])
def test_kda_fp32_d64_ragged(gate_scale):
    """fp32 tokens (fp32 tolerance), segments of 1, 63, 64, 65, 130 and 200 tokens."""
    lengths = [1, 63, 64, 65, 130, 200]
    tk = synth.kda(n_seg=1, L=sum(lengths), n_chain=3, d=64, dtype="f32", gate_scale=gate_scale)
    check_build(tk, "kda_f32_%g" % gate_scale, synth.ragged_offsets(lengths))


def test_kda_bf16_d64():
    tk = synth.kda(n_seg=3, L=100, n_chain=2, d=64)
    check_build(tk, "kda_bf16_d64")


@pytest.mark.parametrize("pattern", ["half", "all"])
def test_kda_strong_and_zero_gates(pattern):
    """Gates of e^-30 per token on a random half of the (token, channel)
    entries and 1 on the rest, or e^-30 everywhere: every factor of the chunk
    form stays within [0, 1], so nothing overflows, and the decay is carried by
    g (hundreds of e-folds over a segment)."""
    tk = synth.kda(n_seg=2, L=130, n_chain=2, d=64, dtype="f32")
    r = np.random.default_rng(11)
    mask = (r.random(tk.log_gate.shape) < 0.5) if pattern == "half" else np.ones(tk.log_gate.shape, bool)
    tk.log_gate = np.where(mask, -30.0, 0.0)
    check_build(tk, "kda_strong_gates_" + pattern)


def test_kda_strong_gates_bf16_d128():
    """Strong and zero gates through the d = 128 factor-record path (fp16 decayed
    keys: entries decayed below fp16's range vanish, which the relative error
    of the unit does not see)."""
    tk = synth.kda(n_seg=2, L=130, n_chain=2)
    r = np.random.default_rng(12)
    tk.log_gate = np.where(r.random(tk.log_gate.shape) < 0.5, -30.0, 0.0)
    check_build(tk, "kda_strong_bf16_d128")


def test_kda_value_channels_of_very_different_scales():
    """Value channels scaled by powers of two from 2^-20 to 2^17 through the d = 128
    factor-record path: each column of S depends on its own value channel only and
    keeps the bf16 bound on its own (the state pass scales its operands per column)."""
    tk = synth.kda(n_seg=2, n_chain=2)
    e = np.array([-20, -9, -3, 0, 5, 11, 17])[np.arange(tk.dv) % 7]
    tk.v = tk.v * np.exp2(e)
    announce("kda_scaled_v", "chains", tk.n_chain, "segs", len(tk.offsets) - 1)
    g, U, S = gpu_build(tk, tk.offsets)
    rg, rU, rS = oracle.build_pairs(KDA, tk.offsets, tk.k, tk.v, tk.beta, tk.log_gate)
    tol = TOL[tk.dtype]
    S = np.asarray(S, np.float64)
    assert np.isfinite(S).all()
    col_err = np.linalg.norm(S - rS, axis=-2) / np.linalg.norm(rS, axis=-2)  # [seg, chain, column]
    worst = float(col_err.max())
    print("  max per-column rel err S %.2e" % worst, flush=True)
    assert worst <= tol, "column %s: %.3e" % (np.unravel_index(int(col_err.argmax()), col_err.shape), worst)
    assert_g_close("kda_scaled_v.g", g, rg, tol)
    assert_units_close("kda_scaled_v.U", U, rU, tol)


def test_kda_bf16_d128_ragged():
    """The factor-record path with segments that are not multiples of the
    64-token chunk (tail chunks of 1, 63, 1, 2 and 8 tokens, a 1-token segment)."""
    lengths = [1, 63, 64, 65, 130, 200]
    tk = synth.kda(n_seg=1, L=sum(lengths), n_chain=3, gate_scale=1.0 / 16)
    check_build(tk, "kda_ragged_d128", synth.ragged_offsets(lengths))


def test_kda_many_ragged_segments_two_launches():
    """300 ragged segments (1..130 tokens) on the factor-record path: two
    launches that reuse one workspace, sized for the larger."""
    rng = np.random.default_rng(5)
    lengths = [int(x) for x in rng.integers(1, 131, 300)]
    tk = synth.kda(n_seg=1, L=sum(lengths), n_chain=2, gate_scale=1.0 / 16)
    check_build(tk, "kda_300seg", synth.ragged_offsets(lengths))


def test_kda_longest_first_across_launches():
    """250 segments, the two longest (2100 and 2400 tokens) last in the batch:
    the first launch (longest first over the batch) holds them and takes the
    single-kernel path, the second launch the 10 shortest, the factor-record path."""
    rng = np.random.default_rng(6)
    lengths = [int(x) for x in rng.integers(1, 200, 248)] + [2100, 2400]
    tk = synth.kda(n_seg=1, L=sum(lengths), n_chain=2, gate_scale=1.0 / 16)
    check_build(tk, "kda_lpt_2launch", synth.ragged_offsets(lengths))


def test_kda_segment_lengths_of_both_paths():
    """2048 tokens (longest of the factor-record path) and 2049 (single kernel)."""
    for L in (2048, 2049):
        tk = synth.kda(n_seg=1, L=L, n_chain=2, gate_scale=1.0 / 64)
        check_build(tk, "kda_long_%d" % L)


def test_kda_build_then_compose_matches_sequential():
    """Cold path end to end on the GPU (KDA build, ordered dense composition)
    against straight recurrence over the whole request, with slow gates."""
    import torch
    tk = synth.kda(n_seg=6, L=192, n_chain=3, gate_scale=1.0 / 64)
    announce("kda_e2e")
    d = upload_tokens(tk)
    g, U, S = api.seg_build(KDA, list(tk.offsets), d["k"], d["v"], d["beta"], d["log_gate"])
    res = api.compose(KDA, g, U, S, want_prefix=True)
    torch.cuda.synchronize()
    Sseq, _ = oracle.sequential(KDA, tk.k, tk.v, tk.beta, tk.log_gate)
    assert_units_close("kda_e2e", host(res["S_out"]), Sseq, TOL["bf16"], unit_dims=1)


def test_kda_cold_full_size_every_unit():
    """The cold request's shape (32 heads x 64 segments x 512 tokens, d = 128,
    bf16) in the launch the benchmark times; every one of the 2048 units against
    one oracle pass over the whole request."""
    tk = synth.kda()
    announce("kda_full", "units", 64 * 32)
    g, U, S = gpu_build(tk, tk.offsets)
    rg, rU, rS = oracle.build_pairs(KDA, tk.offsets, tk.k, tk.v, tk.beta, tk.log_gate)
    compare("full", g, U, S, rg, rU, rS, TOL["bf16"])


def test_kda_seam_with_built_bodies_equals_sequential():
    """Warm reuse of a KDA layer end to end on the GPU: bodies built by the KDA
    build, then the seam step (window tokens on the running state, then each
    body pair) against straight recurrence over [window_0, body_0, window_1, ...]."""
    import torch
    n_seg, w, L, H = 5, 8, 100, 3
    tw = synth.kda(n_seg=n_seg, L=w, n_chain=H, gate_scale=1.0 / 32, want_q=True)
    tb = synth.kda(n_seg=n_seg, L=L, n_chain=H, gate_scale=1.0 / 32)
    tb.k, tb.v, tb.beta, tb.log_gate = tb.k[::-1].copy(), tb.v[::-1].copy(), tb.beta[::-1].copy(), \
        tb.log_gate[::-1].copy()  # other tokens than the windows'
    announce("kda_seam_e2e")
    db = upload_tokens(tb)
    body = api.seg_build(KDA, list(tb.offsets), db["k"], db["v"], db["beta"], db["log_gate"])
    dw = upload_tokens(tw, with_q=True)
    res = api.seam_step(KDA, w, dw["q"], dw["k"], dw["v"], dw["beta"], dw["log_gate"], body=body)
    torch.cuda.synchronize()
    order = []
    for s in range(n_seg):
        order += [("w", s * w + j) for j in range(w)]
        order += [("b", t) for t in range(tb.offsets[s], tb.offsets[s + 1])]
    cat = lambda key: np.stack([getattr(tw if src == "w" else tb, key)[i] for src, i in order])
    q = np.stack([tw.q[i] if src == "w" else np.zeros_like(tw.q[0]) for src, i in order])  # bodies emit nothing
    Sseq, oseq = oracle.sequential(KDA, cat("k"), cat("v"), cat("beta"), cat("log_gate"), q=q)
    assert_units_close("kda_seam_e2e.S", host(res["S_run"]), Sseq, TOL["bf16"], unit_dims=1)
    wpos = [p for p, (src, _) in enumerate(order) if src == "w"]
    ow = host(res["o"]).reshape(n_seg, w, H, -1).transpose(0, 2, 1, 3)
    rw = oseq[wpos].reshape(n_seg, w, H, -1).transpose(0, 2, 1, 3)
    assert_units_close("kda_seam_e2e.o", ow, rw, TOL["bf16"])
