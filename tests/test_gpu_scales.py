"""GPU parity: value channels of very different sizes, on every dense build path, on
the dense composition and on the seam-window step.

The recurrences of the linear layers ([youleyou, linear-layer paragraph]; the
delta rule S <- a (I - b k k^T) S + b k v^T) act on each value channel on its
own (a column of S depends on its own channel of v only), so scaling channel j
by 2^e_j scales column j of every state by the same power of two.  With e_j running from -20 to 17, a
kernel whose fp16 operands share one scale across columns loses the small
columns; each column of S is therefore held to the tolerance on its own
(relative Frobenius error per column).  The d = 128 bf16 state pass has its own
such tests beside the delta and KDA builds.
"""
import numpy as np
import pytest

import oracle
from segment_scan_amd import api, synth
from segment_scan_amd.synth import DELTA, KDA
from tests.gpu_util import TOL, announce, dev_f32, host, upload_tokens

pytestmark = pytest.mark.gpu

EXPONENTS = np.array([-20, -9, -3, 0, 5, 11, 17])


def scale_values(tk):
    tk.v = tk.v * np.exp2(EXPONENTS[np.arange(tk.dv) % len(EXPONENTS)])
    return tk


def column_err(got, ref):
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all()
    return float((np.linalg.norm(got - ref, axis=-2) / np.linalg.norm(ref, axis=-2)).max())


CASES = {
    # segments over 2048 tokens take the one-kernel delta and KDA builds
    "delta_bf16_d128_one_kernel": (DELTA, lambda: synth.gdn_cold(n_seg=1, L=2304, n_chain=2, gate_scale=1 / 16)),
    "delta_f32_d128": (DELTA, lambda: synth.gdn_cold(n_seg=2, L=256, n_chain=2, dtype="f32", gate_scale=1 / 16)),
    "delta_bf16_d64": (DELTA, lambda: synth.gdn_cold(n_seg=2, L=256, n_chain=2, d=64, gate_scale=1 / 16)),
    "kda_bf16_d64": (KDA, lambda: synth.kda(n_seg=2, L=256, n_chain=2, d=64)),
    "kda_bf16_d128_one_kernel": (KDA, lambda: synth.kda(n_seg=1, L=2304, n_chain=2)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_build_columns_of_very_different_scales(case):
    import torch
    fam, make = CASES[case]
    tk = scale_values(make())
    announce(case, "dtype", tk.dtype, "chains", tk.n_chain, "d", tk.dk)
    d = upload_tokens(tk)
    g, U, S = api.seg_build(fam, list(tk.offsets), d["k"], d["v"], d["beta"], d["log_gate"])
    torch.cuda.synchronize()
    _, _, rS = oracle.build_pairs(fam, tk.offsets, tk.k, tk.v, tk.beta, tk.log_gate)
    err = column_err(host(S), rS)
    print("  max per-column rel err S %.2e" % err, flush=True)
    assert err <= TOL[tk.dtype]


def test_compose_columns_of_very_different_scales():
    """fp32 pairs (the oracle's, rounded to fp32) whose S columns span 2^37 in size,
    composed by the dense chain kernel: each column of S_out within the fp32 bound."""
    import torch
    tk = scale_values(synth.gdn_cold(n_seg=12, L=128, n_chain=2, dtype="f32", gate_scale=1 / 64))
    announce("compose_scaled_columns", "segs", 12, "chains", 2)
    g, U, S = oracle.build_pairs(DELTA, tk.offsets, tk.k, tk.v, tk.beta, tk.log_gate)
    g, U, S = np.float32(g), np.float32(U), np.float32(S)
    res = api.compose(DELTA, dev_f32(g), dev_f32(U), dev_f32(S))
    torch.cuda.synchronize()
    ref = oracle.compose(DELTA, g, U, S)["S_out"]
    err = column_err(host(res["S_out"]), ref)
    print("  max per-column rel err S_out %.2e" % err, flush=True)
    assert err <= TOL["f32"]


def test_seam_columns_of_very_different_scales():
    """Seam windows (w = 8, no body pairs) from a start state, values and start
    state scaled per value channel alike: each column of S_run and each output
    channel within the bf16 bound."""
    import torch
    n_seg, w, H = 6, 8, 4
    tk = scale_values(synth.warm_seam_layer(3, n_seg=n_seg, w=w, n_head=H))
    S0 = np.random.default_rng(1).standard_normal((H, tk.dk, tk.dv)).astype(np.float32).astype(np.float64)
    S0 = S0 * np.exp2(EXPONENTS[np.arange(tk.dv) % len(EXPONENTS)])
    announce("seam_scaled_columns", "segs", n_seg, "w", w, "chains", H)
    d = upload_tokens(tk, with_q=True)
    res = api.seam_step(DELTA, w, d["q"], d["k"], d["v"], d["beta"], d["log_gate"], S_run=dev_f32(S0))
    torch.cuda.synchronize()
    ref = oracle.seam(DELTA, n_seg, w, tk.q, tk.k, tk.v, tk.beta, tk.log_gate, S_run=S0)
    eS = column_err(host(res["S_run"]), ref["S_run"])
    o, ro = np.asarray(host(res["o"]), np.float64), ref["o"]  # [n_tok, n_chain, dv]
    assert np.isfinite(o).all()
    eo = float((np.linalg.norm(o - ro, axis=0) / np.linalg.norm(ro, axis=0)).max())
    print("  max per-column rel err S_run %.2e, per output channel %.2e" % (eS, eo), flush=True)
    assert eS <= TOL["bf16"] and eo <= TOL["bf16"]
