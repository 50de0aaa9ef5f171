"""GPU parity: seam-window step (fused with the body-pair composition) vs the oracle."""
import numpy as np
import pytest

import oracle
from segment_scan_amd import api, synth
from segment_scan_amd.synth import DELTA
from tests.gpu_util import TOL, announce, assert_units_close, dev_f32, host, upload_tokens

pytestmark = pytest.mark.gpu


def run_seam(tk, w, body=None, S0=None):
    import torch
    d = upload_tokens(tk, with_q=True)
    S_run = dev_f32(S0) if S0 is not None else None
    b = None if body is None else tuple(dev_f32(x) for x in body)
    res = api.seam_step(DELTA, w, d["q"], d["k"], d["v"], d["beta"], d["log_gate"], body=b, S_run=S_run)
    torch.cuda.synchronize()
    return host(res["S_run"]), host(res["o"])


def check_seam(tk, w, body, S0, name, tol):
    n_seg = tk.n_tok // w
    announce(name, "chains", tk.n_chain, "segs", n_seg, "w", w, "body", body is not None)
    S_run, o = run_seam(tk, w, body, S0)
    ref = oracle.seam(DELTA, n_seg, w, tk.q, tk.k, tk.v, tk.beta, tk.log_gate, body=body, S_run=S0)
    eS = assert_units_close(name + ".S_run", S_run, ref["S_run"], tol, unit_dims=1)
    # outputs per (segment, chain) window
    ow = o.reshape(n_seg, w, tk.n_chain, -1).transpose(0, 2, 1, 3)
    rw = ref["o"].reshape(n_seg, w, tk.n_chain, -1).transpose(0, 2, 1, 3)
    eo = assert_units_close(name + ".o", ow, rw, tol)
    print("  max rel err S %.2e o %.2e" % (eS, eo), flush=True)


def test_warm_reuse_one_layer():
    """One of the 30 layers of the warm 100k-token request: 16 heads, 196 segments, w = 8,
    random fp32 body pairs, bf16 window tokens, zero start."""
    tk = synth.warm_seam_layer(0)
    body = synth.warm_pairs_layer(0)
    check_seam(tk, 8, body, None, "warm_layer0", TOL["bf16"])


@pytest.mark.parametrize("w", [8, 5, 20])
def test_windows_only(w):
    """No body pairs: the window recurrence alone, sub-chunk boundaries at 16 tokens."""
    tk = synth.warm_seam_layer(3, n_seg=6, w=w, n_head=4)
    S0 = np.random.default_rng(1).standard_normal((4, 128, 128)).astype(np.float32).astype(np.float64)
    check_seam(tk, w, None, S0, "windows_w%d" % w, TOL["bf16"])


def test_seam_with_built_bodies_equals_sequential():
    """Body pairs from the oracle's build of the segment bodies: the fused seam
    step must reproduce straight recurrence over [window_0, body_0, window_1, ...]."""
    n_seg, w, L, H = 5, 8, 120, 4
    tw = synth.warm_seam_layer(7, n_seg=n_seg, w=w, n_head=H, gate_scale=1.0 / 64)
    tb = synth.gdn_cold(n_seg=n_seg, L=L, n_chain=H, gate_scale=1.0 / 64)
    body = oracle.build_pairs(DELTA, tb.offsets, tb.k, tb.v, tb.beta, tb.log_gate)
    body32 = tuple(x.astype(np.float32).astype(np.float64) for x in body)
    check_seam(tw, w, body32, None, "built_bodies", TOL["bf16"])


def test_seam_fp32_d64():
    tk = synth.gdn_tiny(n_seg=1, L=4 * 8, gate_scale=1.0 / 16)
    body = synth.warm_pairs_layer(9, n_seg=4, n_head=1, d=64)
    S0 = np.random.default_rng(2).standard_normal((1, 64, 64)).astype(np.float32).astype(np.float64)
    check_seam(tk, 8, body, S0, "seam_f32_d64", TOL["f32"])


def test_warm_reuse_full_size_layers_0_and_29():
    """The full warm request (30 layers x 16 heads = 480 chains) in one launch, as
    the benchmark runs it; layers 0 and 29 are compared element by element."""
    import torch
    parts, pairs = [], []
    for layer in range(synth.WARM_LAYERS):
        if layer in (0, 29):
            parts.append(synth.warm_seam_layer(layer))
            pairs.append(synth.warm_pairs_layer(layer))
    # layers other than 0 and 29 get the same recipe drawn on the GPU (not compared)
    announce("warm_full", "chains", 480)
    H, d, n_seg, w = synth.WARM_HEADS, synth.WARM_D, synth.WARM_SEGS, synth.WARM_W
    gen = torch.Generator(device="cuda").manual_seed(5)
    q = torch.randn((n_seg * w, 480, d), device="cuda", generator=gen)
    q = torch.nn.functional.normalize(q, dim=-1).to(torch.bfloat16)
    k = torch.nn.functional.normalize(torch.randn((n_seg * w, 480, d), device="cuda", generator=gen), dim=-1).to(torch.bfloat16)
    v = torch.randn((n_seg * w, 480, d), device="cuda", generator=gen).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn((n_seg * w, 480), device="cuda", generator=gen)).to(torch.bfloat16)
    lg = (-torch.nn.functional.softplus(torch.randn((n_seg * w, 480), device="cuda", generator=gen)) / 8).to(torch.bfloat16)
    U = torch.randn((n_seg, 480, d, d), device="cuda", generator=gen) * (0.5 / np.sqrt(d))
    S = torch.randn((n_seg, 480, d, d), device="cuda", generator=gen)
    g = torch.zeros((n_seg, 480), device="cuda")
    for li, layer in enumerate((0, 29)):
        sl = slice(layer * H, (layer + 1) * H)
        tk = parts[li]
        up = upload_tokens(tk, with_q=True)
        q[:, sl], k[:, sl], v[:, sl], beta[:, sl], lg[:, sl] = up["q"], up["k"], up["v"], up["beta"], up["log_gate"]
        U[:, sl] = dev_f32(pairs[li][1])
        S[:, sl] = dev_f32(pairs[li][2])
    res = api.seam_step(DELTA, w, q, k, v, beta, lg, body=(g, U, S))
    torch.cuda.synchronize()
    S_run, o = host(res["S_run"]), host(res["o"])
    for li, layer in enumerate((0, 29)):
        sl = slice(layer * H, (layer + 1) * H)
        tk = parts[li]
        ref = oracle.seam(DELTA, n_seg, w, tk.q, tk.k, tk.v, tk.beta, tk.log_gate, body=pairs[li])
        assert_units_close("full.S_run.l%d" % layer, S_run[sl], ref["S_run"], TOL["bf16"], unit_dims=1)
        ow = o[:, sl].reshape(n_seg, w, H, -1).transpose(0, 2, 1, 3)
        rw = ref["o"].reshape(n_seg, w, H, -1).transpose(0, 2, 1, 3)
        assert_units_close("full.o.l%d" % layer, ow, rw, TOL["bf16"])


def test_kda_warm_reuse_full_size_layers_0_and_29():
    """The warm request with KDA layers (480 chains, per-channel gates) in one
    launch, as the benchmark runs it; layers 0 and 29 compared element by element."""
    import torch
    from segment_scan_amd.synth import KDA
    H, d, n_seg, w = synth.WARM_HEADS, synth.WARM_D, synth.WARM_SEGS, synth.WARM_W
    announce("kda_warm_full", "chains", 480)
    gen = torch.Generator(device="cuda").manual_seed(6)
    nt = n_seg * w
    q = torch.nn.functional.normalize(torch.randn((nt, 480, d), device="cuda", generator=gen), dim=-1).to(torch.bfloat16)
    k = torch.nn.functional.normalize(torch.randn((nt, 480, d), device="cuda", generator=gen), dim=-1).to(torch.bfloat16)
    v = torch.randn((nt, 480, d), device="cuda", generator=gen).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn((nt, 480), device="cuda", generator=gen)).to(torch.bfloat16)
    lg = (-torch.nn.functional.softplus(torch.randn((nt, 480, d), device="cuda", generator=gen)) / 8).to(torch.bfloat16)
    U = torch.randn((n_seg, 480, d, d), device="cuda", generator=gen) * (0.5 / np.sqrt(d))
    S = torch.randn((n_seg, 480, d, d), device="cuda", generator=gen)
    g = torch.zeros((n_seg, 480), device="cuda")
    layers = (0, 29)
    parts = [synth.warm_seam_layer_kda(layer) for layer in layers]
    pairs = [synth.warm_pairs_layer(layer) for layer in layers]
    for li, layer in enumerate(layers):
        sl = slice(layer * H, (layer + 1) * H)
        up = upload_tokens(parts[li], with_q=True)
        q[:, sl], k[:, sl], v[:, sl], beta[:, sl], lg[:, sl] = up["q"], up["k"], up["v"], up["beta"], up["log_gate"]
        U[:, sl] = dev_f32(pairs[li][1])
        S[:, sl] = dev_f32(pairs[li][2])
    res = api.seam_step(KDA, w, q, k, v, beta, lg, body=(g, U, S))
    torch.cuda.synchronize()
    S_run, o = host(res["S_run"]), host(res["o"])
    for li, layer in enumerate(layers):
        sl = slice(layer * H, (layer + 1) * H)
        tk = parts[li]
        ref = oracle.seam(KDA, n_seg, w, tk.q, tk.k, tk.v, tk.beta, tk.log_gate, body=pairs[li])
        assert_units_close("kda_full.S_run.l%d" % layer, S_run[sl], ref["S_run"], TOL["bf16"], unit_dims=1)
        ow = o[:, sl].reshape(n_seg, w, H, -1).transpose(0, 2, 1, 3)
        rw = ref["o"].reshape(n_seg, w, H, -1).transpose(0, 2, 1, 3)
        assert_units_close("kda_full.o.l%d" % layer, ow, rw, TOL["bf16"])


def test_seam_many_chains_ragged_window():
    """72 chains (one workgroup per chain), w = 13 (a full and a partial
    8-token sub-chunk), random body pairs, nonzero start state."""
    tk = synth.warm_seam_layer(9, n_seg=3, w=13, n_head=72)
    body = synth.warm_pairs_layer(9, n_seg=3, n_head=72)
    S0 = np.random.default_rng(9).standard_normal((72, 128, 128)).astype(np.float32).astype(np.float64)
    check_seam(tk, 13, body, S0, "many_chains_w13", TOL["bf16"])


def _family_tokens(kind, n_seg, L, n_chain, d=128, dtype="bf16"):
    if kind == "naive":
        return synth.naive(n_seg=n_seg, L=L, n_chain=n_chain, d=d, dtype=dtype)
    if kind == "retnet":
        return synth.retnet(n_seg=n_seg, L=L, n_chain=n_chain, d=d, dtype=dtype)
    if kind == "mamba2":
        return synth.mamba2_like(n_seg=n_seg, L=L, n_chain=n_chain, d=d, dtype=dtype)
    if kind == "gla":
        return synth.gla(n_seg=n_seg, L=L, n_chain=n_chain, d=d, dtype=dtype)
    if kind == "kda":
        return synth.kda(n_seg=n_seg, L=L, n_chain=n_chain, d=d, dtype=dtype, want_q=True)
    return synth.warm_seam_layer(11, n_seg=n_seg, w=L, n_head=n_chain, d=d, dtype=dtype, gate_scale=1.0 / 16)


def _check_family_seam(kind, w, d, dtype, tol):
    import torch
    n_seg, H = 5, 4
    tw = _family_tokens(kind, n_seg, w, H, d, dtype)  # the windows
    tb = _family_tokens(kind, n_seg, 40, H, d, dtype)  # segment bodies -> cached pairs
    fam = tw.fam
    offs = synth.even_offsets(n_seg, 40)
    body = oracle.build_pairs(fam, offs, tb.k, tb.v, tb.beta, tb.log_gate, bool(tb.gate_per_chain))
    body32 = tuple(None if x is None else x.astype(np.float32).astype(np.float64) for x in body)
    S0 = np.random.default_rng(3).standard_normal((H, d, d)).astype(np.float32).astype(np.float64)
    announce("family_seam", kind, "w", w, "d", d, dtype)
    up = upload_tokens(tw, with_q=True)
    res = api.seam_step(fam, w, up["q"], up["k"], up["v"], up["beta"], up["log_gate"], bool(tw.gate_per_chain),
                        body=tuple(None if x is None else dev_f32(x) for x in body32), S_run=dev_f32(S0),
                        want_window_pairs=True)
    torch.cuda.synchronize()
    ref = oracle.seam(fam, n_seg, w, tw.q, tw.k, tw.v, tw.beta, tw.log_gate, bool(tw.gate_per_chain), body=body32,
                      S_run=S0, want_window_pairs=True)
    assert_units_close(kind + ".S_run", host(res["S_run"]), ref["S_run"], tol, unit_dims=1)
    ow = host(res["o"]).reshape(n_seg, w, H, -1).transpose(0, 2, 1, 3)
    rw = ref["o"].reshape(n_seg, w, H, -1).transpose(0, 2, 1, 3)
    assert_units_close(kind + ".o", ow, rw, tol)
    assert_units_close(kind + ".wS", host(res["wS"]), ref["wS"], tol)
    np.testing.assert_allclose(host(res["wg"]), ref["wg"], rtol=tol, atol=tol)
    if ref["wU"] is not None:
        assert_units_close(kind + ".wU", host(res["wU"]), ref["wU"], tol)


@pytest.mark.parametrize("kind", ["naive", "retnet", "mamba2", "gla", "gdn", "kda"])
@pytest.mark.parametrize("w", [8, 13])
def test_seam_every_family_with_window_pairs(kind, w):
    """Window recurrence + body pairs of every family, and each window's own pair."""
    _check_family_seam(kind, w, 128, "bf16", TOL["bf16"])


@pytest.mark.parametrize("kind", ["retnet", "gla", "gdn", "kda"])
def test_seam_families_fp32_d64(kind):
    _check_family_seam(kind, 5, 64, "f32", TOL["f32"])
