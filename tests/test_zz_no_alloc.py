"""hypic_seam_step_noalloc (the seam step on the library's fixed per-device
scratch) against hypic_seam_step with a caller workspace: two calls in a row,
the second with fewer segments and chains, each bit-identical to the entry
point it stands in for and within the bf16-token bound of the oracle."""
import numpy as np
import pytest

import oracle
from segment_scan_amd import api, synth
from segment_scan_amd.synth import DELTA, SCALAR
from tests.gpu_util import TOL, announce, assert_units_close, dev_f32, host, upload_tokens

pytestmark = pytest.mark.gpu


def _pair_of_calls(tw, body, S0, w):
    import torch
    up = upload_tokens(tw, with_q=True)
    n_tok, H = tw.k.shape[0], tw.n_chain
    b = tuple(None if x is None else dev_f32(x) for x in body)
    S_ref = dev_f32(S0)
    ref = api.seam_step(tw.fam, w, up["q"], up["k"], up["v"], up["beta"], up["log_gate"], tw.gate_per_chain,
                        body=b, S_run=S_ref)
    S_na = dev_f32(S0)
    o_na = torch.full((n_tok, H, 128), float("nan"), device="cuda")
    got = api.seam_step_noalloc(tw.fam, w, up["q"], up["k"], up["v"], up["beta"], up["log_gate"],
                                tw.gate_per_chain, body=b, S_run=S_na, o_out=o_na)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("kind", ["gdn", "retnet"])
def test_noalloc_matches_seam_step_two_calls(kind):
    w = 8
    for call, (n_seg, H) in enumerate([(24, 12), (9, 5)]):  # the second call smaller
        announce("noalloc", kind, "call", call, "segs", n_seg, "chains", H)
        if kind == "gdn":
            tw = synth.warm_seam_layer(20 + call, n_seg=n_seg, w=w, n_head=H)
            body = synth.warm_pairs_layer(20 + call, n_seg=n_seg, n_head=H)
        else:
            tw = synth.retnet(n_seg=n_seg, L=w, n_chain=H)
            tb = synth.retnet(n_seg=n_seg, L=40, n_chain=H)
            body = oracle.build_pairs(SCALAR, tb.offsets, tb.k, tb.v, None, tb.log_gate, True)
            body = tuple(None if x is None else x.astype(np.float32).astype(np.float64) for x in body)
        S0 = np.random.default_rng(30 + call).standard_normal((H, 128, 128)).astype(np.float32).astype(np.float64)
        ref, got = _pair_of_calls(tw, body, S0, w)
        import torch
        assert torch.equal(ref["S_run"], got["S_run"]), "S_run differs from hypic_seam_step"
        assert torch.equal(ref["o"], got["o"]), "o differs from hypic_seam_step"
        want = oracle.seam(tw.fam, n_seg, w, tw.q, tw.k, tw.v, tw.beta, tw.log_gate, tw.gate_per_chain, body=body,
                           S_run=S0)
        assert_units_close("noalloc.S_run", host(got["S_run"]), want["S_run"], TOL["bf16"], unit_dims=1)
        ow = host(got["o"]).reshape(n_seg, w, H, -1).transpose(0, 2, 1, 3)
        rw = want["o"].reshape(n_seg, w, H, -1).transpose(0, 2, 1, 3)
        assert_units_close("noalloc.o", ow, rw, TOL["bf16"])
