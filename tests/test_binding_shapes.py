"""The Python binding checks every tensor's shape against the counts it hands
to the library, before any pointer reaches it (no GPU needed: the tensors here
live on the host, so a call that passed the shape checks would stop at the
device check instead, and nothing is ever launched)."""
import pytest
import torch

from segment_scan_amd import api
from segment_scan_amd.synth import DELTA, DIAG, SCALAR

N_TOK, H, D, N_SEG = 128, 3, 64, 2
OFF = [0, 64, 128]


def t(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def bf(*shape):
    return t(*shape, dtype=torch.bfloat16)


def test_seg_build_shapes():
    k, v, b, lg = bf(N_TOK, H, D), bf(N_TOK, H, D), bf(N_TOK, H), bf(N_TOK, H)
    with pytest.raises(ValueError, match="offsets must end"):
        api.seg_build(DELTA, [0, 64, 200], k, v, b, lg)
    with pytest.raises(ValueError, match="v has shape"):
        api.seg_build(DELTA, OFF, k, bf(N_TOK, H, D + 1), b, lg)
    with pytest.raises(ValueError, match="beta has shape"):
        api.seg_build(DELTA, OFF, k, v, bf(N_TOK - 1, H), lg)
    with pytest.raises(ValueError, match="log_gate has shape"):
        api.seg_build(DIAG, OFF, k, v, None, bf(N_TOK, H))
    with pytest.raises(ValueError, match="log_gate has shape"):
        api.seg_build(SCALAR, OFF, k, v, None, t(H + 1), gate_per_chain=True)
    out = (t(N_SEG, H), t(N_SEG, H, D, D), t(N_SEG, H, D, D - 1))
    with pytest.raises(ValueError, match="out.S has shape"):
        api.seg_build(DELTA, OFF, k, v, b, lg, out=out)
    out = (t(N_SEG, H), t(N_SEG, H, D, D, dtype=torch.float64), t(N_SEG, H, D, D))
    with pytest.raises(ValueError, match="out.U has dtype"):
        api.seg_build(DELTA, OFF, k, v, b, lg, out=out)
    # well-formed: stops at the device check, after the shape checks
    with pytest.raises(ValueError, match="GPU device"):
        api.seg_build(DELTA, OFF, k, v, b, lg)


def test_compose_shapes():
    g, U, S = t(N_SEG, H), t(N_SEG, H, D, D), t(N_SEG, H, D, D)
    with pytest.raises(ValueError, match="pairs.U has shape"):
        api.compose(DELTA, g, t(N_SEG + 1, H, D, D), S)
    with pytest.raises(ValueError, match="pairs.g has shape"):
        api.compose(DIAG, g, None, S)
    with pytest.raises(ValueError, match="S_init has shape"):
        api.compose(DELTA, g, U, S, S_init=t(H + 1, D, D))
    with pytest.raises(ValueError, match="prefix_states has shape"):
        api.compose(DELTA, g, U, S, prefix_states=t(N_SEG - 1, H, D, D))
    with pytest.raises(ValueError, match="U_total has shape"):
        api.compose(DELTA, g, U, S, U_total=t(H, D, D + 1))
    with pytest.raises(ValueError, match="GPU device"):
        api.compose(DELTA, g, U, S, workspace=None)


def test_seam_step_shapes():
    w = 8
    n_tok = N_SEG * w
    q, k, v, b, lg = bf(n_tok, H, D), bf(n_tok, H, D), bf(n_tok, H, D), bf(n_tok, H), bf(n_tok, H)
    body = (t(N_SEG, H), t(N_SEG, H, D, D), t(N_SEG, H, D, D))
    with pytest.raises(ValueError, match="n_seg \\* w"):
        api.seam_step(DELTA, 5, q, k, v, b, lg, body=body)
    with pytest.raises(ValueError, match="q has shape"):
        api.seam_step(DELTA, w, bf(n_tok, H, D - 1), k, v, b, lg, body=body)
    with pytest.raises(ValueError, match="body.S has shape"):
        api.seam_step(DELTA, w, q, k, v, b, lg, body=(body[0], body[1], t(N_SEG + 1, H, D, D)))
    with pytest.raises(ValueError, match="S_run has shape"):
        api.seam_step(DELTA, w, q, k, v, b, lg, body=body, S_run=t(H, D, D - 1))
    with pytest.raises(ValueError, match="o_out has shape"):
        api.seam_step(DELTA, w, q, k, v, b, lg, body=body, o_out=t(n_tok - 1, H, D))
    with pytest.raises(ValueError, match="o_out has shape"):
        api.seam_step_noalloc(DELTA, w, q, k, v, b, lg, body=body, S_run=t(H, D, D), o_out=t(n_tok, H + 1, D))
    with pytest.raises(ValueError, match="GPU device"):
        api.seam_step_noalloc(DELTA, w, q, k, v, b, lg, body=body, S_run=t(H, D, D), o_out=t(n_tok, H, D))


def test_rerotate_shapes():
    S = t(N_SEG, H, D, D)
    pos = torch.zeros(N_SEG, dtype=torch.int32)
    with pytest.raises(ValueError, match="U has shape"):
        api.rerotate(DELTA, pos, S, t(N_SEG, H, D, D + 1))
    with pytest.raises(ValueError, match="positions"):
        api.rerotate(DELTA, torch.zeros(N_SEG + 1, dtype=torch.int32), S)
