"""Seeded synthetic inputs for the segment build, composition and seam step.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no arithmetic of the method itself: it only draws random numbers with
the distributions of the workloads and rounds them to the storage dtype.
Every array it returns is fp64 holding values that are exactly representable
in the stated dtype (bf16 or fp32), so the fp64 oracle and the HIP path read
bit-identical inputs.

Random numbers come from numpy's PCG64 seeded with
SeedSequence([20260701, workload_id, tensor_id, layer]).  Values are drawn in
fp64 and rounded to fp32 (round-to-nearest-even); bf16 values are then rounded
from that fp32 value (round-to-nearest-even on the upper 16 bits).

The workloads follow the shapes the pages describe: segments of several
hundred tokens (the seam window is small beside segments usually longer than
512 tokens), a 32k-token cold request, a ~100k-token warm request over 30
linear layers of a hybrid model.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

NAIVE, SCALAR, DIAG, DELTA, KDA = 0, 1, 2, 3, 4
FAMILY_NAMES = {NAIVE: "naive", SCALAR: "scalar", DIAG: "diag", DELTA: "delta", KDA: "kda"}

# tensor ids inside the seed sequence
T_Q, T_K, T_V, T_BETA, T_GATE, T_PG, T_PU, T_PS, T_SINIT, T_LEN = range(10)
SEED_ROOT = 20260701


def rng(workload: int, tensor: int, layer: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, workload, tensor, layer])))


def round_f32(x) -> np.ndarray:
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def _rne_bf16_u32(u: np.ndarray) -> np.ndarray:
    """In place: fp32 bit patterns (uint32) rounded to bf16 (nearest, ties to even),
    low 16 bits cleared.  Finite inputs only."""
    t = u >> 16
    t &= 1
    t += 0x7FFF
    u += t
    u &= np.uint32(0xFFFF0000)
    return u


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.array(x32, dtype=np.float32).view(np.uint32)
    return (_rne_bf16_u32(u) >> 16).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    u = np.asarray(x, np.float64).astype(np.float32).view(np.uint32)
    return _rne_bf16_u32(u).view(np.float32).astype(np.float64)


def round_to(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    raise ValueError(dtype)


def _l2n(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


@dataclass
class Tokens:
    """Token inputs in the library's layout: [n_tok, n_chain, d], token-major."""

    fam: int
    dtype: str
    n_chain: int
    dk: int
    dv: int
    k: np.ndarray
    v: np.ndarray
    q: Optional[np.ndarray] = None
    beta: Optional[np.ndarray] = None
    log_gate: Optional[np.ndarray] = None
    gate_per_chain: bool = False
    offsets: Optional[np.ndarray] = None  # int32 [n_seg + 1] (builds); None for seam windows
    meta: dict = field(default_factory=dict)

    @property
    def n_tok(self) -> int:
        return int(self.k.shape[0])

    def chains(self, idx) -> "Tokens":
        """Sub-batch restricted to the given chain indices (same tokens and offsets)."""
        idx = np.asarray(idx)
        sel = lambda a: None if a is None else a[:, idx]
        lg = self.log_gate
        if lg is not None:
            lg = lg[idx] if self.gate_per_chain else lg[:, idx]
        return Tokens(self.fam, self.dtype, int(idx.size), self.dk, self.dv, sel(self.k), sel(self.v),
                      sel(self.q), sel(self.beta), lg, self.gate_per_chain, self.offsets, dict(self.meta))


def even_offsets(n_seg: int, L: int) -> np.ndarray:
    return (np.arange(n_seg + 1, dtype=np.int64) * L).astype(np.int32)


def _draw_delta_tokens(workload, n_tok, n_chain, d, dtype, gate_scale, layer=0, want_q=True):
    """GDN-style tokens: unit keys/queries, N(0,1) values, beta = sigmoid(N), log alpha = -softplus(N)*scale."""
    shape = (n_tok, n_chain, d)
    k = round_to(_l2n(rng(workload, T_K, layer).standard_normal(shape)), dtype)
    v = round_to(rng(workload, T_V, layer).standard_normal(shape), dtype)
    beta = round_to(_sigmoid(rng(workload, T_BETA, layer).standard_normal((n_tok, n_chain))), dtype)
    lg = None
    if gate_scale is not None:
        lg = round_to(-_softplus(rng(workload, T_GATE, layer).standard_normal((n_tok, n_chain))) * gate_scale,
                      dtype)
    q = round_to(_l2n(rng(workload, T_Q, layer).standard_normal(shape)), dtype) if want_q else None
    return q, k, v, beta, lg


def gdn_tiny(n_seg=4, L=256, gate_scale=1.0, dtype="f32") -> Tokens:
    """Tiny GDN check: 1 layer, 1 head, d=64, 4 segments x 256 tokens, fp32.

    gate_scale multiplies log alpha (0.0 gives DeltaNet, alpha = 1)."""
    n_tok = n_seg * L
    q, k, v, beta, lg = _draw_delta_tokens(1, n_tok, 1, 64, dtype, gate_scale)
    return Tokens(DELTA, dtype, 1, 64, 64, k, v, q, beta, lg, False, even_offsets(n_seg, L),
                  {"workload": "gdn_tiny", "n_seg": n_seg, "L": L, "gate_scale": gate_scale})


def retnet_gammas(n_chain=8) -> np.ndarray:
    """Per-head decays with 1 - gamma log-spaced from 1e-1 to 1e-4 (0.9 .. 0.9999)."""
    h = np.arange(n_chain, dtype=np.float64)
    return 1.0 - 10.0 ** (-(1.0 + 3.0 * h / max(n_chain - 1, 1)))


def retnet(n_seg=16, L=1024, n_chain=8, d=128, dtype="bf16") -> Tokens:
    """RetNet-style scalar decay: q,k,v ~ N(0,1)/sqrt(d), fp32 log gamma per head."""
    n_tok = n_seg * L
    shape = (n_tok, n_chain, d)
    s = 1.0 / np.sqrt(d)
    q = round_to(rng(2, T_Q).standard_normal(shape) * s, dtype)
    k = round_to(rng(2, T_K).standard_normal(shape) * s, dtype)
    v = round_to(rng(2, T_V).standard_normal(shape) * s, dtype)
    lg = round_f32(np.log(retnet_gammas(n_chain)))
    return Tokens(SCALAR, dtype, n_chain, d, d, k, v, q, None, lg, True, even_offsets(n_seg, L),
                  {"workload": "retnet", "n_seg": n_seg, "L": L})


def mamba2_like(n_seg=4, L=256, n_chain=4, d=128, dtype="bf16", gate_scale=1.0 / 8) -> Tokens:
    """Scalar data-dependent decay per token (Mamba2-style): log a = -softplus(N)*scale."""
    n_tok = n_seg * L
    shape = (n_tok, n_chain, d)
    s = 1.0 / np.sqrt(d)
    q = round_to(rng(6, T_Q).standard_normal(shape) * s, dtype)
    k = round_to(rng(6, T_K).standard_normal(shape) * s, dtype)
    v = round_to(rng(6, T_V).standard_normal(shape), dtype)
    lg = round_to(-_softplus(rng(6, T_GATE).standard_normal((n_tok, n_chain))) * gate_scale, dtype)
    return Tokens(SCALAR, dtype, n_chain, d, d, k, v, q, None, lg, False, even_offsets(n_seg, L),
                  {"workload": "mamba2_like", "n_seg": n_seg, "L": L})


def gla(n_seg=64, L=512, n_chain=16, d=128, dtype="bf16", gate_scale=1.0 / 16) -> Tokens:
    """GLA diagonal gating: k,v ~ N(0,1)/sqrt(d); log alpha = -softplus(N)*scale per channel."""
    n_tok = n_seg * L
    shape = (n_tok, n_chain, d)
    s = 1.0 / np.sqrt(d)
    q = round_to(rng(3, T_Q).standard_normal(shape) * s, dtype)
    k = round_to(rng(3, T_K).standard_normal(shape) * s, dtype)
    v = round_to(rng(3, T_V).standard_normal(shape) * s, dtype)
    lg = round_to(-_softplus(rng(3, T_GATE).standard_normal(shape)) * gate_scale, dtype)
    return Tokens(DIAG, dtype, n_chain, d, d, k, v, q, None, lg, False, even_offsets(n_seg, L),
                  {"workload": "gla", "n_seg": n_seg, "L": L, "gate_scale": gate_scale})


def naive(n_seg=4, L=256, n_chain=4, d=128, dtype="bf16") -> Tokens:
    """Naive linear attention (no decay): k,v ~ N(0,1)/sqrt(d)."""
    n_tok = n_seg * L
    shape = (n_tok, n_chain, d)
    s = 1.0 / np.sqrt(d)
    q = round_to(rng(7, T_Q).standard_normal(shape) * s, dtype)
    k = round_to(rng(7, T_K).standard_normal(shape) * s, dtype)
    v = round_to(rng(7, T_V).standard_normal(shape) * s, dtype)
    return Tokens(NAIVE, dtype, n_chain, d, d, k, v, q, None, None, False, even_offsets(n_seg, L),
                  {"workload": "naive", "n_seg": n_seg, "L": L})


def gdn_cold(n_seg=64, L=512, n_chain=32, d=128, dtype="bf16", gate_scale=1.0 / 8, want_q=True) -> Tokens:
    """GDN dense transition, one 32k-token cold request: 32 heads x 64 segments x 512 tokens."""
    n_tok = n_seg * L
    q, k, v, beta, lg = _draw_delta_tokens(4, n_tok, n_chain, d, dtype, gate_scale, want_q=want_q)
    return Tokens(DELTA, dtype, n_chain, d, d, k, v, q, beta, lg, False, even_offsets(n_seg, L),
                  {"workload": "gdn_cold32k", "n_seg": n_seg, "L": L, "gate_scale": gate_scale})


def kda(n_seg=64, L=512, n_chain=32, d=128, dtype="bf16", gate_scale=1.0 / 8, want_q=False) -> Tokens:
    """KDA (delta rule with per-channel gates), the cold request's shape: unit
    keys and queries, v ~ N(0,1), beta = sigmoid(N), log alpha = -softplus(N) *
    scale drawn per token and key channel."""
    n_tok = n_seg * L
    q, k, v, beta, _ = _draw_delta_tokens(14, n_tok, n_chain, d, dtype, None, want_q=want_q)
    lg = round_to(-_softplus(rng(14, T_GATE).standard_normal((n_tok, n_chain, d))) * gate_scale, dtype)
    return Tokens(KDA, dtype, n_chain, d, d, k, v, q, beta, lg, False, even_offsets(n_seg, L),
                  {"workload": "kda_cold32k", "n_seg": n_seg, "L": L, "gate_scale": gate_scale})


def ragged_lengths(n_seg: int, total: int, workload: int = 12, sigma: float = 0.9, min_len: int = 32,
                   max_len: int = 2048):
    """Uneven segment lengths summing to `total`: log-normal shares (log-sd
    sigma), clipped to [min_len, max_len]; the rounding remainder goes to the
    segments in index order, each up to max_len."""
    w = np.exp(rng(workload, T_LEN).standard_normal(n_seg) * sigma)
    lens = np.clip(np.floor(w / w.sum() * total), min_len, max_len).astype(np.int64)
    rest = total - int(lens.sum())
    for i in range(n_seg):
        step = int(np.clip(rest, min_len - lens[i], max_len - lens[i]))
        lens[i] += step
        rest -= step
    assert rest == 0 and lens.min() >= min_len and lens.max() <= max_len and int(lens.sum()) == total
    return lens


def gdn_ragged(n_seg=64, n_chain=32, d=128, total=32768, dtype="bf16", gate_scale=1.0 / 8, want_q=False) -> Tokens:
    """The 32k-token cold GDN request with uneven segments (ragged_lengths)."""
    tk = gdn_cold(n_seg=n_seg, L=total // n_seg, n_chain=n_chain, d=d, dtype=dtype, gate_scale=gate_scale,
                  want_q=want_q)
    t = with_offsets(tk, ragged_offsets(ragged_lengths(n_seg, total)))
    t.meta = {**tk.meta, "workload": "gdn_ragged32k", "lengths": "log-normal, sigma 0.9"}
    return t


def ragged_offsets(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))]).astype(np.int32)


def with_offsets(tok: Tokens, offsets) -> Tokens:
    offsets = np.asarray(offsets, np.int32)
    assert offsets[-1] == tok.n_tok
    t = Tokens(**{**tok.__dict__})
    t.offsets = offsets
    return t


# ---- warm reuse: 30 GDN layers x 16 heads, 196 cached segments, w = 8 ---------

WARM_LAYERS, WARM_HEADS, WARM_SEGS, WARM_W, WARM_D = 30, 16, 196, 8, 128


def warm_pairs_layer(layer: int, n_seg=WARM_SEGS, n_head=WARM_HEADS, d=WARM_D):
    """Random cached body pairs of one layer: g = 0, U ~ N(0, 1/(4d)), S ~ N(0, 1), fp32."""
    g = np.zeros((n_seg, n_head), np.float64)
    U = round_f32(rng(5, T_PU, layer).standard_normal((n_seg, n_head, d, d)) * (0.5 / np.sqrt(d)))
    S = round_f32(rng(5, T_PS, layer).standard_normal((n_seg, n_head, d, d)))
    return g, U, S


def warm_seam_layer(layer: int, n_seg=WARM_SEGS, w=WARM_W, n_head=WARM_HEADS, d=WARM_D, dtype="bf16",
                    gate_scale=1.0 / 8) -> Tokens:
    """Seam-window tokens of one layer: [n_seg*w, n_head, d], GDN distributions (bf16)."""
    q, k, v, beta, lg = _draw_delta_tokens(5, n_seg * w, n_head, d, dtype, gate_scale, layer=layer)
    return Tokens(DELTA, dtype, n_head, d, d, k, v, q, beta, lg, False, None,
                  {"workload": "gdn_warm100k", "layer": layer, "n_seg": n_seg, "w": w})


def warm_seam_layer_kda(layer: int, n_seg=WARM_SEGS, w=WARM_W, n_head=WARM_HEADS, d=WARM_D, dtype="bf16",
                        gate_scale=1.0 / 8) -> Tokens:
    """Seam-window tokens of one KDA layer: as warm_seam_layer, the log gates
    drawn per token and key channel."""
    q, k, v, beta, _ = _draw_delta_tokens(15, n_seg * w, n_head, d, dtype, None, layer=layer)
    lg = round_to(-_softplus(rng(15, T_GATE, layer).standard_normal((n_seg * w, n_head, d))) * gate_scale, dtype)
    return Tokens(KDA, dtype, n_head, d, d, k, v, q, beta, lg, False, None,
                  {"workload": "kda_warm100k", "layer": layer, "n_seg": n_seg, "w": w})


def concat_chains(parts):
    """Concatenate per-layer token batches along the chain axis (chain = layer*heads + head)."""
    p0 = parts[0]
    cat = lambda name: None if getattr(p0, name) is None else np.concatenate([getattr(p, name) for p in parts], axis=1)
    return Tokens(p0.fam, p0.dtype, sum(p.n_chain for p in parts), p0.dk, p0.dv, cat("k"), cat("v"), cat("q"),
                  cat("beta"), cat("log_gate"), p0.gate_per_chain, p0.offsets, dict(p0.meta))
