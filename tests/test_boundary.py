"""C-ABI boundary checks that need no GPU.

The library loads on a host without a GPU; every call below is malformed, so
the library must reject it during host-side validation, before any HIP call,
with the documented status and a message.  Pointers are fake, aligned
integers that are never dereferenced.
"""
import ctypes
import os
import re
import subprocess
import threading

import pytest

from segment_scan_amd import api
from segment_scan_amd.api import Pairs, Tokens

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hypic.h")

INVALID, UNSUPPORTED = api.HYPIC_E_INVALID, api.HYPIC_E_UNSUPPORTED
NAIVE, SCALAR, DIAG, DELTA, KDA = 0, 1, 2, 3, 4
BF16, F32 = api.HYPIC_BF16, api.HYPIC_F32

# fake device addresses, 16-byte aligned, far apart (1 TiB) so nothing overlaps by accident
A = {name: (i + 1) << 40 for i, name in enumerate(
    ["q", "k", "v", "beta", "lg", "g", "U", "S", "Sinit", "Sout", "prefix", "gtot", "Utot", "o", "wg", "wU", "wS",
     "ws"])}
WS_BYTES = 1 << 36


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.LIB_PATH):
        from segment_scan_amd import build
        build.build()
    return api.load_library()


def test_library_exports_every_declared_symbol(lib):
    with open(HEADER) as f:
        text = f.read()
    declared = set(re.findall(r"\b(hypic_[a-z_]+)\s*\(", text))
    assert {"hypic_seg_build", "hypic_seg_build_workspace_size", "hypic_compose", "hypic_compose_workspace_size",
            "hypic_seam_step", "hypic_seam_step_workspace_size", "hypic_rerotate", "hypic_last_error",
            "hypic_abi_version"} <= declared
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\b(hypic_[a-z_]+)\b", out))
    assert declared <= exported, declared - exported
    for name in declared:
        getattr(lib, name)
    assert lib.hypic_abi_version() == 8


def toks(fam, dtype=BF16, q=False, beta=None, lg=None, gate_per_chain=0):
    if beta is None:
        beta = fam in (DELTA, KDA)
    if lg is None:
        lg = fam in (SCALAR, DIAG, DELTA, KDA)
    return Tokens(dtype, A["q"] if q else None, A["k"], A["v"], A["beta"] if beta else None,
                  A["lg"] if lg else None, gate_per_chain)


def pairs(fam, g=True, U=None, S=True):
    if U is None:
        U = fam in (DELTA, KDA)
    return Pairs(A["g"] if g else None, A["U"] if U else None, A["S"] if S else None)


def build_call(lib, fam=DELTA, n_seg=2, offsets=(0, 64, 128), n_chain=2, dk=128, dv=128, t=None, p=None,
               ws=A["ws"], ws_bytes=WS_BYTES):
    off = (ctypes.c_int32 * len(offsets))(*offsets) if offsets is not None else None
    t = toks(fam) if t is None else t
    p = pairs(fam) if p is None else p
    return lib.hypic_seg_build(fam, n_seg, off, n_chain, dk, dv, ctypes.byref(t), ctypes.byref(p), ws, ws_bytes,
                               None)


def ws_size(lib, fam=DELTA, offsets=(0, 64, 128), n_chain=2, d=128, dtype=BF16):
    off = (ctypes.c_int32 * len(offsets))(*offsets)
    out = ctypes.c_size_t(123)
    st = lib.hypic_seg_build_workspace_size(fam, len(offsets) - 1, off, n_chain, d, d, dtype, ctypes.byref(out))
    return st, out.value


def test_compose_workspace_size(lib):
    """The blocked schedule applies to the dense family with few chains: one block
    pair (g, U, S) per (block, chain), about 256 units at d = 128; without prefix
    states also the pairs of the first pairwise reduction level (half as many),
    with prefix states each block's start state instead."""
    def cws(fam=DELTA, n_seg=64, n_chain=32, d=128, prefix=0):
        out = ctypes.c_size_t(7)
        st = lib.hypic_compose_workspace_size(fam, n_seg, n_chain, d, d, prefix, ctypes.byref(out))
        return st, out.value

    def pairs(units):
        return ((units * 4 + 255) // 256) * 256 + 2 * units * 128 * 128 * 4
    units = 8 * 32  # 64 segments in 8 blocks of 8, 32 chains
    assert cws() == (0, pairs(units) + pairs(units // 2))
    assert cws(prefix=1) == (0, pairs(units) + units * 128 * 128 * 4)
    assert cws(n_chain=480) == (0, 0)
    assert cws(n_seg=4) == (0, 0)
    assert cws(fam=SCALAR) == (0, 0)
    assert cws(d=96)[0] == UNSUPPORTED


def test_seam_workspace_size(lib):
    """The delta seam step takes one 576-byte record (inverse factor, gate weights)
    per 8-token sub-window and chain; the other families none."""
    def sws(fam=DELTA, n_seg=196, w=8, n_chain=480, d=128):
        out = ctypes.c_size_t(7)
        st = lib.hypic_seam_step_workspace_size(fam, n_seg, w, n_chain, d, d, ctypes.byref(out))
        return st, out.value
    assert sws() == (0, 196 * 480 * 576)
    assert sws(w=9, n_seg=3, n_chain=2) == (0, 3 * 2 * 2 * 576)
    assert sws(w=1, n_seg=1, n_chain=1, d=64) == (0, 576)
    assert sws(fam=DIAG) == (0, 0)
    assert sws(w=0)[0] == INVALID
    assert sws(d=96)[0] == UNSUPPORTED


def test_piece_split_workspace_size(lib):
    """Few long scalar or diagonal units are built as pieces of whole 64-token
    chunks (at most 4, at most 512 piece units) into the workspace: (g, S) of
    every (segment, piece, chain), the g block padded to 256 bytes."""
    assert ws_size(lib, fam=SCALAR, offsets=(0, 1024, 2048)) == (0, 256 + 2 * 4 * 2 * 128 * 128 * 4)
    assert ws_size(lib, fam=DIAG, offsets=(0, 1024, 2048)) == (0, 2 * 4 * 2 * 128 * 4 + 2 * 4 * 2 * 128 * 128 * 4)
    assert ws_size(lib, fam=NAIVE, offsets=(0, 192), n_chain=1, d=64) == (0, 256 + 3 * 64 * 64 * 4)  # 3 chunks
    assert ws_size(lib, fam=SCALAR, offsets=(0, 64, 1024)) == (0, 0)  # a one-chunk segment: no split
    assert ws_size(lib, fam=SCALAR, offsets=(0, 1024), n_chain=256) == (0, 2 * 256 * 4 + 2 * 256 * 128 * 128 * 4)
    assert ws_size(lib, fam=SCALAR, offsets=(0, 1024), n_chain=512) == (0, 0)  # enough units already


def test_kda_workspace_sizes(lib):
    """The d = 128 bf16 KDA build takes one 42,512-byte factor record per 64-token
    chunk and chain (decayed keys, X, gate factors); other KDA builds and the
    seam step take none; its dense composition takes the delta family's."""
    assert ws_size(lib, fam=KDA) == (0, 2 * 2 * 42512)
    assert ws_size(lib, fam=KDA, offsets=(0, 1, 65, 200), n_chain=3) == (0, (1 + 1 + 3) * 3 * 42512)
    assert ws_size(lib, fam=KDA, offsets=(0, 2049)) == (0, 0)
    assert ws_size(lib, fam=KDA, d=64) == (0, 0)
    assert ws_size(lib, fam=KDA, d=64, dtype=F32) == (0, 0)
    for want_prefix in (0, 1):
        a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
        assert lib.hypic_compose_workspace_size(KDA, 64, 32, 128, 128, want_prefix, ctypes.byref(a)) == 0
        assert lib.hypic_compose_workspace_size(DELTA, 64, 32, 128, 128, want_prefix, ctypes.byref(b)) == 0
        assert a.value == b.value > 0
    out = ctypes.c_size_t(1)
    assert lib.hypic_seam_step_workspace_size(KDA, 4, 8, 2, 128, 128, ctypes.byref(out)) == 0
    assert out.value == 0


def test_workspace_size(lib):
    """Only the d = 128 bf16 delta build takes a workspace: one 8704-byte WY record
    (fp16 A0 [64 x 64], 64 row scales, 64 gate prefixes) per 64-token chunk and chain."""
    lib_ = lib
    assert ws_size(lib_) == (0, 2 * 2 * 8704)
    assert ws_size(lib_, offsets=(0, 1, 65, 200), n_chain=3) == (0, (1 + 1 + 3) * 3 * 8704)
    assert ws_size(lib_, dtype=F32) == (0, 0)
    assert ws_size(lib_, d=64) == (0, 0)
    assert ws_size(lib_, fam=SCALAR) == (0, 0)
    # segments longer than 2048 tokens take the single-kernel path
    assert ws_size(lib_, offsets=(0, 2048)) == (0, 32 * 2 * 8704)
    assert ws_size(lib_, offsets=(0, 2049)) == (0, 0)
    # launches of at most 240 segments reuse one workspace: the largest launch sets the size
    offs = [64 * i for i in range(301)]
    assert ws_size(lib_, offsets=offs, n_chain=1) == (0, 240 * 8704)
    assert ws_size(lib_, offsets=(0, 64, 64))[0] == INVALID
    assert "strictly increase" in api.last_error()
    assert lib_.hypic_seg_build_workspace_size(DELTA, 1, (ctypes.c_int32 * 2)(0, 64), 1, 128, 128, BF16,
                                               None) == INVALID


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(fam=7), INVALID, "unknown family"),
    (dict(n_seg=0, offsets=(0,)), INVALID, "n_seg"),
    (dict(n_chain=0), INVALID, "n_chain"),
    (dict(dk=96, dv=96), UNSUPPORTED, "64, 128"),
    (dict(dk=128, dv=64), UNSUPPORTED, "64, 128"),
    (dict(offsets=None), INVALID, "seg_offsets is NULL"),
    (dict(offsets=(1, 64, 128)), INVALID, "seg_offsets[0]"),
    (dict(offsets=(0, 64, 64)), INVALID, "strictly increase"),
    (dict(offsets=(0, 70, 60)), INVALID, "strictly increase"),
    (dict(fam=SCALAR, t=Tokens(BF16, None, A["k"], A["v"], A["beta"], A["lg"], 0), p=pairs(SCALAR)), INVALID,
     "beta is only defined"),
    (dict(fam=DELTA, t=toks(DELTA, beta=False)), INVALID, "beta is required"),
    (dict(fam=DIAG, t=toks(DIAG, lg=False), p=pairs(DIAG)), INVALID, "log_gate is required"),
    (dict(fam=NAIVE, t=toks(NAIVE, lg=True), p=pairs(NAIVE)), INVALID, "must be NULL"),
    (dict(fam=DELTA, t=toks(DELTA, gate_per_chain=1)), INVALID, "gate_per_chain"),
    (dict(t=Tokens(BF16, None, None, A["v"], A["beta"], A["lg"], 0)), INVALID, "k is NULL"),
    (dict(t=Tokens(BF16, None, A["k"] + 8, A["v"], A["beta"], A["lg"], 0)), INVALID, "aligned"),
    (dict(t=Tokens(9, None, A["k"], A["v"], A["beta"], A["lg"], 0)), INVALID, "dtype"),
    (dict(fam=SCALAR, t=toks(SCALAR), p=pairs(SCALAR, U=True)), INVALID, "only defined for the delta"),
    (dict(fam=DELTA, p=pairs(DELTA, U=False)), INVALID, "required for the delta"),
    (dict(fam=KDA, p=pairs(KDA, U=False), t=toks(KDA)), INVALID, "required for the delta and KDA"),
    (dict(fam=KDA, t=toks(KDA, beta=False), p=pairs(KDA)), INVALID, "beta is required"),
    (dict(fam=KDA, t=toks(KDA, lg=False), p=pairs(KDA)), INVALID, "log_gate is required"),
    (dict(fam=KDA, t=toks(KDA, dtype=F32), p=pairs(KDA)), UNSUPPORTED, "KDA build"),
    (dict(p=Pairs(A["g"], A["U"], None)), INVALID, "out.S is NULL"),
    (dict(p=Pairs(None, A["U"], A["S"])), INVALID, "out.g is NULL"),
    (dict(p=Pairs(A["g"], A["U"], A["k"] + 4096)), INVALID, "overlaps input k"),
    (dict(p=Pairs(A["g"], A["S"] + 4096, A["S"])), INVALID, "overlap"),
    (dict(ws=None), INVALID, "workspace is NULL"),
    (dict(ws_bytes=2 * 2 * 8704 - 1), INVALID, "workspace too small"),
    (dict(ws=A["ws"] + 8), INVALID, "workspace is not 16-byte aligned"),
    (dict(ws=A["k"] + 64), INVALID, "output workspace overlaps input k"),
    (dict(ws=A["S"] + 64), INVALID, "overlap"),
])
def test_seg_build_rejects(lib, kwargs, status, msg):
    st = build_call(lib, **kwargs)
    assert st == status
    assert msg in api.last_error()


def compose_call(lib, fam=DELTA, n_seg=3, n_chain=2, d=128, p=None, S_init=None, S_out=A["Sout"], prefix=None,
                 gtot=None, Utot=None, ws=None, ws_bytes=0):
    p = pairs(fam) if p is None else p
    return lib.hypic_compose(fam, n_seg, n_chain, d, d, ctypes.byref(p), S_init, S_out, prefix, gtot, Utot, ws,
                             ws_bytes, None)


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(n_seg=0), INVALID, "n_seg"),
    (dict(d=32), UNSUPPORTED, "64, 128"),
    (dict(S_out=None), INVALID, "S_out is NULL"),
    (dict(p=Pairs(A["g"], A["U"], None)), INVALID, "in.S is NULL"),
    (dict(p=Pairs(None, A["U"], A["S"])), INVALID, "in.g is NULL"),
    (dict(fam=DELTA, p=Pairs(A["g"], None, A["S"])), INVALID, "required for the delta"),
    (dict(fam=DIAG, p=pairs(DIAG, U=True)), INVALID, "only defined for the delta"),
    (dict(fam=SCALAR, p=pairs(SCALAR), Utot=A["Utot"]), INVALID, "U_total is only defined"),
    (dict(fam=KDA, p=Pairs(A["g"], None, A["S"])), INVALID, "required for the delta and KDA"),
    (dict(S_out=A["S"] + 64), INVALID, "overlaps input pairs.S"),
    (dict(S_init=A["Sinit"], S_out=A["Sinit"] + 16), INVALID, "overlaps input S_init"),
    (dict(prefix=A["Sout"] + 16), INVALID, "overlap"),
    (dict(S_init=A["Sinit"], S_out=A["Sinit"], prefix=A["Sinit"] + 1024), INVALID, "outputs S_out and prefix_states overlap"),
    (dict(gtot=A["gtot"] + 2), INVALID, "aligned"),
    (dict(n_seg=64, ws=A["ws"], ws_bytes=1024), INVALID, "workspace too small"),
    (dict(n_seg=64, ws=A["ws"] + 8, ws_bytes=WS_BYTES), INVALID, "workspace is not 16-byte aligned"),
    (dict(n_seg=64, ws=A["S"] + 64, ws_bytes=WS_BYTES), INVALID, "overlap"),
])
def test_compose_rejects(lib, kwargs, status, msg):
    assert compose_call(lib, **kwargs) == status
    assert msg in api.last_error()


def seam_call(lib, fam=DELTA, n_seg=4, w=8, n_chain=2, d=128, t=None, body="default", S_run=A["Sinit"], o=A["o"],
              win=None, ws=A["ws"], ws_bytes=WS_BYTES):
    t = toks(fam, q=True) if t is None else t
    b = pairs(fam) if body == "default" else body
    return lib.hypic_seam_step(fam, n_seg, w, n_chain, d, d, ctypes.byref(t),
                               ctypes.byref(b) if b is not None else None, S_run, o,
                               ctypes.byref(win) if win is not None else None, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status,msg", [
    (dict(w=0), INVALID, "w must be"),
    (dict(t=toks(DELTA, q=False)), INVALID, "q is NULL"),
    (dict(S_run=None), INVALID, "S_run is NULL"),
    (dict(o=None), INVALID, "o_out is NULL"),
    (dict(o=A["k"] + 128), INVALID, "overlaps input k"),
    (dict(S_run=A["S"]), INVALID, "overlaps input pairs.S"),
    (dict(body=Pairs(A["g"], None, A["S"])), INVALID, "required for the delta"),
    (dict(win=Pairs(A["wg"], None, A["wS"])), INVALID, "window_out.U"),
    (dict(fam=NAIVE, t=toks(NAIVE, q=True), body=pairs(NAIVE), win=Pairs(None, None, A["wS"])), INVALID,
     "window_out needs S and g"),
    (dict(fam=SCALAR, t=toks(SCALAR, q=True), body=pairs(SCALAR), win=Pairs(A["wg"], A["wU"], A["wS"])), INVALID,
     "only defined for the delta"),
    (dict(d=256), UNSUPPORTED, "64, 128"),
    (dict(fam=KDA, t=toks(KDA, q=True, dtype=F32), body=pairs(KDA), win=Pairs(A["wg"], A["wU"], A["wS"]),
          ws=None, ws_bytes=0), UNSUPPORTED, "KDA window pairs"),
    (dict(fam=KDA, t=toks(KDA, q=True), body=pairs(KDA), win=Pairs(A["wg"], None, A["wS"])), INVALID,
     "window_out.U is required"),
    (dict(ws=None), INVALID, "workspace is NULL"),
    (dict(ws_bytes=1024), INVALID, "workspace too small"),
    (dict(ws=A["ws"] + 8), INVALID, "workspace is not 16-byte aligned"),
    (dict(ws=A["o"] + 64), INVALID, "overlap"),
])
def test_seam_rejects(lib, kwargs, status, msg):
    assert seam_call(lib, **kwargs) == status
    assert msg in api.last_error()


def test_last_error_is_per_thread(lib):
    assert build_call(lib, fam=9) == INVALID
    assert "unknown family" in api.last_error()
    seen = {}

    def other():
        seen["msg"] = api.last_error()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert "unknown family" in api.last_error()


def test_binding_requires_gpu_tensors(lib):
    import torch
    k = torch.zeros((4, 1, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        api.seg_build(NAIVE, [0, 4], k, k)


def test_ragged_lengths_recipe():
    """The seeded ragged-segment recipe: exact total, bounds, and a long tail."""
    from segment_scan_amd import synth
    import numpy as np
    lens = synth.ragged_lengths(64, 32768)
    assert int(lens.sum()) == 32768 and lens.min() >= 32 and lens.max() <= 2048
    assert np.array_equal(lens, synth.ragged_lengths(64, 32768))  # seeded
    assert lens.max() / np.median(lens) > 4


def rerotate_call(lib, fam=DELTA, n_seg=2, n_chain=2, dk=128, dv=128, pos=A["q"], base=10000.0, p=None):
    p = pairs(fam, g=False) if p is None else p
    return lib.hypic_rerotate(fam, n_seg, n_chain, dk, dv, pos, base, ctypes.byref(p), None)


@pytest.mark.parametrize("case,status", [
    (dict(fam=DIAG), UNSUPPORTED),
    (dict(fam=KDA), UNSUPPORTED),
    (dict(dk=96, dv=96), UNSUPPORTED),
    (dict(n_seg=0), INVALID),
    (dict(base=0.0), INVALID),
    (dict(base=-2.0), INVALID),
    (dict(base=float("inf")), INVALID),
    (dict(base=float("nan")), INVALID),
    (dict(pos=None), INVALID),
    (dict(p=Pairs(None, A["U"], None)), INVALID),                  # S missing
    (dict(p=Pairs(None, None, A["S"])), INVALID),                  # delta without U
    (dict(fam=SCALAR, p=Pairs(None, A["U"], A["S"])), INVALID),    # U outside the delta family
    (dict(p=Pairs(None, A["U"] + 4, A["S"])), INVALID),            # misaligned
    (dict(pos=A["S"] + 64), INVALID),                              # positions inside S
    (dict(p=Pairs(None, A["S"] + 2 * 128 * 128 * 4, A["S"])), INVALID),  # U overlaps S
    (dict(n_seg=1 << 16, n_chain=1 << 15), INVALID),               # more workgroups than one launch holds
])
def test_rerotate_rejects(lib, case, status):
    assert rerotate_call(lib, **case) == status
    assert lib.hypic_last_error()


def test_seam_noalloc_rejects_more_records_than_its_scratch(lib):
    """The no-allocation seam step refuses, before any HIP call, a call whose
    window records exceed the library's fixed scratch: 1000 segments x 480
    chains x 576 bytes = 276 MB > 64 MiB."""
    t = toks(DELTA, q=True)
    st = lib.hypic_seam_step_noalloc(DELTA, 1000, 8, 480, 128, 128, ctypes.byref(t), ctypes.byref(pairs(DELTA)),
                                     A["Sinit"], A["o"], None, None)
    assert st == INVALID
    msg = api.last_error()
    assert "scratch" in msg and str(1000 * 480 * 576) in msg
    need = ctypes.c_size_t(0)
    assert lib.hypic_seam_step_workspace_size(DELTA, 113, 8, 1024, 128, 128, ctypes.byref(need)) == 0
    assert need.value <= api.NOALLOC_SCRATCH_BYTES  # the largest warm-request-like call that still fits


def test_build_compose_requires_its_workspace(lib):
    """hypic_seg_build_compose refuses a missing or short workspace before any HIP call."""
    off = (ctypes.c_int32 * 3)(0, 64, 128)
    t = toks(DELTA)
    p = pairs(DELTA)
    need = ctypes.c_size_t(0)
    for mode in (0, 1, 2):
        assert lib.hypic_seg_build_compose_workspace_size(DELTA, 2, off, 2, 128, 128, BF16, mode,
                                                          ctypes.byref(need)) == 0
        assert need.value > 0
        st = lib.hypic_seg_build_compose(DELTA, 2, off, 2, 128, 128, ctypes.byref(t), ctypes.byref(p), None,
                                         A["Sout"], None, None, mode, None, 0, None)
        assert st == INVALID and "workspace is NULL" in api.last_error()
        st = lib.hypic_seg_build_compose(DELTA, 2, off, 2, 128, 128, ctypes.byref(t), ctypes.byref(p), None,
                                         A["Sout"], None, None, mode, A["ws"], need.value - 256, None)
        assert st == INVALID and "too small" in api.last_error()
    st = lib.hypic_seg_build_compose(DELTA, 2, off, 2, 128, 128, ctypes.byref(t), ctypes.byref(p), None,
                                     A["Sout"], None, None, 7, A["ws"], WS_BYTES, None)
    assert st == INVALID and "mode" in api.last_error()
