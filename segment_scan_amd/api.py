"""Thin Python binding of the C ABI in include/hypic.h (libhypic.so).

Argument marshalling only: tensors are checked for device, dtype, layout and
contiguity, their data pointers and the current HIP stream are handed to the
library, and missing outputs are allocated with torch.  Every step of the
computation runs in the library's HIP kernels; there is no fallback path.  If
the library is missing the first call raises HypicError.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

import torch

from .synth import NAIVE, SCALAR, DIAG, DELTA, KDA

DENSE = (DELTA, KDA)  # families whose pairs carry a dense U

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhypic.so")

HYPIC_OK, HYPIC_E_INVALID, HYPIC_E_UNSUPPORTED, HYPIC_E_HIP = 0, 1, 2, 3
HYPIC_F32, HYPIC_BF16 = 0, 1
STATUS_NAMES = {0: "HYPIC_OK", 1: "HYPIC_E_INVALID", 2: "HYPIC_E_UNSUPPORTED", 3: "HYPIC_E_HIP"}


class HypicError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), msg))
        self.status = status


class Tokens(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("log_gate", ctypes.c_void_p), ("gate_per_chain", ctypes.c_int)]


class Pairs(ctypes.Structure):
    _fields_ = [("g", ctypes.c_void_p), ("U", ctypes.c_void_p), ("S", ctypes.c_void_p)]


_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH):
    """Load libhypic.so and declare its entry points (no GPU needed)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise HypicError(HYPIC_E_UNSUPPORTED,
                             "%s is not built; run `python -m segment_scan_amd.build`" % path)
        lib = ctypes.CDLL(path)
        P, I = ctypes.c_void_p, ctypes.c_int
        lib.hypic_seg_build.argtypes = [I, I, P, I, I, I, ctypes.POINTER(Tokens), ctypes.POINTER(Pairs), P,
                                        ctypes.c_size_t, P]
        lib.hypic_seg_build_workspace_size.argtypes = [I, I, P, I, I, I, I, ctypes.POINTER(ctypes.c_size_t)]
        lib.hypic_compose.argtypes = [I, I, I, I, I, ctypes.POINTER(Pairs), P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.hypic_seg_build_compose.argtypes = [I, I, P, I, I, I, ctypes.POINTER(Tokens), ctypes.POINTER(Pairs), P,
                                                P, P, P, I, P, ctypes.c_size_t, P]
        lib.hypic_seg_build_compose_workspace_size.argtypes = [I, I, P, I, I, I, I, I,
                                                               ctypes.POINTER(ctypes.c_size_t)]
        lib.hypic_compose_workspace_size.argtypes = [I, I, I, I, I, I, ctypes.POINTER(ctypes.c_size_t)]
        lib.hypic_seam_step.argtypes = [I, I, I, I, I, I, ctypes.POINTER(Tokens), ctypes.POINTER(Pairs), P, P,
                                        ctypes.POINTER(Pairs), P, ctypes.c_size_t, P]
        lib.hypic_seam_step_workspace_size.argtypes = [I, I, I, I, I, I, ctypes.POINTER(ctypes.c_size_t)]
        lib.hypic_seam_step_noalloc.argtypes = [I, I, I, I, I, I, ctypes.POINTER(Tokens), ctypes.POINTER(Pairs), P,
                                                P, ctypes.POINTER(Pairs), P]
        lib.hypic_rerotate.argtypes = [I, I, I, I, I, P, ctypes.c_double, ctypes.POINTER(Pairs), P]
        for f in (lib.hypic_seg_build, lib.hypic_seg_build_workspace_size, lib.hypic_compose,
                  lib.hypic_compose_workspace_size, lib.hypic_seam_step, lib.hypic_seam_step_workspace_size,
                  lib.hypic_seam_step_noalloc, lib.hypic_rerotate, lib.hypic_seg_build_compose,
                  lib.hypic_seg_build_compose_workspace_size):
            f.restype = I
        lib.hypic_last_error.restype = ctypes.c_char_p
        lib.hypic_last_error.argtypes = []
        lib.hypic_abi_version.restype = I
        _lib = lib
        return lib


def last_error() -> str:
    return load_library().hypic_last_error().decode()


def _check(status: int):
    if status != HYPIC_OK:
        raise HypicError(status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _want(name: str, t: Optional[torch.Tensor], shape, dtype=torch.float32):
    """Raise ValueError unless t (if given) has exactly this shape (and dtype).

    The library sizes every device range from the counts it is passed, so a
    tensor of another shape would be read or written out of bounds: the check
    runs here, before any pointer reaches the library."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))


def _check_token_shapes(fam, n_tok, n_chain, d, k, v, q=None, beta=None, log_gate=None, gate_per_chain=False):
    if k.dim() != 3:
        raise ValueError("k must be [n_tok, n_chain, d] (got shape %s)" % (tuple(k.shape),))
    _want("k", k, (n_tok, n_chain, d), None)
    _want("v", v, (n_tok, n_chain, d), None)
    _want("q", q, (n_tok, n_chain, d), None)
    _want("beta", beta, (n_tok, n_chain), None)
    if log_gate is not None:
        if gate_per_chain:
            shape = (n_chain,)
        elif fam in (DIAG, KDA):
            shape = (n_tok, n_chain, d)
        else:
            shape = (n_tok, n_chain)
        _want("log_gate", log_gate, shape, None)


def _check_pair_shapes(fam, what, n_seg, n_chain, d, g, U, S):
    _want(what + ".g", g, _gate_shape(fam, (n_seg, n_chain), d))
    _want(what + ".U", U, (n_seg, n_chain, d, d))
    _want(what + ".S", S, (n_seg, n_chain, d, d))


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HYPIC_BF16
    if t.dtype == torch.float32:
        return HYPIC_F32
    raise ValueError("token tensors must be bfloat16 or float32 (got %s)" % t.dtype)


def _tokens(k, v, q=None, beta=None, log_gate=None, gate_per_chain=False) -> Tokens:
    dt = _dtype_code(k)
    for name, t in (("v", v), ("q", q), ("beta", beta)):
        if t is not None and t.dtype != k.dtype:
            raise ValueError("%s must have the dtype of k" % name)
    if log_gate is not None:
        want = torch.float32 if gate_per_chain else k.dtype
        if log_gate.dtype != want:
            raise ValueError("log_gate must be %s" % want)
    return Tokens(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_gate), int(bool(gate_per_chain)))


def _gate_shape(fam, lead, d):
    return tuple(lead) + ((d,) if fam == DIAG else ())


def _offsets(offsets: Sequence[int]):
    return (ctypes.c_int32 * len(offsets))(*[int(x) for x in offsets])


def seg_build_workspace_size(fam: int, offsets: Sequence[int], n_chain: int, d: int, dtype: torch.dtype) -> int:
    """Bytes of device workspace seg_build needs for this batch (0: none)."""
    out = ctypes.c_size_t(0)
    code = HYPIC_F32 if dtype == torch.float32 else HYPIC_BF16
    _check(load_library().hypic_seg_build_workspace_size(fam, len(offsets) - 1, _offsets(offsets), n_chain, d, d,
                                                         code, ctypes.byref(out)))
    return out.value


def seg_build(fam: int, offsets: Sequence[int], k: torch.Tensor, v: torch.Tensor, beta=None, log_gate=None,
              gate_per_chain: bool = False, out=None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Build (g, U, S) of every (segment, chain): k, v [n_tok, n_chain, d] on the GPU.

    offsets: n_seg + 1 host integers.  Returns (g, U or None, S); `out` may pass
    preallocated (g, U, S) and `workspace` a uint8 device buffer of at least
    seg_build_workspace_size() bytes (otherwise one is taken from torch's
    allocator for the call)."""
    off = _offsets(offsets)
    n_seg = len(offsets) - 1
    if k.dim() != 3:
        raise ValueError("k must be [n_tok, n_chain, d] (got shape %s)" % (tuple(k.shape),))
    n_tok, n_chain, d = k.shape
    if n_seg < 1 or int(offsets[-1]) > n_tok:
        raise ValueError("offsets must end within k.shape[0] = %d (got %s)" % (n_tok, int(offsets[-1])))
    _check_token_shapes(fam, n_tok, n_chain, d, k, v, None, beta, log_gate, gate_per_chain)
    dev = k.device
    if out is not None:
        _check_pair_shapes(fam, "out", n_seg, n_chain, d, *out)
    if out is None:
        g = torch.empty(_gate_shape(fam, (n_seg, n_chain), d), device=dev, dtype=torch.float32)
        U = torch.empty((n_seg, n_chain, d, d), device=dev, dtype=torch.float32) if fam in DENSE else None
        S = torch.empty((n_seg, n_chain, d, v.shape[2]), device=dev, dtype=torch.float32)
    else:
        g, U, S = out
    ws_bytes = 0
    if workspace is None:
        need = seg_build_workspace_size(fam, offsets, n_chain, d, k.dtype)
        if need:
            workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    tk = _tokens(k, v, None, beta, log_gate, gate_per_chain)
    pr = Pairs(_ptr(g), _ptr(U), _ptr(S))
    _check(load_library().hypic_seg_build(fam, n_seg, off, n_chain, d, v.shape[2], ctypes.byref(tk),
                                          ctypes.byref(pr), _ptr(workspace), ws_bytes, _stream(stream)))
    return g, U, S


BC_SEQUENTIAL, BC_PIPELINED, BC_FUSED = 0, 1, 2  # schedules of seg_build_compose


def seg_build_compose_workspace_size(fam: int, offsets: Sequence[int], n_chain: int, d: int,
                                     dtype: torch.dtype, mode: int = BC_SEQUENTIAL) -> int:
    """Bytes of device workspace seg_build_compose needs for this batch and schedule."""
    out = ctypes.c_size_t(0)
    code = HYPIC_F32 if dtype == torch.float32 else HYPIC_BF16
    _check(load_library().hypic_seg_build_compose_workspace_size(fam, len(offsets) - 1, _offsets(offsets), n_chain,
                                                                 d, d, code, int(mode), ctypes.byref(out)))
    return out.value


def seg_build_compose(fam: int, offsets: Sequence[int], k: torch.Tensor, v: torch.Tensor, beta=None,
                      log_gate=None, gate_per_chain: bool = False, out=None, S_init=None, S_out=None,
                      g_total=None, U_total=None, want_total: bool = False, mode: int = BC_SEQUENTIAL,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """Build every (segment, chain) pair and compose each chain's pairs in order
    (hypic_seg_build_compose).  Returns (g, U or None, S) and a dict with S_out,
    g_tot, U_tot; `out` may pass preallocated (g, U, S), `workspace` a uint8
    device buffer of at least seg_build_compose_workspace_size() bytes."""
    off = _offsets(offsets)
    n_seg = len(offsets) - 1
    if k.dim() != 3:
        raise ValueError("k must be [n_tok, n_chain, d] (got shape %s)" % (tuple(k.shape),))
    n_tok, n_chain, d = k.shape
    if n_seg < 1 or int(offsets[-1]) > n_tok:
        raise ValueError("offsets must end within k.shape[0] = %d (got %s)" % (n_tok, int(offsets[-1])))
    _check_token_shapes(fam, n_tok, n_chain, d, k, v, None, beta, log_gate, gate_per_chain)
    if out is not None:
        _check_pair_shapes(fam, "out", n_seg, n_chain, d, *out)
    _want("S_init", S_init, (n_chain, d, d))
    _want("S_out", S_out, (n_chain, d, d))
    _want("g_total", g_total, _gate_shape(fam, (n_chain,), d))
    _want("U_total", U_total, (n_chain, d, d))
    dev = k.device
    if out is None:
        out = (torch.empty(_gate_shape(fam, (n_seg, n_chain), d), device=dev, dtype=torch.float32),
               torch.empty((n_seg, n_chain, d, d), device=dev, dtype=torch.float32) if fam in DENSE else None,
               torch.empty((n_seg, n_chain, d, d), device=dev, dtype=torch.float32))
    g, U, S = out
    if S_out is None:
        S_out = torch.empty((n_chain, d, d), device=dev, dtype=torch.float32)
    if want_total and g_total is None:
        g_total = torch.empty(_gate_shape(fam, (n_chain,), d), device=dev, dtype=torch.float32)
    if want_total and fam in DENSE and U_total is None:
        U_total = torch.empty((n_chain, d, d), device=dev, dtype=torch.float32)
    if workspace is None:
        need = seg_build_compose_workspace_size(fam, offsets, n_chain, d, k.dtype, mode)
        workspace = torch.empty(need, device=dev, dtype=torch.uint8) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    tk = _tokens(k, v, None, beta, log_gate, gate_per_chain)
    pr = Pairs(_ptr(g), _ptr(U), _ptr(S))
    _check(load_library().hypic_seg_build_compose(fam, n_seg, off, n_chain, d, v.shape[2], ctypes.byref(tk),
                                                  ctypes.byref(pr), _ptr(S_init), _ptr(S_out), _ptr(g_total),
                                                  _ptr(U_total), int(mode), _ptr(workspace), ws_bytes,
                                                  _stream(stream)))
    return g, U, S, {"S_out": S_out, "g_tot": g_total, "U_tot": U_total}


def compose_workspace_size(fam: int, n_seg: int, n_chain: int, d: int, want_prefix: bool = False) -> int:
    """Bytes of device workspace that enable compose's blocked schedule (0: none)."""
    out = ctypes.c_size_t(0)
    _check(load_library().hypic_compose_workspace_size(fam, n_seg, n_chain, d, d, int(bool(want_prefix)),
                                                       ctypes.byref(out)))
    return out.value


def compose(fam: int, g, U, S, S_init=None, S_out=None, prefix_states=None, g_total=None, U_total=None,
            want_prefix: bool = False, want_total: bool = False, workspace="auto", stream=None):
    """Ordered composition of pairs [n_seg, n_chain, ...]; returns dict of outputs.

    workspace: "auto" takes one of the size compose_workspace_size() reports from
    torch's allocator, None runs the single-pass schedule, or a uint8 tensor."""
    if S.dim() != 4:
        raise ValueError("S must be [n_seg, n_chain, d_k, d_v] (got shape %s)" % (tuple(S.shape),))
    n_seg, n_chain, dk, dv = S.shape
    _check_pair_shapes(fam, "pairs", n_seg, n_chain, dk, g, U, S)
    _want("S_init", S_init, (n_chain, dk, dv))
    _want("S_out", S_out, (n_chain, dk, dv))
    _want("prefix_states", prefix_states, (n_seg, n_chain, dk, dv))
    _want("g_total", g_total, _gate_shape(fam, (n_chain,), dk))
    _want("U_total", U_total, (n_chain, dk, dk))
    dev = S.device
    if S_out is None:
        S_out = torch.empty((n_chain, dk, dv), device=dev, dtype=torch.float32)
    if want_prefix and prefix_states is None:
        prefix_states = torch.empty((n_seg, n_chain, dk, dv), device=dev, dtype=torch.float32)
    if want_total and g_total is None:
        g_total = torch.empty(_gate_shape(fam, (n_chain,), dk), device=dev, dtype=torch.float32)
    if want_total and fam in DENSE and U_total is None:
        U_total = torch.empty((n_chain, dk, dk), device=dev, dtype=torch.float32)
    if isinstance(workspace, str):
        need = compose_workspace_size(fam, n_seg, n_chain, dk, prefix_states is not None) if fam in DENSE else 0
        workspace = torch.empty(need, device=dev, dtype=torch.uint8) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    pr = Pairs(_ptr(g), _ptr(U), _ptr(S))
    _check(load_library().hypic_compose(fam, n_seg, n_chain, dk, dv, ctypes.byref(pr), _ptr(S_init), _ptr(S_out),
                                        _ptr(prefix_states), _ptr(g_total), _ptr(U_total), _ptr(workspace),
                                        ws_bytes, _stream(stream)))
    return {"S_out": S_out, "prefix": prefix_states, "g_tot": g_total, "U_tot": U_total}


def seam_step_workspace_size(fam: int, n_seg: int, w: int, n_chain: int, d: int) -> int:
    """Bytes of device workspace seam_step needs (0: none)."""
    out = ctypes.c_size_t(0)
    _check(load_library().hypic_seam_step_workspace_size(fam, n_seg, w, n_chain, d, d, ctypes.byref(out)))
    return out.value


def _check_seam_shapes(fam, w, q, k, v, beta, log_gate, gate_per_chain, body, S_run, o_out, window_out):
    if k.dim() != 3:
        raise ValueError("k must be [n_seg * w, n_chain, d] (got shape %s)" % (tuple(k.shape),))
    n_tok, n_chain, d = k.shape
    if w < 1 or n_tok % w:
        raise ValueError("window tokens must be n_seg * w")
    n_seg = n_tok // w
    if q is None:
        raise ValueError("q is required")
    _check_token_shapes(fam, n_tok, n_chain, d, k, v, q, beta, log_gate, gate_per_chain)
    if body is not None:
        _check_pair_shapes(fam, "body", n_seg, n_chain, d, *body)
    if window_out is not None:
        _check_pair_shapes(fam, "window_out", n_seg, n_chain, d, *window_out)
    _want("S_run", S_run, (n_chain, d, d))
    _want("o_out", o_out, (n_tok, n_chain, d))
    return n_seg, n_chain, d


def seam_step(fam: int, w: int, q, k, v, beta=None, log_gate=None, gate_per_chain=False, body=None,
              S_run=None, o_out=None, window_out=None, want_window_pairs=False, workspace=None, stream=None):
    """Seam-window step over [n_seg * w, n_chain, d] window tokens; S_run is updated in place.

    body: None or (g, U, S) cached body pairs.  workspace: a uint8 device buffer
    of at least seam_step_workspace_size() bytes, or None to take one from
    torch's allocator for the call.  Returns dict with S_run, o and window pairs."""
    n_seg, n_chain, d = _check_seam_shapes(fam, w, q, k, v, beta, log_gate, gate_per_chain, body, S_run, o_out,
                                           window_out)
    n_tok = n_seg * w
    dev = k.device
    if S_run is None:
        S_run = torch.zeros((n_chain, d, v.shape[2]), device=dev, dtype=torch.float32)
    if o_out is None:
        o_out = torch.empty((n_tok, n_chain, v.shape[2]), device=dev, dtype=torch.float32)
    if want_window_pairs and window_out is None:
        window_out = (torch.empty(_gate_shape(fam, (n_seg, n_chain), d), device=dev, dtype=torch.float32),
                      torch.empty((n_seg, n_chain, d, d), device=dev, dtype=torch.float32) if fam in DENSE else None,
                      torch.empty((n_seg, n_chain, d, v.shape[2]), device=dev, dtype=torch.float32))
    if workspace is None:
        need = seam_step_workspace_size(fam, n_seg, w, n_chain, d)
        if need:
            workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    tk = _tokens(k, v, q, beta, log_gate, gate_per_chain)
    bp = ctypes.byref(Pairs(_ptr(body[0]), _ptr(body[1]), _ptr(body[2]))) if body is not None else None
    wp = ctypes.byref(Pairs(*[_ptr(x) for x in window_out])) if window_out is not None else None
    _check(load_library().hypic_seam_step(fam, n_seg, w, n_chain, d, v.shape[2], ctypes.byref(tk), bp,
                                          _ptr(S_run), _ptr(o_out), wp, _ptr(workspace), ws_bytes,
                                          _stream(stream)))
    res = {"S_run": S_run, "o": o_out}
    if window_out is not None:
        res.update(wg=window_out[0], wU=window_out[1], wS=window_out[2])
    return res


NOALLOC_SCRATCH_BYTES = 64 << 20  # HYPIC_NOALLOC_SCRATCH_BYTES


def seam_step_noalloc(fam: int, w: int, q, k, v, beta=None, log_gate=None, gate_per_chain=False, body=None,
                      S_run=None, o_out=None, window_out=None, stream=None):
    """seam_step on the library's fixed per-device scratch (hypic_seam_step_noalloc):
    no workspace argument, and the library allocates nothing.  S_run (updated in
    place) and o_out must be given, as must window_out if window pairs are wanted;
    calls that overlap on one GPU race on the scratch."""
    if S_run is None or o_out is None:
        raise ValueError("seam_step_noalloc takes preallocated S_run and o_out")
    n_seg, n_chain, d = _check_seam_shapes(fam, w, q, k, v, beta, log_gate, gate_per_chain, body, S_run, o_out,
                                           window_out)
    tk = _tokens(k, v, q, beta, log_gate, gate_per_chain)
    bp = ctypes.byref(Pairs(_ptr(body[0]), _ptr(body[1]), _ptr(body[2]))) if body is not None else None
    wp = ctypes.byref(Pairs(*[_ptr(x) for x in window_out])) if window_out is not None else None
    _check(load_library().hypic_seam_step_noalloc(fam, n_seg, w, n_chain, d, v.shape[2], ctypes.byref(tk), bp,
                                                  _ptr(S_run), _ptr(o_out), wp, _stream(stream)))
    res = {"S_run": S_run, "o": o_out}
    if window_out is not None:
        res.update(wg=window_out[0], wU=window_out[1], wS=window_out[2])
    return res


def rerotate(fam: int, positions: torch.Tensor, S: torch.Tensor, U: Optional[torch.Tensor] = None,
             rope_base: float = 10000.0, stream=None):
    """Rotary re-rotation of pairs [n_seg, n_chain, ...] in place: S <- R(p) S and,
    for the delta family, U <- R(p) U R(p)^T, with p = positions[s] (int32 on the
    GPU).  Returns (U, S)."""
    if S.dim() != 4:
        raise ValueError("S must be [n_seg, n_chain, d_k, d_v] (got shape %s)" % (tuple(S.shape),))
    n_seg, n_chain, dk, dv = S.shape
    _want("S", S, (n_seg, n_chain, dk, dv))
    _want("U", U, (n_seg, n_chain, dk, dk))
    if positions.dtype != torch.int32 or positions.shape != (n_seg,):
        raise ValueError("positions must be int32 of shape (n_seg,)")
    pr = Pairs(None, _ptr(U), _ptr(S))
    _check(load_library().hypic_rerotate(fam, n_seg, n_chain, dk, dv, _ptr(positions), float(rope_base),
                                         ctypes.byref(pr), _stream(stream)))
    return U, S
