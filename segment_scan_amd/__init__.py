"""segment_scan_amd: MI355X (gfx950) kernels for the linear-attention hot path of
position-independent caching -- segment build of (T_C, S(C|0)), ordered
composition of cached pairs, and the seam-window step.

The compute runs in hand-written HIP kernels behind the C ABI declared in
``include/hypic.h`` (``libhypic.so``).  The Python layer in ``segment_scan_amd.api``
only marshals torch tensors into that ABI.
"""
from .synth import NAIVE, SCALAR, DIAG, DELTA, FAMILY_NAMES  # noqa: F401

__all__ = ["NAIVE", "SCALAR", "DIAG", "DELTA", "FAMILY_NAMES"]
