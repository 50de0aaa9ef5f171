"""Build libhypic.so (gfx950) in-tree with hipcc.

    python -m segment_scan_amd.build [--force] [--verbose]

Compiles every source under csrc/ to an object in csrc/_build/ and links the
shared library next to this file.  Always recompiles sources newer than their
object; `force=True` recompiles everything.  HYPIC_EXTRA_FLAGS (environment)
adds compiler flags, for instance a -D that selects a kernel variant.
"""
from __future__ import annotations

import argparse
import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(HERE, "libhypic.so")
ROOT = os.path.dirname(HERE)
ARCH = os.environ.get("HYPIC_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [*os.environ.get("HYPIC_EXTRA_FLAGS", "").split(), "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-I" + os.path.join(ROOT, "include"),
          "-Wall", "-Wno-unused-function"]
# packed fp32 instructions are kept out of generated code on purpose
DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _sources():
    srcs = sorted(glob.glob(os.path.join(CSRC, "kernels", "*.hip")))
    srcs += sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    srcs += sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    return srcs


def _headers():
    return sorted(glob.glob(os.path.join(CSRC, "**", "*.h"), recursive=True)) + \
        [os.path.join(ROOT, "include", "hypic.h")]


def _compile(src, force, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    newest_dep = max([os.path.getmtime(src)] + [os.path.getmtime(h) for h in _headers()])
    if not force and os.path.exists(obj) and os.path.getmtime(obj) >= newest_dep:
        return obj
    cmd = [HIPCC] + COMMON + (DEVICE if src.endswith(".hip") else []) + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (src, "\n".join(msgs)))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


def build(force: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, force, verbose), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--force", action="store_true")
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.force, args.verbose))
