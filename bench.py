"""Benchmark of the linear-attention hot path of position-independent caching on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one pass of the hot path over one batch of synthetic input already
resident in HBM.  The default workload is one 32k-token cold request of a GDN
layer: 32 heads, d = 128, 64 segments x 512 tokens, bf16 tokens with fp32
accumulation -- every (segment, head) pair (T_C, S(C|0)) built concurrently
(hypic_seg_build), then the 64 pairs of every head composed in order
(hypic_compose).  Other workloads (`--workload`):
  retnet        8 heads x 16 segments x 1024, scalar decay: build + compose
  gla           16 heads x 64 segments x 512, diagonal gates: build + compose
  gdn_cold32k_fused   the cold request in one call, the composition folded into
                the build as a tree (the last build workgroup at a node composes it)
  gdn_warm100k  30 layers x 16 heads, 196 cached segments, w = 8: seam step fused
                with the composition of every cached body pair
  gdn_ragged32k the cold request with uneven segments (58 .. 2048 tokens)
  gdn_warm100k_rerotate  rotary re-rotation of the warm request's cached pairs
                to new offsets
  kda_cold32k   the cold request's shape with KDA (per-channel gated delta rule):
                build + compose
  kda_warm100k  the warm request with KDA layers: seam step
Prints one JSON line.  `value` is segment-tokens/s of the whole step; the
`roofline` object is for the step's dominant kernel, timed with HIP events on
the stream it runs on; `cpu_baseline` times the fp64 oracle on a bounded
sample of the same workload on all of this host's threads, and on one thread.
The default run also carries a `warm` object: the warm request's seam step
(composed segments/s, its roofline and oracle), the metric's second half.
retnet and gla also report their composition alone as single-shot latency
and as back-to-back throughput.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "segment-tokens/s for (T_C,S) build + composed segs/s; % MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "build_delta": ["segment_scan_amd/csrc/kernels/build_delta2.hip"],
    "build_compose": ["segment_scan_amd/csrc/kernels/build_delta2.hip", "segment_scan_amd/csrc/kernels/chain.hip",
                      "segment_scan_amd/csrc/hypic_api.cpp"],
    "build_sd": ["segment_scan_amd/csrc/kernels/build_sd.hip", "segment_scan_amd/csrc/kernels/compose.hip"],
    "seam": ["segment_scan_amd/csrc/kernels/chain.hip", "segment_scan_amd/csrc/kernels/seam_prep.hip"],
    "compose": ["segment_scan_amd/csrc/kernels/compose.hip", "segment_scan_amd/csrc/kernels/chain.hip"],
    "rerotate": ["segment_scan_amd/csrc/kernels/rerotate.hip"],
    "build_kda": ["segment_scan_amd/csrc/kernels/build_kda.hip", "segment_scan_amd/csrc/kernels/build_delta2.hip"],
    "seam_kda": ["segment_scan_amd/csrc/kernels/seam_kda.hip"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel] + ["segment_scan_amd/csrc/kernels/common.h",
                                         "segment_scan_amd/csrc/kernels/split_f16.h"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were
    taken on the current source of the kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel") != kernel or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


# device kernels that make up each timed operation (substrings of their symbol names)
KERNEL_SYMBOLS = {
    "build_delta": ["delta_prep_kernel", "delta_state_kernel", "build_delta_kernel"],
    "build_compose": ["delta_prep_kernel", "delta_state_kernel", "chain_kernel", "chain_wide_kernel",
                      "zero_ints_kernel"],
    "build_sd": ["build_sd_kernel", "compose_elem_kernel"],
    "seam": ["seam_prep_kernel", "chain_kernel", "chain_wide_kernel"],
    "compose": ["chain_kernel", "chain_wide_kernel", "compose_elem_kernel"],
    "rerotate": ["rerotate_kernel"],
    "build_kda": ["kda_prep_kernel", "delta_state_kernel", "build_kda_kernel"],
    "seam_kda": ["seam_kda_kernel"],
}
CALIBRATION_COPIES = 3       # final dispatches of a --copy-calibration run
CALIBRATION_BYTES = 1 << 30  # each reads and writes this many bytes


def ingest_counters(wl, fetch_csv: str, write_csv: str, steps: int, cmds):
    """Turns two rocprofv3 --pmc runs of `bench.py --copy-calibration` (FETCH_SIZE,
    then WRITE_SIZE; counter_collection.csv files) into HBM bytes per launch of the
    timed operation, each counter scaled by what it reads for the plain 1 GiB copy
    kernel that ends the run, and records them in profiles/traffic.json.  The
    library's dispatches are cut into steps of `wl.step_dispatches`; the first
    `wl.op_dispatches` of each of the last `steps` steps are the timed operation."""
    import csv
    workload, kernel = wl.name, wl.kernel

    def per_dispatch(path, counter):
        rows = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                d = int(r["Dispatch_Id"])
                name, val = r["Kernel_Name"], float(r["Counter_Value"])
                rows[d] = (name, rows.get(d, (name, 0.0))[1] + val)
        return [rows[d] for d in sorted(rows)]

    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = per_dispatch(path, counter)
        cal = disp[-CALIBRATION_COPIES:]
        assert len(cal) == CALIBRATION_COPIES and len({n for n, _ in cal}) == 1 and "hypic" not in cal[0][0], \
            "calibration copies not found at the end of %s" % path
        kib_copy = float(np.median([v for _, v in cal]))
        factor = CALIBRATION_BYTES / (kib_copy * 1024.0)
        lib = [(n, v) for n, v in disp[:-CALIBRATION_COPIES] if "hypic" in n]
        sd, od = wl.step_dispatches, wl.op_dispatches
        assert len(lib) % sd == 0 and len(lib) // sd >= steps, \
            "%d library dispatches in %s are not whole steps of %d" % (len(lib), path, sd)
        timed = []
        for i in range(len(lib) - steps * sd, len(lib), sd):
            op = lib[i:i + od]
            assert all(any(k in n for k in KERNEL_SYMBOLS[kernel]) for n, _ in op), [n for n, _ in op]
            timed += op
        kib = sum(v for _, v in timed) / steps
        out[counter] = {"kib_per_launch": round(kib, 1), "copy_kib": round(kib_copy, 1),
                        "scale": round(factor, 4), "bytes_per_launch": int(kib * 1024 * factor),
                        "dispatches_per_launch": od}
    try:
        with open(TRAFFIC_FILE) as f:
            db = json.load(f)
    except (OSError, ValueError):
        db = {}
    db[workload] = {"kernel": kernel, "source_hash": source_hash(kernel),
                    "bytes_per_launch": out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"],
                    "fetch": out["FETCH_SIZE"], "write": out["WRITE_SIZE"], "commands": cmds}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(db, f, indent=1, sort_keys=True)
    return db[workload]


def counter_summary(paths):
    """Markdown table of the library's kernels in rocprofv3 --pmc runs
    (counter_collection.csv files, one pass each): per kernel, the mean of each
    counter per dispatch, and per wave the VALU and MFMA instructions and the
    fraction of wave cycles spent waiting on dependencies."""
    import csv
    import re
    vals = {}
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                if "hypic" not in r["Kernel_Name"]:
                    continue
                name = re.sub(r"hypic::(\(anonymous namespace\)::)?", "", r["Kernel_Name"])
                name = re.sub(r"\(.*", "", name).replace("void ", "")
                key = (name, r["Counter_Name"])
                d = vals.setdefault(key, {})
                d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    kernels = sorted({k for k, _ in vals})
    counters = sorted({c for _, c in vals})
    mean = {key: float(np.mean(list(d.values()))) for key, d in vals.items()}
    lines = ["| counter | " + " | ".join("`%s`" % k for k in kernels) + " |",
             "|---|" + "---|" * len(kernels)]
    for c in counters:
        lines.append("| %s | " % c + " | ".join("%.4g" % mean[(k, c)] if (k, c) in mean else "" for k in kernels)
                     + " |")

    def ratio(k, a, b):
        return mean[(k, a)] / mean[(k, b)] if (k, a) in mean and mean.get((k, b)) else None
    for label, a, b in (("VALU instructions per wave", "SQ_INSTS_VALU", "SQ_WAVES"),
                        ("MFMA instructions per wave", "SQ_INSTS_MFMA", "SQ_WAVES"),
                        ("LDS instructions per wave", "SQ_INSTS_LDS", "SQ_WAVES"),
                        ("wave cycles waiting on dependencies", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")):
        r = [ratio(k, a, b) for k in kernels]
        lines.append("| *%s* | " % label + " | ".join("" if x is None else "%.3g" % x for x in r) + " |")
    return "\n".join(lines)


def trace_summary(path, top=8):
    """Markdown table of a rocprofv3 --kernel-trace --stats kernel_stats.csv: the
    `top` kernels by total time, with calls, total, mean, min and max duration."""
    import csv
    import re
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Name"].replace("(anonymous namespace)::", "").replace("hypic::", "")
            name = re.sub(r"\(.*", "", name).replace("void ", "")
            rows.append((name[:80], int(r["Calls"]), float(r["TotalDurationNs"]), float(r["AverageNs"]),
                         float(r["MinNs"]), float(r["MaxNs"]), float(r["Percentage"])))
    rows.sort(key=lambda x: -x[2])
    lines = ["| kernel | calls | total ms | mean us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|---|"]
    for n, c, t, a, lo, hi, pct in rows[:top]:
        lines.append("| `%s` | %d | %.3f | %.1f | %.1f | %.1f | %.1f |" % (n, c, t / 1e6, a / 1e3, lo / 1e3, hi / 1e3,
                                                                          pct))
    return "\n".join(lines)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def to_dev(arr, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


# ------------------------------------------------------------------ workloads


class Workload:
    name = ""
    kernel = ""          # dominant kernel for the roofline
    op_dispatches = 1    # library dispatches of the timed operation per step
    step_dispatches = 1  # library dispatches per step (the timed operation first)
    tokens = 0           # segment-tokens per step
    composed = 0         # composed segments per step (per chain-group, see config)

    def setup(self):
        raise NotImplementedError

    def step(self, ev0, ev1):
        """Enqueue one step; records ev0/ev1 around the dominant kernel."""
        raise NotImplementedError

    def cpu_sample(self, n_threads=None):
        """Run the oracle on a bounded sample with n_threads threads (all host
        threads when None; the 1-thread run takes a smaller sample of the same
        work); returns (seconds, sample tokens, description)."""
        raise NotImplementedError


def _build_bytes(fam, L, d, es, gate_bytes_per_tok, u_out):
    per_tok = 2 * d * es + gate_bytes_per_tok
    out = d * d * 4 * (2 if u_out else 1) + 4 * (d if fam == 2 else 1)
    return L * per_tok + out


class ColdRequest(Workload):
    """GDN dense transition, one 32k-token cold request (32 heads, 64 x 512, bf16)."""
    name = "gdn_cold32k"
    kernel = "build_delta"
    fam = 3  # delta
    op_dispatches = 2    # factor pass, state pass
    step_dispatches = 6  # + the blocked composition (blocks, two pairwise levels, the last pair)

    def __init__(self):
        self.n_seg, self.L, self.H, self.d = 64, 512, 32, 128
        self.tokens = self.n_seg * self.L
        self.composed = self.n_seg
        units = self.n_seg * self.H
        self.alg_bytes = units * _build_bytes(3, self.L, self.d, 2, 4, True)
        self.alg_flops = units * 8.0 * self.L * self.d ** 2
        # executed MFMA flops of the two build kernels, 32x32x16 MFMAs per 64-token
        # chunk and unit: factor pass Gram 3 tiles x 8 k-steps and the inverse's two
        # 32 x 32 x 32 products in split form (2 x 2 k-steps x 3); state pass per
        # wave (8 waves, one 32-column tile each) K Z 16, A0 R 6, K^T X 16
        chunks = units * (self.L // 64)
        self.exec_flops = chunks * (24 + 12 + 8 * (16 + 6 + 16)) * 32 * 32 * 16 * 2.0

    def setup(self):
        import torch
        from segment_scan_amd import api, synth
        self.api, self.synth = api, synth
        tk = self._tokens()
        self.tk = tk
        self.k, self.v = to_dev(tk.k, "bf16"), to_dev(tk.v, "bf16")
        self.beta, self.lg = to_dev(tk.beta, "bf16"), to_dev(tk.log_gate, "bf16")
        self.offsets = [int(x) for x in tk.offsets]
        dev = "cuda"
        self.g = torch.empty((self.n_seg, self.H), device=dev)
        self.U = torch.empty((self.n_seg, self.H, self.d, self.d), device=dev)
        self.S = torch.empty((self.n_seg, self.H, self.d, self.d), device=dev)
        self.S_out = torch.empty((self.H, self.d, self.d), device=dev)
        n_ws = api.seg_build_workspace_size(self.fam, self.offsets, self.H, self.d, torch.bfloat16)
        self.ws = torch.empty(max(n_ws, 16), device=dev, dtype=torch.uint8)
        n_cws = api.compose_workspace_size(self.fam, self.n_seg, self.H, self.d)
        self.cws = torch.empty(n_cws, device=dev, dtype=torch.uint8) if n_cws else None

    def _tokens(self):
        return self.synth.gdn_cold(want_q=False)

    def step(self, ev0, ev1):
        ev0.record()
        self.api.seg_build(self.fam, self.offsets, self.k, self.v, self.beta, self.lg, out=(self.g, self.U, self.S),
                           workspace=self.ws)
        ev1.record()
        self.api.compose(self.fam, self.g, self.U, self.S, S_out=self.S_out, workspace=self.cws)

    def cpu_sample(self, n_threads=None):
        import oracle
        # all threads: the whole request, every segment and head built and composed;
        # one thread: its first 4 segments (all heads), a sixteenth of the work
        ns = self.n_seg if n_threads is None else 4
        t1 = int(self.tk.offsets[ns])
        sl = slice(0, t1)
        t = time.perf_counter()
        g, U, S = oracle.build_pairs(self.fam, self.tk.offsets[:ns + 1], self.tk.k[sl], self.tk.v[sl],
                                     self.tk.beta[sl], self.tk.log_gate[sl], n_threads=n_threads)
        oracle.compose(self.fam, g, U, S, n_threads=n_threads)
        dt = time.perf_counter() - t
        what = "whole request (64 segments x 32 heads = 2048 units)" if n_threads is None else \
            "segments 0-3 of the request (x 32 heads = 128 units)"
        return dt, int(self.tk.offsets[ns]), what + ": build + ordered compose"

    def config(self):
        return {"workload": self.name, "family": "gdn", "heads": self.H, "d": self.d, "segments": self.n_seg,
                "segment_len": self.L, "tokens": self.tokens, "inputs": "bf16", "accumulate": "fp32",
                "step": "hypic_seg_build (2048 units) + hypic_compose (32 chains x 64)"}


class PipelinedColdRequest(ColdRequest):
    """The cold GDN request in one call (hypic_seg_build_compose): groups of 16
    segments built on the caller's stream, each group composed on a second
    stream while the next is built, the group pairs composed in order last.
    The timed operation is the whole call; its algorithmic bytes are the
    build's (tokens in, pairs out) plus the final states."""
    name = "gdn_cold32k_pipelined"
    kernel = "build_compose"
    op_dispatches = 13   # 4 x (factor pass, state pass, group composition) + final composition
    step_dispatches = 13

    def __init__(self):
        super().__init__()
        self.alg_bytes += self.H * self.d * self.d * 4

    def setup(self):
        import torch
        super().setup()
        n_ws = self.api.seg_build_compose_workspace_size(self.fam, self.offsets, self.H, self.d, torch.bfloat16,
                                                         self.api.BC_PIPELINED)
        self.ws = torch.empty(n_ws, device="cuda", dtype=torch.uint8)

    def step(self, ev0, ev1):
        ev0.record()
        self.api.seg_build_compose(self.fam, self.offsets, self.k, self.v, self.beta, self.lg,
                                   out=(self.g, self.U, self.S), S_out=self.S_out, mode=self.api.BC_PIPELINED,
                                   workspace=self.ws)
        ev1.record()

    def config(self):
        c = super().config()
        c.update(workload=self.name, step="hypic_seg_build_compose (2048 units in 4 groups of 16 segments, "
                                          "each group composed on a second stream while the next is built)")
        return c


class FusedColdRequest(PipelinedColdRequest):
    """The cold GDN request in one call with the composition folded into the
    build (hypic_seg_build_compose, fused schedule): each build workgroup counts
    its pair's arrival at a node of a binary tree over the 64 segments of its
    chain, and the last arrival at a node composes it.  The timed operation is
    the whole call."""
    name = "gdn_cold32k_fused"
    kernel = "build_compose"
    op_dispatches = 3    # counter reset, factor pass, state pass (with the composition)
    step_dispatches = 3

    def setup(self):
        import torch
        ColdRequest.setup(self)
        n_ws = self.api.seg_build_compose_workspace_size(self.fam, self.offsets, self.H, self.d, torch.bfloat16,
                                                         self.api.BC_FUSED)
        self.ws = torch.empty(n_ws, device="cuda", dtype=torch.uint8)

    def step(self, ev0, ev1):
        ev0.record()
        self.api.seg_build_compose(self.fam, self.offsets, self.k, self.v, self.beta, self.lg,
                                   out=(self.g, self.U, self.S), S_out=self.S_out, mode=self.api.BC_FUSED,
                                   workspace=self.ws)
        ev1.record()

    def config(self):
        c = ColdRequest.config(self)
        c.update(workload=self.name, step="hypic_seg_build_compose, fused schedule (2048 units; the composition "
                                          "as a tree per chain, each node composed by the last build workgroup "
                                          "to reach it)")
        return c


class RaggedRequest(ColdRequest):
    """The cold GDN request with uneven segments: 32 heads, 64 segments of 58 .. 2048
    tokens (log-normal lengths, median 366), 32,768 tokens; built longest first."""
    name = "gdn_ragged32k"

    def __init__(self):
        from segment_scan_amd import synth
        super().__init__()
        lens = synth.ragged_lengths(self.n_seg, self.tokens)
        self.alg_bytes = self.H * sum(_build_bytes(3, int(L), self.d, 2, 4, True) for L in lens)
        self.alg_flops = self.H * 8.0 * self.tokens * self.d ** 2
        chunks = self.H * sum((int(L) + 63) // 64 for L in lens)
        self.exec_flops = chunks * (24 + 12 + 8 * (16 + 6 + 16)) * 32 * 32 * 16 * 2.0

    def _tokens(self):
        return self.synth.gdn_ragged(want_q=False)

    def config(self):
        c = super().config()
        c.update(workload=self.name, segment_len="58..2048 (log-normal, median 366)",
                 step="hypic_seg_build (2048 ragged units, longest first) + hypic_compose (32 chains x 64)")
        return c


class KdaRequest(ColdRequest):
    """KDA (delta rule with per-channel gates) at the cold request's shape: 32 heads,
    64 x 512 tokens, d = 128, bf16 tokens and per-channel gates."""
    name = "kda_cold32k"
    kernel = "build_kda"
    fam = 4  # kda
    op_dispatches = 2    # factor pass, state pass
    step_dispatches = 6  # + the blocked composition (blocks, two pairwise levels, the last pair)

    def __init__(self):
        super().__init__()
        units = self.n_seg * self.H
        # per token: k, v and the d channel gates (bf16) and beta
        self.alg_bytes = units * _build_bytes(4, self.L, self.d, 2, 2 * self.d + 2, True)
        # executed 32x32x16 MFMAs per 64-token chunk and unit: factor pass Gram 3
        # tiles x 8 k-steps and the inverse's two 32 x 32 x 32 products (2 k-steps),
        # each in two bf16 terms (3 products); state pass as the delta one, fp16
        # (8 waves: K Z 16, X R 6, K^T X 16)
        chunks = units * (self.L // 64)
        self.exec_flops = chunks * (3 * (3 * 8 + 2 * 2) + 8 * (16 + 6 + 16)) * 32 * 32 * 16 * 2.0

    def _tokens(self):
        return self.synth.kda()

    def config(self):
        c = super().config()
        c.update(workload=self.name, family="kda", gates="per token and key channel (bf16)",
                 step="hypic_seg_build (2048 KDA units) + hypic_compose (32 chains x 64)")
        return c


class ScalarOrDiag(Workload):
    def __init__(self, name, fam, n_seg, L, H, d):
        import torch
        from segment_scan_amd import api, synth
        self.name, self.fam = name, fam
        self.kernel = "build_sd"
        self.n_seg, self.L, self.H, self.d = n_seg, L, H, d
        # few units: the build runs as pieces joined by a grouped composition (a
        # second dispatch, which needs a workspace); the ordered compose follows
        split = api.seg_build_workspace_size(fam, list(synth.even_offsets(n_seg, L)), H, d, torch.bfloat16) > 0
        self.op_dispatches = 2 if split else 1
        self.step_dispatches = self.op_dispatches + 1
        self.tokens = n_seg * L
        self.composed = n_seg
        units = n_seg * H
        gate = 2 * d if fam == 2 else 0
        self.alg_bytes = units * _build_bytes(fam, L, d, 2, gate, False)
        self.alg_flops = units * 2.0 * L * d ** 2
        self.exec_flops = self.alg_flops * 2  # decay-weighted keys in two bf16 terms

    def setup(self):
        import torch
        from segment_scan_amd import api, synth
        self.api = api
        tk = synth.retnet() if self.fam == 1 else synth.gla()
        tk.q = None
        self.tk = tk
        k, v = to_dev(tk.k, "bf16"), to_dev(tk.v, "bf16")
        lg = to_dev(tk.log_gate, "f32") if tk.gate_per_chain else to_dev(tk.log_gate, "bf16")
        self.offsets = [int(x) for x in tk.offsets]
        dev = "cuda"
        gshape = (self.n_seg, self.H, self.d) if self.fam == 2 else (self.n_seg, self.H)
        # Rotate input/output sets whose total exceeds twice the 256 MB last-level
        # cache (MALL), so that repeated steps stream from HBM
        self.n_sets = max(1, -(-2 * (256 << 20) // self.alg_bytes) + 1)
        self.sets = []
        for i in range(self.n_sets):
            self.sets.append(dict(k=k if i == 0 else k.clone(), v=v if i == 0 else v.clone(),
                                  lg=lg if i == 0 else lg.clone(), g=torch.empty(gshape, device=dev),
                                  S=torch.empty((self.n_seg, self.H, self.d, self.d), device=dev),
                                  S_out=torch.empty((self.H, self.d, self.d), device=dev)))
        self.i_set = 0
        n_ws = api.seg_build_workspace_size(self.fam, self.offsets, self.H, self.d, torch.bfloat16)
        self.ws = torch.empty(max(n_ws, 16), device=dev, dtype=torch.uint8)

    def step(self, ev0, ev1):
        b = self.sets[self.i_set]
        self.i_set = (self.i_set + 1) % self.n_sets
        ev0.record()
        self.api.seg_build(self.fam, self.offsets, b["k"], b["v"], None, b["lg"], self.tk.gate_per_chain,
                           out=(b["g"], None, b["S"]), workspace=self.ws)
        ev1.record()
        self.api.compose(self.fam, b["g"], None, b["S"], S_out=b["S_out"])

    def cpu_sample(self, n_threads=None):
        import oracle
        ns = self.n_seg if n_threads is None else max(1, self.n_seg // 8)
        t1 = int(self.tk.offsets[ns])
        sl = slice(0, t1)
        lg = self.tk.log_gate if self.tk.gate_per_chain else self.tk.log_gate[sl]
        t = time.perf_counter()
        g, U, S = oracle.build_pairs(self.fam, self.tk.offsets[:ns + 1], self.tk.k[sl], self.tk.v[sl], None, lg,
                                     self.tk.gate_per_chain, n_threads=n_threads)
        oracle.compose(self.fam, g, U, S, n_threads=n_threads)
        dt = time.perf_counter() - t
        return dt, ns * self.L, "%d of %d segments (x %d heads): build + ordered compose" % (
            ns, self.n_seg, self.H)

    def extra(self):
        """The ordered composition of this workload's pairs on its own: single-shot
        latency (each call alone, synchronised before and after, as a lone
        request sees it) and steady state (back-to-back calls over the rotating
        buffer sets)."""
        import torch
        b = self.sets[0]
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for e0, e1 in ev:
            torch.cuda.synchronize()
            e0.record()
            self.api.compose(self.fam, b["g"], None, b["S"], S_out=b["S_out"])
            e1.record()
            torch.cuda.synchronize()
        single = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        reps = 50
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for i in range(reps):
            bs = self.sets[i % self.n_sets]
            self.api.compose(self.fam, bs["g"], None, bs["S"], S_out=bs["S_out"])
        c1.record()
        torch.cuda.synchronize()
        steady = c0.elapsed_time(c1) / reps
        gbytes = self.n_seg * self.H * (self.d * self.d * 4 + 4 * (self.d if self.fam == 2 else 1)) + \
            self.H * self.d * self.d * 4
        return {"compose": {"single_shot_ms_median": round(single[len(single) // 2], 4),
                            "steady_state_ms": round(steady, 4),
                            "steady_state_gbs": round(gbytes / (steady / 1e3) / 1e9, 1),
                            "alg_bytes": gbytes,
                            "composed_segs_per_s_steady": round(self.n_seg / (steady / 1e3), 1)}}

    def config(self):
        return {"workload": self.name, "family": "retnet" if self.fam == 1 else "gla", "heads": self.H, "d": self.d,
                "segments": self.n_seg, "segment_len": self.L, "tokens": self.tokens, "inputs": "bf16",
                "buffer_sets": getattr(self, "n_sets", None),
                "accumulate": "fp32", "step": "hypic_seg_build + hypic_compose"}


class WarmRequest(Workload):
    """Warm reuse of a 100k-token request: 30 GDN layers x 16 heads, 196 cached segments, w = 8."""
    name = "gdn_warm100k"
    kernel = "seam"
    op_dispatches = 2    # window factor pre-pass, chain
    step_dispatches = 2

    def __init__(self):
        from segment_scan_amd import synth
        self.layers, self.H, self.n_seg, self.w, self.d = (synth.WARM_LAYERS, synth.WARM_HEADS, synth.WARM_SEGS,
                                                           synth.WARM_W, synth.WARM_D)
        self.chains = self.layers * self.H
        self.tokens = self.n_seg * (512 + self.w)
        self.composed = self.n_seg * self.layers  # (layer, segment) compositions
        d, n = self.d, self.chains
        ntok = self.n_seg * self.w
        self.alg_bytes = (self.n_seg * n * (2 * d * d * 4 + 4) + ntok * n * (3 * d * 2 + 4) + ntok * n * d * 4
                          + 2 * n * d * d * 4)
        self.alg_flops = self.n_seg * n * 2.0 * d ** 3 + ntok * n * 6.0 * d * d
        # body products as three fp16 MFMA passes (hi*hi, hi*lo, lo*hi), and per
        # window [K; Q] S (16 rows) and the rank-8 update, three passes each
        # (within 2 % of the MFMA op counters)
        self.exec_flops = self.n_seg * n * 3 * 2.0 * (d ** 3 + (16 + 8) * d * d)

    def setup(self):
        import torch
        from segment_scan_amd import api, synth
        self.api, self.synth = api, synth
        H, d, n_seg, w, n = self.H, self.d, self.n_seg, self.w, self.chains
        # seam tokens and pairs of every layer from the seeded recipe, drawn on the GPU
        gen = torch.Generator(device="cuda").manual_seed(20260701)
        nt = n_seg * w
        f = torch.nn.functional
        self.q = f.normalize(torch.randn((nt, n, d), device="cuda", generator=gen), dim=-1).to(torch.bfloat16)
        self.k = f.normalize(torch.randn((nt, n, d), device="cuda", generator=gen), dim=-1).to(torch.bfloat16)
        self.v = torch.randn((nt, n, d), device="cuda", generator=gen).to(torch.bfloat16)
        self.beta = torch.sigmoid(torch.randn((nt, n), device="cuda", generator=gen)).to(torch.bfloat16)
        self.lg = (-f.softplus(torch.randn((nt, n), device="cuda", generator=gen)) / 8).to(torch.bfloat16)
        self.U = torch.randn((n_seg, n, d, d), device="cuda", generator=gen) * (0.5 / np.sqrt(d))
        self.S = torch.randn((n_seg, n, d, d), device="cuda", generator=gen)
        self.g = torch.zeros((n_seg, n), device="cuda")
        self.S_run = torch.zeros((n, d, d), device="cuda")
        self.o = torch.empty((nt, n, d), device="cuda")
        self.ws = torch.empty(api.seam_step_workspace_size(synth.DELTA, n_seg, w, n, d), device="cuda",
                              dtype=torch.uint8)

    def step(self, ev0, ev1):
        from segment_scan_amd.synth import DELTA
        self.S_run.zero_()
        ev0.record()
        self.api.seam_step(DELTA, self.w, self.q, self.k, self.v, self.beta, self.lg, body=(self.g, self.U, self.S),
                           S_run=self.S_run, o_out=self.o, workspace=self.ws)
        ev1.record()

    def cpu_sample(self, n_threads=None):
        import oracle
        from segment_scan_amd import synth
        from segment_scan_amd.synth import DELTA
        # all threads: layers 0 and 1 in full (196 segments x 16 heads each); one
        # thread: the first 49 segments of layer 0
        n_layers = 2 if n_threads is None else 1
        n_seg = self.n_seg if n_threads is None else self.n_seg // 4
        dt = 0.0
        for layer in range(n_layers):
            tk = synth.warm_seam_layer(layer, n_seg=n_seg)
            body = synth.warm_pairs_layer(layer, n_seg=n_seg)
            t = time.perf_counter()
            oracle.seam(DELTA, n_seg, self.w, tk.q, tk.k, tk.v, tk.beta, tk.log_gate, body=body,
                        n_threads=n_threads)
            dt += time.perf_counter() - t
        # the sample's share of the request's work
        frac = n_layers / self.layers * n_seg / self.n_seg
        what = "layers 0-1 of 30 in full" if n_threads is None else "segments 0-48 of layer 0"
        return dt, self.tokens * frac, what + " (seam + compose), scaled"

    def config(self):
        return {"workload": self.name, "family": "gdn", "layers": self.layers, "heads": self.H, "d": self.d,
                "segments": self.n_seg, "w": self.w, "tokens": self.tokens, "pairs": "fp32", "seam_inputs": "bf16",
                "step": "hypic_seam_step over 480 chains (seam windows + body-pair composition)"}


class KdaWarmRequest(WarmRequest):
    """The warm 100k-token request with KDA layers: 30 layers x 16 heads, 196 cached
    segments, w = 8, window gates per token and key channel."""
    name = "kda_warm100k"
    kernel = "seam_kda"
    op_dispatches = 1
    step_dispatches = 1

    def __init__(self):
        super().__init__()
        d, n = self.d, self.chains
        ntok = self.n_seg * self.w
        # as the GDN warm request plus the per-channel window gates (bf16)
        self.alg_bytes += ntok * n * (2 * d - 2)
        # body products on MFMA in two bf16 terms (three products); windows on the VALU
        self.exec_flops = self.n_seg * n * 3 * 2.0 * d ** 3

    def setup(self):
        import torch
        super().setup()
        gen = torch.Generator(device="cuda").manual_seed(20260703)
        nt, n, d = self.n_seg * self.w, self.chains, self.d
        f = torch.nn.functional
        self.lg = (-f.softplus(torch.randn((nt, n, d), device="cuda", generator=gen)) / 8).to(torch.bfloat16)
        self.ws = None

    def step(self, ev0, ev1):
        from segment_scan_amd.synth import KDA
        self.S_run.zero_()
        ev0.record()
        self.api.seam_step(KDA, self.w, self.q, self.k, self.v, self.beta, self.lg, body=(self.g, self.U, self.S),
                           S_run=self.S_run, o_out=self.o)
        ev1.record()

    def cpu_sample(self, n_threads=None):
        import oracle
        from segment_scan_amd import synth
        from segment_scan_amd.synth import KDA
        n_layers = 2 if n_threads is None else 1
        n_seg = self.n_seg if n_threads is None else self.n_seg // 4
        dt = 0.0
        for layer in range(n_layers):
            tk = synth.kda(n_seg=n_seg, L=self.w, n_chain=self.H, want_q=True)
            body = synth.warm_pairs_layer(layer, n_seg=n_seg)
            t = time.perf_counter()
            oracle.seam(KDA, n_seg, self.w, tk.q, tk.k, tk.v, tk.beta, tk.log_gate, body=body,
                        n_threads=n_threads)
            dt += time.perf_counter() - t
        frac = n_layers / self.layers * n_seg / self.n_seg
        what = "layers 0-1 of 30 in full" if n_threads is None else "segments 0-48 of layer 0"
        return dt, self.tokens * frac, what + " (seam + compose), scaled"

    def config(self):
        c = super().config()
        c.update(workload=self.name, family="kda",
                 step="hypic_seam_step (KDA) over 480 chains (seam windows + body-pair composition)")
        return c


class WarmRerotate(Workload):
    """Rotary re-rotation of the warm 100k-token request's cached pairs (30 GDN
    layers x 16 heads x 196 segments, d = 128, fp32 U and S) to new offsets."""
    name = "gdn_warm100k_rerotate"
    kernel = "rerotate"

    def __init__(self):
        from segment_scan_amd import synth
        self.layers, self.H, self.n_seg, self.d = synth.WARM_LAYERS, synth.WARM_HEADS, synth.WARM_SEGS, synth.WARM_D
        self.chains = self.layers * self.H
        self.tokens = self.n_seg * 512  # cached body tokens moved
        self.composed = 0
        units = self.n_seg * self.chains
        # U and S of every unit read and written once, plus the offsets
        self.alg_bytes = units * 2 * 2 * self.d * self.d * 4 + self.n_seg * 4
        self.alg_flops = 0.0
        self.exec_flops = 0.0

    def setup(self):
        import torch
        from segment_scan_amd import api
        self.api = api
        n_seg, n, d = self.n_seg, self.chains, self.d
        gen = torch.Generator(device="cuda").manual_seed(20260702)
        self.U = torch.randn((n_seg, n, d, d), device="cuda", generator=gen) * (0.5 / np.sqrt(d))
        self.S = torch.randn((n_seg, n, d, d), device="cuda", generator=gen)
        self.pos = torch.randint(-(1 << 20), 1 << 20, (n_seg,), device="cuda", generator=gen, dtype=torch.int32)

    def step(self, ev0, ev1):
        from segment_scan_amd.synth import DELTA
        ev0.record()
        self.api.rerotate(DELTA, self.pos, self.S, self.U)
        ev1.record()

    def cpu_sample(self, n_threads=None):
        import oracle
        from segment_scan_amd import synth
        from segment_scan_amd.synth import DELTA
        n_layers = 2 if n_threads is None else 1
        n_seg = self.n_seg if n_threads is None else self.n_seg // 4
        pos = np.random.default_rng(20260702).integers(-(1 << 20), 1 << 20, n_seg)
        dt = 0.0
        for layer in range(n_layers):
            _, U, S = synth.warm_pairs_layer(layer, n_seg=n_seg)
            t = time.perf_counter()
            oracle.rerotate(DELTA, U, S, pos, n_threads=n_threads)
            dt += time.perf_counter() - t
        frac = n_layers / self.layers * n_seg / self.n_seg
        return dt, self.tokens * frac, "%d layer(s) x %d segments x 16 heads, scaled" % (n_layers, n_seg)

    def config(self):
        return {"workload": self.name, "family": "gdn", "layers": self.layers, "heads": self.H, "d": self.d,
                "segments": self.n_seg, "pairs": "fp32", "rope_base": 10000.0,
                "step": "hypic_rerotate of 196 x 480 cached pairs in place (U <- R U R^T, S <- R S)"}


WORKLOADS = {
    "gdn_cold32k": ColdRequest,
    "gdn_cold32k_pipelined": PipelinedColdRequest,
    "gdn_cold32k_fused": FusedColdRequest,
    "retnet": lambda: ScalarOrDiag("retnet", 1, 16, 1024, 8, 128),
    "gla": lambda: ScalarOrDiag("gla", 2, 64, 512, 16, 128),
    "gdn_warm100k": WarmRequest,
    "gdn_ragged32k": RaggedRequest,
    "gdn_warm100k_rerotate": WarmRerotate,
    "kda_cold32k": KdaRequest,
    "kda_warm100k": KdaWarmRequest,
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gdn_cold32k", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-warm", action="store_true",
                    help="default workload only: skip the warm request's object")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with three plain 1 GiB device copies (for scaling rocprofv3 byte counters)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="record HBM traffic of --workload from two rocprofv3 counter runs (no GPU needed)")
    ap.add_argument("--counter-commands", nargs="*", default=[], help="the rocprofv3 commands, for the record")
    ap.add_argument("--counter-summary", nargs="+", metavar="CSV",
                    help="print per-kernel means of rocprofv3 --pmc counter_collection.csv files and exit")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print the top kernels of a rocprofv3 --stats kernel_stats.csv and exit")
    args = ap.parse_args()
    if args.counter_summary:
        print(counter_summary(args.counter_summary))
        return
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.ingest_counters:
        wl = WORKLOADS[args.workload]()
        rec = ingest_counters(wl, args.ingest_counters[0], args.ingest_counters[1], args.steps,
                              args.counter_commands)
        print(json.dumps(rec))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (how the work would shard across "
              "GPUs is a design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    wl = WORKLOADS[args.workload]()
    ms_per_step, kern_ms = measure(wl, args.steps, args.warmup)

    if args.copy_calibration:
        n = CALIBRATION_BYTES // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(CALIBRATION_COPIES):  # an elementwise kernel (a same-dtype copy_ may become a DMA copy)
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    copy_gbs = None if args.copy_calibration else copy_bandwidth()

    roofline = roofline_obj(wl, kern_ms, copy_gbs)
    cpu = None if args.no_cpu_baseline else cpu_obj(wl)
    out = {"metric": METRIC, "value": round(wl.tokens / (ms_per_step / 1e3), 1), "unit": "segment-tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": wl.config(),
           "composed_segs_per_s": round(wl.composed / (ms_per_step / 1e3), 1),
           "roofline": roofline, "cpu_baseline": cpu}
    if hasattr(wl, "extra") and not args.copy_calibration:  # (the calibration copies end a counter run)
        out.update(wl.extra())

    # The metric's second half, composed segments per second, lives in the warm
    # request: the default run also measures it (as its own object, after the
    # cold request's buffers are released)
    if args.workload == "gdn_cold32k" and not args.no_warm and not args.copy_calibration:
        del wl
        torch.cuda.empty_cache()
        ww = WarmRequest()
        w_ms, w_kern = measure(ww, args.steps, args.warmup)
        out["warm"] = {"config": ww.config(), "ms_per_step": round(w_ms, 4),
                       "composed_segs_per_s": round(ww.composed / (w_ms / 1e3), 1),
                       "composed_head_segs_per_s": round(ww.composed * ww.H / (w_ms / 1e3), 1),
                       "segment_tokens_per_s": round(ww.tokens / (w_ms / 1e3), 1),
                       "roofline": roofline_obj(ww, w_kern, copy_gbs),
                       "cpu_baseline": None if args.no_cpu_baseline else cpu_obj(ww)}
    print(json.dumps(out), flush=True)


def measure(wl, steps, warmup):
    """Set up, run `warmup` untimed steps, then time exactly `steps` (wall clock
    around them, synchronised on both sides) and the dominant operation of each
    with HIP events on the stream it runs on.  Returns (ms per step, op ms list)."""
    import torch
    print("[bench] setting up %s" % wl.name, file=sys.stderr, flush=True)
    wl.setup()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps + warmup)]
    for i in range(warmup):
        wl.step(*evs[i])
    torch.cuda.synchronize()
    print("[bench] warmup done (%s)" % wl.name, file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(steps):
        wl.step(*evs[warmup + i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    return elapsed * 1e3 / steps, [a.elapsed_time(b) for a, b in evs[warmup:]]


def copy_bandwidth():
    """Achievable HBM bandwidth on this machine: an elementwise kernel reading and
    writing 1 GiB each (out of place), timed with events."""
    import torch
    n = CALIBRATION_BYTES // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    c1.record()
    torch.cuda.synchronize()
    gbs = round(5 * 2 * CALIBRATION_BYTES / (c0.elapsed_time(c1) / 1e3) / 1e9, 1)
    del src, dst
    return gbs


def roofline_obj(wl, kern_ms, copy_gbs):
    k_ms = float(np.mean(kern_ms))
    achieved = wl.alg_bytes / (k_ms / 1e3) / 1e9
    return {"bound": "hbm", "kernel": wl.kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl.name, wl.kernel),
            "alg_bytes_per_launch": wl.alg_bytes, "kernel_ms": round(k_ms, 4),
            "kernel_ms_median": round(float(np.median(kern_ms)), 4),
            "kernel_ms_p10": round(float(np.percentile(kern_ms, 10)), 4),
            "kernel_ms_p90": round(float(np.percentile(kern_ms, 90)), 4),
            "mfma_alg_tflops": round(wl.alg_flops / (k_ms / 1e3) / 1e12, 1),
            "mfma_exec_tflops": round(wl.exec_flops / (k_ms / 1e3) / 1e12, 1),
            "mfma_exec_frac": round(wl.exec_flops / (k_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "copy_gbs": copy_gbs, "frac_of_copy": None if not copy_gbs else round(achieved / copy_gbs, 4)}


def cpu_obj(wl):
    """The oracle timed on this host: all threads on the bounded sample, and one
    thread on a smaller sample of the same work."""
    import oracle
    print("[bench] timing the oracle on a sample (%s)" % wl.name, file=sys.stderr, flush=True)
    dt, tokens, desc = wl.cpu_sample()
    dt1, tokens1, desc1 = wl.cpu_sample(n_threads=1)
    return {"value": round(tokens / dt, 2), "unit": "segment-tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle", "sample": desc, "seconds": round(dt, 2), "cpu_model": cpu_model(),
            "single_thread": {"value": round(tokens1 / dt1, 2), "cores": 1, "sample": desc1,
                              "seconds": round(dt1, 2)}}


if __name__ == "__main__":
    main()
