"""bench.py's byte-counter ingestion (no GPU): synthetic rocprofv3 counter files.

The ingestion cuts the library's dispatches into steps, takes the timed
operation's dispatches from the last `steps` steps and scales each counter by
what it reads for the 1 GiB calibration copies at the end of the run.
"""
import csv
import json
import os

import pytest

import bench


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, val) in enumerate(rows):
            # two counter rows per dispatch (per-XCD partial values), summed by the ingestion
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val / 2})
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val / 2})


def _run(tmp_path, monkeypatch, wl, step_kernels, op_kib, other_kib, steps, warmup, copy_kib):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = [("void at::native::fill", 99.0)]  # torch work before the steps
        for _ in range(warmup + steps):
            for j, name in enumerate(step_kernels):
                rows.append((name, op_kib if j < wl.op_dispatches else other_kib))
        rows += [("void at::native::vectorized_elementwise_kernel<mul>", copy_kib)] * bench.CALIBRATION_COPIES
        _write(tmp_path / (counter + ".csv"), counter, rows)
    return bench.ingest_counters(wl, str(tmp_path / "FETCH_SIZE.csv"), str(tmp_path / "WRITE_SIZE.csv"), steps,
                                 ["cmd"])


def test_cold_request_two_op_dispatches_of_six(tmp_path, monkeypatch):
    wl = bench.WORKLOADS["gdn_cold32k"]()
    kernels = ["hypic::delta_prep_kernel(x)", "hypic::delta_state_kernel<1>(x)"] + \
        ["hypic::chain_wide_kernel<2, false, true>(x)"] * 4
    rec = _run(tmp_path, monkeypatch, wl, kernels, op_kib=1000.0, other_kib=7777.0, steps=20, warmup=5,
               copy_kib=524288.0)
    # two op dispatches of 1000 KiB per step; 1 GiB copy reads 512 MiB -> scale 2
    assert rec["fetch"]["dispatches_per_launch"] == 2
    assert rec["fetch"]["scale"] == 2.0
    assert rec["fetch"]["bytes_per_launch"] == 2 * 1000 * 1024 * 2
    assert rec["bytes_per_launch"] == 2 * (2 * 1000 * 1024 * 2)
    with open(tmp_path / "traffic.json") as f:
        assert json.load(f)["gdn_cold32k"]["source_hash"] == bench.source_hash("build_delta")


def test_same_kernel_inside_and_outside_the_operation(tmp_path, monkeypatch):
    """retnet's split build ends with a grouped composition by the same kernel
    that the ordered compose after the timed region uses: only the first one counts."""
    wl = bench.WORKLOADS["retnet"]()
    assert (wl.op_dispatches, wl.step_dispatches) == (2, 3)
    kernels = ["hypic::build_sd_kernel<1>(x)", "hypic::compose_elem_kernel<1, 128>(x)",
               "hypic::compose_elem_kernel<1, 128>(x)"]
    rec = _run(tmp_path, monkeypatch, wl, kernels, op_kib=10.0, other_kib=5000.0, steps=4, warmup=1,
               copy_kib=1048576.0)
    assert rec["write"]["bytes_per_launch"] == 2 * 10 * 1024


def test_wrong_step_structure_is_refused(tmp_path, monkeypatch):
    wl = bench.WORKLOADS["gdn_cold32k"]()
    kernels = ["hypic::delta_prep_kernel(x)", "hypic::delta_state_kernel<1>(x)", "hypic::chain_kernel<128, 4>(x)"]
    with pytest.raises(AssertionError):
        _run(tmp_path, monkeypatch, wl, kernels, op_kib=1.0, other_kib=1.0, steps=3, warmup=1, copy_kib=1.0)
