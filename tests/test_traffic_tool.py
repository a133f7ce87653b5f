"""The counter summary behind the benchmark's `traffic` figure (CPU): on small synthetic rocprofv3
counter and trace CSVs, `summarize` scales each kernel's mean per-dispatch counter by the plain
copy's calibration factor (true bytes / counted bytes of the run's last dispatch), keys the two
products of a layer by their grids, attaches mean durations and the algorithmic bytes, and
`bytes_per_launch` returns the scaled bytes only while the kernel sources are unchanged."""
import csv
import json
import os

import pytest

from two_tower_cross_amd import traffic

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]
ATTN = "void tt::block_attn_bf16_kernel<128>(tt::AttnParams)"
LIN = "void tt::linear_kernel<2>(tt::LinearParams, int)"
COPY = "__amd_rocclr_copyBuffer"
QKV_GRID, OUT_GRID = 216 * 512, 256 * 512      # the QKV product runs on the smaller grid


def write_counters(path, counter, rows):
    """rows: (kernel name, grid size, KiB counted); dispatch ids in order, one row each."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, (name, grid, kib) in enumerate(rows, start=1):
            w.writerow({k: 0 for k in FIELDS} | {"Dispatch_Id": d, "Grid_Size": grid,
                                                  "Kernel_Name": name, "Counter_Name": counter,
                                                  "Counter_Value": kib})


def write_trace(path, rows):
    """rows: (kernel name, grid size, duration ns)."""
    fields = ["Kernel_Name", "Grid_Size", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        t = 1000
        for name, grid, ns in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Start_Timestamp": t,
                        "End_Timestamp": t + ns})
            t += ns + 10


@pytest.fixture()
def csvs(tmp_path):
    f, w, t = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.csv"
    # two launches of each kernel, then the 1 MiB calibration copy, counted as half its bytes
    # by the fetch counter and exactly by the write counter
    write_counters(f, "FETCH_SIZE", [(ATTN, 2048 * 512, 100.0), (LIN, QKV_GRID, 10.0),
                                     (LIN, OUT_GRID, 20.0), (ATTN, 2048 * 512, 300.0),
                                     (LIN, QKV_GRID, 30.0), (LIN, OUT_GRID, 40.0),
                                     (COPY, 4096, 512.0)])
    write_counters(w, "WRITE_SIZE", [(ATTN, 2048 * 512, 8.0), (LIN, QKV_GRID, 1.0),
                                     (LIN, OUT_GRID, 2.0), (ATTN, 2048 * 512, 8.0),
                                     (LIN, QKV_GRID, 3.0), (LIN, OUT_GRID, 4.0),
                                     (COPY, 4096, 1024.0)])
    write_trace(t, [(ATTN, 2048 * 512, 70_000), (LIN, QKV_GRID, 10_000), (LIN, OUT_GRID, 12_000),
                    (ATTN, 2048 * 512, 80_000), (LIN, QKV_GRID, 14_000), (LIN, OUT_GRID, 16_000)])
    return str(f), str(w), str(t)


def test_counts_are_scaled_by_the_copy_calibration(csvs):
    s = traffic.summarize(*csvs[:2], 1, csvs[2])
    assert s["calibration"]["FETCH_SIZE"]["factor"] == pytest.approx(2.0)
    assert s["calibration"]["WRITE_SIZE"]["factor"] == pytest.approx(1.0)
    k = s["kernels"]
    attn = k["block_attn_bf16_kernel<128>"]
    # mean of the two dispatches, KiB -> bytes, times the factor
    assert attn["dispatches"] == 2
    assert attn["FETCH_SIZE"] == int(200.0 * 1024 * 2.0)
    assert attn["WRITE_SIZE"] == int(8.0 * 1024)
    assert attn["traffic_bytes"] == attn["FETCH_SIZE"] + attn["WRITE_SIZE"]
    assert attn["mean_us"] == pytest.approx(75.0)
    alg = traffic.ALGORITHMIC_LOOP32K["block_attn_bf16_kernel<128>"]
    assert attn["algorithmic_bytes"] == alg
    assert attn["algorithmic_GBps"] == pytest.approx(round(alg / 75.0 / 1e3, 1))
    # the two products of a layer: one kernel on two grids, told apart by grid
    qkv, out = k["linear_kernel<2>@qkv"], k["linear_kernel<2>@out"]
    assert qkv["FETCH_SIZE"] == int(20.0 * 1024 * 2.0) and out["FETCH_SIZE"] == int(30.0 * 1024 * 2.0)
    assert qkv["WRITE_SIZE"] == int(2.0 * 1024) and out["WRITE_SIZE"] == int(3.0 * 1024)
    assert qkv["mean_us"] == pytest.approx(12.0) and out["mean_us"] == pytest.approx(14.0)
    # the calibration copy itself is not a kernel of the library
    assert not any("copyBuffer" in name for name in k)


def test_bytes_per_launch_follows_the_sources(csvs, tmp_path, monkeypatch):
    s = traffic.summarize(*csvs[:2], 1, csvs[2])
    md = tmp_path / "summary.md"
    md.write_text("# summary\n\n" + json.dumps(s) + "\n")
    attn = s["kernels"]["block_attn_bf16_kernel<128>"]["traffic_bytes"]
    assert traffic.bytes_per_launch(str(md), ["block_attn_bf16_kernel<128>"]) == attn
    # a kernel that is not in the summary, or a missing summary: no figure
    assert traffic.bytes_per_launch(str(md), ["lm_unmask_kernel"]) is None
    assert traffic.bytes_per_launch(str(tmp_path / "none.md"), ["block_attn_bf16_kernel<128>"]) is None
    # a changed source file: the stored hash no longer matches, so no figure either
    s["source_sha256"]["block_attn.hip"] = "0" * 64
    md.write_text("# summary\n\n" + json.dumps(s) + "\n")
    assert traffic.bytes_per_launch(str(md), ["block_attn_bf16_kernel<128>"]) is None


def test_short_names():
    assert traffic.short_name(ATTN) == "block_attn_bf16_kernel<128>"
    assert traffic.short_name("void tt::attn_reduce_kernel<128, 1>(tt::AttnParams)") == \
        "attn_reduce_kernel<128,1>"
    assert traffic.source_of("attn_reduce_kernel<128,1>") == "block_attn.hip"
    assert traffic.source_of("__amd_rocclr_copyBuffer") is None
