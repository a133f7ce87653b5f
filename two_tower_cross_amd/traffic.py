"""HBM traffic of the step's kernels from rocprofv3 byte counters.

Two counter runs of the same command (``--pmc FETCH_SIZE``, then ``--pmc WRITE_SIZE``; the counters
report KiB per dispatch) are scaled by what the same counter reads for a plain device copy of known
size in the same run (``bench.py --copy-calibration MIB``): factor = true bytes / counted bytes.
Optionally the kernel trace of the same command (``--kernel-trace``; its kernel_trace CSV, or
the kernel_stats CSV of ``--stats``) adds each kernel's mean duration, so that counted bytes per
second can be put next to the algorithmic rate.

    python -m two_tower_cross_amd.traffic [--by-grid] FETCH_CSV WRITE_CSV COPY_MIB OUT_MD "COMMAND" [TRACE_CSV]
    python -m two_tower_cross_amd.traffic --sq SQ_CSV_1 SQ_CSV_2 TRACE_CSV OUT_MD "COMMAND"
    python -m two_tower_cross_amd.traffic --stats STATS_CSV OUT_MD "TITLE" "COMMAND"

writes a short summary (a table plus one JSON line) that ``bench.py`` reads back. Kernels are keyed
by name and grid size (the two projections of a layer are the same kernel on different grids);
the JSON records the SHA-256 of each kernel's source file, so that a stale measurement is never
reported for a changed kernel.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "two_tower_cross_amd", "csrc")

# kernel name prefix -> source file
SOURCES = [("block_attn", "block_attn.hip"), ("attn_reduce", "block_attn.hip"),
           ("linear", "linear.hip"), ("lm_unmask", "linear.hip"), ("pack_weight", "linear.hip"),
           ("unmask", "unmask.hip"), ("nll", "unmask.hip"), ("mask_corrupt", "unmask.hip"),
           ("kv_", "kv_append.hip"), ("stream_read", "probe.hip")]

# Algorithmic bytes per dispatch of the 32K-context block loop (batch 8, S 16, Hq 32 / Hkv 2,
# head_dim 128, hidden 2048, vocab 131072, L 32768), by (kernel, grid size in work-items):
# what the method itself must move through that kernel (inputs read once, outputs written once);
# split partials and re-reads are overhead, counted by the counters but not here.
_B, _S, _HQ, _HKV, _D, _H, _V, _L = 8, 16, 32, 2, 128, 2048, 131072, 32768
_M = _B * _S
ALGORITHMIC_LOOP32K = {
    # context K+V, block K+V and Q (the O write is the merge's)
    "block_attn_bf16_kernel<128>": 2 * _B * _HKV * _L * _D * 2 + 2 * _B * _HKV * _S * _D * 2
    + _B * _S * _HQ * _D * 2,
    "attn_reduce_kernel<128>": _B * _S * _HQ * _D * 2,                     # O write
    # QKV product: W_qkv + H (its fp32 K partials are overhead); the reduce writes Q, K_blk, V_blk
    "linear_kernel<2>@qkv": (_HQ + 2 * _HKV) * _D * _H * 2 + _M * _H * 2,
    "linear_reduce_kernel@qkv": _M * (_HQ + 2 * _HKV) * _D * 2,
    # output product: W_o + O; the reduce reads the residual and writes H
    "linear_kernel<2>@out": _H * _HQ * _D * 2 + _M * _HQ * _D * 2,
    "linear_reduce_kernel@out": 2 * _M * _H * 2,
    # fused lm-head: W_lm + H_final, then 12-byte row triples per 256-logit tile (their round trip
    # is the fused path's own overhead, not counted)
    "lm_unmask_kernel": _V * _H * 2 + _M * _H * 2,
    "unmask_tiles_finalize_kernel": 0,
}


def _algorithmic(key):
    """Algorithmic bytes of a kernel key (the merge is one entry whatever its partition groups)."""
    if key.startswith("attn_reduce_kernel<128,"):
        key = "attn_reduce_kernel<128>"
    return ALGORITHMIC_LOOP32K.get(key)


def _lookup(kernels, name):
    """The entry of `name`, or of the one key that starts with it followed by ',' (template
    arguments beyond the first)."""
    if name in kernels:
        return kernels[name]
    hits = [v for k, v in kernels.items() if k.startswith(name.rstrip(">") + ",")]
    return hits[0] if len(hits) == 1 else None


def source_of(kernel):
    k = kernel.replace("tt::", "")
    for prefix, src in SOURCES:
        if k.startswith(prefix):
            return src
    return None


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def short_name(kernel):
    """`void tt::block_attn_bf16_kernel<128>(tt::AttnParams)` -> `block_attn_bf16_kernel<128>`."""
    k = kernel.strip()
    if k.startswith("void "):
        k = k[5:]
    k = k.replace("tt::", "").replace(" ", "")
    depth, out = 0, []
    for ch in k:
        if ch == "(" and depth == 0:
            break
        out.append(ch)
        depth += ch == "<"
        depth -= ch == ">"
    return "".join(out)


def _grid(r):
    """Total work-items of a CSV row (one Grid_Size column, or one per dimension)."""
    if r.get("Grid_Size"):
        return int(r["Grid_Size"])
    n = 1
    for ax in ("X", "Y", "Z"):
        n *= int(r.get(f"Grid_Size_{ax}", 1) or 1)
    return n


def _per_dispatch(path, counter):
    """{dispatch id: (kernel name, grid size, value)} for one counter of a counter CSV."""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, _, v = out.get(d, (short_name(r["Kernel_Name"]), _grid(r), 0.0))
            out[d] = (name, _grid(r), v + float(r["Counter_Value"]))
    return out


def _durations(trace_csv):
    """{kernel key: mean duration in us} from a rocprofv3 kernel_trace CSV of the same command
    (keys as for the counters), or from a kernel_stats CSV (by name only)."""
    if not trace_csv:
        return {}
    with open(trace_csv) as f:
        rows = list(csv.DictReader(f))
    if rows and "AverageNs" in rows[0]:
        return {short_name(r["Name"]): float(r["AverageNs"]) / 1e3 for r in rows}
    grids = {}
    for r in rows:
        grids.setdefault(short_name(r["Kernel_Name"]), set()).add(_grid(r))
    durs = {}
    for r in rows:
        name = short_name(r["Kernel_Name"])
        k = _key(name, _grid(r), grids)
        durs.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return {k: statistics.mean(v) for k, v in durs.items()}


BY_GRID = False   # key every kernel by name and grid (several workloads in one run)


def _key(name, grid, grids):
    """Kernel key: the name, with the projection's role when one name runs on several grids."""
    if BY_GRID:
        return f"{name}@{grid}" if len(grids[name]) > 1 else name
    if name in ("linear_kernel<2>", "linear_reduce_kernel") and len(grids[name]) == 2:
        # at this workload the QKV product runs on the smaller grid (72 feature tiles x 3 K
        # partitions against 32 x 8) and its reduce on the larger one (4608 against 2048 features)
        qkv = min(grids[name]) if name == "linear_kernel<2>" else max(grids[name])
        return name + ("@qkv" if grid == qkv else "@out")
    return name


def summarize(fetch_csv, write_csv, copy_mib, stats_csv=None):
    copy_bytes = copy_mib << 20
    per = {}
    factors = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = _per_dispatch(path, counter)
        last = disp[max(disp)]                      # the calibration copy: the run's last dispatch
        factor = copy_bytes / (last[2] * 1024.0)
        factors[counter] = {"copy_kernel": last[0][:60], "copy_counted_kib": round(last[2], 1),
                            "factor": round(factor, 4)}
        grids = {}
        for name, grid, _ in disp.values():
            grids.setdefault(name, set()).add(grid)
        vals = {}
        for d, (name, grid, v) in disp.items():
            if d == max(disp) or source_of(name) is None:
                continue
            vals.setdefault(_key(name, grid, grids), []).append(v)
        for k, vs in vals.items():
            e = per.setdefault(k, {"dispatches": len(vs)})
            e[counter] = int(statistics.mean(vs) * 1024 * factor)
    dur = _durations(stats_csv)
    hashes = {}
    for k, e in per.items():
        src = source_of(k)
        hashes[src] = source_hash(os.path.join(CSRC, src))
        e["source"] = src
        e["traffic_bytes"] = e.get("FETCH_SIZE", 0) + e.get("WRITE_SIZE", 0)
        alg = _algorithmic(k)
        if alg is not None:
            e["algorithmic_bytes"] = alg
            if alg:
                e["traffic_over_algorithmic"] = round(e["traffic_bytes"] / alg, 3)
        base = k if k in dur else k.split("@")[0]
        if base in dur:
            e["mean_us"] = round(dur[base], 2)
            if alg:
                e["algorithmic_GBps"] = round(alg / dur[base] / 1e3, 1)
                e["algorithmic_frac_of_8TBps"] = round(alg / dur[base] / 1e3 / 8000.0, 4)
            e["counted_GBps"] = round(e["traffic_bytes"] / dur[base] / 1e3, 1)
    return {"kernels": per, "source_sha256": hashes, "copy_mib": copy_mib, "calibration": factors}


def bytes_per_launch(summary_md, kernels):
    """Scaled fetch + write bytes per call summed over ``kernels`` (short names), or None (no
    summary, a kernel missing, or a changed source file)."""
    if not os.path.exists(summary_md):
        return None
    with open(summary_md) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{") and '"kernels"' in line:
                s = json.loads(line)
                total = 0
                for k in kernels:
                    e = _lookup(s["kernels"], k)
                    if e is None:
                        return None
                    src = e["source"]
                    if s["source_sha256"].get(src) != source_hash(os.path.join(CSRC, src)):
                        return None
                    total += e["traffic_bytes"]
                return total
    return None


# SQ counters: units as read on gfx950 (each checked against a known quantity): SQ_BUSY_CYCLES
# sums the shader clock over the 32 shader engines (8 XCDs x 4), so /32 gives the kernel's cycles;
# SQ_VALU_MFMA_BUSY_CYCLES and SQ_VALU_MFMA_COEXEC_CYCLES sum cycles over the 1024 SIMDs (busy =
# MFMA instructions x 32 cycles for 32x32x16 bf16); SQ_WAVE_CYCLES, SQ_ACTIVE_INST_* and SQ_WAIT_*
# are in 4-cycle units summed over waves.
N_SE, N_SIMD, MFMA_FLOPS, PEAK_TFLOPS = 32, 1024, 32 * 32 * 16 * 2, 2500.0


def sq_summary(csvs, trace_csv):
    vals = {}
    for path in csvs:
        per = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                name = short_name(r["Kernel_Name"])
                if source_of(name) is None:
                    continue
                d = (name, _grid(r), int(r["Dispatch_Id"]))
                c = per.setdefault(d, {})
                c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        grids = {}
        for name, grid, _ in per:
            grids.setdefault(name, set()).add(grid)
        for (name, grid, _), c in per.items():
            e = vals.setdefault(_key(name, grid, grids), {})
            for k, v in c.items():
                e.setdefault(k, []).append(v)
    dur = _durations(trace_csv)
    out = {}
    for k, cs in vals.items():
        m = {c: statistics.mean(v) for c, v in cs.items()}
        e = {"counters": {c: round(v) for c, v in m.items()}}
        us = dur.get(k, dur.get(k.split("@")[0]))
        cyc = m.get("SQ_BUSY_CYCLES", 0) / N_SE
        if us:
            e["mean_us"] = round(us, 2)
            if cyc:
                e["clock_GHz"] = round(cyc / us / 1e3, 3)
            if m.get("SQ_INSTS_MFMA"):
                tf = m["SQ_INSTS_MFMA"] * MFMA_FLOPS / us / 1e6
                e["mfma_TFLOPs"] = round(tf, 1)
                e["mfma_frac_of_peak"] = round(tf / PEAK_TFLOPS, 4)
        if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            e["mfma_busy_frac"] = round(m["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / cyc, 4)
        valu = m.get("SQ_ACTIVE_INST_VALU", 0) * 4 / N_SIMD
        if valu and "SQ_VALU_MFMA_COEXEC_CYCLES" in m:
            e["valu_cycles_per_simd"] = round(valu)
            e["valu_coexec_frac"] = round(m["SQ_VALU_MFMA_COEXEC_CYCLES"] / N_SIMD / valu, 4)
        if m.get("SQ_WAVE_CYCLES"):
            e["wait_frac"] = round(m.get("SQ_WAIT_ANY", 0) / m["SQ_WAVE_CYCLES"], 4)
            e["issue_blocked_frac"] = round(m.get("SQ_WAIT_INST_ANY", 0) / m["SQ_WAVE_CYCLES"], 4)
        out[k] = e
    return out


def main_sq(argv):
    sq1, sq2, trace_csv, out_md, command = argv[:5]
    s = sq_summary([sq1, sq2], trace_csv)
    with open(out_md, "w") as f:
        f.write("# SQ counters of the denoise-step kernels, 32K-context block loop\n\n")
        f.write("Two counter passes (8 SQ counters each) and a kernel trace for durations, of\n\n")
        f.write(f"    {command}\n\n")
        f.write("Units: SQ_BUSY_CYCLES / 32 shader engines = the kernel's cycles (so clock = that "
                "/ mean duration); SQ_VALU_MFMA_BUSY / COEXEC cycles summed over 1024 SIMDs; "
                "SQ_WAVE_CYCLES, SQ_ACTIVE_INST_* and SQ_WAIT_* in 4-cycle units summed over "
                "waves. MFMA TFLOP/s = SQ_INSTS_MFMA x 32768 flops (32x32x16 bf16) / mean "
                "duration, against 2.5 PFLOP/s dense bf16.\n\n")
        f.write("| kernel | mean us | clock GHz | MFMA busy | MFMA TFLOP/s (% peak) | VALU cycles / SIMD "
                "| VALU co-exec with MFMA | waves waiting | issue-blocked |\n")
        f.write("|---|---:|---:|---:|---:|---:|---:|---:|---:|\n")
        pct = lambda x: "-" if x is None else f"{100 * x:.1f}%"
        for k, e in sorted(s.items(), key=lambda kv: -kv[1].get("mean_us", 0)):
            tf = (f"{e['mfma_TFLOPs']} ({100 * e['mfma_frac_of_peak']:.1f}%)"
                  if "mfma_TFLOPs" in e else "-")
            f.write(f"| `{k}` | {e.get('mean_us', '-')} | {e.get('clock_GHz', '-')} | "
                    f"{pct(e.get('mfma_busy_frac')) if e.get('counters', {}).get('SQ_INSTS_MFMA') else '-'} | {tf} | "
                    f"{e.get('valu_cycles_per_simd', '-')} | "
                    f"{pct(e.get('valu_coexec_frac')) if e.get('counters', {}).get('SQ_INSTS_MFMA') else '-'} | "
                    f"{pct(e.get('wait_frac'))} | {pct(e.get('issue_blocked_frac'))} |\n")
        f.write("\nMachine-readable:\n\n" + json.dumps(s) + "\n")


def main_stats(argv):
    """Kernel-time table from a rocprofv3 kernel_stats CSV (the library's kernels and the rest)."""
    stats_csv, out_md, title, command = argv[:4]
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    with open(out_md, "w") as f:
        f.write(f"# Kernel time, {title}\n\nCommand (MI355X, one GPU):\n\n    {command}\n\n")
        f.write("| kernel | calls | avg us | min us | max us | % of GPU time |\n")
        f.write("|---|---:|---:|---:|---:|---:|\n")
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            name = short_name(r["Name"])
            name = name if len(name) <= 60 else name[:57] + "..."
            f.write(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                    f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                    f"{100 * float(r['TotalDurationNs']) / total:.2f} |\n")


def main(argv):
    global BY_GRID
    if len(argv) > 1 and argv[1] == "--sq":
        return main_sq(argv[2:])
    if len(argv) > 1 and argv[1] == "--stats":
        return main_stats(argv[2:])
    if "--by-grid" in argv:
        BY_GRID = True
        argv = [a for a in argv if a != "--by-grid"]
    fetch_csv, write_csv, copy_mib, out_md, command = argv[1:6]
    stats_csv = argv[6] if len(argv) > 6 else None
    s = summarize(fetch_csv, write_csv, int(copy_mib), stats_csv)
    title = ("the attention and unmasking workloads (kernels keyed by name and grid size in "
             "work-items)" if BY_GRID else "the denoise-step kernels, 32K-context block loop")
    with open(out_md, "w") as f:
        f.write(f"# HBM traffic of {title}\n\n")
        f.write("Counters: rocprofv3 `--pmc FETCH_SIZE` and `--pmc WRITE_SIZE`, one run each"
                + (", and a `--kernel-trace --stats` run for durations" if stats_csv else "")
                + ", of\n\n")
        f.write(f"    {command}\n\n")
        for c, r in s["calibration"].items():
            f.write(f"- {c}: a plain copy of {s['copy_mib']} MiB (`{r['copy_kernel']}`) counted "
                    f"{r['copy_counted_kib']} KiB -> scale factor {r['factor']}\n")
        f.write("\nBytes per dispatch, scaled; algorithmic = what the method itself moves through "
                "the kernel at this workload.\n\n")
        f.write("| kernel | dispatches | fetch B | write B | traffic B | algorithmic B | "
                "traffic / alg. | mean us | alg. GB/s | alg. % of 8 TB/s |\n")
        f.write("|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|\n")
        for k, e in sorted(s["kernels"].items(), key=lambda kv: -kv[1]["traffic_bytes"]):
            f.write(f"| `{k}` | {e['dispatches']} | {e.get('FETCH_SIZE', 0):,} | "
                    f"{e.get('WRITE_SIZE', 0):,} | {e['traffic_bytes']:,} | "
                    f"{e.get('algorithmic_bytes', '-') if 'algorithmic_bytes' not in e else format(e['algorithmic_bytes'], ',')} | "
                    f"{e.get('traffic_over_algorithmic', '-')} | {e.get('mean_us', '-')} | "
                    f"{e.get('algorithmic_GBps', '-')} | "
                    f"{round(100 * e['algorithmic_frac_of_8TBps'], 1) if 'algorithmic_frac_of_8TBps' in e else '-'} |\n")
        f.write("\nMachine-readable (bench.py reports a kernel's traffic only while the hash of "
                "its source file matches):\n\n")
        f.write(json.dumps(s) + "\n")
    print(json.dumps(s))


if __name__ == "__main__":
    main(sys.argv)
