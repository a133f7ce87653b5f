"""HBM traffic of the block-attention kernel from rocprofv3 byte counters.

Two counter runs of the same command (``--pmc FETCH_SIZE``, then ``--pmc WRITE_SIZE``; the counters
report KiB per dispatch) are scaled by what the same counter reads for a plain device copy of known
size in the same run (``bench.py --copy-calibration MIB``): factor = true bytes / counted bytes.

    python -m two_tower_cross_amd.traffic FETCH_CSV WRITE_CSV COPY_MIB OUT_MD "COMMAND"

writes a short summary (text plus one JSON line) that ``bench.py`` reads back; the JSON records the
SHA-256 of the kernel source so that a stale measurement is never reported for a changed kernel.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys

KERNEL = "block_attn_bf16_kernel<128>"


def _per_dispatch(path, counter):
    """{dispatch id: (kernel name, value)} for one counter of a counter_collection CSV."""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, v = out.get(d, (r["Kernel_Name"], 0.0))
            out[d] = (name, v + float(r["Counter_Value"]))
    return out


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def summarize(fetch_csv, write_csv, copy_mib, kernel_source):
    copy_bytes = copy_mib << 20
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = _per_dispatch(path, counter)
        attn = [v for n, v in disp.values() if KERNEL in n.replace(" ", "")]
        # the calibration copy: the last dispatch of the run
        last = disp[max(disp)]
        factor = copy_bytes / (last[1] * 1024.0)
        kib = sum(attn) / len(attn)
        res[counter] = {"dispatches": len(attn), "kib_per_dispatch": round(kib, 1),
                        "copy_kernel": last[0][:80], "copy_counted_kib": round(last[1], 1),
                        "factor": round(factor, 4), "bytes_per_launch": int(kib * 1024 * factor)}
    total = res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]
    return {"kernel": KERNEL, "source_sha256": source_hash(kernel_source), "copy_mib": copy_mib,
            "fetch": res["FETCH_SIZE"], "write": res["WRITE_SIZE"], "traffic_bytes": total}


def bytes_per_launch(summary_md, kernel_source):
    """Scaled fetch + write bytes per launch, or None (no summary / different kernel source)."""
    if not os.path.exists(summary_md):
        return None
    with open(summary_md) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{") and '"traffic_bytes"' in line:
                s = json.loads(line)
                if s.get("source_sha256") == source_hash(kernel_source):
                    return int(s["traffic_bytes"])
    return None


def main(argv):
    fetch_csv, write_csv, copy_mib, out_md, command = argv[1:6]
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = os.path.join(root, "two_tower_cross_amd", "csrc", "block_attn.hip")
    s = summarize(fetch_csv, write_csv, int(copy_mib), src)
    with open(out_md, "w") as f:
        f.write(f"# HBM traffic of {KERNEL}, 32K-context block loop\n\n")
        f.write("Counters: rocprofv3 `--pmc FETCH_SIZE` and `--pmc WRITE_SIZE`, one run each, of\n\n")
        f.write(f"    {command}\n\n")
        for k in ("fetch", "write"):
            r = s[k]
            f.write(f"- {k.upper()}: {r['kib_per_dispatch']} KiB counted per dispatch over "
                    f"{r['dispatches']} dispatches; plain copy of {s['copy_mib']} MiB "
                    f"(`{r['copy_kernel']}`) counted {r['copy_counted_kib']} KiB -> factor "
                    f"{r['factor']}; scaled: {r['bytes_per_launch']} bytes per launch\n")
        f.write(f"- traffic (fetch + write, scaled): {s['traffic_bytes']} bytes per launch\n\n")
        f.write("Machine-readable (bench.py reports it only while the kernel source hash matches):\n\n")
        f.write(json.dumps(s) + "\n")
    print(json.dumps(s))


if __name__ == "__main__":
    main(sys.argv)
