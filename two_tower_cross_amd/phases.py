"""Per-work-group phase timelines of the attention and projection kernels.

Loads the profiling build (``python -m two_tower_cross_amd.build --phase-stamps``: the same
sources compiled with TT_PHASE_STAMPS, where wave 0 of every work-group stamps the 100 MHz wall
clock at each phase of its kernel) instead of the product library, runs the block attention at the
32K-context layer (batch 8, Hq 32 / Hkv 2, head_dim 128, automatic partitions) and at a single
131072-token context (automatic and 64 partitions), each call after a 1 GiB write so that nothing
is served from the last-level cache, and the QKV and output projections at the block loop's shape
(128 rows, hidden 2048, Q width 4096), each call after a 1 GiB non-temporal read, as in the block
loop between two uses of a layer's weights (the KV caches and the lm-head weight are read
non-temporally): the caches of the XCDs hold nothing useful, while the weights may stay in the
last-level cache. Writes the phase percentiles over the work-groups of the last of six calls as
markdown.

Usage (on an MI355X): ``python -m two_tower_cross_amd.phases OUT.md 'COMMAND'``.
"""
from __future__ import annotations

import ctypes as C
import math
import os
import sys

import numpy as np
import torch

from . import _lib
from .build import STAMPS_LIB

ROWS = 8192

ATTN_PHASES = [
    ("start", None, 0),
    ("to the partition's tile indices (first memory round trip, plan)", 0, 1),
    ("issuing the ring's first DMA (and the block tile)", 1, 2),
    ("until tile 0 has landed", 2, 3),
    ("ring (every context tile)", 3, 4),
    ("epilogue (normalize, partials or output)", 4, 5),
    ("end", None, 5),
]
LINEAR_PHASES = [
    ("start", None, 0),
    ("until chunk 0 has landed", 0, 1),
    ("K loop", 1, 2),
    ("drain of the last loads, barrier", 2, 3),
    ("partial stores, arrival and wait, merge of a share of the tile's rows", 3, 4),
    ("until the stores are done", 4, 5),
    ("end", None, 5),
]


def _stamps_fn(L, name):
    f = getattr(L, name)
    f.restype = C.c_int
    f.argtypes = [C.c_void_p, C.c_size_t, C.c_int]
    return f


def _read(f):
    buf = np.zeros((ROWS, 8), np.uint64)
    if f(buf.ctypes.data, buf.nbytes, 0) != 0:
        raise RuntimeError("reading the phase stamps failed")
    rows = buf[buf[:, 0] != 0].astype(np.float64)
    return rows


def _pct(x):
    return (f"{np.percentile(x, 0):.2f} | {np.median(x):.2f} | {np.percentile(x, 90):.2f} | "
            f"{np.max(x):.2f}")


def _table(rows, phases, title, call_us):
    t0 = rows[:, 0].min()
    us = (rows[:, :6] - t0) / 100.0                    # 100 MHz counter
    # a phase a work-group skipped (no full tile: no ring) takes the previous stamp
    for k in range(1, 6):
        miss = rows[:, k] == 0
        us[miss, k] = us[miss, k - 1]
    cyc = rows[:, 7] - rows[:, 6]
    lines = [f"**{title}** — {len(rows)} work-groups; event-timed call {call_us:.1f} us; "
             f"work-group span {us[:, 5].max():.1f} us", "",
             "| phase | min us | median | p90 | max |", "|---|---:|---:|---:|---:|"]
    for name, a, b in phases:
        x = us[:, b] if a is None else us[:, b] - us[:, a]
        lines.append(f"| {name} | {_pct(x)} |")
    return lines, cyc, us


def main(argv):
    out_md, command = argv[1], argv[2]
    if not os.path.exists(STAMPS_LIB):
        raise SystemExit(f"{STAMPS_LIB} is missing: python -m two_tower_cross_amd.build --phase-stamps")
    _lib.LIB_PATH = STAMPS_LIB
    L = _lib.lib()
    attn_f, lin_f = _stamps_fn(L, "tt_phase_stamps_attn"), _stamps_fn(L, "tt_phase_stamps_linear")
    import two_tower_cross_amd as tt

    dev = torch.device("cuda", 0)
    scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    g = torch.Generator(device=dev).manual_seed(1)
    bf = torch.bfloat16
    from .timing import TimingEvent
    ev = [TimingEvent() for _ in range(2)]
    report = ["# Per-work-group phase timelines: block attention and projections", "",
              "Command (MI355X, one GPU; the profiling build is compiled beforehand on any host with "
              "`python -m two_tower_cross_amd.build --phase-stamps`):", "", f"    {command}", "",
              "Phases from wall_clock64 stamps of wave 0 of every work-group, relative to the "
              "earliest work-group start of the call (the last of six calls, each right after a 1 GiB "
              "write on the same stream for the attention, a 1 GiB non-temporal read for the "
              "projections); the event-timed call (fence-free events, the launch from Python "
              "included) adds dispatch and drain.", ""]

    sink = torch.zeros(2048, dtype=torch.int32, device=dev)

    def timed(call, clear, nt_read=False):
        # stamps cleared, then the 1 GiB write (or non-temporal read) and the call back to back on
        # the stream (the compute units are awake, as in the block loop)
        us = 0.0
        for it in range(6):
            clear(None, 0, 1)
            if nt_read:
                tt.probe_stream_read(scrub, 2048, sink)
            else:
                scrub.fill_(it)
            ev[0].record()
            call()
            ev[1].record()
            torch.cuda.synchronize()
            us = 1e3 * ev[0].elapsed_time(ev[1])
        return us

    def attn_case(B, Lctx, splits, S=16, Hq=32, Hkv=2, D=128):
        k = torch.randn(tt.k_pages_shape(B, Hkv, Lctx, D), generator=g, device=dev).to(bf)
        v = torch.randn(tt.v_pages_shape(B, Hkv, Lctx, D), generator=g, device=dev).to(bf)
        q = torch.randn((B, S, Hq, D), generator=g, device=dev).to(bf)
        kb = torch.randn((B, Hkv, S, D), generator=g, device=dev).to(bf)
        vb = torch.randn((B, Hkv, D, S), generator=g, device=dev).to(bf)
        table = torch.arange(B, dtype=torch.int32, device=dev).view(B, 1)
        lens = torch.full((B,), Lctx, dtype=torch.int32, device=dev)
        out = torch.empty((B, S, Hq, D), dtype=bf, device=dev)
        return lambda: tt.block_attn(q, k, v, table, lens, kb, vb, scale=1 / math.sqrt(D),
                                     max_ctx_len=Lctx, num_splits=splits, out=out)

    for title, args in [("Attention, 32K-context layer: batch 8, L 32768, automatic partitions",
                         (8, 32768, 0)),
                        ("Attention, one 131072-token context, automatic partitions",
                         (1, 131072, 0)),
                        ("Attention, one 131072-token context, 64 partitions", (1, 131072, 64))]:
        call = attn_case(*args)
        us = timed(call, attn_f)
        rows = _read(attn_f)
        lines, cyc, span = _table(rows, ATTN_PHASES, title, us)
        ring_us = span[:, 4] - span[:, 3]
        ok = ring_us > 0
        clock = np.median(cyc[ok] / ring_us[ok]) / 1e3 if ok.any() else float("nan")
        report += lines + ["", f"Shader clock in the ring: {clock:.3f} GHz.", ""]
        del call
        torch.cuda.empty_cache()

    B, S, H, Hq, Hkv, D = 8, 16, 2048, 32, 2, 128
    h = torch.randn((B, S, H), generator=g, device=dev).to(bf)
    wq = tt.pack_weight((torch.randn(((Hq + 2 * Hkv) * D, H), generator=g, device=dev) * 0.02).to(bf))
    wo = tt.pack_weight((torch.randn((H, Hq * D), generator=g, device=dev) * 0.02).to(bf))
    o = torch.randn((B, S, Hq, D), generator=g, device=dev).to(bf)
    for title, call in [("QKV projection: 128 x 4608 x 2048 (K split in 3, the K partials "
                         "merged inside the kernel)", lambda: tt.qkv_projection(h, wq, Hq, Hkv, D)),
                        ("Output projection: 128 x 2048 x 4096 (K split in 8, the K partials "
                         "and the residual merged inside the kernel)",
                         lambda: tt.out_projection(h, o, wo))]:
        us = timed(call, lin_f, nt_read=True)
        rows = _read(lin_f)
        lines, cyc, span = _table(rows, LINEAR_PHASES, title, us)
        clock = np.median(cyc / np.maximum(span[:, 5] - span[:, 0], 1e-3)) / 1e3
        report += lines + ["", f"Shader clock over the work-group: {clock:.3f} GHz.", ""]

    with open(out_md, "w") as f:
        f.write("\n".join(report) + "\n")
    print(out_md)


if __name__ == "__main__":
    main(sys.argv)
