"""Benchmark: committed tokens/s of the TwoTower denoise-step block loop on one MI355X, plus the
attention and unmasking workloads at their own shapes.

Headline workload (one "step" of this benchmark = one block): batch 8, 6 attention layers, context
32768 tokens per sequence (resident bf16 KV caches, 1.61 GB), block S = 16, T = 16 denoise steps,
hidden 2048, Hq = 32 / Hkv = 2, head_dim 128, vocab 131072, threshold 0.9 with the one-commit
fallback and commit-all at the last step. Every denoise step rewrites the block KV of every layer
(QKV projection), runs the block attention over [context KV ; block KV] of the same layer, the
output projection with the residual add, the lm-head and the confidence unmasking. Inputs are
synthetic (seeded on-device draws) and resident in HBM before timing starts.

Prints one JSON line. ``value`` is committed tokens/s over the timed blocks. ``roofline`` reports
the block-attention call of the loop (main kernel + partition merge, the dominant work of a step)
as algorithmic HBM bytes per call (context K+V, block K+V, Q read, O write) over the call's mean
duration, from HIP events that the library records on its launch stream in a second timed pass
of the same K blocks (the headline pass carries no per-call events): every other denoise step
brackets one layer's call (before the kernel, after the merge), the others one layer's main
kernel alone (``roofline.kernel_only``), the layers rotating over the steps.
The events are created with hipEventDisableSystemFence: a default event's record writes back and
invalidates the caches, which costs about 5 us of idle GPU per record and slows the next kernel. ``workloads`` holds the other
shapes (tiny fp32; 4K context with the 16 x 131072 unmasking; a ragged paged batch of 32; a 131072-
token context at 64/128/256/auto partitions), each timed over 50 calls with a 1 GiB write between
calls (outside the timed events) so that no input is served from the 256 MB last-level cache, as
median and minimum, with the fp64 CPU oracle's time and its max-abs deviation on the same inputs.
``stream_read_ceiling`` is a plain streaming read of 2 GiB measured in the same run, and
``mfma_ceiling`` the issue rate of 32x32x16 bf16 MFMA chains at 2 and 4 waves per SIMD, with and
without an LDS operand read per MFMA (both probes are part of the library).
``cpu_baseline`` times the oracle on a bounded sample of the headline workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense bf16
THRESHOLD = 0.9
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "step_kernels_loop32k_traffic.md")
TIMED_CALLS = 50
SCRUB_BYTES = 1 << 30


def attn_bytes(ctx_lens, S, Hq, Hkv, D, e=2):
    """Algorithmic bytes of one attention call: context K+V of every sequence, block K+V, the Q
    read and the O write."""
    B = len(ctx_lens)
    ctx = sum(2 * Hkv * int(L) * D * e for L in ctx_lens)
    return ctx + 2 * B * Hkv * S * D * e + 2 * B * S * Hq * D * e


def attn_flops(ctx_lens, S, Hq, D):
    """QK^T and PV over every (context + block) key of every query row: 4 flops per row, key, dim."""
    return sum(4 * Hq * S * (int(L) + S) * D for L in ctx_lens)


def make_event(fenced=False):
    import torch
    from two_tower_cross_amd.timing import TimingEvent
    return torch.cuda.Event(enable_timing=True) if fenced else TimingEvent()


def stats_us(xs):
    return {"median": round(statistics.median(xs), 2), "min": round(min(xs), 2),
            "n": len(xs)}


def host_description():
    return {"sched_getaffinity": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(),
            "blas_threads": blas_threads()}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    for var in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS"):
        if os.environ.get(var, "").isdigit():
            return int(os.environ[var])
    return len(os.sched_getaffinity(0))


def cpu_baseline(m, steps=2):
    """The fp64 oracle on the whole batch for the first ``steps`` denoise steps of a block (each:
    6 layers of QKV projection, block attention and output projection; lm-head; unmasking with
    the one-commit fallback). tokens/s = tokens committed / seconds."""
    import numpy as np
    from oracle import step as ostep

    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    layers = [(f64(m.w_qkv[l]), f64(m.w_o[l]), f64(m.k_pages[l]), f64(m.v_pages[l]))
              for l in range(m.layers)]
    w_lm = f64(m.w_lm)
    hs = [f64(m.h_steps[t]) for t in range(steps)]
    bt = m.block_table.cpu().numpy()
    lens = m.ctx_lens.cpu().numpy()
    masked = np.ones((m.B, m.S), np.uint8)
    tokens = np.full((m.B, m.S), -1, np.int32)
    n_tok = 0
    t0 = time.perf_counter()
    for t in range(steps):
        tokens, masked, _, n, _ = ostep.denoise_step(
            hs[t], layers, bt, lens, w_lm, masked, tokens, Hq=m.Hq, Hkv=m.Hkv, D=m.D,
            scale=1.0 / math.sqrt(m.D), threshold=THRESHOLD, min_commit=True)
        n_tok += int(n.sum())
    dt = time.perf_counter() - t0
    host = host_description()
    return {"value": n_tok / dt, "unit": "committed tokens/s", "cores": host["blas_threads"],
            "kind": "oracle",
            "sample": f"the first {steps} of {m.T} denoise steps of one block, whole batch of "
                      f"{m.B} at context {m.L} (6 layers, lm-head {m.vocab}, unmask): "
                      f"{dt:.2f} s for {n_tok} committed tokens",
            "host": host}


def measured_traffic(kernels):
    """HBM bytes per call summed over ``kernels`` from the committed counter summary, or None
    when there is none or the kernel source changed since the counters were taken."""
    try:
        from two_tower_cross_amd import traffic
        return traffic.bytes_per_launch(TRAFFIC_SUMMARY, kernels)
    except Exception:
        return None


class Timer:
    """Timed calls of a workload, each preceded by a 1 GiB write (outside the events)."""

    def __init__(self, torch, dev, fenced=False):
        self.torch = torch
        self.fenced = fenced
        self.scrub = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device=dev)

    def events(self, n):
        evs = [make_event(self.fenced) for _ in range(n)]
        for e in evs:
            e.record()          # materialize the underlying hipEvent_t
        return evs

    def run(self, call, *, calls=TIMED_CALLS, warmup=3, n_events=3, reset=None):
        """call(events) enqueues one call and records the events; returns per-call lists of
        elapsed microseconds between event 0 and every later event."""
        torch = self.torch
        for _ in range(warmup):
            if reset:
                reset()
            call(None)
        torch.cuda.synchronize()
        evs = [self.events(n_events) for _ in range(calls)]
        torch.cuda.synchronize()
        for i in range(calls):
            if reset:
                reset()
            self.scrub.fill_(i & 0xFF)
            call(evs[i])
        torch.cuda.synchronize()
        return [[1e3 * e[0].elapsed_time(e[k]) for e in evs] for k in range(1, n_events)]


def attention_workload(name, case, timer, splits_list, *, out_dtype, oracle_time=True):
    """Times twotower_block_attn on ``case`` for each partition count; oracle time and max-abs
    deviation of the last GPU output."""
    import numpy as np
    import torch
    import two_tower_cross_amd as tt
    from oracle import attention as oattn

    dev = torch.device("cuda", 0)
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    f = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt)
    d = dict(q=f(case.q), k_pages=f(case.k_pages), v_pages=f(case.v_pages),
             block_table=torch.from_numpy(case.block_table).to(dev),
             ctx_lens=torch.from_numpy(case.ctx_lens).to(dev), k_blk=f(case.k_blk),
             v_blk=f(case.v_blk))
    lens = [int(x) for x in case.ctx_lens]
    e = 2 if case.dtype == "bf16" else 4
    nbytes = attn_bytes(lens, case.S, case.Hq, case.Hkv, case.D, e)
    flops = attn_flops(lens, case.S, case.Hq, case.D)
    out = torch.empty((case.B, case.S, case.Hq, case.D), dtype=out_dtype, device=dev)
    res = {"bytes": nbytes, "flops": flops, "calls": {}}
    for splits in splits_list:
        def call(evs, splits=splits):
            tt.block_attn(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["ctx_lens"],
                          d["k_blk"], d["v_blk"], scale=case.scale, max_ctx_len=max(lens),
                          num_splits=splits, out=out,
                          timing_events=None if evs is None else [x.cuda_event for x in evs])
        kern, whole = timer.run(call)
        med = statistics.median(whole)
        res["calls"]["auto" if splits == 0 else str(splits)] = {
            "us": stats_us(whole), "kernel_us": stats_us(kern),
            "GBps": round(nbytes / med / 1e3, 1),
            "frac": round(nbytes / med / 1e3 / HBM_PEAK_GBPS, 4),
            "kernel_frac": round(nbytes / statistics.median(kern) / 1e3 / HBM_PEAK_GBPS, 4),
            "TFLOPs": round(flops / med / 1e6, 1)}
    if oracle_time:
        t0 = time.perf_counter()
        ref, _ = oattn.block_attention_case(case)
        res["oracle_s"] = round(time.perf_counter() - t0, 3)
        res["max_abs_err_last_call"] = float(np.abs(out.float().cpu().numpy() - ref).max())
    res["workload"] = name
    return res


def unmask_workload(name, logits_np, timer):
    import numpy as np
    import torch
    import two_tower_cross_amd as tt
    from oracle import unmask as ounmask

    dev = torch.device("cuda", 0)
    B, S, V = logits_np.shape
    logits = torch.from_numpy(logits_np).to(dev)
    masked = torch.ones((B, S), dtype=torch.uint8, device=dev)
    tokens = torch.full((B, S), -1, dtype=torch.int32, device=dev)
    conf = torch.empty((B, S), dtype=torch.float32, device=dev)
    ncom = torch.empty((B,), dtype=torch.int32, device=dev)

    def reset():
        masked.fill_(1)
        tokens.fill_(-1)

    def call(evs):
        if evs is not None:
            evs[0].record()
        tt.unmask(logits, masked, tokens, THRESHOLD, min_commit=True, confidence=conf,
                  n_committed=ncom)
        if evs is not None:
            evs[1].record()

    (whole,) = timer.run(call, reset=reset, n_events=2)
    nbytes = B * S * V * 4
    med = statistics.median(whole)
    t0 = time.perf_counter()
    ot, om, _, _ = ounmask.confidence_unmask(logits_np, np.ones((B, S), np.uint8),
                                             np.full((B, S), -1, np.int32), np.float32(THRESHOLD),
                                             min_commit=True)
    oracle_s = time.perf_counter() - t0
    same = bool(np.array_equal(tokens.cpu().numpy(), ot) and np.array_equal(masked.cpu().numpy(), om))
    return {"workload": name, "bytes": nbytes, "us": stats_us(whole),
            "GBps": round(nbytes / med / 1e3, 1),
            "frac": round(nbytes / med / 1e3 / HBM_PEAK_GBPS, 4),
            "oracle_s": round(oracle_s, 3), "commits_equal_oracle": same}


def stream_ceiling(timer, dev):
    import torch
    import two_tower_cross_amd as tt

    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3)
    sink = torch.zeros(65536, dtype=torch.int32, device=dev)
    best = None
    for wg in (256, 512, 1024, 2048, 4096):
        def call(evs, wg=wg):
            if evs is not None:
                evs[0].record()
            tt.probe_stream_read(src, wg, sink)
            if evs is not None:
                evs[1].record()
        (us,) = timer.run(call, calls=10, n_events=2)
        gbps = nbytes / statistics.median(us) / 1e3
        if best is None or gbps > best[0]:
            best = (gbps, wg)
    del src
    return {"GBps": round(best[0], 1), "frac_of_peak": round(best[0] / HBM_PEAK_GBPS, 4),
            "workgroups": best[1], "bytes": nbytes}


def mfma_ceiling(timer, dev):
    """Issue rate of 32x32x16 bf16 MFMA chains (twotower_probe_mfma_rate) with the GPU filled at 2
    and at 4 waves per SIMD, with and without a 1 KB LDS operand read per MFMA."""
    import torch
    import two_tower_cross_amd as tt

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(2 * cus * 512, dtype=torch.float32, device=dev)
    iters = 2048
    out = {"compute_units": cus, "iters": iters}
    for name, mode in (("2_waves_per_simd", 0), ("4_waves_per_simd", 2),
                       ("2_waves_per_simd_lds_operand", 1), ("4_waves_per_simd_lds_operand", 3)):
        wg = cus * (2 if mode & 2 else 1)
        flops = wg * 8 * iters * 16 * 32768

        def call(evs, mode=mode, wg=wg):
            if evs is not None:
                evs[0].record()
            tt.probe_mfma_rate(mode, wg, iters, sink)
            if evs is not None:
                evs[1].record()
        (us,) = timer.run(call, calls=5, n_events=2)
        tf = flops / statistics.median(us) / 1e6
        out[name] = {"TFLOPs": round(tf, 1), "frac_of_dense_peak": round(tf / MFMA_PEAK_TFLOPS, 4),
                     "us": round(statistics.median(us), 2)}
    return out


def workloads(dev, fenced=False):
    import synth
    import torch

    timer = Timer(torch, dev, fenced)
    out = {}
    out["stream_read_ceiling"] = stream_ceiling(timer, dev)
    out["mfma_ceiling"] = mfma_ceiling(timer, dev)
    print("bench: stream and MFMA ceilings done", file=sys.stderr, flush=True)
    out["tiny_fp32"] = attention_workload(
        "tiny fp32: L 256, S 16, Hq 4 / Hkv 1, head_dim 64", synth.config_attn("tiny_fp32"),
        timer, [0], out_dtype=torch.float32)
    out["tiny_fp32_unmask"] = unmask_workload("tiny fp32 unmask: 16 x 1024 logits ~ N(0, 3)",
                                              synth.config_logits("tiny_fp32"), timer)
    out["ctx4k"] = attention_workload(
        "4K context bf16: B 1, L 4096, S 16, Hq 32 / Hkv 2, head_dim 128",
        synth.config_attn("ctx4k_bf16"), timer, [0], out_dtype=torch.bfloat16)
    out["ctx4k_unmask"] = unmask_workload(
        "4K-context unmask: 16 x 131072 logits ~ N(0, 4) + one planted peak per row",
        synth.config_logits("ctx4k_bf16"), timer)
    print("bench: tiny and 4K workloads done", file=sys.stderr, flush=True)
    out["ragged32"] = attention_workload(
        "ragged paged batch bf16: B 32, L ~ U[1024, 8192], 256-token pages in random order",
        synth.config_attn("ragged32_paged"), timer, [0], out_dtype=torch.bfloat16)
    print("bench: ragged workload done", file=sys.stderr, flush=True)
    out["ctx128k"] = attention_workload(
        "131072-token context bf16: B 1, S 16, Hq 32 / Hkv 2, head_dim 128, 1% outlier keys x8",
        synth.config_attn("long128k"), timer, [64, 128, 256, 0], out_dtype=torch.bfloat16)
    print("bench: 128K workload done", file=sys.stderr, flush=True)
    del timer
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed blocks (T denoise steps each)")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the tiny / 4K / ragged / 128K workloads after the block loop")
    ap.add_argument("--no-events", action="store_true",
                    help="do not record per-call attention events")
    ap.add_argument("--fenced-events", action="store_true",
                    help="time with default HIP events (a system-scope cache write-back and "
                         "invalidate at every record) instead of fence-free timing events")
    ap.add_argument("--block-size", type=int, default=16, metavar="S",
                    help="block size S (16 is the benchmark's workload; the pages also use 32 and "
                         "128)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed region, copy MIB MiB device to device once (the plain "
                         "copy of known size that scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is "
              "single-GPU by design and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    import two_tower_cross_amd as tt
    from synth.device import loop_model

    dev = torch.device("cuda", 0)
    m = loop_model(5, S=args.block_size, device=dev)
    step = tt.DenoiseStep(k_pages=m.k_pages, v_pages=m.v_pages, w_qkv=m.w_qkv, w_o=m.w_o,
                          w_lm=m.w_lm, block_table=m.block_table, ctx_lens=m.ctx_lens,
                          max_ctx_len=m.L, num_q_heads=m.Hq, num_kv_heads=m.Hkv, head_dim=m.D,
                          batch=m.B, S=m.S)
    masked = torch.ones((m.B, m.S), dtype=torch.uint8, device=dev)
    tokens = torch.full((m.B, m.S), -1, dtype=torch.int32, device=dev)
    # per-step commit counts of the timed blocks, each step writing its own slice (summed after
    # timing, so that counting adds no work to the timed region)
    counts = torch.zeros((args.steps, m.T, m.B), dtype=torch.int32, device=dev)

    L = m.layers

    def step_events(s):
        """Events of timed denoise step s. Even steps bracket one layer's attention call (main
        kernel + merge), odd steps one layer's main kernel alone, the layers rotating; so each
        sampled call carries two events and a step records two (every record still costs about
        2 us of idle GPU, so the timing is spread thin over the timed region)."""
        ev = [None] * (3 * L)
        e0, e1 = make_event(args.fenced_events), make_event(args.fenced_events)
        layer = (s // 2) % L
        if s % 2 == 0:
            ev[3 * layer], ev[3 * layer + 2] = e0.cuda_event, e1.cuda_event
        else:
            layer = (layer + L // 2) % L
            ev[3 * layer], ev[3 * layer + 1] = e0.cuda_event, e1.cuda_event
        return ev, s % 2, (e0, e1)

    def run_block(events=None, k=None):
        masked.fill_(1)
        tokens.fill_(-1)
        for t in range(m.T):
            step(m.h_steps[t], masked, tokens, threshold=THRESHOLD, min_commit=True,
                 commit_all=(t == m.T - 1), timing_events=None if events is None else events[t][0],
                 n_committed=None if k is None else counts[k, t])

    for _ in range(args.warmup):
        run_block()
    torch.cuda.synchronize()

    def timed_pass(events=None):
        """K timed blocks (bracketed by synchronize); returns (ms total, committed tokens, ms per
        block, host enqueue ms)."""
        counts.zero_()
        marks = [make_event() for _ in range(args.steps + 1)]   # block boundaries (fence-free)
        for e in marks:
            e.record()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_host = time.perf_counter()
        start.record()
        marks[0].record()
        for k in range(args.steps):
            run_block(None if events is None else events[k * m.T:(k + 1) * m.T], k)
            marks[k + 1].record()
        stop.record()
        enqueue_ms = (time.perf_counter() - t_host) * 1e3
        torch.cuda.synchronize()
        total = start.elapsed_time(stop)
        per_block = [round(marks[k].elapsed_time(marks[k + 1]), 3) for k in range(args.steps)]
        n = int(counts.sum().item())
        assert not masked.any().item(), "a block ended with masked positions"
        return total, n, per_block, enqueue_ms

    # The headline pass carries no per-call events (a record on the launch stream between two
    # kernels costs idle GPU time and, now and then, a long host-side stall in the runtime).
    ms_total, n_tokens, block_ms, host_enqueue_ms = timed_pass()
    ms_per_block = ms_total / args.steps
    value = n_tokens / (ms_total / 1e3)
    print(f"bench: block loop timed, {value:.1f} committed tokens/s", file=sys.stderr, flush=True)

    # The attention roofline comes from a second timed pass of the same K blocks, with the
    # library recording the sampled events on its launch stream.
    events = None
    ev_pass = None
    if not args.no_events:
        events = [step_events(s) for s in range(args.steps * m.T)]
        for _, _, pair in events:
            for e in pair:
                e.record()      # materialize
        torch.cuda.synchronize()
        ev_total, ev_tokens, ev_blocks, ev_enqueue = timed_pass(events)
        ev_pass = {"value": round(ev_tokens / (ev_total / 1e3), 1),
                   "ms_per_timed_block": ev_blocks, "host_enqueue_ms": round(ev_enqueue, 2)}

    roofline = None
    if events is not None:
        whole = [1e3 * a.elapsed_time(b) for _, kind, (a, b) in events if kind == 0]
        kern = [1e3 * a.elapsed_time(b) for _, kind, (a, b) in events if kind == 1]
        n_calls = len(whole)
        lens = [m.L] * m.B
        nbytes = attn_bytes(lens, m.S, m.Hq, m.Hkv, m.D)
        flops = attn_flops(lens, m.S, m.Hq, m.D)
        call_us, kern_us = sum(whole) / len(whole), sum(kern) / len(kern)
        kernels = ["block_attn_bf16_kernel<128>", "attn_reduce_kernel<128>"]
        if flops / nbytes <= MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
            achieved = nbytes / call_us / 1e3
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                        "traffic": measured_traffic(kernels) if m.S == 16 else None,
                        "kernel": " + ".join(kernels), "call_us": round(call_us, 2),
                        "call_us_median_min": stats_us(whole), "bytes_per_call": nbytes,
                        "timed_calls": n_calls, "timing_pass": ev_pass,
                        "timing": "a second timed pass of the same blocks: every other denoise "
                        "step brackets one attention call, the others one main kernel "
                        "(layers rotating), "
                        + ("default" if args.fenced_events else "fence-free") + " HIP events "
                        "recorded by the library on its launch stream",
                        "kernel_only": {"kernel": kernels[0], "launch_us": round(kern_us, 2),
                                        "launch_us_median_min": stats_us(kern),
                                        "achieved": round(nbytes / kern_us / 1e3, 1),
                                        "frac": round(nbytes / kern_us / 1e3 / HBM_PEAK_GBPS, 4)}}
        else:   # past the ridge (larger blocks): the matrix cores bound the attention
            achieved = flops / call_us / 1e6
            roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                        "traffic": None, "kernel": " + ".join(kernels),
                        "call_us": round(call_us, 2), "flops_per_call": flops,
                        "kernel_only": {"kernel": kernels[0], "launch_us": round(kern_us, 2),
                                        "frac": round(flops / kern_us / 1e6 / MFMA_PEAK_TFLOPS, 4)}}

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # one denoise step with every sequence live, then with half of them finished (no masked
    # position left): a finished sequence gets no attention work, the live ones spread over the GPU
    half = None
    if not args.no_workloads:
        timer = Timer(torch, dev, args.fenced_events)
        hm = torch.ones((m.B, m.S), dtype=torch.uint8, device=dev)
        ht = torch.full((m.B, m.S), -1, dtype=torch.int32, device=dev)

        def step_with(n_finished):
            def reset():
                hm.fill_(1)
                hm[:n_finished] = 0
                ht.fill_(-1)

            def call(evs):
                if evs is not None:
                    evs[0].record()
                step(m.h_steps[0], hm, ht, threshold=THRESHOLD, min_commit=True)
                if evs is not None:
                    evs[1].record()
            (us,) = timer.run(call, calls=20, n_events=2, reset=reset)
            return stats_us(us)
        half = {"workload": "one denoise step of the block loop (6 layers, lm-head, unmask)",
                "all_live_us": step_with(0), f"{m.B // 2}_of_{m.B}_finished_us": step_with(m.B // 2)}
        del timer

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(m)
        print("bench: cpu baseline done", file=sys.stderr, flush=True)

    extra = None
    if not args.no_workloads:
        del step
        extra = workloads(dev, args.fenced_events)
        extra["step_half_finished"] = half

    if args.copy_calibration > 0 and not args.no_workloads:
        n = args.copy_calibration << 20   # again: the calibration must be the run's last dispatch
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    line = {
        "metric": "denoise-step attn HBM GB/s (% of peak) + committed tokens/s at 32K ctx",
        "value": round(value, 1),
        "unit": "committed tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_block, 4),
        "ms_per_timed_block": block_ms,
        "host_enqueue_ms": round(host_enqueue_ms, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded on-device N(0,1) KV caches, hidden states and scaled weights; "
                "seeded host draws for the other workloads)",
        "config": {"workload": f"block loop: batch 8, 6 attention layers, context 32768, S={m.S}, "
                               "T=16, hidden 2048, Hq 32 / Hkv 2, head_dim 128, vocab 131072, "
                               "threshold 0.9", "global_batch": m.B, "seq_len": m.L,
                   "parallelism": "single GPU"},
        "attn_GBps": None if roofline is None or roofline["bound"] != "hbm" else roofline["achieved"],
        "attn_frac_of_hbm_peak": (None if roofline is None or roofline["bound"] != "hbm"
                                  else roofline["frac"]),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "workloads": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
