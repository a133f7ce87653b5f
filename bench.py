"""Benchmark: committed tokens/s of the TwoTower denoise-step block loop on one MI355X.

Workload (one "step" of this benchmark = one block): batch 8, 6 attention layers, context 32768
tokens per sequence (resident bf16 KV caches, 1.61 GB), block S = 16, T = 16 denoise steps, hidden
2048, Hq = 32 / Hkv = 2, head_dim 128, vocab 131072, threshold 0.9 with the one-commit fallback and
commit-all at the last step. Every denoise step rewrites the block KV of every layer (QKV
projection), runs the block attention over [context KV ; block KV] of the same layer, the output
projection with the residual add, the lm-head to fp32 logits and the confidence unmasking.
Inputs are synthetic (seeded on-device draws) and resident in HBM before timing starts.

Prints one JSON line. ``value`` is committed tokens/s over the timed blocks; ``roofline``
reports the block-attention kernel (the dominant kernel) as algorithmic HBM bytes per launch over
its average launch duration, taken from HIP events recorded around every launch of it inside the
timed region; ``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense bf16
THRESHOLD = 0.9
ATTN_SOURCE = os.path.join(ROOT, "two_tower_cross_amd", "csrc", "block_attn.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "block_attn_bf16_128_loop32k_traffic.md")


def attn_bytes_per_launch(B, L, S, Hq, Hkv, D, e=2):
    """Algorithmic bytes the block-attention kernel must move per launch: context K+V, block K+V
    and Q (its reads; the output is written by the partition merge)."""
    ctx = 2 * B * Hkv * L * D * e
    blk = 2 * B * Hkv * S * D * e
    q = B * S * Hq * D * e
    return ctx + blk + q


def attn_flops_per_launch(B, L, S, Hq, D):
    """QK^T and PV over every (context + block) key of every query row: 4 flops per row, key, dim."""
    return 4 * B * Hq * S * (L + S) * D


def cpu_baseline(m, threads_note, steps=2):
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
    return {"value": n_tok / dt, "unit": "committed tokens/s", "cores": threads_note,
            "kind": "oracle",
            "sample": f"the first {steps} of {m.T} denoise steps of one block, whole batch of "
                      f"{m.B} at context {m.L} (6 layers, lm-head {m.vocab}, unmask): "
                      f"{dt:.2f} s for {n_tok} committed tokens"}


def measured_traffic():
    """HBM bytes per launch of the attention kernel from the committed counter summary, or None
    when there is none or the kernel source changed since the counters were taken."""
    try:
        from two_tower_cross_amd import traffic
        return traffic.bytes_per_launch(TRAFFIC_SUMMARY, ATTN_SOURCE)
    except Exception:
        return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed blocks (T denoise steps each)")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-events", action="store_true",
                    help="do not record per-launch attention events")
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

    def make_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record()          # materialize the underlying hipEvent_t
        return evs

    def run_block(events=None, k=None):
        masked.fill_(1)
        tokens.fill_(-1)
        for t in range(m.T):
            ev = None
            if events is not None:
                base = t * 2 * m.layers
                ev = [events[base + i].cuda_event for i in range(2 * m.layers)]
            step(m.h_steps[t], masked, tokens, threshold=THRESHOLD, min_commit=True,
                 commit_all=(t == m.T - 1), timing_events=ev,
                 n_committed=None if k is None else counts[k, t])

    for _ in range(args.warmup):
        run_block()
    torch.cuda.synchronize()

    per_block = 2 * m.layers * m.T
    events = None if args.no_events else make_events(per_block * args.steps)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        run_block(None if events is None else events[k * per_block:(k + 1) * per_block], k)
    stop.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    n_tokens = int(counts.sum().item())
    assert not masked.any().item(), "a block ended with masked positions"
    ms_per_block = ms_total / args.steps
    value = n_tokens / (ms_total / 1e3)

    roofline = None
    attn_us = None
    if events is not None:
        durs = [events[2 * i].elapsed_time(events[2 * i + 1]) for i in range(len(events) // 2)]
        attn_us = 1e3 * sum(durs) / len(durs)
        nbytes = attn_bytes_per_launch(m.B, m.L, m.S, m.Hq, m.Hkv, m.D)
        flops = attn_flops_per_launch(m.B, m.L, m.S, m.Hq, m.D)
        if flops / nbytes <= MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
            achieved = nbytes / (attn_us * 1e-6) / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                        "traffic": measured_traffic() if m.S == 16 else None,
                        "kernel": "block_attn_bf16_kernel<128>", "launch_us": round(attn_us, 2),
                        "bytes_per_launch": nbytes}
        else:   # past the ridge (larger blocks): the matrix cores bound the kernel
            achieved = flops / (attn_us * 1e-6) / 1e12
            roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                        "traffic": None, "kernel": "block_attn_bf16_kernel<128>",
                        "launch_us": round(attn_us, 2), "flops_per_launch": flops}

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(m, blas_threads())

    line = {
        "metric": "denoise-step attn HBM GB/s (% of peak) + committed tokens/s at 32K ctx",
        "value": round(value, 1),
        "unit": "committed tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_block, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded on-device N(0,1) KV caches, hidden states and scaled weights)",
        "config": {"workload": f"block loop: batch 8, 6 attention layers, context 32768, S={m.S}, "
                               "T=16, hidden 2048, Hq 32 / Hkv 2, head_dim 128, vocab 131072, "
                               "threshold 0.9", "global_batch": m.B, "seq_len": m.L,
                   "parallelism": "single GPU"},
        "attn_GBps": (None if roofline is None else
                      round(attn_bytes_per_launch(m.B, m.L, m.S, m.Hq, m.Hkv, m.D) / attn_us / 1e3, 1)),
        "attn_frac_of_hbm_peak": (None if roofline is None else
                                  round(attn_bytes_per_launch(m.B, m.L, m.S, m.Hq, m.Hkv, m.D)
                                        / attn_us / 1e3 / HBM_PEAK_GBPS, 4)),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
