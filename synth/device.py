"""Seeded on-device inputs for the 6-layer, 32K-context block loop (bulk data too large to
generate on the host). Distributions and layouts only; no method arithmetic.

Model (one reading, stated with the library): residual stream H [B, S, hidden]; per layer
W_qkv [(Hq + 2 Hkv) D, hidden] and W_o [hidden, Hq D] ~ N(0, 1/fan_in); lm-head W_lm
[V, hidden] ~ N(0, 1/hidden); context KV per layer ~ N(0, 1) as a contiguous cache (one page per
sequence, in the library's tiled page layouts: k [B, Hkv, L/64, D/8, 64, 8], v [B, Hkv, L/64, 8,
D, 8]); a fresh H ~ N(0, 1) per denoise step.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass
class LoopModel:
    B: int
    S: int
    L: int
    layers: int
    Hq: int
    Hkv: int
    D: int
    hidden: int
    vocab: int
    T: int
    k_pages: list
    v_pages: list
    w_qkv: list
    w_o: list
    w_lm: torch.Tensor
    block_table: torch.Tensor
    ctx_lens: torch.Tensor
    h_steps: list
    free_pages: torch.Tensor = None   # paged variant: stack of unused pool pages
    free_count: torch.Tensor = None


def _randn(shape, gen, device, std=1.0):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def loop_model(seed: int = 5, *, B=8, S=16, L=32768, layers=6, Hq=32, Hkv=2, D=128, hidden=2048,
               vocab=131072, T=16, device="cuda", page_size=None, spare_pages=0,
               max_pages=None) -> LoopModel:
    """page_size None: one contiguous page per sequence. Otherwise a pool of page_size-token pages,
    sequence b holding pages b*n .. b*n + n - 1 (n = ceil(L / page_size)) in its table of
    max_pages entries (-1 beyond), plus spare_pages free pages on a stack for the cache to grow."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    if page_size is None:
        P = max(64, -(-L // 64) * 64)
        pool, n = B, 1
    else:
        P = page_size
        n = -(-L // P)
        pool = B * n + spare_pages
    k_pages, v_pages, w_qkv, w_o = [], [], [], []
    for _ in range(layers):
        k_pages.append(_randn((pool, Hkv, P // 64, D // 8, 64, 8), g, dev))
        v_pages.append(_randn((pool, Hkv, P // 64, 8, D, 8), g, dev))
        w_qkv.append(_randn(((Hq + 2 * Hkv) * D, hidden), g, dev, 1.0 / math.sqrt(hidden)))
        w_o.append(_randn((hidden, Hq * D), g, dev, 1.0 / math.sqrt(Hq * D)))
    w_lm = _randn((vocab, hidden), g, dev, 1.0 / math.sqrt(hidden))
    h_steps = []
    for t in range(T):
        gt = torch.Generator(device=dev)
        gt.manual_seed(seed * 1000 + t)
        h_steps.append(_randn((B, S, hidden), gt, dev))
    ctx_lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    if page_size is None:
        block_table = torch.arange(B, dtype=torch.int32, device=dev).view(B, 1)
        return LoopModel(B, S, L, layers, Hq, Hkv, D, hidden, vocab, T, k_pages, v_pages, w_qkv,
                         w_o, w_lm, block_table, ctx_lens, h_steps)
    mp = max_pages if max_pages is not None else n + 1
    block_table = torch.full((B, mp), -1, dtype=torch.int32, device=dev)
    block_table[:, :n] = torch.arange(B * n, dtype=torch.int32, device=dev).view(B, n)
    free_pages = torch.arange(B * n, pool, dtype=torch.int32, device=dev)
    free_count = torch.tensor([pool - B * n], dtype=torch.int32, device=dev)
    return LoopModel(B, S, L, layers, Hq, Hkv, D, hidden, vocab, T, k_pages, v_pages, w_qkv, w_o,
                     w_lm, block_table, ctx_lens, h_steps, free_pages, free_count)
