"""Seeded synthetic inputs for the block-diffusion denoise step.

This module is shared by the oracle tests, the GPU parity tests and the benchmark. It holds
distributions, shapes, memory layouts and the fp32 -> bf16 rounding of stored values, and nothing
of the method's own arithmetic (no attention, softmax, argmax or threshold). Every random draw is
made from a NumPy PCG64 generator with an explicit seed, so the same call gives the same bits on
every machine.

Layouts produced here (the library's layouts, documented in ``include/twotower.h``):

* ``q``        ``[B, S, Hq, D]``
* ``k_pages``  ``[num_pages, Hkv, page_size // T, D // CK, T, CK]`` (tiles of T tokens made of
  CK-element chunks: element (o, d) at [page, g, o // T, d // CK, o % T, d % CK])
* ``v_pages``  ``[num_pages, Hkv, page_size // T, T // CV, D, CV]`` (tiles of T tokens made of
  CV-token chunks: element (o, d) at [page, g, o // T, (o % T) // CV, d, o % CV])

  (T, CK, CV) = (64, 8, 8), the library's widths, whenever page_size is a multiple of 64 and D
  of 8; otherwise a width falls back to the whole extent (T = page_size, CK = D, CV = T), which
  only the oracle reads (small hand-sized cases).
* ``k_blk``    ``[B, Hkv, S, D]``
* ``v_blk``    ``[B, Hkv, D, S]``
* ``block_table`` ``[B, max_pages]`` int32, ``ctx_lens`` ``[B]`` int32
* ``logits``   ``[B, S, V]`` fp32

Floating arrays are returned as float32. For bf16 cases every stored value is already exactly
representable in bf16 (rounded to nearest even), so ``bf16_bits`` gives the bits the GPU sees and
the oracle upcasts the very same values.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "rng", "round_to_bf16", "bf16_bits", "bits_to_f32", "tile_widths", "tile_k", "untile_k",
    "tile_v", "untile_v", "AttnCase",
    "attn_case",
    "logits_normal", "logits_planted", "config_attn", "config_logits",
]


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even); NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(x)
    out[nan] = np.float32("nan")
    return out


def bf16_bits(x_bf16_exact: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exactly representable in bf16."""
    u = np.ascontiguousarray(x_bf16_exact, dtype=np.float32).view(np.uint32)
    low = u & 0xFFFF
    if np.any(low[~np.isnan(x_bf16_exact)] != 0):
        raise ValueError("values are not bf16-exact")
    return (u >> 16).astype(np.uint16)


def tile_widths(page_size: int, D: int) -> tuple[int, int, int]:
    """(T, CK, CV): tokens per tile, K elements per chunk, V tokens per chunk."""
    T = 64 if page_size % 64 == 0 else page_size
    CK = 8 if D % 8 == 0 else D
    CV = 8 if T % 8 == 0 else T
    return T, CK, CV


def tile_k(k: np.ndarray) -> np.ndarray:
    """[..., page, D] (token-major page) -> [..., page // T, D // CK, T, CK] (the K page layout)."""
    *lead, P, D = k.shape
    T, CK, _ = tile_widths(P, D)
    nd = len(lead)
    x = k.reshape(*lead, P // T, T, D // CK, CK)
    return np.ascontiguousarray(np.swapaxes(x, nd + 1, nd + 2))


def untile_k(kt: np.ndarray) -> np.ndarray:
    """Inverse of tile_k."""
    *lead, nt, nck, T, CK = kt.shape
    nd = len(lead)
    return np.ascontiguousarray(np.swapaxes(kt, nd + 1, nd + 2)).reshape(*lead, nt * T, nck * CK)


def tile_v(v_dim_major: np.ndarray) -> np.ndarray:
    """[..., D, page] (dim-major page) -> [..., page // T, T // CV, D, CV] (the V page layout)."""
    *lead, D, P = v_dim_major.shape
    T, _, CV = tile_widths(P, D)
    nd = len(lead)
    x = v_dim_major.reshape(*lead, D, P // T, T // CV, CV)
    perm = list(range(nd)) + [nd + 1, nd + 2, nd, nd + 3]
    return np.ascontiguousarray(x.transpose(perm))


def untile_v(vt: np.ndarray) -> np.ndarray:
    """Inverse of tile_v: [..., page // T, T // CV, D, CV] -> [..., D, page]."""
    *lead, nt, ncv, D, CV = vt.shape
    nd = len(lead)
    perm = list(range(nd)) + [nd + 2, nd, nd + 1, nd + 3]
    return np.ascontiguousarray(vt.transpose(perm)).reshape(*lead, D, nt * ncv * CV)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class AttnCase:
    """One block-attention problem in the library's memory layout (see module docstring)."""
    dtype: str                 # "bf16" or "fp32"
    q: np.ndarray
    k_pages: np.ndarray
    v_pages: np.ndarray
    block_table: np.ndarray
    ctx_lens: np.ndarray
    k_blk: np.ndarray
    v_blk: np.ndarray
    scale: float

    @property
    def B(self): return self.q.shape[0]

    @property
    def S(self): return self.q.shape[1]

    @property
    def Hq(self): return self.q.shape[2]

    @property
    def D(self): return self.q.shape[3]

    @property
    def Hkv(self): return self.k_pages.shape[1]

    @property
    def page_size(self): return self.k_pages.shape[2] * self.k_pages.shape[4]


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = x.astype(np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def attn_case(seed: int, *, B: int, S: int, Hq: int, Hkv: int, D: int, ctx_lens,
              page_size: int | None = None, dtype: str = "bf16", shuffle_pages: bool = True,
              spare_frac: float = 0.0, nan_poison: bool = False, outlier_frac: float = 0.0,
              outlier_scale: float = 8.0, scale: float | None = None, q_scale: float = 1.0,
              v_scale: float = 1.0) -> AttnCase:
    """Q/K/V ~ N(0, 1) in the paged layout.

    ``ctx_lens``: sequence of B context lengths. ``page_size`` None means one page per sequence
    (contiguous context, page_size = max length rounded up to a multiple of 64). With ``shuffle_pages`` the
    pages of all sequences sit in the pool in a random order. ``spare_frac`` adds unused pool
    pages; ``nan_poison`` fills unused pages and the tail of every last page with NaN.
    ``outlier_frac`` of the context positions, drawn independently per KV head, get their whole
    key vector multiplied by ``outlier_scale`` before rounding. ``q_scale`` / ``v_scale`` multiply
    the queries / all values (context and block) before rounding: Q ~ N(0, q_scale^2),
    V ~ N(0, v_scale^2).
    """
    g = rng(seed)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32).reshape(B)
    Lmax = int(ctx_lens.max()) if B else 0
    if page_size is None:
        page_size = max(64, -(-Lmax // 64) * 64)
    pages_per_seq = [-(-int(L) // page_size) for L in ctx_lens]
    n_used = sum(pages_per_seq)
    n_pool = max(1, n_used + int(math.ceil(spare_frac * n_used)))
    max_pages = max(1, max(pages_per_seq) if B else 1)

    qs, vs = np.float32(q_scale), np.float32(v_scale)
    q = _store(g.standard_normal((B, S, Hq, D), dtype=np.float32) * qs, dtype)
    k_blk = _store(g.standard_normal((B, Hkv, S, D), dtype=np.float32), dtype)
    v_blk = _store(g.standard_normal((B, Hkv, D, S), dtype=np.float32) * vs, dtype)

    seqs = []
    for b in range(B):
        L = int(ctx_lens[b])
        k = g.standard_normal((L, Hkv, D), dtype=np.float32)
        v = g.standard_normal((L, Hkv, D), dtype=np.float32) * vs
        if outlier_frac > 0.0:
            hit = g.random((L, Hkv)) < outlier_frac
            k = np.where(hit[:, :, None], k * np.float32(outlier_scale), k)
        seqs.append((_store(k, dtype), _store(v, dtype)))

    fill = np.float32("nan") if nan_poison else np.float32(0.0)
    k_pages = np.full((n_pool, Hkv, page_size, D), fill, dtype=np.float32)   # both tiled below
    v_pages = np.full((n_pool, Hkv, D, page_size), fill, dtype=np.float32)
    order = g.permutation(n_pool) if shuffle_pages else np.arange(n_pool)
    block_table = np.zeros((B, max_pages), dtype=np.int32)
    nxt = 0
    for b in range(B):
        L = int(ctx_lens[b])
        k, v = seqs[b]
        for p in range(pages_per_seq[b]):
            slot = int(order[nxt]); nxt += 1
            block_table[b, p] = slot
            t0, t1 = p * page_size, min(L, (p + 1) * page_size)
            n = t1 - t0
            k_pages[slot, :, :n, :] = k[t0:t1].transpose(1, 0, 2)
            v_pages[slot, :, :, :n] = v[t0:t1].transpose(1, 2, 0)
    k_pages, v_pages = tile_k(k_pages), tile_v(v_pages)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return AttnCase(dtype, q, k_pages, v_pages, block_table, ctx_lens, k_blk, v_blk, float(scale))


def logits_normal(seed: int, B: int, S: int, V: int, sigma: float) -> np.ndarray:
    """fp32 logits ~ N(0, sigma^2)."""
    return (rng(seed).standard_normal((B, S, V), dtype=np.float32) * np.float32(sigma))


def logits_planted(seed: int, B: int, S: int, V: int, sigma: float,
                   conf_lo: float = 0.3, conf_hi: float = 0.999) -> np.ndarray:
    """N(0, sigma^2) logits plus one planted peak per row.

    The peak position is uniform. Its height is ln V + sigma^2/2 + ln(c / (1 - c)) with
    c ~ U(conf_lo, conf_hi): ln V + sigma^2/2 is the log of the expected partition sum of the
    normal background, so the peak's share of the row lands near c and rows spread over both
    sides of a threshold in (conf_lo, conf_hi).
    """
    g = rng(seed)
    x = g.standard_normal((B, S, V), dtype=np.float32) * np.float32(sigma)
    pos = g.integers(0, V, size=(B, S))
    c = g.uniform(conf_lo, conf_hi, size=(B, S))
    height = math.log(V) + 0.5 * sigma * sigma + np.log(c / (1.0 - c))
    bi, si = np.meshgrid(np.arange(B), np.arange(S), indexing="ij")
    x[bi, si, pos] = height.astype(np.float32)
    return x


# ---------------------------------------------------------------------------------------------
# The workload shapes: a tiny fp32 case, a 4K-context bf16 case, a ragged paged batch of 32,
# a 128K-token long context and the 6-layer 32K-context block loop (built on the device by the
# benchmark; its attention shapes are also available here at reduced length for parity).

def config_attn(name: str, *, ctx_len: int | None = None, seed: int | None = None) -> AttnCase:
    if name == "tiny_fp32":
        return attn_case(1 if seed is None else seed, B=1, S=16, Hq=4, Hkv=1, D=64,
                         ctx_lens=[256 if ctx_len is None else ctx_len], page_size=256,
                         dtype="fp32", scale=1.0 / 8.0)
    if name == "ctx4k_bf16":
        L = 4096 if ctx_len is None else ctx_len
        return attn_case(2 if seed is None else seed, B=1, S=16, Hq=32, Hkv=2, D=128,
                         ctx_lens=[L], page_size=None, dtype="bf16")
    if name == "ragged32_paged":
        g = rng(3 if seed is None else seed)
        lo, hi = (1024, 8192) if ctx_len is None else (max(1, ctx_len // 8), ctx_len)
        lens = g.integers(lo, hi + 1, size=32)
        return attn_case(int(g.integers(1 << 30)), B=32, S=16, Hq=32, Hkv=2, D=128, ctx_lens=lens,
                         page_size=256, dtype="bf16", shuffle_pages=True, spare_frac=0.1,
                         nan_poison=True)
    if name == "long128k":
        L = 131072 if ctx_len is None else ctx_len
        return attn_case(4 if seed is None else seed, B=1, S=16, Hq=32, Hkv=2, D=128,
                         ctx_lens=[L], page_size=None, dtype="bf16", outlier_frac=0.01,
                         outlier_scale=8.0)
    if name == "loop32k_layer":
        L = 32768 if ctx_len is None else ctx_len
        return attn_case(5 if seed is None else seed, B=8, S=16, Hq=32, Hkv=2, D=128,
                         ctx_lens=[L] * 8, page_size=None, dtype="bf16")
    raise KeyError(name)


def config_logits(name: str, *, seed: int | None = None, vocab: int | None = None) -> np.ndarray:
    if name == "tiny_fp32":
        return logits_normal(1 if seed is None else seed, 1, 16, vocab or 1024, math.sqrt(3.0))
    if name == "ctx4k_bf16":
        return logits_planted(2 if seed is None else seed, 1, 16, vocab or 131072, 2.0)
    raise KeyError(name)
