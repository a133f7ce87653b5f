"""Reference block attention of the denoiser tower (float64, NumPy).

Definition followed (Nemotron-TwoTower explainer, gist.science, sections "Architektur" and
"Generierungsprozess"; dgnews.ru, architecture section; gotburnout.io, "2. Denoiser Tower"):
at every denoise step and every attention layer, the queries of the S positions of the current
block attend to the frozen context tower's KV cache of the *same* layer (prompt and committed
tokens, i.e. everything before the block) and to the block's own KV (bidirectional inside the
block). Readings taken where the pages are silent:

* one softmax over the concatenation [context keys ; block keys];
* no mask: the context cache holds only earlier tokens, every block query sees every block key
  including its own position;
* GQA: query head h reads KV head floor(h / (Hq / Hkv));
* the scale is a parameter (1/sqrt(D) in all workloads); Q and K arrive position-encoded.

For every (b, query head h, block position i), with g = h // G and keys K_cat = [K_ctx(b, g) ;
K_blk(b, g)], values V_cat likewise:

    s_j = scale * <q, K_cat[j]>,  m = max_j s_j,  w_j = exp(s_j - m)
    o   = sum_j w_j V_cat[j] / sum_j w_j,   lse = m + ln(sum_j w_j)

Context row t of sequence b sits in page block_table[b, t // page_size] at offset
o = t % page_size. A page holds tiles of T tokens made of element chunks (the cache layout this
build chooses; the pages prescribe none): K pages are [pool, Hkv, page_size // T, D // CK, T, CK]
(element (o, d) at [page, g, o // T, d // CK, o % T, d % CK]), V pages
[pool, Hkv, page_size // T, T // CV, D, CV] (element (o, d) at [page, g, o // T, (o % T) // CV,
d, o % CV]). The library uses T = CK = ... = 64, 8, 8; the tile and chunk widths are read from the
array shapes here, so that small cases can use pages of a few tokens. The block's V is
[B, Hkv, D, S]. Only rows t < ctx_lens[b] are read.
"""
from __future__ import annotations

import numpy as np


def gather_context(k_pages, v_pages, block_table, ctx_len, b, g):
    """Rows 0..ctx_len-1 of sequence b, KV head g, as float64 [L, D] keys and [L, D] values."""
    n_tiles, nck, T, CK = k_pages.shape[2:]
    n_tiles_v, ncv, D, CV = v_pages.shape[2:]
    if n_tiles_v != n_tiles or ncv * CV != T or nck * CK != D:
        raise ValueError("K and V pages disagree on the page or tile shape")
    page_size = n_tiles * T
    t = np.arange(int(ctx_len))
    page = np.asarray(block_table)[b, t // page_size]
    o = t % page_size
    kp = np.asarray(k_pages[:, g], dtype=np.float64)   # [pool, tiles, D // CK, T, CK]
    vp = np.asarray(v_pages[:, g], dtype=np.float64)   # [pool, tiles, T // CV, D, CV]
    d = np.arange(D)
    keys = kp[page[:, None], (o // T)[:, None], d[None, :] // CK, (o % T)[:, None], d[None, :] % CK]
    vals = vp[page[:, None], (o // T)[:, None], ((o % T) // CV)[:, None], d[None, :],
              (o % CV)[:, None]]
    return keys, vals                                   # [L, D] each


def _softmax_attend(qrows, keys, vals, scale):
    """qrows [R, D], keys/vals [N, D] -> (out [R, D], lse [R]) with one softmax over N keys."""
    s = scale * (qrows @ keys.T)                     # [R, N]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    z = w.sum(axis=1, keepdims=True)
    return (w @ vals) / z, (m + np.log(z))[:, 0]


def block_attention(q, k_pages, v_pages, block_table, ctx_lens, k_blk, v_blk, scale):
    """Full output: O float64 [B, S, Hq, D] and LSE float64 [B, Hq, S] (natural log)."""
    q = np.asarray(q, dtype=np.float64)
    B, S, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    out = np.empty((B, S, Hq, D))
    lse = np.empty((B, Hq, S))
    for b in range(B):
        for g in range(Hkv):
            kc, vc = gather_context(k_pages, v_pages, block_table, ctx_lens[b], b, g)
            keys = np.concatenate([kc, np.asarray(k_blk[b, g], dtype=np.float64)], axis=0)
            vals = np.concatenate([vc, np.asarray(v_blk[b, g], dtype=np.float64).T], axis=0)
            if keys.shape[0] == 0:
                raise ValueError("no keys: context and block are both empty")
            for h in range(g * G, (g + 1) * G):
                o, l = _softmax_attend(q[b, :, h, :], keys, vals, scale)
                out[b, :, h, :] = o
                lse[b, h, :] = l
    return out, lse


def block_attention_case(case):
    """``block_attention`` on a ``synth.AttnCase``."""
    return block_attention(case.q, case.k_pages, case.v_pages, case.block_table, case.ctx_lens,
                           case.k_blk, case.v_blk, case.scale)
