"""Reference denoise step and T-step block loop of a synthetic attention-only denoiser (float64).

The generation loop followed (Nemotron-TwoTower explainer, gist.science, section
"Generierungsprozess", and the same section of the Chinese page): a new block starts as S masked
tokens; the denoiser refines it over T steps; in each step it attends, layer by layer, to the
context tower's KV cache of past blocks and to its own bidirectional KV of the current block
(rewritten every step, because the block changes); confident tokens are committed (confidence
unmasking, see ``unmask``). The context cache is the frozen tower's and is only read.

The pages give no shapes for the denoiser's layers; the synthetic model used here (a reading,
not the pages') is a residual stream H [B, S, hidden] with, per attention layer l,

    [Q | K_blk | V_blk] = H W_qkv[l]^T          (W_qkv[l]: [Hq*D + 2*Hkv*D, hidden])
    O                   = block attention of the block queries over [ctx KV[l] ; block KV]
    H                   = H + O W_o[l]^T          (W_o[l]: [hidden, Hq*D])

and finally logits = H W_lm^T (W_lm: [V, hidden]). Weight matrices are stored [out, in]. The
columns of W_qkv^T are ordered Q (head-major, h*D + d), then K (g*D + d), then V (g*D + d).
"""
from __future__ import annotations

import numpy as np

from . import attention, unmask


def linear(x, w):
    """x [..., in] times w [out, in]^T in float64."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def qkv_projection(h, w_qkv, Hq, Hkv, D):
    """H [B,S,hidden] -> Q [B,S,Hq,D], K_blk [B,Hkv,S,D], V_blk [B,Hkv,D,S]."""
    y = linear(h, w_qkv)                              # [B, S, Hq*D + 2*Hkv*D]
    B, S, _ = y.shape
    q = y[..., :Hq * D].reshape(B, S, Hq, D)
    k = y[..., Hq * D:(Hq + Hkv) * D].reshape(B, S, Hkv, D).transpose(0, 2, 1, 3)
    v = y[..., (Hq + Hkv) * D:].reshape(B, S, Hkv, D).transpose(0, 2, 3, 1)
    return q, k, v


def residual_output(h, o, w_o):
    """H + O W_o^T with O [B,S,Hq,D] flattened to [B,S,Hq*D]."""
    B, S = o.shape[:2]
    return np.asarray(h, dtype=np.float64) + linear(np.asarray(o).reshape(B, S, -1), w_o)


def lm_head(h, w_lm):
    return linear(h, w_lm)


def denoise_step(h0, layers, block_table, ctx_lens, w_lm, masked, tokens, *, Hq, Hkv, D, scale,
                 threshold, min_commit=False, commit_all=False):
    """One step. ``layers`` is a list of (w_qkv, w_o, k_pages, v_pages), one per attention layer.

    Returns (tokens', masked', confidence, n_committed, logits).
    """
    h = np.asarray(h0, dtype=np.float64)
    for w_qkv, w_o, k_pages, v_pages in layers:
        q, kb, vb = qkv_projection(h, w_qkv, Hq, Hkv, D)
        o, _ = attention.block_attention(q, k_pages, v_pages, block_table, ctx_lens, kb, vb, scale)
        h = residual_output(h, o, w_o)
    logits = lm_head(h, w_lm)
    t, m, c, n = unmask.confidence_unmask(logits, masked, tokens, threshold, min_commit, commit_all)
    return t, m, c, n, logits


def block_loop(h_steps, layers, block_table, ctx_lens, w_lm, *, Hq, Hkv, D, scale, threshold,
               min_commit=True, mask_token=-1):
    """T steps over one block; h_steps[t] is the step-t hidden input [B,S,hidden].

    The block starts fully masked; the last step commits every position still masked.
    Returns (tokens, n_committed per step [T, B]).
    """
    T = len(h_steps)
    B, S = h_steps[0].shape[:2]
    tokens = np.full((B, S), mask_token, dtype=np.int32)
    masked = np.ones((B, S), dtype=np.uint8)
    per_step = np.zeros((T, B), dtype=np.int32)
    for t in range(T):
        tokens, masked, _, n, _ = denoise_step(
            h_steps[t], layers, block_table, ctx_lens, w_lm, masked, tokens, Hq=Hq, Hkv=Hkv, D=D,
            scale=scale, threshold=threshold, min_commit=min_commit, commit_all=(t == T - 1))
        per_step[t] = n
    return tokens, per_step
