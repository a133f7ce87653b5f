"""Pure-Python brute force for tiny shapes (no NumPy, no max subtraction).

Independent restatements of the two definitions, used only to pin the NumPy oracle:

* attention: o = sum_j e^{s_j} v_j / sum_j e^{s_j} over the concatenated keys, s_j = scale*<q,k_j>
  (the denoiser's block attention, Nemotron-TwoTower explainer, section "Generierungsprozess");
* confidence: p_j = e^{x_j} / sum e^{x_k}, confidence = max_j p_j at the first maximising j
  (confidence unmasking, explainer, section "Training und Konditionierung").
"""
from __future__ import annotations

import math


def attend(q, keys, vals, scale):
    """q: list[D]; keys, vals: list of list[D] -> list[D]."""
    e = [math.exp(scale * sum(a * b for a, b in zip(q, k))) for k in keys]
    z = math.fsum(e)
    D = len(vals[0])
    return [math.fsum(e[j] * vals[j][d] for j in range(len(keys))) / z for d in range(D)]


def block_attention(q, ctx_k, ctx_v, blk_k, blk_v, scale):
    """Nested lists: q[B][S][Hq][D], ctx_k/ctx_v[B][Hkv][L_b][D] (token-major, already gathered),
    blk_k/blk_v[B][Hkv][S][D]. Returns out[B][S][Hq][D]."""
    B, S, Hq = len(q), len(q[0]), len(q[0][0])
    Hkv = len(blk_k[0])
    G = Hq // Hkv
    out = []
    for b in range(B):
        ob = []
        for i in range(S):
            oi = []
            for h in range(Hq):
                g = h // G
                keys = list(ctx_k[b][g]) + list(blk_k[b][g])
                vals = list(ctx_v[b][g]) + list(blk_v[b][g])
                oi.append(attend(q[b][i][h], keys, vals, scale))
            ob.append(oi)
        out.append(ob)
    return out


def confidence(row):
    """(token, confidence) with an explicit softmax."""
    e = [math.exp(x) for x in row]
    z = math.fsum(e)
    best = 0
    for j in range(1, len(row)):
        if row[j] > row[best]:
            best = j
    return best, e[best] / z
