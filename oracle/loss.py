"""Reference masked-diffusion training objective (NumPy; fp64 for the likelihood).

Test infrastructure only: imported by tests/, never by the library.

Definition followed (Nemotron-TwoTower explainer, gist.science, "Training und Konditionierung",
masked-diffusion paragraph): clean blocks are corrupted by replacing tokens with [MASK] according
to a linear schedule, and the denoiser minimizes the negative log-likelihood of the original
tokens at the masked positions. Readings taken where the pages are silent:

* linear schedule: a block's diffusion time t is uniform in [0, 1) and each position is masked
  independently with probability t; the uniform draws are inputs (u_time per sequence, u_mask per
  position) and position i is masked iff u_mask < t, compared in fp32 as given;
* the objective is the plain mean of the per-position NLL over all masked positions of the batch
  (no time-dependent weight; the pages name none), and 0 when nothing is masked.
"""
from __future__ import annotations

import numpy as np


def corrupt(clean, u_time, u_mask, mask_id):
    """Returns (noisy int32 [B,S], masked uint8 [B,S], t float32 [B])."""
    clean = np.asarray(clean, dtype=np.int32)
    t = np.asarray(u_time, dtype=np.float32)
    u = np.asarray(u_mask, dtype=np.float32)
    masked = u < t[:, None]
    noisy = np.where(masked, np.int32(mask_id), clean).astype(np.int32)
    return noisy, masked.astype(np.uint8), t.copy()


def masked_nll(logits, targets, masked):
    """Per-row NLL (float64 [B,S], 0 at unmasked rows), mean over masked rows, their number."""
    x = np.asarray(logits, dtype=np.float64)
    B, S, V = x.shape
    nll = np.zeros((B, S))
    for b in range(B):
        for i in range(S):
            if masked[b, i]:
                row = x[b, i]
                m = row.max()
                lse = m + np.log(np.exp(row - m).sum())
                tg = int(targets[b, i])
                nll[b, i] = lse - row[tg] if 0 <= tg < V else np.nan
    n = int(np.count_nonzero(masked))
    loss = float(nll[np.asarray(masked) != 0].sum() / n) if n else 0.0
    return nll, loss, n
