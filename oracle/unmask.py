"""Reference confidence unmasking (float64, NumPy).

Definition followed (Nemotron-TwoTower explainer, gist.science, section "Training und
Konditionierung", sampling paragraph, and the same section of the Chinese page; lay summary
"Der Konfidenz-Trick"; dgnews.ru, test-results section, threshold 0.8 at block size 16): at each
step the denoiser predicts every still-masked position in parallel; positions whose confidence is
above the threshold gamma are committed, uncertain ones stay masked, so the number of commits per
step adapts. Readings taken where the pages are silent:

* confidence = the largest softmax probability of the row = 1 / sum_j exp(x_j - max x);
* the predicted token is the lowest vocabulary index attaining the maximum logit;
* "above" is strict: commit iff conf > gamma;
* commits are final: committed positions are neither read nor changed;
* ``min_commit``: if no masked position clears gamma, the masked position with the largest
  confidence is committed (lowest position on ties), so every step makes progress;
* ``commit_all``: commit every masked position (the last step of a block).
"""
from __future__ import annotations

import numpy as np


def row_confidence(row):
    """(token, confidence) of one logits row, in float64."""
    x = np.asarray(row, dtype=np.float64)
    k = int(np.argmax(x))                   # first index attaining the maximum
    return k, 1.0 / float(np.sum(np.exp(x - x[k])))


def confidence_unmask(logits, masked, tokens, threshold, min_commit=False, commit_all=False):
    """Returns (tokens', masked', confidence [B,S] float64 (NaN where not masked), n_committed [B])."""
    logits = np.asarray(logits)
    B, S, _ = logits.shape
    tokens = np.array(tokens, dtype=np.int32, copy=True)
    masked = np.array(masked, dtype=np.uint8, copy=True)
    conf = np.full((B, S), np.nan)
    n_committed = np.zeros(B, dtype=np.int32)
    gamma = float(threshold)
    for b in range(B):
        cand = []
        for i in range(S):
            if masked[b, i]:
                k, c = row_confidence(logits[b, i])
                conf[b, i] = c
                cand.append((i, k, c))
        if commit_all:
            chosen = cand
        else:
            chosen = [e for e in cand if e[2] > gamma]
            if min_commit and not chosen and cand:
                best = cand[0]
                for e in cand[1:]:
                    if e[2] > best[2]:          # strict: the lowest position wins a tie
                        best = e
                chosen = [best]
        for i, k, _ in chosen:
            tokens[b, i] = k
            masked[b, i] = 0
        n_committed[b] = len(chosen)
    return tokens, masked, conf, n_committed
