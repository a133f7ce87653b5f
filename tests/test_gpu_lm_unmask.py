"""GPU parity of the lm-head fused with the unmasking (twotower_lm_head_unmask).

Every masked position is predicted at once and the confident ones are committed (Nemotron-TwoTower
explainer, "Training und Konditionierung", sampling paragraph). The fused call reduces each
256-logit tile of a row to (max, first argmax, sum of exp) inside the product. The logits it
stores on request must match twotower_lm_head within fp32 rounding (the two calls may split K
differently), and twotower_unmask run on those stored logits must agree with it: the same tokens
wherever a row is committed by both (the argmax of identical fp32 values), confidences within fp32
rounding of the reordered sum, and the same commit decisions wherever no confidence lies within
that rounding of the threshold or of the fallback's rival. The decisions are also checked against
the oracle's unmasking of the same logits.
"""
import math

import numpy as np
import pytest
import torch

import synth
import two_tower_cross_amd as tt
from oracle import unmask as ounmask
from gpu_util import DEV

pytestmark = pytest.mark.gpu

CONF_RTOL = 1e-5     # fp32 sum of exp, tile order vs chunk order
GUARD = 1e-4         # relative margin under which a decision is a near tie


def make(seed, B, S, hidden, V, sigma, committed_frac):
    g = torch.Generator(device=DEV).manual_seed(seed)
    h = torch.randn((B, S, hidden), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((V, hidden), generator=g, device=DEV) * (sigma / math.sqrt(hidden))).to(torch.bfloat16)
    r = synth.rng(seed)
    masked = torch.from_numpy((r.random((B, S)) >= committed_frac).astype(np.uint8)).to(DEV)
    tokens = torch.from_numpy(np.where(masked.cpu().numpy() == 0, 7, -1).astype(np.int32)).to(DEV)
    return h, tt.pack_weight(w), masked, tokens


def exempt(conf_ref, m0, gamma, min_commit, commit_all):
    """Sequences whose decisions sit within rounding of the threshold or of a fallback rival."""
    out = set()
    for b in range(conf_ref.shape[0]):
        c = conf_ref[b][m0[b] != 0]
        if commit_all or c.size == 0:
            continue
        if np.any(np.abs(c - gamma) <= GUARD * gamma):
            out.add(b)
        elif min_commit and not np.any(c > gamma) and c.size > 1:
            top = np.sort(c)[::-1]
            if top[0] - top[1] <= GUARD * top[0]:
                out.add(b)
    return out


CASES = [
    # B, S, hidden, V, logit sigma, threshold, committed fraction, min_commit, commit_all
    (2, 16, 512, 8192, 3.0, 0.15, 0.0, True, False),
    (3, 5, 136, 1004, 4.0, 0.05, 0.3, True, False),      # ragged last tile, S != 16
    (8, 16, 2048, 131072, 1.0, 0.9, 0.0, True, False),   # the 32K loop's lm-head: fallback only
    (4, 16, 264, 4096, 5.0, 0.5, 0.5, False, False),
    (2, 64, 128, 2048, 2.0, 0.3, 0.2, True, True),       # commit-all, 64 positions
    (2, 128, 256, 2048, 3.0, 0.2, 0.3, True, False),     # block size 128 (two row tiles)
    (2, 16, 128, 1100, 3.0, 0.2, 0.0, True, False),      # 35 slabs: last tile past the weight
    # two row blocks, 300 tiles over 128 persistent work-groups (2 or 3 each), K tail
    (16, 16, 136, 76800, 2.0, 0.3, 0.2, True, False),
]


@pytest.mark.parametrize("keep", [True, False], ids=["logits", "no-logits"])
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}S{c[1]}V{c[3]}" for c in CASES])
def test_fused_matches_two_call_path_and_oracle(case, keep):
    """keep: the call also stores the logits (and unmask runs on them); else the logits come from
    a second, storing call (the same products in the same order, so the same fp32 values)."""
    B, S, hidden, V, sigma, gamma, frac, min_commit, commit_all = case
    h, w, masked, tokens = make(17 + V % 97, B, S, hidden, V, sigma, frac)
    m0, t0 = masked.cpu().numpy().copy(), tokens.cpu().numpy().copy()
    m1, t1 = masked.clone(), tokens.clone()
    conf, n, logits = tt.lm_head_unmask(h, w, masked, tokens, gamma, min_commit=min_commit,
                                        commit_all=commit_all, keep_logits=keep)
    if not keep:
        assert logits is None
        _, _, logits = tt.lm_head_unmask(h, w, masked.new_tensor(m0), tokens.new_tensor(t0), gamma,
                                         min_commit=min_commit, commit_all=commit_all,
                                         keep_logits=True)
    ref_logits = tt.lm_head(h, w)
    conf2, n2 = tt.unmask(logits, m1, t1, gamma, min_commit=min_commit, commit_all=commit_all)
    torch.cuda.synchronize()
    err = (logits - ref_logits).abs().max().item()
    assert err <= 1e-4 + 1e-5 * ref_logits.abs().max().item(), err

    live = m0 != 0
    c, c2 = conf.cpu().numpy(), conf2.cpu().numpy()
    assert np.all(np.abs(c[live] - c2[live]) <= CONF_RTOL * np.abs(c2[live]))
    assert np.all(np.isnan(c[~live]))                    # committed rows are not touched

    gm, gt, gn = masked.cpu().numpy(), tokens.cpu().numpy(), n.cpu().numpy()
    rm, rt, rn = m1.cpu().numpy(), t1.cpu().numpy(), n2.cpu().numpy()
    both = (gm == 0) & (rm == 0) & live
    assert np.array_equal(gt[both], rt[both])
    assert np.array_equal(gt[~live], t0[~live]) and np.all(gm[~live] == 0)
    skip = exempt(c2.astype(np.float64), m0, gamma, min_commit, commit_all)
    for b in range(B):
        if b not in skip:
            assert np.array_equal(gm[b], rm[b]) and np.array_equal(gt[b], rt[b]) and gn[b] == rn[b]

    # the oracle's unmasking of the same logits (fp64 confidences)
    ot, om, oc, on = ounmask.confidence_unmask(logits.cpu().numpy(), m0, t0, np.float32(gamma),
                                               min_commit=min_commit, commit_all=commit_all)
    assert np.all(np.abs(c[live] - oc[live]) <= CONF_RTOL * oc[live])
    skip = exempt(oc, m0, gamma, min_commit, commit_all)
    for b in range(B):
        if b not in skip:
            assert np.array_equal(gm[b], om[b]) and np.array_equal(gt[b], ot[b]) and gn[b] == on[b]
    assert len(skip) < B                                  # the case decides something


def test_logits_not_stored_gives_the_same_decisions():
    h, w, masked, tokens = make(23, 2, 16, 512, 8192, 3.0, 0.25)
    m1, t1 = masked.clone(), tokens.clone()
    conf, n, logits = tt.lm_head_unmask(h, w, masked, tokens, 0.15, min_commit=True)
    conf2, n2, logits2 = tt.lm_head_unmask(h, w, m1, t1, 0.15, min_commit=True, keep_logits=True)
    torch.cuda.synchronize()
    assert logits is None and logits2 is not None
    assert torch.equal(masked, m1) and torch.equal(tokens, t1) and torch.equal(n, n2)
    # the two reduce the sums of exponentials in different orders (fp32 rounding)
    c, c2 = conf.cpu().numpy(), conf2.cpu().numpy()
    assert np.array_equal(np.isnan(c), np.isnan(c2))
    ok = ~np.isnan(c)
    assert np.all(np.abs(c[ok] - c2[ok]) <= CONF_RTOL * np.abs(c2[ok]))


def test_fully_committed_block_is_left_alone():
    h, w, masked, tokens = make(29, 2, 16, 256, 1024, 3.0, 1.1)   # every position committed
    assert not masked.any()
    t0 = tokens.clone()
    conf, n, _ = tt.lm_head_unmask(h, w, masked, tokens, 0.5, min_commit=True)
    torch.cuda.synchronize()
    assert torch.equal(tokens, t0) and not masked.any()
    assert torch.isnan(conf).all() and (n == 0).all()
