"""GPU parity of the lm-head fused with the unmasking (twotower_lm_head_unmask).

Every masked position is predicted at once and the confident ones are committed (Nemotron-TwoTower
explainer, "Training und Konditionierung", sampling paragraph). The fused call reduces each
256-logit tile of a row to (max, first argmax, sum of exp) inside the product. The logits it
stores on request must match twotower_lm_head within fp32 rounding (the two calls may split K
differently), twotower_unmask run on those stored logits must take the same decisions with
confidences within fp32 rounding of the reordered sum, and the decisions must be those of the
oracle's unmasking of its own fp64 logits of the same bf16 inputs. The inputs are guarded as the
parity bar asks: on the oracle's fp64 logits no live confidence lies within 1e-3 of the threshold,
no row's top two token probabilities are within 1e-4 (relative) of each other, and where the
one-commit fallback fires the two best confidences differ by 1e-3 (relative); so no decision
depends on rounding and every sequence is checked.
"""
import functools
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
CONF_RTOL_F64 = 1e-4  # GPU (fp32 product and sums) against the oracle's fp64 logits
MARGIN = 1e-3        # every live confidence at least this far from the threshold
TOKEN_GAP = 1e-4     # top-1 / top-2 probability of a row differ by at least this (relative)
RIVAL_GAP = 1e-3     # where the fallback fires, the two best confidences differ by this (relative)


def _oracle_rows(h_rows, w64):
    """Row confidence, top-1 / top-2 relative probability gap of fp64 logits h W^T."""
    x = h_rows.astype(np.float64) @ w64.T
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    conf = 1.0 / e.sum(axis=1)
    top2 = np.partition(e, -2, axis=1)[:, -2] if x.shape[1] > 1 else np.zeros(len(x))
    return conf, 1.0 - top2          # e of the top token is 1


@functools.lru_cache(maxsize=None)
def _guarded(seed, B, S, hidden, V, sigma, committed_frac, gamma, min_commit, commit_all):
    """Host inputs guarded on the oracle's fp64 logits of the same bf16 values (rows redrawn until
    no decision lies near a tie), so the fused call's decisions are fixed by the definition."""
    r = synth.rng(seed)
    w = synth.round_to_bf16(r.standard_normal((V, hidden), dtype=np.float32)
                            * np.float32(sigma / math.sqrt(hidden)))
    w64 = w.astype(np.float64)
    masked = (r.random((B, S)) >= committed_frac).astype(np.uint8)
    h = synth.round_to_bf16(r.standard_normal((B, S, hidden), dtype=np.float32))
    conf = np.zeros((B, S))
    gap = np.ones((B, S))
    todo = np.ones((B, S), bool)
    for _ in range(64):
        c, gp = _oracle_rows(h[todo], w64)
        conf[todo], gap[todo] = c, gp
        live = masked.astype(bool)
        bad = live & (gap < TOKEN_GAP)
        if not commit_all:
            bad |= live & (np.abs(conf - np.float64(np.float32(gamma))) < MARGIN)
            if min_commit:
                for b in range(B):
                    cb = np.where(live[b], conf[b], -1.0)
                    if live[b].sum() > 1 and not np.any(cb > gamma):
                        top = np.sort(cb)[::-1]
                        if top[0] - top[1] < RIVAL_GAP * top[0]:
                            bad[b, int(np.argmax(cb))] = True
        if not bad.any():
            ref64 = (h.reshape(B * S, hidden).astype(np.float64) @ w64.T).reshape(B, S, V)
            return h, w, masked, ref64
        h[bad] = synth.round_to_bf16(r.standard_normal((int(bad.sum()), hidden), dtype=np.float32))
        todo = bad
    raise RuntimeError("could not guard the inputs")


def make(*key):
    """Fresh device tensors (hidden, packed weight, masked, tokens) of the guarded inputs, and the
    oracle's fp64 logits of the same bf16 values."""
    h, w, masked, ref64 = _guarded(*key)
    tokens = np.where(masked == 0, 7, -1).astype(np.int32)
    to = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dt)
    return (to(h, torch.bfloat16), tt.pack_weight(to(w, torch.bfloat16)), to(masked, torch.uint8),
            to(tokens, torch.int32), ref64)


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


def _random_cases(seed, n):
    """Seeded random cases within the documented limits (the same every run)."""
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        out.append((int(g.integers(1, 9)), int(g.choice([1, 5, 16, 33, 64, 100])),
                    8 * int(g.integers(8, 65)), 4 * int(g.integers(25, 5001)),
                    float(g.choice([2.0, 3.0, 4.0, 5.0])),
                    float(g.choice([0.05, 0.1, 0.2, 0.3, 0.5, 0.9])),
                    float(g.choice([0.0, 0.2, 0.5])), bool(g.random() < 0.8),
                    bool(g.random() < 0.15)))
    return out


CASES += _random_cases(41, 6)


@pytest.mark.parametrize("keep", [True, False], ids=["logits", "no-logits"])
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}S{c[1]}V{c[3]}" for c in CASES])
def test_fused_matches_two_call_path_and_oracle(case, keep):
    """keep: the call also stores the logits (and unmask runs on them); else the logits come from
    a second, storing call (the same products in the same order, so the same fp32 values). On the
    guarded inputs every sequence's decisions are those of the oracle on its own fp64 logits."""
    B, S, hidden, V, sigma, gamma, frac, min_commit, commit_all = case
    h, w, masked, tokens, ref64 = make(17 + V % 97, B, S, hidden, V, sigma, frac, gamma,
                                       min_commit, commit_all)
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
    assert np.array_equal(gm, rm) and np.array_equal(gt, rt) and np.array_equal(gn, rn)
    assert np.array_equal(gt[~live], t0[~live]) and np.all(gm[~live] == 0)

    # the oracle's unmasking of its own fp64 logits of the same bf16 inputs: every sequence
    ot, om, oc, on = ounmask.confidence_unmask(ref64, m0, t0, np.float32(gamma),
                                               min_commit=min_commit, commit_all=commit_all)
    assert np.all(np.abs(c[live] - oc[live]) <= CONF_RTOL_F64 * oc[live])
    assert np.array_equal(gm, om) and np.array_equal(gt, ot) and np.array_equal(gn, on)


def test_logits_not_stored_gives_the_same_decisions():
    h, w, masked, tokens, _ = make(23, 2, 16, 512, 8192, 3.0, 0.25, 0.15, True, False)
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
    h, w, masked, tokens, _ = make(29, 2, 16, 256, 1024, 3.0, 1.1, 0.5, True, False)  # all committed
    assert not masked.any()
    t0 = tokens.clone()
    conf, n, _ = tt.lm_head_unmask(h, w, masked, tokens, 0.5, min_commit=True)
    torch.cuda.synchronize()
    assert torch.equal(tokens, t0) and not masked.any()
    assert torch.isnan(conf).all() and (n == 0).all()
