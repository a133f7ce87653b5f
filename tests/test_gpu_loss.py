"""GPU parity of the masked-diffusion training objective's two kernels.

Clean blocks are corrupted with [MASK] on a linear schedule and the denoiser minimizes the NLL of
the original tokens at the masked positions (Nemotron-TwoTower explainer, "Training und
Konditionierung"). The corruption is compared bit for bit with oracle/loss.py on the same uniform
draws (both compare the same fp32 values); the NLL is compared with the fp64 oracle on the same
fp32 logits (fp32 log-sum-exp: relative 1e-5 plus an absolute term for the cancellation
lse - x_target), the masked count exactly.
"""
import math

import numpy as np
import pytest
import torch

import synth
import two_tower_cross_amd as tt
from oracle import loss as oloss
from gpu_util import DEV

pytestmark = pytest.mark.gpu


def test_corruption_matches_the_oracle():
    r = synth.rng(80)
    B, S = 64, 16
    clean = r.integers(0, 131072, (B, S)).astype(np.int32)
    u_t = r.random(B).astype(np.float32)
    u_t[:3] = [0.0, 0.999999, 0.5]
    u_m = r.random((B, S)).astype(np.float32)
    u_m[2, 5] = 0.5                                    # equal to t: stays clean
    d = lambda x: torch.from_numpy(x).to(DEV)
    noisy, masked, t = tt.mask_corrupt(d(clean), d(u_t), d(u_m), mask_id=131071)
    torch.cuda.synchronize()
    rn, rm, rt = oloss.corrupt(clean, u_t, u_m, 131071)
    assert np.array_equal(noisy.cpu().numpy(), rn) and np.array_equal(masked.cpu().numpy(), rm)
    assert np.array_equal(t.cpu().numpy(), rt)
    assert masked[2, 5].item() == 0 and not masked[0].any()


@pytest.mark.parametrize("seed", range(84, 88))
def test_random_corruptions_match_the_oracle(seed):
    """Seeded random batch and block sizes (up to 300 positions), vocabularies and mask ids."""
    r = synth.rng(seed)
    B, S, V = int(r.integers(1, 65)), int(r.integers(1, 301)), int(r.integers(2, 200001))
    clean = r.integers(0, V - 1, (B, S)).astype(np.int32)
    u_t = r.random(B).astype(np.float32)
    u_m = r.random((B, S)).astype(np.float32)
    d = lambda x: torch.from_numpy(x).to(DEV)
    noisy, masked, t = tt.mask_corrupt(d(clean), d(u_t), d(u_m), mask_id=V - 1)
    torch.cuda.synchronize()
    rn, rm, rt = oloss.corrupt(clean, u_t, u_m, V - 1)
    assert np.array_equal(noisy.cpu().numpy(), rn) and np.array_equal(masked.cpu().numpy(), rm)
    assert np.array_equal(t.cpu().numpy(), rt)


CASES = [  # B, S, V, ld, sigma, masked fraction
    (8, 16, 131072, 131072, 2.0, 0.5),
    (3, 5, 1004, 1010, 4.0, 0.7),        # ragged vocabulary, padded rows
    (2, 100, 8192, 8192, 1.0, 0.3),      # more than 64 positions
    (4, 16, 4096, 4096, 3.0, 0.0),       # nothing masked
]


def _random_cases(seed, n):
    """Seeded random cases (the same every run): batch, block size up to 300, vocabulary and row
    padding, logit scale and masked fraction."""
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        V = int(g.integers(1, 60001))
        out.append((int(g.integers(1, 9)), int(g.integers(1, 301)), V, V + int(g.integers(0, 9)),
                    float(g.choice([0.5, 1.0, 2.0, 4.0])), float(g.choice([0.1, 0.5, 0.9, 1.0]))))
    return out


CASES += _random_cases(61, 5)


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}S{c[1]}V{c[2]}" for c in CASES])
def test_masked_nll_matches_the_oracle(case):
    B, S, V, ld, sigma, frac = case
    r = synth.rng(81 + V % 89)
    store = r.standard_normal((B, S, ld)).astype(np.float32) * sigma
    targets = r.integers(0, V, (B, S)).astype(np.int32)
    masked = (r.random((B, S)) < frac).astype(np.uint8)
    logits = torch.from_numpy(store).to(DEV)[..., :V]
    nll, mean, n = tt.masked_nll(logits, torch.from_numpy(targets).to(DEV),
                                 torch.from_numpy(masked).to(DEV))
    torch.cuda.synchronize()
    rn, rmean, rcount = oloss.masked_nll(store[..., :V], targets, masked)
    got = nll.cpu().numpy().astype(np.float64)
    assert int(n.item()) == rcount
    assert np.all(got[masked == 0] == 0)
    tol = 1e-5 * np.abs(rn) + 1e-5 * (math.log(V) + sigma)
    assert np.all(np.abs(got - rn) <= tol), float(np.abs(got - rn).max())
    assert abs(mean.item() - rmean) <= 1e-5 * abs(rmean) + 1e-5 * (math.log(V) + sigma)


def test_target_outside_the_vocabulary_gives_nan():
    logits = torch.zeros((1, 3, 512), device=DEV)
    targets = torch.tensor([[5, 512, -1]], dtype=torch.int32, device=DEV)
    masked = torch.ones((1, 3), dtype=torch.uint8, device=DEV)
    nll, mean, n = tt.masked_nll(logits, targets, masked)
    torch.cuda.synchronize()
    assert abs(nll[0, 0].item() - math.log(512)) < 1e-5
    assert math.isnan(nll[0, 1].item()) and math.isnan(nll[0, 2].item()) and n.item() == 3
