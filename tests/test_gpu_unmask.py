"""GPU parity of twotower_unmask against the fp64 oracle.

Definition checked: masked positions whose confidence (largest softmax probability) is above the
threshold are committed with their argmax token, the others stay masked (Nemotron-TwoTower
explainer, "Training und Konditionierung"). Committed ids and the mask must match bit for bit;
inputs are guarded so that no confidence lies within 1e-3 of the threshold and, where the
one-commit fallback fires, the two best confidences differ by more than 1e-3 relative.
"""
import math

import numpy as np
import pytest
import torch

import synth
import two_tower_cross_amd as tt
from oracle import unmask as ounmask
from gpu_util import DEV, guarded_logits

pytestmark = pytest.mark.gpu


def gpu_unmask(logits, masked, tokens, threshold, **kw):
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(DEV)
    m = torch.from_numpy(masked.astype(np.uint8)).to(DEV)
    t = torch.from_numpy(tokens.astype(np.int32)).to(DEV)
    conf, n = tt.unmask(lg, m, t, threshold, **kw)
    torch.cuda.synchronize()
    return t.cpu().numpy(), m.cpu().numpy(), conf.cpu().numpy().astype(np.float64), n.cpu().numpy()


def compare(logits, masked, tokens, threshold, **kw):
    gt, gm, gc, gn = gpu_unmask(logits, masked, tokens, threshold, **kw)
    ot, om, oc, on = ounmask.confidence_unmask(logits, masked, tokens, np.float32(threshold), **kw)
    np.testing.assert_array_equal(gm, om)
    np.testing.assert_array_equal(gt, ot)
    np.testing.assert_array_equal(gn, on)
    sel = masked.astype(bool)
    np.testing.assert_allclose(gc[sel], oc[sel], rtol=1e-5)
    return gt, gm, gc, gn


@pytest.mark.parametrize("min_commit", [False, True])
def test_tiny_config(min_commit):
    make = lambda s: synth.logits_normal(s, 1, 16, 1024, math.sqrt(3.0))
    x = guarded_logits(make, 0.9, 1, min_commit=min_commit)
    masked = np.ones((1, 16), np.uint8)
    compare(x, masked, np.full((1, 16), -1, np.int32), 0.9, min_commit=min_commit)


@pytest.mark.parametrize("threshold", [0.9, 0.8])
def test_ctx4k_planted_peaks(threshold):
    make = lambda s: synth.logits_planted(s, 1, 16, 131072, 2.0)
    x = guarded_logits(make, threshold, 2)
    masked = np.ones((1, 16), np.uint8)
    gt, gm, _, gn = compare(x, masked, np.full((1, 16), -1, np.int32), threshold)
    assert 0 < gn[0] < 16      # both sides of the threshold occur


def test_batch_with_partial_masks_and_fallback():
    B, S, V = 6, 16, 20000
    make = lambda s: synth.logits_planted(s, B, S, V, 2.0, 0.05, 0.95)
    g = synth.rng(8)
    masked = (g.random((B, S)) < 0.7).astype(np.uint8)
    masked[0] = 0                              # a finished sequence
    x = guarded_logits(make, 0.9, 7, min_commit=True, masked=masked)
    tokens = g.integers(0, V, size=(B, S)).astype(np.int32)
    x[masked == 0] = np.nan                    # committed rows must never be read
    compare(x, masked, tokens, 0.9, min_commit=True)
    compare(x, masked, tokens, 0.9, commit_all=True)


def test_constant_and_single_peak_rows():
    V = 4096
    x = np.zeros((1, 3, V), np.float32)
    a95 = math.log(0.95 * (V - 1) / 0.05)
    a85 = math.log(0.85 * (V - 1) / 0.15)
    x[0, 1, 77] = a95
    x[0, 2, 4000] = a85
    masked = np.ones((1, 3), np.uint8)
    gt, gm, gc, gn = compare(x, masked, np.full((1, 3), -1, np.int32), 0.9)
    np.testing.assert_allclose(gc[0], [1.0 / V, 0.95, 0.85], rtol=1e-5)
    assert gt[0, 0] == -1 and gt[0, 1] == 77 and gm[0].tolist() == [1, 0, 1]
    # the constant row: argmax is index 0 when committed
    gt, gm, _, _ = compare(x, masked, np.full((1, 3), -1, np.int32), 0.0)
    assert gt[0, 0] == 0


def test_fallback_ties_pick_lowest_position():
    V = 3000
    x = synth.logits_normal(9, 1, 8, V, 1.0)
    x[0, 5] = x[0, 2]           # identical rows -> identical confidences
    x[0, 2, 17] = x[0, 5, 17] = 30.0
    masked = np.ones((1, 8), np.uint8)
    gt, gm, _, gn = compare(x, masked, np.full((1, 8), -1, np.int32), 1.5, min_commit=True)
    assert gn[0] == 1 and gm[0, 2] == 0 and gm[0, 5] == 1 and gt[0, 2] == 17


def test_exact_ties_inside_a_row_pick_lowest_index():
    V = 50000
    x = synth.logits_normal(10, 1, 4, V, 1.0)
    for i, (a, b) in enumerate([(3, 40000), (9000, 9001), (8191, 8192), (0, 49999)]):
        x[0, i, a] = x[0, i, b] = 12.0
    gt, _, _, _ = compare(x, np.ones((1, 4), np.uint8), np.full((1, 4), -1, np.int32), 0.0)
    assert gt[0].tolist() == [3, 9000, 8191, 0]


def _random_vocab(seed, n):
    """Seeded random vocabulary sizes and row paddings (the same every run)."""
    g = np.random.default_rng(seed)
    return [(int(g.integers(1, 200001)), int(g.integers(0, 17))) for _ in range(n)]


@pytest.mark.parametrize("V,pad", [(1000, 0), (1003, 0), (8192, 4), (12345, 7), (1, 3)]
                         + _random_vocab(51, 5))
def test_vocab_sizes_and_row_strides(V, pad):
    B, S = 2, 5
    base = synth.logits_normal(11 + V, B, S, V + pad, 2.0)
    x = base[:, :, :V]
    masked = np.ones((B, S), np.uint8)
    masked[1, 3] = 0
    lg = torch.from_numpy(np.ascontiguousarray(base)).to(DEV)[:, :, :V]
    m = torch.from_numpy(masked).to(DEV)
    t = torch.full((B, S), -1, dtype=torch.int32, device=DEV)
    conf, n = tt.unmask(lg, m, t, 0.5, commit_all=True)
    torch.cuda.synchronize()
    ot, om, oc, on = ounmask.confidence_unmask(x, masked, np.full((B, S), -1, np.int32),
                                               np.float32(0.5), commit_all=True)
    np.testing.assert_array_equal(t.cpu().numpy(), ot)
    np.testing.assert_array_equal(m.cpu().numpy(), om)
    np.testing.assert_allclose(conf.cpu().numpy()[masked == 1], oc[masked == 1], rtol=1e-5)


@pytest.mark.parametrize("S", [65, 128, 256])
def test_blocks_larger_than_a_wavefront(S):
    """Block sizes 32 / 128 of the pages and up to 256: the decisions span several wavefronts."""
    B, V = 3, 4096
    make = lambda s: synth.logits_planted(s, B, S, V, 2.0, 0.05, 0.95)
    g = synth.rng(90 + S)
    masked = (g.random((B, S)) < 0.8).astype(np.uint8)
    x = guarded_logits(make, 0.9, 91 + S, min_commit=True, masked=masked)
    tokens = g.integers(0, V, size=(B, S)).astype(np.int32)
    compare(x, masked, tokens, 0.9, min_commit=True)
    # the fallback, with the best position in a later wavefront
    y = synth.logits_normal(95 + S, 1, S, V, 1.0)
    y[0, S - 3, 11] = 12.0
    compare(y, np.ones((1, S), np.uint8), np.full((1, S), -1, np.int32), 0.999, min_commit=True)
