"""GPU parity of the dense projections and of the denoise step / T-step block loop.

The generation loop checked: the block starts fully masked, each step rewrites the block's own
KV at every layer, attends to the resident context caches and commits confident tokens
(Nemotron-TwoTower explainer, "Generierungsprozess"). Stage-wise parity: each stage is compared
with the oracle fed the GPU's own inputs for that stage; the step is compared bit for bit with the
composition of the per-stage entry points; the loop is checked by its invariants.
"""
import math

import numpy as np
import pytest
import torch

import synth
import two_tower_cross_amd as tt
from oracle import attention as oattn, step as ostep, unmask as ounmask
from synth.device import loop_model
from gpu_util import DEV, TOL_BF16, max_abs

pytestmark = pytest.mark.gpu


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def bf16_ok(got, ref):
    """bf16 result of an fp32-accumulated product: one rounding (<= 2^-8 relative) plus slack."""
    err = np.abs(got - ref)
    return bool(np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-3)), float(err.max())


def small_model(seed=3, L=1000, layers=2, B=2, Hq=8, Hkv=2, D=128, hidden=512, V=8192):
    return loop_model(seed, B=B, S=16, L=L, layers=layers, Hq=Hq, Hkv=Hkv, D=D, hidden=hidden,
                      vocab=V, T=16, device=DEV)


def pack_reference(w):
    """The packed layout written out from its definition in include/twotower.h (numpy)."""
    N, K = w.shape
    nbk, ks = -(-N // 32), -(-K // 16)
    wp = np.zeros((nbk * 32, ks * 16), dtype=w.dtype)
    wp[:N, :K] = w
    # [nb, r, s, hh, e] -> [nb, s, hh, r, e]: lane = hh * 32 + r; one 1 KB unit per (nb, s)
    units = wp.reshape(nbk, 32, ks, 2, 8).transpose(0, 2, 3, 1, 4).reshape(nbk, ks, 512)
    # groups of 8 slabs, each group's units step-major: unit 8 gi ks + s gsize + nb % 8
    return np.concatenate([units[g:g + 8].transpose(1, 0, 2).reshape(-1)
                           for g in range(0, nbk, 8)])


@pytest.mark.parametrize("N,K", [(64, 64), (1004, 136), (4608, 2048), (37, 8), (300, 40)])
def test_pack_weight_matches_the_documented_layout(N, K):
    g = torch.Generator(device=DEV).manual_seed(15)
    w = torch.randn((N, K), generator=g, device=DEV).to(torch.bfloat16)
    pw = tt.pack_weight(w)
    torch.cuda.synchronize()
    got = pw.data.cpu().numpy().view(np.uint16)
    ref = pack_reference(w.cpu().view(torch.int16).numpy().view(np.uint16))
    assert got.shape == ref.shape and np.array_equal(got, ref)


@pytest.mark.parametrize("shape", [(2, 16, 512, 8, 2, 128), (8, 16, 2048, 32, 2, 128),
                                   (3, 5, 264, 4, 1, 64)])
def test_qkv_projection(shape):
    B, S, hidden, Hq, Hkv, D = shape
    g = torch.Generator(device=DEV).manual_seed(11)
    h = torch.randn((B, S, hidden), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn(((Hq + 2 * Hkv) * D, hidden), generator=g, device=DEV) / math.sqrt(hidden)).to(torch.bfloat16)
    q, kb, vb = tt.qkv_projection(h, w, Hq, Hkv, D)
    torch.cuda.synchronize()
    rq, rk, rv = ostep.qkv_projection(f64(h), f64(w), Hq, Hkv, D)
    for got, ref in ((q, rq), (kb, rk), (vb, rv)):
        ok, err = bf16_ok(f64(got), ref)
        assert ok, err


@pytest.mark.parametrize("rows,hidden,inf", [(32, 512, 1024), (128, 2048, 4096), (80, 264, 136)])
def test_out_projection(rows, hidden, inf):
    g = torch.Generator(device=DEV).manual_seed(12)
    h = torch.randn((rows, hidden), generator=g, device=DEV).to(torch.bfloat16)
    o = torch.randn((rows, inf), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((hidden, inf), generator=g, device=DEV) / math.sqrt(inf)).to(torch.bfloat16)
    out = tt.out_projection(h, o, w)
    torch.cuda.synchronize()
    ref = ostep.residual_output(f64(h)[:, None], f64(o).reshape(rows, 1, inf), f64(w))[:, 0]
    ok, err = bf16_ok(f64(out), ref)
    assert ok, err
    # in place (the residual stream of the step)
    h2 = h.clone()
    tt.out_projection(h2, o, w, out=h2)
    torch.cuda.synchronize()
    assert torch.equal(h2, out)


# (96: 3 slabs of 32 features in 64-feature tiles; 70000: 2188 slabs in 256-feature tiles: the last
# tile of each reaches past the packed weight and must read nothing there)
@pytest.mark.parametrize("rows,hidden,V", [(32, 512, 8192), (128, 2048, 131072), (7, 136, 1004),
                                           (5, 128, 96), (128, 256, 70000)])
def test_lm_head(rows, hidden, V):
    g = torch.Generator(device=DEV).manual_seed(13)
    h = torch.randn((rows, hidden), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((V, hidden), generator=g, device=DEV) / math.sqrt(hidden)).to(torch.bfloat16)
    logits = tt.lm_head(h, w)
    torch.cuda.synchronize()
    cols = np.sort(synth.rng(14).choice(V, size=min(V, 4096), replace=False))
    ref = ostep.lm_head(f64(h), f64(w[torch.from_numpy(cols).to(DEV)]))
    got = f64(logits)[:, cols]
    err = max_abs(got, ref)
    assert err <= 1e-4 + 1e-5 * np.abs(ref).max(), err


def compose_step(m, t, masked, tokens, threshold, min_commit, commit_all):
    """The step written out with the per-stage entry points."""
    h = m.h_steps[t]
    outs = {}
    for l in range(m.layers):
        q, kb, vb = tt.qkv_projection(h, m.w_qkv[l], m.Hq, m.Hkv, m.D)
        o = tt.block_attn(q, m.k_pages[l], m.v_pages[l], m.block_table, m.ctx_lens, kb, vb,
                          max_ctx_len=m.L, out_dtype=torch.bfloat16)
        outs[l] = (q, kb, vb, o, h)
        h = tt.out_projection(h, o, m.w_o[l])
    conf, n, logits = tt.lm_head_unmask(h, m.w_lm, masked, tokens, threshold,
                                        min_commit=min_commit, commit_all=commit_all,
                                        keep_logits=True)
    return h, logits, conf, n, outs


def make_step(m, **kw):
    return tt.DenoiseStep(k_pages=m.k_pages, v_pages=m.v_pages, w_qkv=m.w_qkv, w_o=m.w_o,
                          w_lm=m.w_lm, block_table=m.block_table, ctx_lens=m.ctx_lens,
                          max_ctx_len=m.L, num_q_heads=m.Hq, num_kv_heads=m.Hkv, head_dim=m.D,
                          batch=m.B, S=m.S, **kw)


def test_step_equals_composition_of_stages_bit_for_bit():
    m = small_model()
    step = make_step(m, keep_logits=True)
    masked = torch.ones((m.B, m.S), dtype=torch.uint8, device=DEV)
    tokens = torch.full((m.B, m.S), -1, dtype=torch.int32, device=DEV)
    masked2, tokens2 = masked.clone(), tokens.clone()
    conf, n = step(m.h_steps[0], masked, tokens, threshold=0.9, min_commit=True)
    h, logits, conf2, n2, _ = compose_step(m, 0, masked2, tokens2, 0.9, True, False)
    torch.cuda.synchronize()
    assert torch.equal(step.h_work, h)
    assert torch.equal(step.logits, logits)
    assert torch.equal(masked, masked2) and torch.equal(tokens, tokens2)
    assert torch.equal(n, n2)
    assert torch.equal(conf, conf2)


def test_step_stages_against_oracle():
    m = small_model(seed=4, L=777)
    masked = torch.ones((m.B, m.S), dtype=torch.uint8, device=DEV)
    tokens = torch.full((m.B, m.S), -1, dtype=torch.int32, device=DEV)
    m0 = masked.cpu().numpy().copy()
    t0 = tokens.cpu().numpy().copy()
    h, logits, conf, n, outs = compose_step(m, 0, masked, tokens, 0.9, True, False)
    torch.cuda.synchronize()
    for l, (q, kb, vb, o, hin) in outs.items():
        # projection stage on the GPU's own input
        rq, rk, rv = ostep.qkv_projection(f64(hin), f64(m.w_qkv[l]), m.Hq, m.Hkv, m.D)
        assert bf16_ok(f64(q), rq)[0] and bf16_ok(f64(kb), rk)[0] and bf16_ok(f64(vb), rv)[0]
        # attention stage on the GPU's own q / block KV
        ref, _ = oattn.block_attention(f64(q), f64(m.k_pages[l]), f64(m.v_pages[l]),
                                       m.block_table.cpu().numpy(), m.ctx_lens.cpu().numpy(),
                                       f64(kb), f64(vb), 1.0 / math.sqrt(m.D))
        ref16 = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
        assert max_abs(f64(o), ref16) <= TOL_BF16
    # lm-head on the GPU's final residual stream
    ref_logits = ostep.lm_head(f64(h), f64(m.w_lm))
    assert max_abs(f64(logits), ref_logits) <= 1e-4 + 1e-5 * np.abs(ref_logits).max()
    # unmasking on the GPU's logits: bit-exact where the fallback choice is not a near tie
    ot, om, oc, on = ounmask.confidence_unmask(logits.cpu().numpy(), m0, t0, np.float32(0.9),
                                               min_commit=True)
    gm, gt, gn = masked.cpu().numpy(), tokens.cpu().numpy(), n.cpu().numpy()
    for b in range(m.B):
        c = np.sort(oc[b])[::-1]
        if c[0] - c[1] >= 1e-4 * c[0]:
            assert np.array_equal(gm[b], om[b]) and np.array_equal(gt[b], ot[b]) and gn[b] == on[b]
        else:   # near tie: any best position is valid
            assert gn[b] == 1 and m0[b].sum() - gm[b].sum() == 1


def checksum(ts):
    return [int(t.view(torch.int16).to(torch.int64).sum().item()) for t in ts]


def run_block(m, step, threshold=0.9, count_slices=False):
    """One block of T steps. With count_slices every step writes its commit counts into its own
    row of a [T, B] tensor (as the benchmark does) instead of the step's own buffer."""
    masked = torch.ones((m.B, m.S), dtype=torch.uint8, device=DEV)
    tokens = torch.full((m.B, m.S), -1, dtype=torch.int32, device=DEV)
    counts = torch.full((m.T, m.B), -7, dtype=torch.int32, device=DEV)
    per_step, history = [], []
    for t in range(m.T):
        _, n = step(m.h_steps[t], masked, tokens, threshold=threshold, min_commit=True,
                    commit_all=(t == m.T - 1), n_committed=counts[t] if count_slices else None)
        per_step.append(n.clone())
        history.append(masked.clone())
    torch.cuda.synchronize()
    per_step = torch.stack(per_step).cpu().numpy()
    if count_slices:
        assert np.array_equal(per_step, counts.cpu().numpy())
    return masked, tokens, per_step, [h.cpu().numpy() for h in history]


def test_block_loop_invariants_small():
    m = small_model(seed=6)
    before = checksum(m.k_pages + m.v_pages)
    masked, tokens, per_step, hist = run_block(m, make_step(m))
    assert (per_step >= 1).all() and (per_step.sum(0) == m.S).all()
    assert not masked.any()
    t = tokens.cpu().numpy()
    assert ((t >= 0) & (t < m.vocab)).all()
    for a, b in zip(hist, hist[1:]):
        assert (b <= a).all()                  # a committed position never becomes masked again
    assert checksum(m.k_pages + m.v_pages) == before


def test_full_size_loop_32k_one_block():
    """6 layers, batch 8, context 32768, S = T = 16, vocab 131072: the benchmark's workload."""
    m = loop_model(5, device=DEV)
    step = make_step(m, keep_logits=True)
    before = checksum(m.k_pages[:1] + m.v_pages[-1:])
    masked, tokens, per_step, hist = run_block(m, step, count_slices=True)
    # near-uniform logits of a random model: exactly one commit per step per sequence
    assert (per_step == 1).all()
    assert not masked.any()
    t = tokens.cpu().numpy()
    assert ((t >= 0) & (t < m.vocab)).all()
    assert checksum(m.k_pages[:1] + m.v_pages[-1:]) == before
    # last layer's attention (its q and block KV are still in the step's buffers), sampled (b, g)
    l = m.layers - 1
    for b, g in ((0, 0), (5, 1)):
        heads = slice(g * 16, (g + 1) * 16)
        ref, _ = oattn.block_attention(
            f64(step.q[b:b + 1, :, heads]), f64(m.k_pages[l][b:b + 1, g:g + 1]),
            f64(m.v_pages[l][b:b + 1, g:g + 1]), np.zeros((1, 1), np.int32),
            np.array([m.L], np.int32), f64(step.k_blk[l][b:b + 1, g:g + 1]),
            f64(step.v_blk[l][b:b + 1, g:g + 1]), 1.0 / math.sqrt(m.D))
        ref16 = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
        assert max_abs(f64(step.attn_out[b:b + 1, :, heads]), ref16) <= TOL_BF16
    # lm-head on the final residual stream, sampled vocabulary columns
    cols = np.sort(synth.rng(15).choice(m.vocab, size=2048, replace=False))
    ref = ostep.lm_head(f64(step.h_work), f64(m.w_lm[torch.from_numpy(cols).to(DEV)]))
    got = f64(step.logits)[..., cols]
    assert max_abs(got, ref) <= 1e-4 + 1e-5 * np.abs(ref).max()


def test_full_size_loop_32k_as_benchmarked():
    """The benchmark's exact step (logits not kept: the persistent fused lm-head) commits the same
    tokens at the same steps as the step that keeps its logits (checked against the oracle
    above); the two differ only in the fp32 order of the sums of exponentials."""
    m = loop_model(5, device=DEV)
    _, tok_kept, per_kept, _ = run_block(m, make_step(m, keep_logits=True))
    masked, tok, per, _ = run_block(m, make_step(m), count_slices=True)
    assert not masked.any()
    assert np.array_equal(per, per_kept)
    assert torch.equal(tok, tok_kept)


@pytest.mark.parametrize("S", [32, 128])
def test_block_sizes_of_the_pages(S):
    """The block sizes the pages train and sample with besides 16 (32 in training, 128 at
    sampling): a block decodes to completion and the last layer's attention matches the oracle."""
    m = loop_model(9 + S, B=2, S=S, L=700, layers=2, Hq=8, Hkv=2, D=128, hidden=256, vocab=2048,
                   T=4, device=DEV)
    step = make_step(m)
    masked, tokens, per_step, _ = run_block(m, step)
    assert not masked.any() and (per_step >= 1).all() and (per_step.sum(0) == S).all()
    l = m.layers - 1
    for b, g in ((0, 0), (1, 1)):
        heads = slice(g * (m.Hq // m.Hkv), (g + 1) * (m.Hq // m.Hkv))
        ref, _ = oattn.block_attention(
            f64(step.q[b:b + 1, :, heads]), f64(m.k_pages[l][b:b + 1, g:g + 1]),
            f64(m.v_pages[l][b:b + 1, g:g + 1]), np.zeros((1, 1), np.int32),
            np.array([m.L], np.int32), f64(step.k_blk[l][b:b + 1, g:g + 1]),
            f64(step.v_blk[l][b:b + 1, g:g + 1]), 1.0 / math.sqrt(m.D))
        ref16 = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
        assert max_abs(f64(step.attn_out[b:b + 1, :, heads]), ref16) <= TOL_BF16
