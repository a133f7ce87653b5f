"""Pins of the CPU oracle against closed forms, invariants, brute force and library routines.

None of these compares the oracle with itself: each check is a fact fixed by the definition of
the denoiser's block attention (one softmax over the context tower's same-layer KV and the block's
own KV; Nemotron-TwoTower explainer, sections "Architektur" / "Generierungsprozess") or of
confidence unmasking (explainer, section "Training und Konditionierung"), chosen so that a dropped
term, a wrong sign, a wrong index or a transposed operand in the oracle fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

import synth
from oracle import attention, bruteforce, cache, loss, step, unmask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_case(seed=0, B=2, S=3, Hq=4, Hkv=2, D=5, lens=(7, 4), page_size=3, **kw):
    return synth.attn_case(seed, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, ctx_lens=list(lens),
                           page_size=page_size, dtype="fp32", **kw)


def run(case, **over):
    args = dict(q=case.q, k_pages=case.k_pages, v_pages=case.v_pages, block_table=case.block_table,
                ctx_lens=case.ctx_lens, k_blk=case.k_blk, v_blk=case.v_blk, scale=case.scale)
    args.update(over)
    return attention.block_attention(**args)


def all_values(case, b, g):
    """Context values (token-major) followed by the block values, float64 [L+S, D]."""
    _, vc = attention.gather_context(case.k_pages, case.v_pages, case.block_table,
                                     case.ctx_lens[b], b, g)
    return np.concatenate([vc, case.v_blk[b, g].T.astype(np.float64)], axis=0)


# ------------------------------------------------------------------------------- attention pins

def test_identical_keys_give_mean_of_values():
    c = small_case(1)
    c.k_pages[...] = 0.37
    c.k_blk[...] = 0.37
    out, lse = run(c)
    G = c.Hq // c.Hkv
    for b in range(c.B):
        for h in range(c.Hq):
            mean = all_values(c, b, h // G).mean(axis=0)
            np.testing.assert_allclose(out[b, :, h, :], np.broadcast_to(mean, (c.S, c.D)),
                                       rtol=0, atol=1e-12)


def test_single_key_returns_its_value():
    # one context key, no block keys
    c = small_case(2, B=1, lens=(1,), S=2)
    out, lse = run(c, k_blk=c.k_blk[:, :, :0], v_blk=c.v_blk[:, :, :, :0])
    G = c.Hq // c.Hkv
    for h in range(c.Hq):
        v = synth.untile_v(c.v_pages)[c.block_table[0, 0], h // G, :, 0]
        np.testing.assert_allclose(out[0, :, h, :], np.broadcast_to(v, (2, c.D)), atol=1e-15)
    # empty context, one block key
    c = small_case(3, B=1, lens=(0,), S=1)
    out, _ = run(c)
    for h in range(c.Hq):
        np.testing.assert_allclose(out[0, 0, h, :], c.v_blk[0, h // G, :, 0], atol=1e-15)


def test_zero_query_gives_mean_and_log_count():
    c = small_case(4)
    c.q[...] = 0.0
    out, lse = run(c)
    G = c.Hq // c.Hkv
    for b in range(c.B):
        n = int(c.ctx_lens[b]) + c.S
        np.testing.assert_allclose(lse[b], math.log(n), atol=1e-13)
        for h in range(c.Hq):
            np.testing.assert_allclose(out[b, 0, h], all_values(c, b, h // G).mean(axis=0),
                                       atol=1e-13)


def test_permutation_invariance_block_context_and_pages():
    c = small_case(5, lens=(9, 6), page_size=2)
    ref, ref_lse = run(c)
    g = synth.rng(99)
    # permute block rows (K and V together)
    perm = g.permutation(c.S)
    out, lse = run(c, k_blk=c.k_blk[:, :, perm, :], v_blk=c.v_blk[:, :, :, perm])
    np.testing.assert_allclose(out, ref, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, atol=1e-13)
    # permute the order of pages in the pool, remapping the block table
    pool_perm = g.permutation(c.k_pages.shape[0])
    inv = np.argsort(pool_perm)
    out, _ = run(c, k_pages=c.k_pages[pool_perm], v_pages=c.v_pages[pool_perm],
                 block_table=inv[c.block_table].astype(np.int32))
    np.testing.assert_allclose(out, ref, atol=1e-13)
    # permute context rows: rebuild a contiguous context with shuffled token order
    B, Hkv, D = c.B, c.Hkv, c.D
    Lmax = int(c.ctx_lens.max())
    kp = np.zeros((B, Hkv, Lmax, D), np.float32)
    vp = np.zeros((B, Hkv, D, Lmax), np.float32)       # dim-major, tiled below
    for b in range(B):
        L = int(c.ctx_lens[b])
        p = g.permutation(L)
        for h in range(Hkv):
            kc, vc = attention.gather_context(c.k_pages, c.v_pages, c.block_table, L, b, h)
            kp[b, h, :L] = kc[p]
            vp[b, h, :, :L] = vc[p].T
    out, _ = run(c, k_pages=synth.tile_k(kp), v_pages=synth.tile_v(vp),
                 block_table=np.arange(B, dtype=np.int32)[:, None])
    np.testing.assert_allclose(out, ref, atol=1e-13)


def test_matches_pure_python_bruteforce():
    for seed in range(4):
        g = synth.rng(100 + seed)
        B, S, Hkv = 2, int(g.integers(1, 5)), int(g.integers(1, 3))
        Hq = Hkv * int(g.integers(1, 3))
        D = int(g.integers(1, 9))
        lens = [int(x) for x in g.integers(0, 9, size=B)]
        c = small_case(seed, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, lens=lens, page_size=3)
        out, _ = run(c)
        ctx_k, ctx_v = [], []
        for b in range(B):
            kk, vv = [], []
            for h in range(Hkv):
                kc, vc = attention.gather_context(c.k_pages, c.v_pages, c.block_table,
                                                  c.ctx_lens[b], b, h)
                kk.append(kc.tolist()); vv.append(vc.tolist())
            ctx_k.append(kk); ctx_v.append(vv)
        blk_v = c.v_blk.transpose(0, 1, 3, 2)
        bf = bruteforce.block_attention(c.q.astype(np.float64).tolist(), ctx_k, ctx_v,
                                        c.k_blk.astype(np.float64).tolist(),
                                        blk_v.astype(np.float64).tolist(), c.scale)
        np.testing.assert_allclose(out, np.array(bf), rtol=0, atol=1e-12)


def test_key_shift_invariance():
    c = small_case(6)
    ref, _ = run(c)
    u = synth.rng(7).standard_normal((c.Hkv, c.D)).astype(np.float32)
    kp = synth.tile_k(synth.untile_k(c.k_pages) + u[None, :, None, :])
    kb = c.k_blk + u[None, :, None, :]
    out, _ = run(c, k_pages=kp, k_blk=kb)
    np.testing.assert_allclose(out, ref, atol=1e-6)


def test_lse_merge_identity():
    """attn over A u B equals the LSE-weighted merge of attn over A and attn over B."""
    c = small_case(8, lens=(10, 7), page_size=4)
    full, full_lse = run(c)
    # A: context only (no block keys); B: block only (empty context)
    oa, la = run(c, k_blk=c.k_blk[:, :, :0], v_blk=c.v_blk[:, :, :, :0])
    ob, lb = run(c, ctx_lens=np.zeros_like(c.ctx_lens))
    la_t, lb_t = la.transpose(0, 2, 1)[..., None], lb.transpose(0, 2, 1)[..., None]  # [B,S,Hq,1]
    m = np.maximum(la_t, lb_t)
    wa, wb = np.exp(la_t - m), np.exp(lb_t - m)
    merged = (wa * oa + wb * ob) / (wa + wb)
    np.testing.assert_allclose(merged, full, atol=1e-12)
    np.testing.assert_allclose((m + np.log(wa + wb))[..., 0].transpose(0, 2, 1), full_lse,
                               atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    c = small_case(9, Hq=6, Hkv=2)
    G = 3
    out, lse = run(c)
    rep = lambda x: np.repeat(x, G, axis=1)  # KV head g serves query heads g*G .. g*G+G-1
    out2, lse2 = run(c, k_pages=rep(c.k_pages), v_pages=rep(c.v_pages), k_blk=rep(c.k_blk),
                     v_blk=rep(c.v_blk))
    np.testing.assert_allclose(out, out2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)


def test_affine_values():
    c = small_case(10)
    ref, _ = run(c)
    alpha = -1.75
    beta = synth.rng(11).standard_normal(c.D).astype(np.float32)
    vp = alpha * c.v_pages + beta[None, None, None, None, :, None]
    vb = alpha * c.v_blk + beta[None, None, :, None]
    out, _ = run(c, v_pages=vp.astype(np.float32), v_blk=vb.astype(np.float32))
    np.testing.assert_allclose(out, alpha * ref + beta, atol=1e-5)


def test_matches_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    c = small_case(12, B=2, S=4, Hq=6, Hkv=3, D=8, lens=(11, 5), page_size=4)
    out, _ = run(c)
    G = c.Hq // c.Hkv
    for b in range(c.B):
        keys, vals = [], []
        for g in range(c.Hkv):
            kc, vc = attention.gather_context(c.k_pages, c.v_pages, c.block_table,
                                              c.ctx_lens[b], b, g)
            keys.append(np.concatenate([kc, c.k_blk[b, g]], 0))
            vals.append(np.concatenate([vc, c.v_blk[b, g].T], 0))
        K = torch.tensor(np.stack(keys)).repeat_interleave(G, 0)        # [Hq, N, D]
        V = torch.tensor(np.stack(vals)).repeat_interleave(G, 0)
        Q = torch.tensor(c.q[b].astype(np.float64)).permute(1, 0, 2)    # [Hq, S, D]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=c.scale)
        np.testing.assert_allclose(out[b], ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_tile_layout_addresses():
    """Element (o, d) of a 128-token page sits at [page, g, o // 64, d // 8, o % 64, d % 8] of the
    K pages and at [page, g, o // 64, (o % 64) // 8, d, o % 8] of the V pages."""
    c = small_case(14, B=1, Hq=2, Hkv=1, D=16, lens=(150,), page_size=128)
    L = 150
    kc, vc = attention.gather_context(c.k_pages, c.v_pages, c.block_table, L, 0, 0)
    for t in (0, 7, 8, 63, 64, 127, 128, 149):
        page, o = c.block_table[0, t // 128], t % 128
        for d in (0, 7, 8, 15):
            assert kc[t, d] == c.k_pages[page, 0, o // 64, d // 8, o % 64, d % 8]
            assert vc[t, d] == c.v_pages[page, 0, o // 64, (o % 64) // 8, d, o % 8]
    dm = synth.rng(1).standard_normal((2, 3, 5, 192))
    tv = synth.tile_v(dm)
    assert tv.shape == (2, 3, 3, 8, 5, 8)
    assert tv[1, 2, 2, 3, 4, 7] == dm[1, 2, 4, 2 * 64 + 3 * 8 + 7]
    np.testing.assert_array_equal(synth.untile_v(tv), dm)
    tm = synth.rng(2).standard_normal((2, 3, 192, 24))
    tk = synth.tile_k(tm)
    assert tk.shape == (2, 3, 3, 3, 64, 8)
    assert tk[1, 2, 2, 1, 5, 6] == tm[1, 2, 2 * 64 + 5, 8 + 6]
    np.testing.assert_array_equal(synth.untile_k(tk), tm)


def test_paged_layout_equals_contiguous():
    base = small_case(13, lens=(13, 8), page_size=5)
    ref, _ = run(base)
    for ps in (1, 2, 16):
        c = small_case(13, lens=(13, 8), page_size=ps)
        out, _ = run(c)
        np.testing.assert_allclose(out, ref, atol=1e-13)


def test_golden_attention_closed_form():
    rows = {}
    with open(os.path.join(GOLDEN, "attention_closed_form.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(None, 1)
                rows[k] = v
    q = np.array(rows["q"].split(), float).reshape(1, 1, 1, 2)
    w = [float(x) for x in rows["ctx_key_weights"].split()]
    sec = [float(x) for x in rows["ctx_key_second"].split()]
    vals = [[float(x) for x in part.split()] for part in rows["ctx_values"].split("|")]
    L = len(w)
    k_pages = np.zeros((L, 1, 1, 1, 1, 2)); v_pages = np.zeros((L, 1, 1, 1, 2, 1))   # 1-token pages
    order = [1, 0]  # token 0 in pool page 1, token 1 in pool page 0
    for t in range(L):
        k_pages[order[t], 0, 0, 0, 0] = [math.log(w[t]), sec[t]]
        v_pages[order[t], 0, 0, 0, :, 0] = vals[t]
    bw = float(rows["blk_key_weights"]); bs = float(rows["blk_key_second"])
    k_blk = np.array([math.log(bw), bs]).reshape(1, 1, 1, 2)
    v_blk = np.array([float(x) for x in rows["blk_values"].split()]).reshape(1, 1, 2, 1)
    out, lse = attention.block_attention(q, k_pages, v_pages, np.array([order], np.int32),
                                         np.array([L], np.int32), k_blk, v_blk, 1.0)
    np.testing.assert_allclose(out[0, 0, 0], [float(x) for x in rows["expect_out"].split()],
                               atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 0], math.log(float(rows["expect_lse_exp"])), atol=1e-15)


# ---------------------------------------------------------------------------------- unmask pins

def test_constant_row_confidence_is_one_over_vocab():
    V = 1000
    logits = np.full((1, 2, V), 3.25, np.float32)
    t, m, c, n = unmask.confidence_unmask(logits, np.ones((1, 2), np.uint8),
                                          np.full((1, 2), -1, np.int32), 0.5)
    np.testing.assert_allclose(c, 1.0 / V, rtol=1e-14)
    assert n[0] == 0 and m.all()
    k, conf = unmask.row_confidence(logits[0, 0])
    assert k == 0


@pytest.mark.parametrize("target", [0.95, 0.85])
def test_single_peak_closed_form(target):
    V = 4096
    a = math.log(target * (V - 1) / (1 - target))        # e^a / (e^a + V - 1) = target
    logits = np.zeros((1, 1, V), np.float64)
    logits[0, 0, 1234] = a
    t, m, c, n = unmask.confidence_unmask(logits, np.ones((1, 1), np.uint8),
                                          np.full((1, 1), -1, np.int32), 0.9)
    np.testing.assert_allclose(c[0, 0], math.exp(a) / (math.exp(a) + V - 1), rtol=1e-13)
    np.testing.assert_allclose(c[0, 0], target, rtol=1e-12)
    assert (n[0] == 1) == (target > 0.9)
    if target > 0.9:
        assert t[0, 0] == 1234 and m[0, 0] == 0


def test_commits_monotone_in_threshold():
    logits = synth.logits_planted(21, 3, 16, 2048, 2.0)
    masked = (synth.rng(22).random((3, 16)) < 0.8).astype(np.uint8)
    tok = np.full((3, 16), -1, np.int32)
    prev = None
    for gamma in (0.2, 0.5, 0.8, 0.9, 0.95, 0.99):
        _, m, _, _ = unmask.confidence_unmask(logits, masked, tok, gamma)
        committed = (masked == 1) & (m == 0)
        if prev is not None:
            assert np.all(committed <= prev)
        prev = committed


def test_extreme_thresholds():
    V = 512
    logits = synth.logits_normal(23, 2, 8, V, 1.0)
    masked = np.ones((2, 8), np.uint8)
    tok = np.full((2, 8), -1, np.int32)
    _, m, _, n = unmask.confidence_unmask(logits, masked, tok, 1.0)
    assert m.all() and (n == 0).all()
    _, m, _, n = unmask.confidence_unmask(logits, masked, tok, 0.999 / V)
    assert not m.any() and (n == 8).all()


def test_committed_rows_untouched_and_counts():
    logits = synth.logits_planted(24, 4, 16, 1024, 2.0)
    g = synth.rng(25)
    masked = (g.random((4, 16)) < 0.6).astype(np.uint8)
    tok = g.integers(0, 1024, size=(4, 16)).astype(np.int32)
    logits[masked == 0] = np.nan   # committed rows must not be read
    t, m, c, n = unmask.confidence_unmask(logits, masked, tok, 0.7, min_commit=True)
    assert np.all(t[masked == 0] == tok[masked == 0])
    assert np.all(m[masked == 0] == 0)
    assert np.all(np.isnan(c[masked == 0]))
    np.testing.assert_array_equal(n, masked.sum(1) - m.sum(1))
    assert np.all(m <= masked)


def test_min_commit_takes_best_and_lowest_position_on_ties():
    V = 64
    logits = np.zeros((1, 4, V), np.float32)
    logits[0, 1, 5] = 2.0
    logits[0, 3, 7] = 2.0       # same confidence as position 1
    logits[0, 2, 9] = 1.0
    masked = np.ones((1, 4), np.uint8)
    t, m, _, n = unmask.confidence_unmask(logits, masked, np.full((1, 4), -1, np.int32), 0.9,
                                          min_commit=True)
    assert n[0] == 1 and m[0].tolist() == [1, 0, 1, 1] and t[0, 1] == 5
    # nothing masked: the fallback does nothing
    t, m, _, n = unmask.confidence_unmask(logits, np.zeros((1, 4), np.uint8),
                                          np.zeros((1, 4), np.int32), 0.9, min_commit=True)
    assert n[0] == 0


def test_matches_torch_softmax_argmax():
    torch = pytest.importorskip("torch")
    logits = synth.logits_planted(26, 2, 16, 4096, 2.0)
    masked = np.ones((2, 16), np.uint8)
    t, _, c, _ = unmask.confidence_unmask(logits, masked, np.full((2, 16), -1, np.int32), 0.9,
                                          commit_all=True)
    x = torch.tensor(logits.astype(np.float64))
    p = torch.softmax(x, dim=-1)
    np.testing.assert_allclose(c, p.max(-1).values.numpy(), rtol=1e-12)
    np.testing.assert_array_equal(t, x.argmax(-1).numpy())


def test_confidence_matches_bruteforce():
    g = synth.rng(27)
    for _ in range(20):
        row = (g.standard_normal(50) * 3).tolist()
        if g.random() < 0.3:
            row[7] = row[31] = max(row) + 1.0        # exact tie: first index wins
        k1, c1 = unmask.row_confidence(row)
        k2, c2 = bruteforce.confidence(row)
        assert k1 == k2
        assert abs(c1 - c2) <= 1e-14


def test_golden_unmask_closed_form():
    rows, cases = [], []
    with open(os.path.join(GOLDEN, "unmask_closed_form.txt")) as f:
        for line in f:
            line = line.strip()
            if line.startswith("row "):
                w, tk, cf = line[4:].split("|")
                num, den = cf.split()[1].split("/")
                rows.append(([math.log(float(x)) for x in w.split()], int(tk.split()[1]),
                             float(num) / float(den)))
            elif line.startswith("case "):
                lhs, rhs = line[5:].split("->")
                gamma, mc, ca = lhs.split()
                cases.append((float(gamma), bool(int(mc)), bool(int(ca)),
                              [int(x) for x in rhs.split()]))
    logits = np.array([[r[0] for r in rows]])
    S = len(rows)
    for gamma, mc, ca, expect in cases:
        t, m, c, n = unmask.confidence_unmask(logits, np.ones((1, S), np.uint8),
                                              np.full((1, S), -1, np.int32), gamma, mc, ca)
        assert sorted(np.nonzero(m[0] == 0)[0].tolist()) == expect, (gamma, mc, ca)
        for i in expect:
            assert t[0, i] == rows[i][1]
        np.testing.assert_allclose(c[0], [r[2] for r in rows], rtol=1e-14)
        assert n[0] == len(expect)


# ------------------------------------------------------------------------------------ step pins

def test_linear_matches_explicit_loop():
    g = synth.rng(30)
    x = g.standard_normal((2, 3, 5))
    w = g.standard_normal((4, 5))
    y = step.linear(x, w)
    for a in range(2):
        for b in range(3):
            for o in range(4):
                assert abs(y[a, b, o] - math.fsum(x[a, b, i] * w[o, i] for i in range(5))) < 1e-12


def test_qkv_projection_column_order():
    Hq, Hkv, D = 4, 2, 3
    hidden = (Hq + 2 * Hkv) * D
    h = synth.rng(31).standard_normal((2, 5, hidden))
    q, k, v = step.qkv_projection(h, np.eye(hidden), Hq, Hkv, D)
    for b in range(2):
        for i in range(5):
            for hh in range(Hq):
                np.testing.assert_array_equal(q[b, i, hh], h[b, i, hh * D:(hh + 1) * D])
            for g in range(Hkv):
                np.testing.assert_array_equal(k[b, g, i], h[b, i, (Hq + g) * D:(Hq + g + 1) * D])
                for d in range(D):
                    assert v[b, g, d, i] == h[b, i, (Hq + Hkv + g) * D + d]


def test_residual_output():
    g = synth.rng(32)
    h = g.standard_normal((2, 3, 6))
    o = g.standard_normal((2, 3, 2, 4))
    np.testing.assert_array_equal(step.residual_output(h, o, np.zeros((6, 8))), h)
    w = g.standard_normal((6, 8))
    r = step.residual_output(h, o, w)
    for b in range(2):
        for i in range(3):
            flat = o[b, i].reshape(-1)
            for c in range(6):
                assert abs(r[b, i, c] - h[b, i, c] - math.fsum(flat * w[c])) < 1e-12


def _tiny_model(seed, B=2, S=4, Hq=4, Hkv=2, D=8, hidden=16, V=50, L=9, layers=2):
    g = synth.rng(seed)
    case = small_case(seed, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, lens=[L] * B, page_size=4)
    lay = []
    for _ in range(layers):
        c = small_case(int(g.integers(1 << 20)), B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, lens=[L] * B,
                       page_size=4, shuffle_pages=False)
        w_qkv = g.standard_normal(((Hq + 2 * Hkv) * D, hidden)) / math.sqrt(hidden)
        w_o = g.standard_normal((hidden, Hq * D)) / math.sqrt(Hq * D)
        lay.append((w_qkv, w_o, c.k_pages, c.v_pages, c.block_table))
    w_lm = g.standard_normal((V, hidden)) / math.sqrt(hidden)
    return case, lay, w_lm


def test_block_loop_finishes_and_keeps_context_read_only():
    B, S, T = 2, 4, 4
    case, lay, w_lm = _tiny_model(33, B=B, S=S)
    # all layers share one page table in this synthetic model
    bt = lay[0][4]
    layers = [(a, b, c, d) for a, b, c, d, _ in lay]
    for l in lay:
        assert np.array_equal(l[4], bt)
    before = [(c.copy(), d.copy()) for _, _, c, d in layers]
    g = synth.rng(34)
    hs = [g.standard_normal((B, S, 16)) for _ in range(T)]
    tokens, per_step = step.block_loop(hs, layers, bt, case.ctx_lens, w_lm, Hq=4, Hkv=2, D=8,
                                       scale=1 / math.sqrt(8), threshold=0.9, min_commit=True)
    assert np.all(per_step.sum(0) == S)
    assert np.all(per_step >= 1)
    assert np.all((tokens >= 0) & (tokens < 50))
    for (c0, d0), (_, _, c1, d1) in zip(before, layers):
        assert np.array_equal(c0, c1, equal_nan=True) and np.array_equal(d0, d1, equal_nan=True)


def test_denoise_step_matches_stagewise_composition():
    B, S = 2, 4
    case, lay, w_lm = _tiny_model(35, B=B, S=S)
    bt = lay[0][4]
    layers = [(a, b, c, d) for a, b, c, d, _ in lay]
    h0 = synth.rng(36).standard_normal((B, S, 16))
    masked = np.ones((B, S), np.uint8)
    tok = np.full((B, S), -1, np.int32)
    t, m, c, n, logits = step.denoise_step(h0, layers, bt, case.ctx_lens, w_lm, masked, tok,
                                           Hq=4, Hkv=2, D=8, scale=0.35, threshold=0.05)
    # the same chain written out with the pages' stages, checked against brute force attention
    h = h0.copy()
    for w_qkv, w_o, kp, vp in layers:
        q, kb, vb = step.qkv_projection(h, w_qkv, 4, 2, 8)
        o = np.zeros((B, S, 4, 8))
        for b in range(B):
            for hh in range(4):
                kc, vc = attention.gather_context(kp, vp, bt, case.ctx_lens[b], b, hh // 2)
                keys = np.concatenate([kc, kb[b, hh // 2]]).tolist()
                vals = np.concatenate([vc, vb[b, hh // 2].T]).tolist()
                for i in range(S):
                    o[b, i, hh] = bruteforce.attend(q[b, i, hh].tolist(), keys, vals, 0.35)
        h = h + o.reshape(B, S, -1) @ w_o.T
    np.testing.assert_allclose(logits, h @ w_lm.T, atol=1e-10)


# ------------------------------------------------------------------------------ generator pins

def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = synth.rng(40).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 65504.0]   # ties to even
    r = synth.round_to_bf16(x)
    t = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(r, t)
    np.testing.assert_array_equal(synth.bits_to_f32(synth.bf16_bits(r)), r)


def test_paged_generator_places_tokens_where_the_table_says():
    c = synth.attn_case(41, B=3, S=2, Hq=2, Hkv=1, D=4, ctx_lens=[5, 0, 9], page_size=2,
                        dtype="fp32", spare_frac=0.5, nan_poison=True)
    used = set()
    for b in range(3):
        L = int(c.ctx_lens[b])
        for p in range(-(-L // 2)):
            used.add(int(c.block_table[b, p]))
        kc, vc = attention.gather_context(c.k_pages, c.v_pages, c.block_table, L, b, 0)
        assert not np.isnan(kc).any() and not np.isnan(vc).any()
    assert len(used) == sum(-(-int(L) // 2) for L in c.ctx_lens)
    spare = [p for p in range(c.k_pages.shape[0]) if p not in used]
    assert spare and all(np.isnan(c.k_pages[p]).all() for p in spare)
    # tail of the last page of sequence 0 (length 5, page 2) is poisoned
    assert np.isnan(synth.untile_k(c.k_pages)[c.block_table[0, 2], 0, 1]).all()


# ------------------------------------------------------------------------------ cache append

def _paged_cache(seed, pool, Hkv, page, D, layers=2):
    r = synth.rng(seed)
    T, CK, CV = synth.tile_widths(page, D)
    k = [r.standard_normal((pool, Hkv, page // T, D // CK, T, CK)) for _ in range(layers)]
    v = [r.standard_normal((pool, Hkv, page // T, T // CV, D, CV)) for _ in range(layers)]
    return k, v


def test_append_extends_every_gathered_context_by_the_block_rows():
    """Independent of the page bookkeeping: reading the cache back through the new table gives the
    old context followed by the block rows (K row-major, V transposed from [D, S])."""
    B, Hkv, D, S, page = 3, 2, 8, 16, 64
    k, v = _paged_cache(50, 12, Hkv, page, D)
    lens = np.array([60, 128, 0], np.int32)
    table = np.full((B, 4), -1, np.int32)
    table[0, 0], table[1, :2] = 3, [5, 7]
    free = np.array([0, 1, 2, 4, 6, 8, 9, 10, 11], np.int32)
    r = synth.rng(51)
    kn = [r.standard_normal((B, Hkv, S, D)) for _ in range(2)]
    vn = [r.standard_normal((B, Hkv, D, S)) for _ in range(2)]
    k2, v2, t2, l2, top, st = cache.append_block(k, v, table, lens, free, len(free), kn, vn)
    assert st == 0 and list(l2) == [76, 144, 16]
    for layer in range(2):
        for b in range(B):
            for g in range(Hkv):
                old_k, old_v = attention.gather_context(k[layer], v[layer], table, lens[b], b, g)
                new_k, new_v = attention.gather_context(k2[layer], v2[layer], t2, l2[b], b, g)
                np.testing.assert_array_equal(new_k, np.concatenate([old_k, kn[layer][b, g]]))
                np.testing.assert_array_equal(new_v, np.concatenate([old_v, vn[layer][b, g].T]))


def test_append_page_assignment_worked_example():
    """page 64, S 16, free stack [10, 11, 12, 13] (top = 13): sequence 0 (60 rows) crosses into a
    new page -> 13; sequence 1 (128 rows, pages full) needs one -> 12; sequence 2 (empty) -> 11."""
    k, v = _paged_cache(52, 16, 1, 64, 4, layers=1)
    table = np.full((3, 3), -1, np.int32)
    table[0, 0], table[1, :2] = 0, [1, 2]
    z = [np.zeros((3, 1, 16, 4))], [np.zeros((3, 1, 4, 16))]
    _, _, t2, l2, top, st = cache.append_block(k, v, table, [60, 128, 0], [10, 11, 12, 13], 4, *z)
    assert st == 0 and top == 1 and list(l2) == [76, 144, 16]
    assert t2[0].tolist() == [0, 13, -1] and t2[1].tolist() == [1, 2, 12] and t2[2].tolist() == [11, -1, -1]


def test_append_skips_what_does_not_fit_and_leaves_it_untouched():
    k, v = _paged_cache(53, 8, 1, 64, 4, layers=1)
    r = synth.rng(54)
    kn, vn = [r.standard_normal((4, 1, 16, 4))], [r.standard_normal((4, 1, 4, 16))]
    table = np.array([[0, -1], [1, -1], [2, -1], [3, 4]], np.int32)
    lens = np.array([64, 10, 64, 120], np.int32)
    # seq 0 pops page 7; seq 1 needs none; seq 2 finds the stack empty; seq 3's table is full
    k2, v2, t2, l2, top, st = cache.append_block(k, v, table, lens, [7], 1, kn, vn)
    assert top == 0 and list(l2) == [80, 26, 64, 120]
    assert st == cache.OUT_OF_PAGES | cache.NO_ROOM_IN_TABLE
    assert t2[2].tolist() == [2, -1] and t2[3].tolist() == [3, 4]
    np.testing.assert_array_equal(k2[0][[2, 3, 4]], k[0][[2, 3, 4]])
    np.testing.assert_array_equal(v2[0][[2, 3, 4]], v[0][[2, 3, 4]])
    # a page id outside the pool is refused before anything is written
    _, _, t3, l3, top3, st3 = cache.append_block(k, v, table, lens, [99], 1, kn, vn)
    assert st3 & cache.BAD_PAGE and l3[0] == 64 and t3[0].tolist() == [0, -1] and top3 == 1


# ------------------------------------------------------------------- masked-diffusion objective

def test_nll_of_uniform_logits_is_log_vocab():
    B, S, V = 2, 5, 1000
    x = np.full((B, S, V), 3.25)
    masked = np.array([[1, 0, 1, 1, 0], [0, 0, 0, 0, 1]], np.uint8)
    targets = synth.rng(55).integers(0, V, (B, S))
    nll, mean, n = loss.masked_nll(x, targets, masked)
    assert n == 4 and abs(mean - math.log(V)) < 1e-12
    np.testing.assert_allclose(nll[masked == 1], math.log(V), rtol=0, atol=1e-12)
    assert np.all(nll[masked == 0] == 0)


def test_nll_closed_form_single_peak():
    # target logit c, all others 0: nll = ln(e^c + V - 1) - c
    V, c = 257, 4.5
    x = np.zeros((1, 2, V))
    x[0, 0, 17] = c
    x[0, 1, 3] = c
    nll, mean, n = loss.masked_nll(x, np.array([[17, 9]]), np.ones((1, 2), np.uint8))
    assert abs(nll[0, 0] - (math.log(math.exp(c) + V - 1) - c)) < 1e-12
    assert abs(nll[0, 1] - math.log(math.exp(c) + V - 1)) < 1e-12     # target is a 0 logit
    assert n == 2 and abs(mean - nll.mean()) < 1e-15


def test_nll_matches_torch_cross_entropy_and_is_shift_invariant():
    torch = pytest.importorskip("torch")
    r = synth.rng(56)
    B, S, V = 3, 7, 513
    x = r.standard_normal((B, S, V)) * 3
    targets = r.integers(0, V, (B, S))
    masked = (r.random((B, S)) < 0.6).astype(np.uint8)
    nll, mean, n = loss.masked_nll(x, targets, masked)
    sel = masked.reshape(-1) == 1
    ce = torch.nn.functional.cross_entropy(torch.tensor(x.reshape(-1, V)[sel]),
                                           torch.tensor(targets.reshape(-1)[sel]), reduction="none")
    np.testing.assert_allclose(nll.reshape(-1)[sel], ce.numpy(), rtol=1e-12, atol=1e-12)
    assert abs(mean - ce.mean().item()) < 1e-12
    shifted, _, _ = loss.masked_nll(x + r.standard_normal((B, S, 1)) * 100, targets, masked)
    np.testing.assert_allclose(shifted, nll, rtol=0, atol=1e-9)


def test_linear_schedule_corruption():
    r = synth.rng(57)
    B, S = 4000, 16
    clean = r.integers(0, 1000, (B, S)).astype(np.int32)
    u_t = r.random(B).astype(np.float32)
    u_m = r.random((B, S)).astype(np.float32)
    noisy, masked, t = loss.corrupt(clean, u_t, u_m, mask_id=999999)
    assert np.array_equal(noisy[masked == 1], np.full(int(masked.sum()), 999999))
    assert np.array_equal(noisy[masked == 0], clean[masked == 0])
    # masking probability equals t: the masked fraction of each time bin tracks its mean time
    bins = np.minimum((u_t * 10).astype(int), 9)
    for k in range(10):
        sel = bins == k
        frac, tm = masked[sel].mean(), u_t[sel].mean()
        assert abs(frac - tm) < 4 * math.sqrt(tm * (1 - tm) / (sel.sum() * S)) + 1e-3
    # t = 0 masks nothing; the comparison is strict (u == t stays clean)
    _, m0, _ = loss.corrupt(clean[:2], np.zeros(2, np.float32), u_m[:2], 0)
    assert not m0.any()
    _, m1, _ = loss.corrupt(clean[:1], u_m[0, :1].copy(), u_m[:1], 0)
    assert m1[0, 0] == 0
