"""GPU parity of the context-cache append after a block is committed, and of two blocks decoded
back to back at a growing context.

Once a block is fully committed, its keys and values join the context cache that the next block
attends to (Nemotron-TwoTower explainer, "Generierungsprozess"). twotower_kv_append is compared bit
for bit with the oracle's append (oracle/cache.py: same rows, same page assignment from the
free-page stack, same flags); then a second block is decoded against the grown cache and its
attention is compared with the oracle over the concatenated context.
"""
import math

import numpy as np
import pytest
import torch

import synth
import two_tower_cross_amd as tt
from oracle import attention as oattn, cache as ocache
from synth.device import loop_model
from gpu_util import DEV, TOL_BF16, max_abs

pytestmark = pytest.mark.gpu


def to_np(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def setup_case(seed, *, B, Hkv, D, S, page, lens, layers, pool, max_pages, dtype, free=None):
    r = synth.rng(seed)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    mk = lambda shape: torch.from_numpy(r.standard_normal(shape).astype(np.float32)).to(DEV).to(dt)
    k = [mk(tt.k_pages_shape(pool, Hkv, page, D)) for _ in range(layers)]
    v = [mk(tt.v_pages_shape(pool, Hkv, page, D)) for _ in range(layers)]
    kn = [mk((B, Hkv, S, D)) for _ in range(layers)]
    vn = [mk((B, Hkv, D, S)) for _ in range(layers)]
    # pages in use: a random permutation of the pool (minus an explicit free stack), the rest free
    perm = r.permutation([p for p in range(pool) if free is None or p not in free]).astype(np.int32)
    table = np.full((B, max_pages), -1, np.int32)
    used = 0
    for b, L in enumerate(lens):
        n = -(-L // page)
        table[b, :n] = perm[used:used + n]
        used += n
    if free is None:
        free = perm[used:]
    t = lambda x: torch.from_numpy(np.ascontiguousarray(np.asarray(x, np.int32))).to(DEV)
    return dict(k=k, v=v, kn=kn, vn=vn, table=t(table), lens=t(lens), free=t(free),
                count=t([len(free)]), status=t([0]))


def run_both(c):
    ref = ocache.append_block([to_np(x) for x in c["k"]], [to_np(x) for x in c["v"]],
                              c["table"].cpu().numpy(), c["lens"].cpu().numpy(),
                              c["free"].cpu().numpy(), int(c["count"].item()),
                              [to_np(x) for x in c["kn"]], [to_np(x) for x in c["vn"]])
    tt.kv_append(c["k"], c["v"], c["kn"], c["vn"], c["table"], c["lens"], c["free"], c["count"],
                 c["status"])
    torch.cuda.synchronize()
    k2, v2, table2, lens2, top2, st2 = ref
    assert np.array_equal(c["table"].cpu().numpy(), table2)
    assert np.array_equal(c["lens"].cpu().numpy(), lens2)
    assert int(c["count"].item()) == top2 and int(c["status"].item()) == st2
    for layer in range(len(c["k"])):   # exact copies (bf16 values are exact in float64)
        assert np.array_equal(to_np(c["k"][layer]), k2[layer])
        assert np.array_equal(to_np(c["v"][layer]), v2[layer])
    return st2


@pytest.mark.parametrize("dtype,D,page", [("bf16", 128, 256), ("bf16", 64, 64), ("fp32", 128, 128)])
def test_append_matches_the_oracle(dtype, D, page):
    # lengths: empty, page-aligned, crossing one page, ending exactly on a boundary, mid-page
    lens = [0, 2 * page, page - 5, page - 16, 3 * page + 7]
    c = setup_case(60 + D + page, B=len(lens), Hkv=2, D=D, S=16, page=page, lens=lens, layers=3,
                   pool=24, max_pages=6, dtype=dtype)
    assert run_both(c) == 0
    # a second append on top of the first (the pages just allocated are now partly filled)
    c["kn"] = [x.flip(2).contiguous() for x in c["kn"]]
    c["vn"] = [x.flip(3).contiguous() for x in c["vn"]]
    assert run_both(c) == 0


def _random_append(seed):
    """A seeded random append within the documented limits: block sizes up to 128, both head
    sizes, pages of 64 to 256 tokens, random lengths that leave room in each table, and a pool
    whose free stack covers every sequence (so every append goes through)."""
    g = np.random.default_rng(seed)
    page = int(g.choice([64, 128, 192, 256]))
    S = int(g.choice([1, 5, 16, 32, 100, 128]))
    max_pages = int(g.integers(-(-S // page) + 1, 7))
    B = int(g.integers(1, 7))
    lens = [int(x) for x in g.integers(0, max_pages * page - S + 1, size=B)]
    used = sum(-(-L // page) for L in lens)
    need = sum(-(-(L + S) // page) - (-(-L // page)) for L in lens)
    return dict(B=B, Hkv=int(g.integers(1, 4)), D=int(g.choice([64, 128])), S=S, page=page,
                lens=lens, layers=int(g.integers(1, 4)), pool=used + need + int(g.integers(0, 4)),
                max_pages=max_pages, dtype="bf16" if g.random() < 0.7 else "fp32")


@pytest.mark.parametrize("seed", range(110, 118))
def test_random_appends_match_the_oracle(seed):
    c = setup_case(seed, **_random_append(seed))
    assert run_both(c) == 0


def test_append_flags_and_skips_like_the_oracle():
    # stack of 2 pages for 3 sequences that each need one; the last table is too short
    c = setup_case(70, B=4, Hkv=1, D=64, S=16, page=64, lens=[64, 64, 60, 120], layers=2,
                   pool=12, max_pages=2, dtype="bf16", free=[9, 10])
    st = run_both(c)
    assert st == ocache.OUT_OF_PAGES | ocache.NO_ROOM_IN_TABLE
    # a page id outside the pool is refused before anything is written
    c = setup_case(71, B=2, Hkv=1, D=64, S=16, page=64, lens=[64, 10], layers=1, pool=4,
                   max_pages=3, dtype="bf16", free=[3, 77])
    assert run_both(c) == ocache.BAD_PAGE


def test_two_blocks_at_a_growing_context():
    """Block 1, append its final block KV as the context rows of its tokens, block 2 at L + S."""
    m = loop_model(8, B=2, S=16, L=1018, layers=2, Hq=8, Hkv=2, D=128, hidden=512, vocab=8192,
                   T=4, device=DEV, page_size=256, spare_pages=4, max_pages=5)
    step = tt.DenoiseStep(k_pages=m.k_pages, v_pages=m.v_pages, w_qkv=m.w_qkv, w_o=m.w_o,
                          w_lm=m.w_lm, block_table=m.block_table, ctx_lens=m.ctx_lens,
                          max_ctx_len=m.L + m.S, num_q_heads=m.Hq, num_kv_heads=m.Hkv,
                          head_dim=m.D, batch=m.B, S=m.S)
    l = m.layers - 1
    before = [oattn.gather_context(to_np(m.k_pages[l]), to_np(m.v_pages[l]),
                                   m.block_table.cpu().numpy(), m.L, b, g)
              for b in range(m.B) for g in range(m.Hkv)]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    for blk in range(2):
        masked = torch.ones((m.B, m.S), dtype=torch.uint8, device=DEV)
        tokens = torch.full((m.B, m.S), -1, dtype=torch.int32, device=DEV)
        for t in range(m.T):
            step(m.h_steps[t], masked, tokens, threshold=0.9, min_commit=True,
                 commit_all=(t == m.T - 1))
        torch.cuda.synchronize()
        assert not masked.any()
        if blk == 0:
            kb1, vb1 = step.k_blk[l].clone(), step.v_blk[l].clone()
            tt.kv_append(m.k_pages, m.v_pages, step.k_blk, step.v_blk, m.block_table, m.ctx_lens,
                         m.free_pages, m.free_count, status)
            torch.cuda.synchronize()
            assert m.ctx_lens.tolist() == [m.L + m.S] * m.B and int(status.item()) == 0
            assert int(m.free_count.item()) == 4 - m.B       # 1018 + 16 crosses into a 5th page
    # block 2's last step, last layer: oracle over [original context ; block-1 rows] + block 2
    Lc = m.L + m.S
    Lp = -(-Lc // 64) * 64
    kc = np.zeros((m.B, m.Hkv, Lp, m.D))
    vc = np.zeros((m.B, m.Hkv, Lp, m.D))
    for b in range(m.B):
        for g in range(m.Hkv):
            ok, ov = before[b * m.Hkv + g]
            kc[b, g, :Lc] = np.concatenate([ok, to_np(kb1)[b, g]])
            vc[b, g, :Lc] = np.concatenate([ov, to_np(vb1)[b, g].T])
    vtiles = synth.tile_v(vc.transpose(0, 1, 3, 2))
    ref, _ = oattn.block_attention(to_np(step.q), synth.tile_k(kc), vtiles,
                                   np.arange(m.B, dtype=np.int32).reshape(m.B, 1),
                                   np.full(m.B, Lc, np.int32), to_np(step.k_blk[l]),
                                   to_np(step.v_blk[l]), 1.0 / math.sqrt(m.D))
    ref16 = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    assert max_abs(to_np(step.attn_out), ref16) <= TOL_BF16
