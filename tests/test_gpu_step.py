"""GPU parity of the dense projections and of the denoise step / T-step block loop.

The generation loop checked: the block starts fully masked, each step rewrites the block's own
KV at every layer, attends to the resident context caches and commits confident tokens
(Nemotron-TwoTower explainer, "Generierungsprozess"). Stage-wise parity: each stage is compared
with the oracle fed the GPU's own inputs for that stage; the step is compared bit for bit with the
composition of the per-stage entry points; the loop is checked by its invariants.
"""
import itertools
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


def random_shapes(seed, n, draw):
    """n shapes drawn by draw(generator), seeded: the same every run."""
    g = np.random.default_rng(seed)
    return [draw(g) for _ in range(n)]


def _ri(g, lo, hi):
    return int(g.integers(lo, hi + 1))


# batch, S, hidden (multiple of 8), Hq = G Hkv, Hkv, head_dim (multiple of 4)
RANDOM_QKV = random_shapes(31, 6, lambda g: (lambda hkv: (_ri(g, 1, 4), _ri(g, 1, 40),
                                                          8 * _ri(g, 1, 160), hkv * _ri(g, 1, 8),
                                                          hkv, 4 * _ri(g, 1, 32)))(_ri(g, 1, 3)))
# rows, hidden (multiple of 4), in_features (multiple of 8)
RANDOM_OUT = random_shapes(32, 6, lambda g: (_ri(g, 1, 300), 4 * _ri(g, 1, 300),
                                             8 * _ri(g, 1, 200)))
# rows, hidden (multiple of 8), vocab (multiple of 4)
RANDOM_LM = random_shapes(33, 6, lambda g: (_ri(g, 1, 200), 8 * _ri(g, 1, 100),
                                            4 * _ri(g, 1, 5000)))


# (3, 100, 1024, 2, 1, 48): 300 rows in three 128-row tiles, 192 features in three tiles, K in 4
# parts merged inside the kernel; then seeded random shapes within the documented limits
@pytest.mark.parametrize("shape", [(2, 16, 512, 8, 2, 128), (8, 16, 2048, 32, 2, 128),
                                   (3, 5, 264, 4, 1, 64), (3, 100, 1024, 2, 1, 48)] + RANDOM_QKV)
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


# (300, 200, 1024): three row tiles, the last feature tile 8 wide, K in 4 parts merged inside
@pytest.mark.parametrize("rows,hidden,inf", [(32, 512, 1024), (128, 2048, 4096), (80, 264, 136),
                                             (300, 200, 1024)] + RANDOM_OUT)
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


def test_projection_merge_needs_no_clean_workspace():
    """The K partials of the projections are summed inside the product's kernel; its work-groups
    meet at arrival counters kept in the caller's workspace, which nobody clears. A workspace of
    arbitrary bytes, all ones, or left over by the previous call (complete counts of another launch)
    gives the same outputs bit for bit, and they match the oracle."""
    g = torch.Generator(device=DEV).manual_seed(21)
    B, S, hidden, Hq, Hkv, D = 8, 16, 2048, 32, 2, 128
    h = torch.randn((B, S, hidden), generator=g, device=DEV).to(torch.bfloat16)
    wq = tt.pack_weight((torch.randn(((Hq + 2 * Hkv) * D, hidden), generator=g, device=DEV)
                         / math.sqrt(hidden)).to(torch.bfloat16))
    o = torch.randn((B * S, Hq * D), generator=g, device=DEV).to(torch.bfloat16)
    wo_dense = (torch.randn((hidden, Hq * D), generator=g, device=DEV) / math.sqrt(Hq * D)).to(torch.bfloat16)
    wo = tt.pack_weight(wo_dense)
    ws = torch.empty(16 << 20, dtype=torch.uint8, device=DEV)
    outs = []
    for fill in ("random", "ones", "previous", "previous"):
        if fill == "random":
            ws.copy_(torch.randint(0, 256, ws.shape, generator=g, device=DEV, dtype=torch.int32)
                     .to(torch.uint8))
        elif fill == "ones":
            ws.fill_(255)
        q, kb, vb = tt.qkv_projection(h, wq, Hq, Hkv, D, workspace=ws)
        ho = tt.out_projection(h.view(B * S, hidden), o, wo, workspace=ws)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (q, kb, vb, ho)])
    for later in outs[1:]:
        for a, b in zip(outs[0], later):
            assert torch.equal(a, b)
    ref = ostep.residual_output(f64(h.view(B * S, hidden))[:, None], f64(o).reshape(B * S, 1, Hq * D),
                                f64(wo_dense))[:, 0]
    ok, err = bf16_ok(f64(outs[0][3]), ref)
    assert ok, err


def test_projection_merge_inside_equals_separate_merge_kernel(monkeypatch):
    """The K partials summed inside the product kernel (each partition its share of the rows), by
    the last partition to arrive after every other one handed its share over
    (TWOTOWER_MERGE_WAIT_POLLS=0: the path taken when partitions cannot all be resident) and by the
    separate merge kernel (TWOTOWER_MERGE_IN_KERNEL=0) give the same outputs bit for bit: one sum,
    in partition order."""
    g = torch.Generator(device=DEV).manual_seed(23)
    for B, S, hidden, Hq, Hkv, D in ((8, 16, 2048, 32, 2, 128), (3, 5, 264, 4, 1, 64)):
        h = torch.randn((B, S, hidden), generator=g, device=DEV).to(torch.bfloat16)
        wq = tt.pack_weight((torch.randn(((Hq + 2 * Hkv) * D, hidden), generator=g, device=DEV)
                             / math.sqrt(hidden)).to(torch.bfloat16))
        o = torch.randn((B * S, Hq * D), generator=g, device=DEV).to(torch.bfloat16)
        wo = tt.pack_weight((torch.randn((hidden, Hq * D), generator=g, device=DEV)
                             / math.sqrt(Hq * D)).to(torch.bfloat16))
        outs = []
        for inside, polls in (("1", "256"), ("1", "0"), ("0", "256")):
            monkeypatch.setenv("TWOTOWER_MERGE_IN_KERNEL", inside)
            monkeypatch.setenv("TWOTOWER_MERGE_WAIT_POLLS", polls)
            q, kb, vb = tt.qkv_projection(h, wq, Hq, Hkv, D)
            ho = tt.out_projection(h.view(B * S, hidden), o, wo)
            torch.cuda.synchronize()
            outs.append((q, kb, vb, ho))
        for other in outs[1:]:
            for a, b in zip(outs[0], other):
                assert torch.equal(a, b)


def test_projections_on_two_streams_at_once():
    """Two output projections launched at the same time on two streams (each grid fills the GPU,
    so their work-groups share the compute units and a tile's partitions need not all be resident
    at once): both finish, and each equals the same call made alone, bit for bit."""
    g = torch.Generator(device=DEV).manual_seed(24)
    rows, hidden, inf = 128, 2048, 4096
    wo = tt.pack_weight((torch.randn((hidden, inf), generator=g, device=DEV) / math.sqrt(inf))
                        .to(torch.bfloat16))
    hs = [torch.randn((rows, hidden), generator=g, device=DEV).to(torch.bfloat16) for _ in range(2)]
    os_ = [torch.randn((rows, inf), generator=g, device=DEV).to(torch.bfloat16) for _ in range(2)]
    refs = [tt.out_projection(h, o, wo) for h, o in zip(hs, os_)]
    outs = [torch.empty_like(r) for r in refs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(5):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        for st, h, o, out in zip(streams, hs, os_, outs):
            with torch.cuda.stream(st):
                tt.out_projection(h, o, wo, out=out)
        torch.cuda.synchronize()
        for out, ref in zip(outs, refs):
            assert torch.equal(out, ref)


def test_stages_from_several_host_threads_at_once():
    """Four host threads, each with its own stream (and the binding's own workspaces), run QKV,
    attention and the output projection concurrently (the ctypes calls release the interpreter
    lock): the library's per-device caches are shared by all of them, and every thread's results
    equal the same calls made from one thread, bit for bit."""
    import threading
    m = small_model(seed=9)
    l = 0
    hs = [m.h_steps[t] for t in range(4)]

    def stages(h):
        q, kb, vb = tt.qkv_projection(h, m.w_qkv[l], m.Hq, m.Hkv, m.D)
        o = tt.block_attn(q, m.k_pages[l], m.v_pages[l], m.block_table, m.ctx_lens, kb, vb,
                          max_ctx_len=m.L, out_dtype=torch.bfloat16)
        return q, o, tt.out_projection(h, o, m.w_o[l])

    refs = [stages(h) for h in hs]
    torch.cuda.synchronize()
    results, errors = [None] * len(hs), []
    barrier = threading.Barrier(len(hs))

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            barrier.wait()
            with torch.cuda.stream(stream):
                outs = [stages(hs[i]) for _ in range(3)]
            stream.synchronize()
            results[i] = outs
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(hs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    for outs, ref in zip(results, refs):
        for got in outs:
            for a, b in zip(got, ref):
                assert torch.equal(a, b)

def test_projection_graph_replays_match_eager_calls():
    """Both projections captured in one graph (every replay of a captured product carries the same
    launch tag, so each finds the previous replay's complete arrival counts) and replayed several
    times, with eager work in between: every replay equals the eager calls bit for bit."""
    g = torch.Generator(device=DEV).manual_seed(22)
    B, S, hidden, Hq, Hkv, D = 8, 16, 2048, 32, 2, 128
    h = torch.randn((B, S, hidden), generator=g, device=DEV).to(torch.bfloat16)
    wq = tt.pack_weight((torch.randn(((Hq + 2 * Hkv) * D, hidden), generator=g, device=DEV)
                         / math.sqrt(hidden)).to(torch.bfloat16))
    o = torch.randn((B * S, Hq * D), generator=g, device=DEV).to(torch.bfloat16)
    wo = tt.pack_weight((torch.randn((hidden, Hq * D), generator=g, device=DEV)
                         / math.sqrt(Hq * D)).to(torch.bfloat16))
    qkv = (torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=DEV),
           torch.empty((B, Hkv, S, D), dtype=torch.bfloat16, device=DEV),
           torch.empty((B, Hkv, D, S), dtype=torch.bfloat16, device=DEV))
    ho = torch.empty((B * S, hidden), dtype=torch.bfloat16, device=DEV)

    def calls():
        tt.qkv_projection(h, wq, Hq, Hkv, D, out=qkv)
        tt.out_projection(h.view(B * S, hidden), o, wo, out=ho)

    calls()                               # eager first: every one-time setup is done
    torch.cuda.synchronize()
    ref = [t.clone() for t in (*qkv, ho)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for _ in range(3):
        for t in (*qkv, ho):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((*qkv, ho), ref):
            assert torch.equal(a, b)
        calls()                           # eager calls between the replays
        torch.cuda.synchronize()


# (96: 3 slabs of 32 features in 64-feature tiles; 70000: 2188 slabs in 256-feature tiles: the last
# tile of each reaches past the packed weight and must read nothing there)
@pytest.mark.parametrize("rows,hidden,V", [(32, 512, 8192), (128, 2048, 131072), (7, 136, 1004),
                                           (5, 128, 96), (128, 256, 70000)] + RANDOM_LM)
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


def test_step_timing_events_change_nothing():
    """The profiling hook of the step (events around each layer's attention, NULL entries
    skipped; fence-free timing events as the benchmark creates them) records time and leaves every
    output bit for bit as without events."""
    from two_tower_cross_amd.timing import TimingEvent
    m = small_model()
    step = make_step(m, keep_logits=True)
    runs = []
    for with_events in (False, True):
        masked = torch.ones((m.B, m.S), dtype=torch.uint8, device=DEV)
        tokens = torch.full((m.B, m.S), -1, dtype=torch.int32, device=DEV)
        evs, handles = None, None
        if with_events:
            evs = [TimingEvent() for _ in range(4)]
            handles = [None] * (3 * m.layers)
            handles[0], handles[2] = evs[0].cuda_event, evs[1].cuda_event        # layer 0: call
            handles[3 * (m.layers - 1)], handles[3 * (m.layers - 1) + 1] = (
                evs[2].cuda_event, evs[3].cuda_event)                           # last: kernel
        conf, n = step(m.h_steps[0], masked, tokens, threshold=0.9, min_commit=True,
                       timing_events=handles)
        torch.cuda.synchronize()
        runs.append((conf.clone(), n.clone(), masked.clone(), tokens.clone(), step.logits.clone()))
        if with_events:
            assert evs[0].elapsed_time(evs[1]) > 0.0 and evs[2].elapsed_time(evs[3]) > 0.0
    for a, b in zip(*runs):
        assert torch.equal(a, b)


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


def test_finished_sequences_get_no_attention_work():
    """A sequence with no masked position left gets no attention work in the step (the live
    sequences' context is re-planned over the whole GPU): its state and its attention output rows
    are untouched, and the live sequences' attention and decisions still match the oracle on the
    step's own inputs."""
    m = small_model(seed=8, B=4, L=1500)
    step = make_step(m, keep_logits=True)
    masked = torch.ones((m.B, m.S), dtype=torch.uint8, device=DEV)
    tokens = torch.full((m.B, m.S), -1, dtype=torch.int32, device=DEV)
    for b in (1, 3):
        masked[b] = 0
        tokens[b] = 10 + b
    m0, t0 = masked.clone(), tokens.clone()
    step.attn_out.fill_(7.0)
    conf, n = step(m.h_steps[0], masked, tokens, threshold=0.9, min_commit=True)
    torch.cuda.synchronize()
    for b in (1, 3):
        assert torch.equal(masked[b], m0[b]) and torch.equal(tokens[b], t0[b]) and int(n[b]) == 0
        assert bool((step.attn_out[b] == 7.0).all())       # no attention work for it
    l = m.layers - 1
    G = m.Hq // m.Hkv
    for b in (0, 2):
        for g in range(m.Hkv):
            heads = slice(g * G, (g + 1) * G)
            ref, _ = oattn.block_attention(
                f64(step.q[b:b + 1, :, heads]), f64(m.k_pages[l][b:b + 1, g:g + 1]),
                f64(m.v_pages[l][b:b + 1, g:g + 1]), np.zeros((1, 1), np.int32),
                np.array([m.L], np.int32), f64(step.k_blk[l][b:b + 1, g:g + 1]),
                f64(step.v_blk[l][b:b + 1, g:g + 1]), 1.0 / math.sqrt(m.D))
            ref16 = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
            assert max_abs(f64(step.attn_out[b:b + 1, :, heads]), ref16) <= TOL_BF16
    ot, om, oc, on = ounmask.confidence_unmask(step.logits.cpu().numpy(), m0.cpu().numpy(),
                                               t0.cpu().numpy(), np.float32(0.9), min_commit=True)
    gm, gt = masked.cpu().numpy(), tokens.cpu().numpy()
    for b in (0, 2):
        c = np.sort(oc[b])[::-1]
        if c[0] - c[1] >= 1e-4 * c[0]:
            assert np.array_equal(gm[b], om[b]) and np.array_equal(gt[b], ot[b])
        else:
            assert int(n[b]) == 1


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


def test_block_of_steps_replays_from_a_graph_like_eager_calls():
    """The T steps of a block captured in one graph (the library records no memset and allocates
    nothing per call) replay bit for bit like eager calls: commits, counts, confidence and the
    residual stream, on every replay, with the program's own eager work in between."""
    m = small_model(seed=8)
    step = make_step(m)
    masked = torch.ones((m.B, m.S), dtype=torch.uint8, device=DEV)
    tokens = torch.full((m.B, m.S), -1, dtype=torch.int32, device=DEV)
    counts = torch.zeros((m.T, m.B), dtype=torch.int32, device=DEV)

    def steps():
        for t in range(m.T):
            step(m.h_steps[t], masked, tokens, threshold=0.9, min_commit=True,
                 commit_all=(t == m.T - 1), n_committed=counts[t])

    def reset():
        masked.fill_(1)
        tokens.fill_(-1)
        counts.fill_(-7)

    def state():
        return [x.clone() for x in (masked, tokens, counts, step.confidence, step.h_work)]

    reset()
    steps()
    torch.cuda.synchronize()
    ref = state()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        steps()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(graph):
        steps()
    for _ in range(3):
        reset()
        graph.replay()
        torch.cuda.synchronize()
        got = state()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        assert not masked.any()

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
    # last layer's attention (its q and block KV are still in the step's buffers), every (b, g)
    l = m.layers - 1
    for b, g in itertools.product(range(m.B), range(m.Hkv)):
        G = m.Hq // m.Hkv
        heads = slice(g * G, (g + 1) * G)
        ref, _ = oattn.block_attention(
            f64(step.q[b:b + 1, :, heads]), f64(m.k_pages[l][b:b + 1, g:g + 1]),
            f64(m.v_pages[l][b:b + 1, g:g + 1]), np.zeros((1, 1), np.int32),
            np.array([m.L], np.int32), f64(step.k_blk[l][b:b + 1, g:g + 1]),
            f64(step.v_blk[l][b:b + 1, g:g + 1]), 1.0 / math.sqrt(m.D))
        ref16 = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
        assert max_abs(f64(step.attn_out[b:b + 1, :, heads]), ref16) <= TOL_BF16
    # lm-head on the final residual stream, sampled vocabulary columns
    cols = np.sort(synth.rng(15).choice(m.vocab, size=8192, replace=False))
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


def test_full_size_first_step_logits_and_decisions_against_oracle():
    """First denoise step of the 32K loop at full size (8 sequences x 16 positions, vocabulary
    131072): every logit against the oracle's lm-head on the step's final residual stream, every
    row's confidence against the oracle on the step's own fp32 logits, and the commit decisions.
    A random model's confidences are all far below the threshold, so each sequence commits its
    most confident position (the fallback); the token is the row's first argmax over the same
    fp32 logits on both sides, hence exact. Where a sequence's top two confidences are closer than
    1e-4 (relative) the fp32 and fp64 sums may order them differently: the commit must then be
    one of those positions."""
    m = loop_model(5, device=DEV)
    step = make_step(m, keep_logits=True)
    masked = torch.ones((m.B, m.S), dtype=torch.uint8, device=DEV)
    tokens = torch.full((m.B, m.S), -1, dtype=torch.int32, device=DEV)
    m0, t0 = masked.cpu().numpy(), tokens.cpu().numpy()
    conf, n = step(m.h_steps[0], masked, tokens, threshold=0.9, min_commit=True)
    torch.cuda.synchronize()
    logits = step.logits.cpu().numpy()
    assert logits.shape == (m.B, m.S, m.vocab)
    ref = ostep.lm_head(f64(step.h_work), f64(m.w_lm))
    assert max_abs(logits, ref) <= 1e-4 + 1e-5 * np.abs(ref).max()
    del ref
    ot, om, oc, on = ounmask.confidence_unmask(logits, m0, t0, np.float32(0.9), min_commit=True)
    gc = conf.cpu().numpy().astype(np.float64)
    assert np.all(oc < 0.5)                                # far below the threshold
    np.testing.assert_allclose(gc, oc, rtol=1e-5, atol=0)
    gm, gt, gn = masked.cpu().numpy(), tokens.cpu().numpy(), n.cpu().numpy()
    assert (gn == 1).all() and np.array_equal(gn, on)
    first_argmax = logits.argmax(axis=2)
    for b in range(m.B):
        (i,) = np.flatnonzero(gm[b] == 0)                  # exactly one commit
        assert gt[b, i] == first_argmax[b, i]
        assert (gt[b, gm[b] == 1] == -1).all()             # the rest untouched
        c = np.sort(oc[b])[::-1]
        if c[0] - c[1] >= 1e-4 * c[0]:
            assert np.array_equal(gm[b], om[b]) and np.array_equal(gt[b], ot[b])
        else:
            assert oc[b, i] >= c[0] * (1 - 1e-4)


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


def test_empty_batch_through_every_entry_point():
    """A batch of 0 sequences (PyTorch's empty tensors: null data pointers) is a no-op for every
    call: empty results, no error, no launch; the caches and pools stay as they are."""
    bf, i32, u8, f32 = torch.bfloat16, torch.int32, torch.uint8, torch.float32
    S, Hq, Hkv, D, hidden, V, page = 16, 8, 2, 64, 512, 1000, 64
    g = torch.Generator(device=DEV).manual_seed(21)
    kp = torch.randn(tt.k_pages_shape(3, Hkv, page, D), generator=g, device=DEV).to(bf)
    vp = torch.randn(tt.v_pages_shape(3, Hkv, page, D), generator=g, device=DEV).to(bf)
    before = (kp.clone(), vp.clone())
    out = tt.block_attn(torch.empty((0, S, Hq, D), dtype=bf, device=DEV), kp, vp,
                        torch.empty((0, 2), dtype=i32, device=DEV),
                        torch.empty((0,), dtype=i32, device=DEV),
                        torch.empty((0, Hkv, S, D), dtype=bf, device=DEV),
                        torch.empty((0, Hkv, D, S), dtype=bf, device=DEV))
    assert tuple(out.shape) == (0, S, Hq, D)
    conf, ncom = tt.unmask(torch.empty((0, S, V), dtype=f32, device=DEV),
                           torch.empty((0, S), dtype=u8, device=DEV),
                           torch.empty((0, S), dtype=i32, device=DEV), 0.9, min_commit=True)
    assert conf.numel() == 0 and ncom.numel() == 0
    w_qkv = (torch.randn(((Hq + 2 * Hkv) * D, hidden), generator=g, device=DEV) / 16).to(bf)
    q, kb, vb = tt.qkv_projection(torch.empty((0, S, hidden), dtype=bf, device=DEV), w_qkv, Hq,
                                  Hkv, D)
    assert q.numel() == kb.numel() == vb.numel() == 0
    w_o = (torch.randn((hidden, Hq * D), generator=g, device=DEV) / 16).to(bf)
    h = tt.out_projection(torch.empty((0, hidden), dtype=bf, device=DEV),
                          torch.empty((0, Hq * D), dtype=bf, device=DEV), w_o)
    assert tuple(h.shape) == (0, hidden)
    w_lm = (torch.randn((V, hidden), generator=g, device=DEV) / 16).to(bf)
    assert tuple(tt.lm_head(torch.empty((0, S, hidden), dtype=bf, device=DEV), w_lm).shape) == \
        (0, S, V)
    for keep in (False, True):
        c, n, lg = tt.lm_head_unmask(torch.empty((0, S, hidden), dtype=bf, device=DEV), w_lm,
                                     torch.empty((0, S), dtype=u8, device=DEV),
                                     torch.empty((0, S), dtype=i32, device=DEV), 0.9,
                                     keep_logits=keep)
        assert c.numel() == 0 and n.numel() == 0 and (lg is None or lg.numel() == 0)
    noisy, masked, t = tt.mask_corrupt(torch.empty((0, S), dtype=i32, device=DEV),
                                       torch.empty((0,), dtype=f32, device=DEV),
                                       torch.empty((0, S), dtype=f32, device=DEV), V)
    assert noisy.numel() == masked.numel() == t.numel() == 0
    nll, loss, count = tt.masked_nll(torch.empty((0, S, V), dtype=f32, device=DEV),
                                     torch.empty((0, S), dtype=i32, device=DEV),
                                     torch.empty((0, S), dtype=u8, device=DEV))
    assert nll.numel() == 0 and loss.item() == 0.0 and count.item() == 0
    free_count = torch.tensor([3], dtype=i32, device=DEV)
    status = torch.zeros((1,), dtype=i32, device=DEV)
    tt.kv_append([kp], [vp], [torch.empty((0, Hkv, S, D), dtype=bf, device=DEV)],
                 [torch.empty((0, Hkv, D, S), dtype=bf, device=DEV)],
                 torch.empty((0, 2), dtype=i32, device=DEV), torch.empty((0,), dtype=i32, device=DEV),
                 torch.arange(3, dtype=i32, device=DEV), free_count, status)
    torch.cuda.synchronize()
    assert free_count.item() == 3 and status.item() == 0
    assert torch.equal(kp, before[0]) and torch.equal(vp, before[1])
