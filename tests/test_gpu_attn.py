"""GPU parity of twotower_block_attn against the fp64 oracle (element by element).

Definition checked: the block queries attend, under one softmax, to the context tower's same-layer
KV rows and the block's own KV rows (Nemotron-TwoTower explainer, "Architektur" /
"Generierungsprozess"). Tolerances: max-abs 1e-5 for fp32 inputs, 2e-2 for bf16 inputs (fp32
output; bf16 output is compared with the oracle rounded to bf16 at the same 2e-2).
"""
import math

import numpy as np
import pytest
import torch

import synth
import two_tower_cross_amd as tt
from oracle import attention as oattn
from gpu_util import DEV, TOL_BF16, TOL_FP32, dev_case, gpu_attn, max_abs, to_dev

pytestmark = pytest.mark.gpu


def check(case, out, lse, tol, lse_tol=None):
    ref, ref_lse = oattn.block_attention_case(case)
    err = max_abs(out, ref)
    assert err <= tol, f"max-abs {err:.3g} > {tol}"
    if lse is not None:
        lerr = max_abs(lse, ref_lse)
        assert lerr <= (lse_tol or tol), f"lse max-abs {lerr:.3g}"
    return ref


# ------------------------------------------------------------------ the workload configurations

def test_tiny_fp32():
    case = synth.config_attn("tiny_fp32")
    out, lse = gpu_attn(case)
    check(case, out, lse, TOL_FP32)


def test_tiny_fp32_ragged_and_empty_context():
    for L in (0, 1, 37, 255):
        case = synth.config_attn("tiny_fp32", ctx_len=L)
        out, lse = gpu_attn(case)
        check(case, out, lse, TOL_FP32)


@pytest.mark.parametrize("splits", [0, 1, 3, 16, 64])
def test_ctx4k_bf16_splits(splits):
    case = synth.config_attn("ctx4k_bf16")
    out, lse = gpu_attn(case, num_splits=splits)
    check(case, out, lse, TOL_BF16)


def test_ctx4k_bf16_output_in_bf16():
    case = synth.config_attn("ctx4k_bf16")
    out, _ = gpu_attn(case, out_dtype=torch.bfloat16)
    ref, _ = oattn.block_attention_case(case)
    ref16 = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    assert max_abs(out, ref16) <= TOL_BF16


def test_ragged_paged_batch():
    case = synth.config_attn("ragged32_paged")
    assert np.isnan(case.k_pages).any()          # unused pages and page tails are poisoned
    for splits in (0, 8):
        out, lse = gpu_attn(case, num_splits=splits)
        assert not np.isnan(out).any()
        check(case, out, lse, TOL_BF16)


@pytest.mark.parametrize("splits", [0, 64, 128, 256])
def test_long_context_131072(splits):
    case = synth.config_attn("long128k")
    out, lse = gpu_attn(case, num_splits=splits)
    check(case, out, lse, TOL_BF16)


def test_loop32k_layer_shape():
    case = synth.config_attn("loop32k_layer")
    out, lse = gpu_attn(case, out_dtype=torch.float32)
    check(case, out, lse, TOL_BF16)


# ------------------------------------------------------------------------------- the merge

@pytest.mark.parametrize("B,Hkv,D,lens,splits", [
    (32, 2, 128, (2048, 1500), 16),      # 64 (b, g) units: one partition group per row
    (64, 2, 64, (1024, 700), 16),        # head_dim 64, one partition group
    (8, 2, 128, (4096, 3000), 40),       # 4 partition groups, partitions past a short sequence
    (1, 2, 128, (40960,), 600),          # 16 groups, 320 partitions: two load batches per thread
    (2, 1, 64, (20000, 9000), 313),      # 16 groups at head_dim 64, 313 partitions, ragged
])
def test_merge_partition_groups(B, Hkv, D, lens, splits):
    """The partition merge spreads a row's partitions over 1, 4 or 16 thread groups depending on
    the number of rows and partitions; every variant must give the oracle's result."""
    ctx = [lens[b % len(lens)] for b in range(B)]
    case = synth.attn_case(61 + B, B=B, S=16, Hq=16 * Hkv, Hkv=Hkv, D=D, ctx_lens=ctx,
                           page_size=None if B == 1 else 512, dtype="bf16")
    out, lse = gpu_attn(case, num_splits=splits)
    check(case, out, lse, TOL_BF16)


@pytest.mark.parametrize("B,Hq,Hkv,hi", [
    (100, 8, 2, 3000),   # two lanes' worth of sequences per wave in the plan
    (256, 4, 1, 1500),   # the largest batch the balanced plan takes (four per lane)
    (300, 4, 1, 600),    # beyond it: the uniform split by the longest context
])
def test_balanced_plan_batches(B, Hq, Hkv, hi):
    """The automatic partition count cuts every sequence's context from the actual lengths so
    that the work-groups get nearly equal shares: empty, one-token, tile-boundary and random
    lengths, against the oracle."""
    g = synth.rng(70 + B)
    lens = g.integers(0, hi + 1, size=B)
    lens[:6] = [0, 1, 63, 64, 65, hi]
    case = synth.attn_case(71 + B, B=B, S=16, Hq=Hq, Hkv=Hkv, D=128, ctx_lens=lens,
                           page_size=256, dtype="bf16", nan_poison=True, spare_frac=0.05)
    out, lse = gpu_attn(case)
    assert not np.isnan(out).any()
    check(case, out, lse, TOL_BF16)


# ----------------------------------------------------------------------------- value range

@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("splits", [1, 16, 64])
@pytest.mark.parametrize("v_scale", [1e5, 1e-6])
def test_value_range(v_scale, splits, out_dtype):
    """The output is defined for any bf16 values: V ~ N(0, v_scale^2) far above fp16's largest
    value (65504) and far below its smallest normal (6.1e-5). The queries are scaled by 4 so that
    the softmax concentrates on a few keys and the partition outputs reach max|V|. Attention is
    linear in V, so the bf16 tolerance scales with v_scale; a bf16 output adds its own rounding
    (2^-8 relative)."""
    case = synth.attn_case(60, B=1, S=16, Hq=32, Hkv=2, D=128, ctx_lens=[4096], dtype="bf16",
                           q_scale=4.0, v_scale=v_scale)
    ref, ref_lse = oattn.block_attention_case(case)
    if v_scale > 1.0:
        # each output row is a convex combination of the partitions' rows, so some partition
        # row exceeds fp16's range wherever the result does
        assert np.abs(ref).max() > 65504.0
    out, lse = gpu_attn(case, num_splits=splits, out_dtype=out_dtype)
    assert np.isfinite(out).all()
    tol = TOL_BF16 * v_scale
    if out_dtype == torch.float32:
        err = max_abs(out, ref)
        assert err <= tol, f"max-abs {err:.3g} > {tol:.3g}"
    else:
        excess = np.abs(out - ref) - (tol + 2.0 ** -8 * np.abs(ref))
        assert excess.max() <= 0.0, f"bf16 output off by {excess.max():.3g} beyond the bound"
    assert max_abs(lse, ref_lse) <= TOL_BF16


# ------------------------------------------------------------------------ closed forms on the GPU

def test_identical_keys_give_mean_of_values():
    case = synth.attn_case(50, B=2, S=16, Hq=32, Hkv=2, D=128, ctx_lens=[700, 64], page_size=256,
                           dtype="bf16")
    case.k_pages[...] = 0.5
    case.k_blk[...] = 0.5
    out, lse = gpu_attn(case)
    ref = check(case, out, lse, TOL_BF16)
    # every weight is exactly 1 on the GPU too: the result is the plain mean of the values
    for b in range(2):
        n = int(case.ctx_lens[b]) + 16
        s = case.scale * 0.5 * case.q[b].astype(np.float64).sum(-1)        # [S, Hq]
        np.testing.assert_allclose(lse[b], math.log(n) + s.T, atol=1e-4)


def test_zero_query_gives_mean_and_log_count():
    case = synth.attn_case(51, B=1, S=16, Hq=16, Hkv=1, D=64, ctx_lens=[1000], page_size=1024,
                           dtype="bf16")
    case.q[...] = 0.0
    out, lse = gpu_attn(case, num_splits=3)
    check(case, out, lse, TOL_BF16)
    np.testing.assert_allclose(lse, math.log(1016), atol=1e-5)


def test_single_dominant_key_returns_its_value():
    case = synth.attn_case(52, B=1, S=16, Hq=2, Hkv=1, D=128, ctx_lens=[512], page_size=512,
                           dtype="bf16")
    # key 300 is 8 * q-direction with a margin of >= 40 in score over every other key
    qdir = np.zeros(128, np.float32); qdir[0] = 1.0
    case.q[...] = 0.0
    case.q[..., 0] = 8.0
    case.k_pages[...] = synth.round_to_bf16(case.k_pages * 0.01)
    case.k_blk[...] = synth.round_to_bf16(case.k_blk * 0.01)
    k = synth.untile_k(case.k_pages)                      # [pool, Hkv, page, D]
    k[case.block_table[0, 0], 0, 300, :] = 0.0
    k[case.block_table[0, 0], 0, 300, 0] = 64.0
    case.k_pages = synth.tile_k(k)
    out, lse = gpu_attn(case)
    v = synth.untile_v(case.v_pages)[case.block_table[0, 0], 0, :, 300]
    for h in range(2):
        np.testing.assert_allclose(out[0, :, h, :], np.broadcast_to(v, (16, 128)), atol=1e-5)


def test_page_order_is_bit_invariant_and_block_order_within_tolerance():
    case = synth.attn_case(53, B=3, S=16, Hq=32, Hkv=2, D=128, ctx_lens=[1000, 3000, 64],
                           page_size=256, dtype="bf16", spare_frac=0.5)
    d = dev_case(case)
    ref, ref_lse = gpu_attn(case, d)
    g = synth.rng(54)
    P = case.k_pages.shape[0]
    perm = g.permutation(P)
    inv = np.argsort(perm)
    d2 = dict(d, k_pages=d["k_pages"][torch.from_numpy(perm).to(DEV)].contiguous(),
              v_pages=d["v_pages"][torch.from_numpy(perm).to(DEV)].contiguous(),
              block_table=torch.from_numpy(inv[case.block_table].astype(np.int32)).to(DEV))
    out, lse = gpu_attn(case, d2)
    assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)
    bp = torch.from_numpy(g.permutation(16)).to(DEV)
    d3 = dict(d, k_blk=d["k_blk"][:, :, bp].contiguous(), v_blk=d["v_blk"][:, :, :, bp].contiguous())
    out, _ = gpu_attn(case, d3)
    assert max_abs(out, ref) <= 2e-3


def test_split_count_only_changes_rounding():
    case = synth.attn_case(55, B=2, S=16, Hq=32, Hkv=2, D=128, ctx_lens=[5000, 2000],
                           page_size=256, dtype="bf16")
    outs = [gpu_attn(case, num_splits=s)[0] for s in (1, 2, 7, 20, 79)]
    for o in outs[1:]:
        assert max_abs(o, outs[0]) <= 2e-3


# -------------------------------------------------------------------------------- shapes / edges

@pytest.mark.parametrize("S,Hq,Hkv,D", [
    (16, 4, 4, 128),    # MHA: 16 query rows per KV head, padded to one 32-row wavefront
    (1, 8, 1, 128),     # a single block position
    (5, 6, 2, 64),      # rows = 15, head_dim 64
    (32, 32, 2, 128),   # 512 rows: two row groups per KV head
    (64, 4, 1, 64),
    (16, 16, 1, 64),
    (128, 32, 2, 128),  # block size 128: two block-key tiles, 2048 rows = 8 row groups
    (100, 8, 2, 128),   # block keys 64 + 36, S not a multiple of 8 (scalar block-V loads)
    (256, 4, 1, 64),    # the largest block: four block-key tiles
])
def test_shapes_bf16(S, Hq, Hkv, D):
    case = synth.attn_case(60 + S, B=2, S=S, Hq=Hq, Hkv=Hkv, D=D, ctx_lens=[333, 1200],
                           page_size=128, dtype="bf16")
    for splits in (1, 0):
        out, lse = gpu_attn(case, num_splits=splits)
        check(case, out, lse, TOL_BF16)


@pytest.mark.parametrize("S,Hq,Hkv,D", [(16, 8, 2, 128), (3, 3, 1, 64), (128, 4, 2, 64)])
def test_shapes_fp32(S, Hq, Hkv, D):
    case = synth.attn_case(70 + S, B=2, S=S, Hq=Hq, Hkv=Hkv, D=D, ctx_lens=[300, 5],
                           page_size=64, dtype="fp32")
    out, lse = gpu_attn(case)
    check(case, out, lse, TOL_FP32)


def _random_attn(seed):
    """A seeded random configuration within the documented limits: ragged paged contexts
    (empty ones included), any block size up to 256, GQA groups, both head sizes, page sizes that
    are multiples of 64, and a partition count."""
    g = np.random.default_rng(seed)
    hkv = int(g.integers(1, 4))
    B = int(g.integers(1, 7))
    return dict(B=B, S=int(g.choice([1, 2, 5, 16, 17, 31, 48, 64, 100, 128, 200, 256])),
                Hq=hkv * int(g.integers(1, 9)), Hkv=hkv, D=int(g.choice([64, 128])),
                ctx_lens=[int(x) for x in g.integers(0, 1500, size=B)],
                page_size=int(g.choice([64, 128, 192, 256, 512])),
                dtype="bf16" if g.random() < 0.75 else "fp32",
                splits=int(g.choice([0, 1, 2, 5])))


@pytest.mark.parametrize("seed", range(90, 102))
def test_random_shapes_within_the_limits(seed):
    cfg = _random_attn(seed)
    splits = cfg.pop("splits")
    dtype = cfg["dtype"]
    case = synth.attn_case(seed, shuffle_pages=True, spare_frac=0.25, **cfg)
    for s in sorted({0, splits}):
        out, lse = gpu_attn(case, num_splits=s)
        check(case, out, lse, TOL_BF16 if dtype == "bf16" else TOL_FP32)


def test_empty_context_and_tiny_tails():
    case = synth.attn_case(80, B=4, S=16, Hq=32, Hkv=2, D=128, ctx_lens=[0, 1, 63, 65],
                           page_size=64, dtype="bf16", nan_poison=True, spare_frac=1.0)
    for splits in (0, 1, 2):
        out, lse = gpu_attn(case, num_splits=splits, max_ctx_len=128)
        check(case, out, lse, TOL_BF16)


def test_bad_lengths_and_pages_give_nan_rows_only():
    case = synth.attn_case(81, B=3, S=16, Hq=32, Hkv=2, D=128, ctx_lens=[500, 700, 900],
                           page_size=256, dtype="bf16")
    d = dev_case(case)
    lens = d["ctx_lens"].clone()
    lens[1] = 5000                        # above max_ctx_len
    bt = d["block_table"].clone()
    bt[2, 1] = 10_000                     # page index outside the pool
    d.update(ctx_lens=lens, block_table=bt)
    ref, _ = oattn.block_attention_case(case)
    for splits in (1, 0):
        out, lse = gpu_attn(case, d, num_splits=splits, max_ctx_len=1024)
        assert np.isnan(out[1]).all() and np.isnan(out[2]).all() and np.isnan(lse[1:]).all()
        assert max_abs(out[0], ref[0]) <= TOL_BF16


@pytest.mark.parametrize("L", [4096, 4160])
def test_partition_tile_index_paths(L):
    """One partition of 64 tiles keeps its tile indices in registers and one of 65 stages them in
    LDS. Both must match the oracle, and both must catch a bad page in the partition's last tile."""
    case = synth.attn_case(83, B=2, S=16, Hq=8, Hkv=2, D=128, ctx_lens=[L, L - 100], page_size=64,
                           dtype="bf16")
    out, lse = gpu_attn(case, num_splits=1, max_ctx_len=L)
    ref = check(case, out, lse, TOL_BF16)
    d = dev_case(case)
    bt = d["block_table"].clone()
    bt[0, L // 64 - 1] = 10_000           # the last page of sequence 0, outside the pool
    d.update(block_table=bt)
    out, lse = gpu_attn(case, d, num_splits=1, max_ctx_len=L)
    assert np.isnan(out[0]).all() and np.isnan(lse[0]).all()
    assert max_abs(out[1], ref[1]) <= TOL_BF16


def test_deterministic_and_outputs_stay_in_bounds():
    case = synth.config_attn("ctx4k_bf16", ctx_len=3000)
    d = dev_case(case)
    guard = torch.full((2, 16 * 32 * 128 + 64), 7.0, dtype=torch.float32, device=DEV)
    outs = []
    for _ in range(3):
        out = guard[0, 32:32 + 16 * 32 * 128].view(1, 16, 32, 128)
        tt.block_attn(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["ctx_lens"],
                      d["k_blk"], d["v_blk"], scale=case.scale, max_ctx_len=3000, out=out)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy().copy())
        assert (guard[0, :32] == 7.0).all() and (guard[0, -32:] == 7.0).all()
        assert (guard[1] == 7.0).all()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


def test_timing_event_hook_skips_null_entries():
    """The profiling hook records the events it is given around the main kernel and after the
    merge; a None entry is skipped, and the output is the same as without events."""
    case = synth.attn_case(81, B=2, S=16, Hq=32, Hkv=2, D=128, ctx_lens=[4096, 3000],
                           page_size=256, dtype="bf16")
    ref_out, _ = gpu_attn(case, num_splits=8)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in evs:
        e.record()          # materialize the handles
    torch.cuda.synchronize()
    out_a, _ = gpu_attn(case, num_splits=8,
                        timing_events=[evs[0].cuda_event, None, evs[1].cuda_event])
    out_b, _ = gpu_attn(case, num_splits=8,
                        timing_events=[evs[2].cuda_event, evs[3].cuda_event, None])
    torch.cuda.synchronize()
    assert evs[0].elapsed_time(evs[1]) > 0.0 and evs[2].elapsed_time(evs[3]) > 0.0
    assert np.array_equal(out_a, ref_out) and np.array_equal(out_b, ref_out)


# ------------------------------------------------------------- workspace content, graph replays

def _attn_into(case, d, out, lse, workspace=None, **kw):
    tt.block_attn(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["ctx_lens"], d["k_blk"],
                  d["v_blk"], scale=case.scale, max_ctx_len=int(case.ctx_lens.max()), out=out,
                  return_lse=True, lse_out=lse, workspace=workspace, **kw)


def test_attention_output_does_not_depend_on_workspace_content():
    """The caller's workspace is never cleared: a workspace of arbitrary bytes, all ones, or left
    over by the previous call gives the same output bit for bit, and it matches the oracle."""
    case = synth.attn_case(91, B=4, S=16, Hq=32, Hkv=2, D=128, ctx_lens=[4096, 3000, 5000, 100],
                           page_size=256, dtype="bf16")
    d = dev_case(case)
    outs = []
    ws = torch.empty(32 << 20, dtype=torch.uint8, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(5)
    for fill in ("random", "ones", "previous", "previous"):
        if fill == "random":
            ws.copy_(torch.randint(0, 256, ws.shape, generator=g, device=DEV, dtype=torch.int32)
                     .to(torch.uint8))
        elif fill == "ones":
            ws.fill_(255)
        out = torch.empty((4, 16, 32, 128), dtype=torch.float32, device=DEV)
        lse = torch.empty((4, 32, 16), dtype=torch.float32, device=DEV)
        _attn_into(case, d, out, lse, workspace=ws)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)))
    check(case, outs[0][0], outs[0][1], TOL_BF16)
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])


def test_graph_replays_of_the_attention_match_eager_calls():
    """A captured attention call replayed several times, with eager work in between, and again
    after the lengths changed on the device (the partitions of every sequence are planned on the
    device, so they change without a new capture): every replay equals the eager call."""
    case = synth.attn_case(92, B=4, S=16, Hq=32, Hkv=2, D=128, ctx_lens=[4096, 4096, 4096, 4096],
                           page_size=256, dtype="bf16")
    d = dev_case(case)
    out = torch.empty((4, 16, 32, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((4, 32, 16), dtype=torch.float32, device=DEV)
    _attn_into(case, d, out, lse)                 # eager first: every one-time setup is done
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _attn_into(case, d, out, lse)
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    d["ctx_lens"].copy_(torch.tensor([4096, 900, 2500, 64], dtype=torch.int32, device=DEV))
    e_out, e_lse = torch.empty_like(out), torch.empty_like(lse)
    _attn_into(case, d, e_out, e_lse)
    torch.cuda.synchronize()
    for _ in range(2):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, e_out) and torch.equal(lse, e_lse)
    case.ctx_lens[:] = [4096, 900, 2500, 64]
    check(case, e_out.cpu().numpy().astype(np.float64), e_lse.cpu().numpy().astype(np.float64),
          TOL_BF16)
