"""The C ABI without a GPU: symbols, struct layouts, host-side validation and workspace sizing.

Every call here either fails validation or is a workspace-size query (ws == NULL), both of which
return before any HIP call, so nothing runs on a device.
"""
import ctypes as C
import os
import re

import pytest

from two_tower_cross_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "twotower.h")

FAKE = 0x10000  # a 256-byte aligned fake device address; never dereferenced by these calls


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(twotower_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert "twotower_block_attn" in names and "twotower_unmask" in names
    assert "twotower_denoise_step" in names
    for n in names:
        assert hasattr(L, n), n


def test_struct_layouts_match_the_header(L):
    for i, st in enumerate(_lib.STRUCTS):
        assert C.sizeof(st) == L.twotower_struct_size(i), st.__name__
        for j, (name, _) in enumerate(st._fields_):
            assert getattr(st, name).offset == L.twotower_struct_offset(i, j), (st.__name__, name)
        assert L.twotower_struct_offset(i, len(st._fields_)) == -1
    assert L.twotower_struct_size(99) == -1


def test_status_strings(L):
    assert [_lib.status_string(s) for s in range(5)] == [
        "TT_OK", "TT_EINVAL", "TT_ENOTSUP", "TT_ENOSPACE", "TT_EHIP"]
    assert _lib.status_string(1234) == "TT_UNKNOWN"


def attn_args(**over):
    a = _lib.BlockAttnArgs()
    vals = dict(batch=8, S=16, num_q_heads=32, num_kv_heads=2, head_dim=128, dtype=_lib.TT_BF16,
                out_dtype=_lib.TT_FP32, scale=128 ** -0.5, q=FAKE, k_pages=FAKE, v_pages=FAKE,
                num_pages=8, page_size=32768, max_pages_per_seq=1, max_ctx_len=32768,
                block_table=FAKE, ctx_lens=FAKE, k_blk=FAKE, v_blk=FAKE, out=FAKE, lse=None,
                num_splits=0)
    vals.update(over)
    for k, v in vals.items():
        setattr(a, k, v)
    return a


def query(name, a):
    n = C.c_size_t(12345)
    st = _lib.call(name, a, None, n, None)
    return st, n.value


def test_attention_workspace_query_and_plan():
    st, n = query("twotower_block_attn", attn_args())
    assert st == _lib.TT_OK
    # automatic (balanced) plan for 8 sequences x 2 KV heads at 32768 tokens: 128 partitions per KV
    # head (16 per sequence), 256-row fp16 partials + an fp32 (lse, scale exponent) pair per row,
    # plus the plan record (2 int32) of every sequence
    items = 8 * 2 * 16
    expect = (-(-items * 256 * 128 * 2 // 256) * 256 + -(-items * 256 * 8 // 256) * 256
              + -(-8 * 2 * 4 // 256) * 256)
    assert n == expect
    # one partition needs no workspace
    st, n = query("twotower_block_attn", attn_args(num_splits=1))
    assert st == _lib.TT_OK and n == 0
    st, n = query("twotower_block_attn", attn_args(dtype=_lib.TT_FP32, out_dtype=_lib.TT_FP32))
    assert st == _lib.TT_OK and n == 0


def ws_bytes(slots, rows, batch):
    up = lambda x: -(-x // 256) * 256
    return up(slots * rows * 128 * 2) + up(slots * rows * 8) + up(batch * 2 * 4)


def test_attention_short_partitions_use_128_row_groups():
    # one sequence of 131072 tokens: at 256 query rows the automatic plan would cut each KV head's
    # 2048 tiles into 128 partitions of 16 tiles (< 24), so the rows go into two groups of 128 and
    # every (KV head, row group) gets 64 partitions of 32 tiles: 2 x 2 x 64 slots of 128 rows
    a = attn_args(batch=1, page_size=131072, max_ctx_len=131072)
    st, n = query("twotower_block_attn", a)
    assert st == _lib.TT_OK and n == ws_bytes(2 * 2 * 64, 128, 1)
    # an explicit partition count keeps one group of 256 rows
    st, n = query("twotower_block_attn", attn_args(batch=1, page_size=131072, max_ctx_len=131072,
                                                   num_splits=128))
    assert st == _lib.TT_OK
    up = lambda x: -(-x // 256) * 256
    assert n == up(2 * 128 * 256 * 128 * 2) + up(2 * 128 * 256 * 8)
    # 4096 tokens: 64 tiles per KV head, one tile per partition either way
    st, n = query("twotower_block_attn", attn_args(batch=1, page_size=4096, max_ctx_len=4096))
    assert st == _lib.TT_OK and n == ws_bytes(2 * 2 * 64, 128, 1)
    # the 32K loop (32 tiles per partition) keeps 256 rows: the workspace pinned above
    st, n = query("twotower_block_attn", attn_args())
    assert st == _lib.TT_OK and n == ws_bytes(8 * 2 * 16, 256, 8)
    # 128 rows or fewer (G * S <= 128) are one group already
    st, n = query("twotower_block_attn", attn_args(batch=1, num_q_heads=16, page_size=131072,
                                                   max_ctx_len=131072))
    assert st == _lib.TT_OK and n == ws_bytes(2 * 128, 128, 1)


def test_attention_workspace_too_small_reports_size():
    a = attn_args()
    st, need = query("twotower_block_attn", a)
    n = C.c_size_t(need - 1)
    st = _lib.call("twotower_block_attn", a, C.c_void_p(FAKE), n, None)
    assert st == _lib.TT_ENOSPACE and n.value == need


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=96), _lib.TT_ENOTSUP),
    (dict(S=257), _lib.TT_ENOTSUP),
    (dict(page_size=100, max_ctx_len=100), _lib.TT_ENOTSUP),
    (dict(out_dtype=_lib.TT_BF16, dtype=_lib.TT_FP32), _lib.TT_ENOTSUP),
    (dict(num_q_heads=31), _lib.TT_EINVAL),
    (dict(S=0), _lib.TT_EINVAL),
    (dict(scale=-1.0), _lib.TT_EINVAL),
    (dict(scale=float("nan")), _lib.TT_EINVAL),
    (dict(max_ctx_len=32769), _lib.TT_EINVAL),
    (dict(q=FAKE + 8), _lib.TT_EINVAL),
    (dict(v_pages=None), _lib.TT_EINVAL),
    (dict(ctx_lens=None), _lib.TT_EINVAL),
    (dict(num_splits=-1), _lib.TT_EINVAL),
    (dict(dtype=7), _lib.TT_EINVAL),
])
def test_attention_argument_errors(over, code):
    st, _ = query("twotower_block_attn", attn_args(**over))
    assert st == code, _lib.status_string(st)


def unmask_args(**over):
    a = _lib.UnmaskArgs()
    vals = dict(batch=8, S=16, vocab=131072, ld=131072, logits=FAKE, masked=FAKE, tokens=FAKE,
                confidence=None, n_committed=None, threshold=0.9, min_commit=1, commit_all=0)
    vals.update(over)
    for k, v in vals.items():
        setattr(a, k, v)
    return a


def test_unmask_workspace_and_errors():
    st, n = query("twotower_unmask", unmask_args())
    assert st == _lib.TT_OK and n == 8 * 16 * 16 * 16
    for over, code in [(dict(S=257), _lib.TT_ENOTSUP), (dict(ld=100), _lib.TT_EINVAL),
                       (dict(threshold=float("nan")), _lib.TT_EINVAL),
                       (dict(tokens=None), _lib.TT_EINVAL), (dict(vocab=0), _lib.TT_EINVAL),
                       (dict(tokens=FAKE + 2), _lib.TT_EINVAL)]:
        assert query("twotower_unmask", unmask_args(**over))[0] == code, over


def test_packed_weight_size_and_validation(L):
    # ceil(out / 32) slabs of ceil(in / 16) 1 KB blocks
    assert L.twotower_packed_weight_bytes(4608, 2048) == 144 * 128 * 1024
    assert L.twotower_packed_weight_bytes(1004, 136) == 32 * 9 * 1024
    assert L.twotower_packed_weight_bytes(0, 16) == 0
    assert L.twotower_packed_weight_bytes(16, -1) == 0
    # argument errors are reported before anything is enqueued
    assert L.twotower_pack_weight(FAKE, 64, 12, FAKE, None) == _lib.TT_ENOTSUP   # 12 % 8 != 0
    assert L.twotower_pack_weight(None, 64, 64, FAKE, None) == _lib.TT_EINVAL
    assert L.twotower_pack_weight(FAKE, 64, 64, None, None) == _lib.TT_EINVAL
    assert L.twotower_pack_weight(FAKE + 8, 64, 64, FAKE, None) == _lib.TT_EINVAL
    assert L.twotower_pack_weight(FAKE, 0, 64, FAKE, None) == _lib.TT_EINVAL


def test_projection_queries_and_errors():
    q = _lib.QkvArgs(8, 16, 2048, 32, 2, 128, FAKE, FAKE, FAKE, FAKE, FAKE)
    st, n = query("twotower_qkv_projection", q)
    # 72 tiles of 64 features -> K in 3 partitions (one work-group per compute unit): fp32 partials,
    # then one arrival counter (a 128-byte line) per tile for the merge inside the kernel
    assert st == _lib.TT_OK and n == 3 * 128 * 4608 * 4 + 72 * 128
    q.hidden = 2044
    assert query("twotower_qkv_projection", q)[0] == _lib.TT_ENOTSUP
    o = _lib.OutProjArgs(128, 2048, 4096, 0, FAKE, FAKE, FAKE, FAKE)
    st, n = query("twotower_out_projection", o)
    assert st == _lib.TT_OK and n == 8 * 128 * 2048 * 4 + 32 * 128   # 32 tiles x 8 K partitions
    o.o = FAKE + 4
    assert query("twotower_out_projection", o)[0] == _lib.TT_EINVAL
    lm = _lib.LmHeadArgs(128, 2048, 131072, 0, 131072, FAKE, FAKE, FAKE)
    st, n = query("twotower_lm_head", lm)
    assert st == _lib.TT_OK and n == 0   # 512 tiles of 256 features fill the GPU without K partitions
    lm.ld = 131070
    assert query("twotower_lm_head", lm)[0] == _lib.TT_EINVAL


def lm_unmask_args(**over):
    a = _lib.LmHeadUnmaskArgs()
    a.lm = _lib.LmHeadArgs(128, 2048, 131072, 0, 131072, FAKE, FAKE, FAKE)
    a.unmask = unmask_args(logits=None, vocab=0, ld=0)   # ignored by the fused call
    for k, v in over.items():
        obj, f = k.split("__")
        setattr(getattr(a, obj), f, v)
    return a


def test_lm_head_unmask_workspace_and_errors():
    st, n = query("twotower_lm_head_unmask", lm_unmask_args())
    # one (max, index, sum) slot of 16 bytes per row and 256-logit tile
    assert st == _lib.TT_OK and n == 128 * 512 * 16
    assert query("twotower_lm_head_unmask", lm_unmask_args(lm__logits=None, lm__ld=0))[0] == _lib.TT_OK
    for over, code in [(dict(lm__rows=127), _lib.TT_EINVAL),          # rows != batch * S
                       (dict(unmask__S=257, lm__rows=8 * 257), _lib.TT_ENOTSUP),
                       (dict(lm__ld=131070), _lib.TT_EINVAL),
                       (dict(lm__vocab=131074, lm__ld=131076), _lib.TT_ENOTSUP),
                       (dict(lm__h=FAKE + 8), _lib.TT_EINVAL),
                       (dict(lm__logits=FAKE + 4), _lib.TT_EINVAL),
                       (dict(unmask__masked=None), _lib.TT_EINVAL),
                       (dict(unmask__threshold=float("nan")), _lib.TT_EINVAL)]:
        assert query("twotower_lm_head_unmask", lm_unmask_args(**over))[0] == code, over


def test_denoise_step_validation():
    a = _lib.DenoiseStepArgs()
    a.num_layers, a.hidden, a.vocab = 6, 2048, 131072
    a.attn = attn_args()
    assert query("twotower_denoise_step", a)[0] == _lib.TT_EINVAL   # layer arrays missing
    arr = (C.c_void_p * 6)(*([FAKE] * 6))
    vpp = C.POINTER(C.c_void_p)
    for f in ("k_pages", "v_pages", "w_qkv", "w_o", "k_blk", "v_blk"):
        setattr(a, f, C.cast(arr, vpp))
    for f in ("w_lm", "h_in", "h_work", "q", "attn_out", "logits"):
        setattr(a, f, FAKE)
    a.logits_ld = 131072
    a.unmask = unmask_args()
    st, n = query("twotower_denoise_step", a)
    assert st == _lib.TT_OK and n > 0
    a.logits = None   # logits are optional: the unmasking is fused into the lm-head
    assert query("twotower_denoise_step", a)[0] == _lib.TT_OK
    a.attn = attn_args(dtype=_lib.TT_FP32)
    assert query("twotower_denoise_step", a)[0] == _lib.TT_ENOTSUP


def append_args(**over):
    a = _lib.KvAppendArgs()
    arr = (C.c_void_p * 6)(*([FAKE] * 6))
    vpp = C.POINTER(C.c_void_p)
    a.num_layers, a.batch, a.num_kv_heads, a.head_dim, a.S = 6, 8, 2, 128, 16
    a.dtype, a.num_pages, a.page_size, a.max_pages_per_seq = _lib.TT_BF16, 1100, 256, 130
    for f in ("k_pages", "v_pages", "k_new", "v_new"):
        setattr(a, f, C.cast(arr, vpp))
    for f in ("block_table", "ctx_lens", "free_pages", "free_count", "status"):
        setattr(a, f, FAKE)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_kv_append_workspace_and_errors():
    st, n = query("twotower_kv_append", append_args())
    assert st == _lib.TT_OK and n == 256          # one int32 per sequence, 256-byte aligned
    for over, code in [(dict(num_layers=0), _lib.TT_EINVAL), (dict(num_layers=17), _lib.TT_ENOTSUP),
                       (dict(page_size=100), _lib.TT_ENOTSUP), (dict(S=0), _lib.TT_EINVAL),
                       (dict(dtype=5), _lib.TT_EINVAL), (dict(free_count=None), _lib.TT_EINVAL),
                       (dict(status=None), _lib.TT_EINVAL), (dict(k_new=None), _lib.TT_EINVAL)]:
        assert query("twotower_kv_append", append_args(**over))[0] == code, over
    arr = (C.c_void_p * 6)(*([FAKE] * 5 + [FAKE + 1]))   # misaligned last layer
    a = append_args(v_pages=C.cast(arr, C.POINTER(C.c_void_p)))
    assert query("twotower_kv_append", a)[0] == _lib.TT_EINVAL


def test_loss_entry_points_validate_and_size():
    c = _lib.MaskCorruptArgs(8, 16, 131071, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    st, n = query("twotower_mask_corrupt", c)
    assert st == _lib.TT_OK and n == 0
    c.u_mask = None
    assert query("twotower_mask_corrupt", c)[0] == _lib.TT_EINVAL
    a = _lib.MaskedNllArgs(8, 16, 131072, 0, 131072, FAKE, FAKE, FAKE, FAKE, None, None)
    st, n = query("twotower_masked_nll", a)
    assert st == _lib.TT_OK and n == 8 * 16 * 16 * 16     # the unmasking's chunk triples
    a.S = 200
    assert query("twotower_masked_nll", a)[0] == _lib.TT_OK   # no 64-position limit here
    for over, code in [(dict(targets=None), _lib.TT_EINVAL), (dict(nll=FAKE + 2), _lib.TT_EINVAL),
                       (dict(ld=100), _lib.TT_EINVAL), (dict(S=0), _lib.TT_EINVAL)]:
        b = _lib.MaskedNllArgs(8, 16, 131072, 0, 131072, FAKE, FAKE, FAKE, FAKE, None, None)
        for k, v in over.items():
            setattr(b, k, v)
        assert query("twotower_masked_nll", b)[0] == code, over


def test_cache_shape_helpers_match_the_tiled_layouts():
    """k_pages_shape / v_pages_shape are the shapes of the header's tiled caches: a token-major
    [pages, Hkv, page, D] K cache tiled by synth.tile_k and a dim-major V cache tiled by
    synth.tile_v (64-token tiles of 8-wide chunks) land exactly there, and the binding's shape
    check accepts them and refuses the untiled layouts."""
    import numpy as np
    import torch

    import synth
    import two_tower_cross_amd as tt

    P, Hkv, page, D = 3, 2, 128, 64
    k = np.zeros((P, Hkv, page, D), np.float32)
    v = np.zeros((P, Hkv, D, page), np.float32)
    assert synth.tile_k(k).shape == tt.k_pages_shape(P, Hkv, page, D)
    assert synth.tile_v(v).shape == tt.v_pages_shape(P, Hkv, page, D)
    assert tt._cache_dims(torch.empty(tt.k_pages_shape(P, Hkv, page, D))) == (P, Hkv, page, D)
    for bad in [(P, Hkv, page, D), (P, Hkv, page // 64, D, 64), (P, Hkv, 2, 8, 32, 8)]:
        with pytest.raises(ValueError):
            tt._cache_dims(torch.empty(bad))


def test_stream_read_probe_validation(L):
    f = L.twotower_probe_stream_read
    assert f(None, 1 << 20, 256, C.c_void_p(FAKE), None) == _lib.TT_EINVAL
    assert f(C.c_void_p(FAKE), 0, 256, C.c_void_p(FAKE), None) == _lib.TT_EINVAL
    assert f(C.c_void_p(FAKE), 1000, 256, C.c_void_p(FAKE), None) == _lib.TT_EINVAL   # not x16
    assert f(C.c_void_p(FAKE + 8), 1 << 20, 256, C.c_void_p(FAKE), None) == _lib.TT_EINVAL
    assert f(C.c_void_p(FAKE), 1 << 20, 0, C.c_void_p(FAKE), None) == _lib.TT_EINVAL
    assert f(C.c_void_p(FAKE), 1 << 20, 65537, C.c_void_p(FAKE), None) == _lib.TT_EINVAL
    assert f(C.c_void_p(FAKE), 1 << 20, 256, None, None) == _lib.TT_EINVAL


def test_mfma_rate_probe_validation(L):
    f = L.twotower_probe_mfma_rate
    assert f(0, 256, 64, None, None) == _lib.TT_EINVAL
    assert f(0, 256, 64, C.c_void_p(FAKE + 2), None) == _lib.TT_EINVAL   # misaligned
    assert f(-1, 256, 64, C.c_void_p(FAKE), None) == _lib.TT_EINVAL
    assert f(4, 256, 64, C.c_void_p(FAKE), None) == _lib.TT_EINVAL
    assert f(0, 0, 64, C.c_void_p(FAKE), None) == _lib.TT_EINVAL
    assert f(0, 65537, 64, C.c_void_p(FAKE), None) == _lib.TT_EINVAL
    assert f(0, 256, 0, C.c_void_p(FAKE), None) == _lib.TT_EINVAL
    assert f(0, 256, (1 << 20) + 1, C.c_void_p(FAKE), None) == _lib.TT_EINVAL


def test_static_attention_entry_validates_before_touching_the_device(L):
    """The no-allocation entry point checks its arguments and the scratch size on the host first
    (here no device is ever touched): bad arguments give TT_EINVAL, an explicit partition count
    whose partials exceed the 32 MiB scratch TT_ENOSPACE."""
    f = L.twotower_block_attn_static
    assert f(None, None) == _lib.TT_EINVAL
    assert f(C.byref(attn_args(head_dim=96)), None) == _lib.TT_ENOTSUP
    assert f(C.byref(attn_args(q=FAKE + 8)), None) == _lib.TT_EINVAL
    # 8 x 2 units x 256 partitions x 256 rows x (256 + 8) B = 276 MB of partials
    assert f(C.byref(attn_args(num_splits=256)), None) == _lib.TT_ENOSPACE
    assert _lib.STATIC_SCRATCH_BYTES == 32 << 20


def run_empty(name, a):
    """Size query, then a run with a (never dereferenced) workspace pointer: both TT_OK with 0
    bytes; the run returns before any HIP call, so it needs no device."""
    st, n = query(name, a)
    assert (st, n) == (_lib.TT_OK, 0), (name, _lib.status_string(st), n)
    m = C.c_size_t(0)
    st = _lib.call(name, a, C.c_void_p(FAKE), m, None)
    assert st == _lib.TT_OK, (name, _lib.status_string(st))


def test_empty_batch_is_a_no_op_with_null_device_pointers():
    """batch = 0 (rows = 0): sizes still checked, no workspace, nothing launched, TT_OK, and the
    device pointers may be NULL (as PyTorch's empty tensors give); a nonzero batch still needs
    them."""
    nulls = dict(q=None, k_pages=None, v_pages=None, k_blk=None, v_blk=None, out=None,
                 block_table=None, ctx_lens=None)
    run_empty("twotower_block_attn", attn_args(batch=0, **nulls))
    assert _lib.lib().twotower_block_attn_static(C.byref(attn_args(batch=0, **nulls)), None) == \
        _lib.TT_OK
    assert query("twotower_block_attn", attn_args(batch=0, S=0, **nulls))[0] == _lib.TT_EINVAL
    assert query("twotower_block_attn", attn_args(batch=1, **nulls))[0] == _lib.TT_EINVAL
    run_empty("twotower_unmask", unmask_args(batch=0, logits=None, masked=None, tokens=None))
    assert query("twotower_unmask", unmask_args(batch=1, tokens=None))[0] == _lib.TT_EINVAL
    run_empty("twotower_qkv_projection", _lib.QkvArgs(0, 16, 2048, 32, 2, 128, None, None, None,
                                                      None, None))
    run_empty("twotower_out_projection", _lib.OutProjArgs(0, 2048, 4096, 0, None, None, None, None))
    run_empty("twotower_lm_head", _lib.LmHeadArgs(0, 2048, 131072, 0, 131072, None, None, None))
    lu = lm_unmask_args(lm__rows=0, lm__h=None, lm__w_lm=None, lm__logits=None, unmask__batch=0,
                        unmask__masked=None, unmask__tokens=None)
    run_empty("twotower_lm_head_unmask", lu)
    run_empty("twotower_mask_corrupt",
              _lib.MaskCorruptArgs(0, 16, 131071, 0, None, None, None, None, None, None))
    run_empty("twotower_masked_nll",
              _lib.MaskedNllArgs(0, 16, 131072, 0, 131072, None, None, None, None, None, None))
    empty = (C.c_void_p * 6)()   # host arrays of null layer pointers
    vpp = C.POINTER(C.c_void_p)
    ap = append_args(batch=0, block_table=None, ctx_lens=None, free_pages=None, free_count=None,
                     status=None, **{f: C.cast(empty, vpp) for f in ("k_pages", "v_pages", "k_new",
                                                                    "v_new")})
    run_empty("twotower_kv_append", ap)
    ap.k_pages = None                        # the host arrays themselves are still required
    assert query("twotower_kv_append", ap)[0] == _lib.TT_EINVAL
    s = _lib.DenoiseStepArgs()
    s.num_layers, s.hidden, s.vocab = 6, 2048, 131072
    s.attn = attn_args(batch=0, **nulls)
    for f in ("k_pages", "v_pages", "w_qkv", "w_o", "k_blk", "v_blk"):
        setattr(s, f, C.cast(empty, vpp))
    s.unmask = unmask_args(batch=0, logits=None, masked=None, tokens=None)
    run_empty("twotower_denoise_step", s)
    s.attn = attn_args(batch=1, **nulls)
    assert query("twotower_denoise_step", s)[0] == _lib.TT_EINVAL
