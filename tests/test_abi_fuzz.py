"""Host-side argument checking of every entry point under random and extreme arguments (CPU).

Each case starts from valid arguments and overwrites one to three fields with values drawn from
edge sets (zero, negative, powers of two and their neighbours, the int32 limits, NaN and
infinities, null and misaligned pointers). Every call is a workspace-size query (ws == NULL),
which never launches anything, so no device is needed. A call must return one of the five
status codes, and a size it reports must be a multiple of the 256-byte workspace alignment; a
crash (for instance a division by zero in the planning) ends the test process. The sanitizer
build runs this file too, so undefined behaviour in the same code (signed overflow, invalid
enum loads, out-of-bounds reads) fails it there.
"""
import ctypes as C
import math
import random

import pytest

from two_tower_cross_amd import _lib

FAKE = 0x10000
LAYERS_MAX = 64           # host pointer arrays are this long, whatever num_layers says
INTS = [-(2 ** 31), -65536, -2, -1, 0, 1, 2, 3, 4, 7, 8, 15, 16, 17, 31, 32, 48, 63, 64, 65, 96,
        100, 127, 128, 129, 255, 256, 257, 1000, 1024, 4095, 4096, 4160, 8192, 32768, 65535,
        65536, 131072, 1 << 20, 1 << 24, 2 ** 31 - 1]
I64S = INTS + [2 ** 32, 2 ** 40, 2 ** 62]
FLOATS = [0.0, -0.0, -1.0, 1e-30, 1e-3, 0.088, 0.5, 0.9, 1.0, 2.0, 1e30, math.inf, -math.inf,
          math.nan]
PTRS = [None, FAKE, FAKE + 2, FAKE + 4, FAKE + 8, FAKE + 16, FAKE + 256]
CASES = 1500


def host_array(rng):
    """A host array of LAYERS_MAX device pointers, mostly valid, or a null array."""
    if rng.random() < 0.05:
        return None
    vals = [rng.choice(PTRS) if rng.random() < 0.1 else FAKE for _ in range(LAYERS_MAX)]
    return C.cast((C.c_void_p * LAYERS_MAX)(*vals), C.POINTER(C.c_void_p))


def draw(rng, ctype):
    if ctype is C.c_int32:
        return rng.choice(INTS) if rng.random() < 0.8 else rng.randint(-(2 ** 31), 2 ** 31 - 1)
    if ctype is C.c_int64:
        return rng.choice(I64S) if rng.random() < 0.8 else rng.randint(-(2 ** 40), 2 ** 40)
    if ctype is C.c_float:
        return rng.choice(FLOATS) if rng.random() < 0.8 else rng.uniform(-10.0, 10.0)
    if ctype is C.c_void_p:
        return rng.choice(PTRS)
    return None


def leaf_fields(struct, prefix=()):
    """(path, ctype) of every scalar or pointer field, nested structs flattened."""
    out = []
    for name, ctype in struct._fields_:
        if isinstance(ctype, type) and issubclass(ctype, C.Structure):
            out += leaf_fields(ctype, prefix + (name,))
        else:
            out.append((prefix + (name,), ctype))
    return out


def set_field(obj, path, value):
    for p in path[:-1]:
        obj = getattr(obj, p)
    setattr(obj, path[-1], value)


def fill(obj, values):
    for k, v in values.items():
        set_field(obj, tuple(k.split("__")), v)
    return obj


def attn_valid():
    return dict(batch=8, S=16, num_q_heads=32, num_kv_heads=2, head_dim=128, dtype=_lib.TT_BF16,
                out_dtype=_lib.TT_FP32, scale=0.088, q=FAKE, k_pages=FAKE, v_pages=FAKE,
                num_pages=1024, page_size=256, max_pages_per_seq=128, max_ctx_len=32768,
                block_table=FAKE, ctx_lens=FAKE, k_blk=FAKE, v_blk=FAKE, out=FAKE, lse=None,
                num_splits=0)


def unmask_valid():
    return dict(batch=8, S=16, vocab=131072, ld=131072, logits=FAKE, masked=FAKE, tokens=FAKE,
                confidence=FAKE, n_committed=FAKE, threshold=0.9, min_commit=1, commit_all=0)


def base(name, rng):
    """Valid arguments of entry point `name` (host arrays drawn fresh)."""
    if name == "twotower_block_attn":
        return fill(_lib.BlockAttnArgs(), attn_valid())
    if name == "twotower_unmask":
        return fill(_lib.UnmaskArgs(), unmask_valid())
    if name == "twotower_qkv_projection":
        return _lib.QkvArgs(8, 16, 2048, 32, 2, 128, FAKE, FAKE, FAKE, FAKE, FAKE)
    if name == "twotower_out_projection":
        return _lib.OutProjArgs(128, 2048, 4096, 0, FAKE, FAKE, FAKE, FAKE)
    if name == "twotower_lm_head":
        return _lib.LmHeadArgs(128, 2048, 131072, 0, 131072, FAKE, FAKE, FAKE)
    if name == "twotower_lm_head_unmask":
        a = _lib.LmHeadUnmaskArgs()
        a.lm = _lib.LmHeadArgs(128, 2048, 131072, 0, 131072, FAKE, FAKE, None)
        a.unmask = fill(_lib.UnmaskArgs(), unmask_valid())
        return a
    if name == "twotower_denoise_step":
        a = _lib.DenoiseStepArgs()
        a.num_layers, a.hidden, a.vocab = 6, 2048, 131072
        a.attn = fill(_lib.BlockAttnArgs(), attn_valid())
        a.attn.out_dtype = _lib.TT_BF16
        for f in ("w_lm", "h_in", "h_work", "q", "attn_out"):
            setattr(a, f, FAKE)
        a.logits, a.logits_ld = None, 131072
        a.unmask = fill(_lib.UnmaskArgs(), unmask_valid())
        return a
    if name == "twotower_kv_append":
        a = _lib.KvAppendArgs()
        a.num_layers, a.batch, a.num_kv_heads, a.head_dim, a.S = 6, 8, 2, 128, 16
        a.dtype, a.num_pages, a.page_size, a.max_pages_per_seq = _lib.TT_BF16, 1100, 256, 130
        for f in ("block_table", "ctx_lens", "free_pages", "free_count", "status"):
            setattr(a, f, FAKE)
        return a
    if name == "twotower_mask_corrupt":
        return _lib.MaskCorruptArgs(8, 16, 131071, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    if name == "twotower_masked_nll":
        return _lib.MaskedNllArgs(8, 16, 131072, 0, 131072, FAKE, FAKE, FAKE, FAKE, None, None)
    raise KeyError(name)


HOST_ARRAYS = {
    "twotower_denoise_step": ("k_pages", "v_pages", "w_qkv", "w_o", "k_blk", "v_blk"),
    "twotower_kv_append": ("k_pages", "v_pages", "k_new", "v_new"),
}
LAYER_FIELD = {"twotower_denoise_step": "num_layers", "twotower_kv_append": "num_layers"}


@pytest.mark.parametrize("name", sorted(_lib.ENTRY_POINTS))
def test_size_queries_survive_random_and_extreme_arguments(name):
    struct = _lib.ENTRY_POINTS[name][0]
    fields = [(p, t) for p, t in leaf_fields(struct)
              if t in (C.c_int32, C.c_int64, C.c_float, C.c_void_p) and "reserved" not in p[-1]]
    rng = random.Random(f"fuzz-{name}")
    statuses = set()
    for case in range(CASES):
        a = base(name, rng)
        keep = []   # host arrays must outlive the call
        for f in HOST_ARRAYS.get(name, ()):
            arr = host_array(rng)
            keep.append(arr)
            setattr(a, f, arr)
        for _ in range(rng.randint(1 if case else 0, 3)):
            path, ctype = rng.choice(fields)
            set_field(a, path, draw(rng, ctype))
        if name in LAYER_FIELD and getattr(a, LAYER_FIELD[name]) > LAYERS_MAX:
            setattr(a, LAYER_FIELD[name], LAYERS_MAX)   # the arrays hold LAYERS_MAX entries
        n = C.c_size_t(12345)
        st = _lib.call(name, a, None, n, None)
        assert st in (_lib.TT_OK, _lib.TT_EINVAL, _lib.TT_ENOTSUP), (name, case, st)
        if st == _lib.TT_OK:
            assert n.value % 256 == 0, (name, case, n.value)
        statuses.add(st)
    # the draws reach both the accepting and the rejecting paths
    assert _lib.TT_OK in statuses and _lib.TT_EINVAL in statuses, statuses
