"""ctypes view of ``libtwotower.so``: struct mirrors of ``include/twotower.h`` and the loader.

Argument marshalling only; every step of the computation runs in the library's HIP kernels.
Loading fails loudly (``LibraryNotBuilt``) when the shared library is missing: there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("TWOTOWER_LIB", os.path.join(HERE, "libtwotower.so"))

TT_OK, TT_EINVAL, TT_ENOTSUP, TT_ENOSPACE, TT_EHIP = range(5)
TT_FP32, TT_BF16 = 0, 1
TT_APPEND_OUT_OF_PAGES, TT_APPEND_NO_ROOM_IN_TABLE, TT_APPEND_BAD_PAGE = 1, 2, 4
STATIC_SCRATCH_BYTES = 32 << 20
ABI_VERSION = 9

i32, i64, f32, vp = C.c_int32, C.c_int64, C.c_float, C.c_void_p


class BlockAttnArgs(C.Structure):
    _fields_ = [("batch", i32), ("S", i32), ("num_q_heads", i32), ("num_kv_heads", i32),
                ("head_dim", i32), ("dtype", i32), ("out_dtype", i32), ("scale", f32),
                ("q", vp), ("k_pages", vp), ("v_pages", vp),
                ("num_pages", i32), ("page_size", i32), ("max_pages_per_seq", i32),
                ("max_ctx_len", i32),
                ("block_table", vp), ("ctx_lens", vp), ("k_blk", vp), ("v_blk", vp),
                ("out", vp), ("lse", vp), ("num_splits", i32), ("reserved0", i32),
                ("timing_events", C.POINTER(vp))]


class UnmaskArgs(C.Structure):
    _fields_ = [("batch", i32), ("S", i32), ("vocab", i32), ("reserved0", i32), ("ld", i64),
                ("logits", vp), ("masked", vp), ("tokens", vp), ("confidence", vp),
                ("n_committed", vp), ("threshold", f32), ("min_commit", i32),
                ("commit_all", i32), ("reserved1", i32)]


class QkvArgs(C.Structure):
    _fields_ = [("batch", i32), ("S", i32), ("hidden", i32), ("num_q_heads", i32),
                ("num_kv_heads", i32), ("head_dim", i32), ("h", vp), ("w_qkv", vp), ("q", vp),
                ("k_blk", vp), ("v_blk", vp)]


class OutProjArgs(C.Structure):
    _fields_ = [("rows", i32), ("hidden", i32), ("in_features", i32), ("reserved0", i32),
                ("h_in", vp), ("o", vp), ("w_o", vp), ("h_out", vp)]


class LmHeadArgs(C.Structure):
    _fields_ = [("rows", i32), ("hidden", i32), ("vocab", i32), ("reserved0", i32), ("ld", i64),
                ("h", vp), ("w_lm", vp), ("logits", vp)]


class LmHeadUnmaskArgs(C.Structure):
    _fields_ = [("lm", LmHeadArgs), ("unmask", UnmaskArgs)]


class KvAppendArgs(C.Structure):
    _fields_ = [("num_layers", i32), ("batch", i32), ("num_kv_heads", i32), ("head_dim", i32),
                ("S", i32), ("dtype", i32), ("num_pages", i32), ("page_size", i32),
                ("max_pages_per_seq", i32), ("reserved0", i32),
                ("k_pages", C.POINTER(vp)), ("v_pages", C.POINTER(vp)),
                ("k_new", C.POINTER(vp)), ("v_new", C.POINTER(vp)),
                ("block_table", vp), ("ctx_lens", vp), ("free_pages", vp), ("free_count", vp),
                ("status", vp)]


class MaskCorruptArgs(C.Structure):
    _fields_ = [("batch", i32), ("S", i32), ("mask_id", i32), ("reserved0", i32),
                ("clean", vp), ("u_time", vp), ("u_mask", vp), ("noisy", vp), ("masked", vp),
                ("t_out", vp)]


class MaskedNllArgs(C.Structure):
    _fields_ = [("batch", i32), ("S", i32), ("vocab", i32), ("reserved0", i32), ("ld", i64),
                ("logits", vp), ("targets", vp), ("masked", vp), ("nll", vp), ("loss", vp),
                ("n_masked", vp)]


class DenoiseStepArgs(C.Structure):
    _fields_ = [("num_layers", i32), ("hidden", i32), ("vocab", i32), ("reserved0", i32),
                ("attn", BlockAttnArgs),
                ("k_pages", C.POINTER(vp)), ("v_pages", C.POINTER(vp)),
                ("w_qkv", C.POINTER(vp)), ("w_o", C.POINTER(vp)),
                ("k_blk", C.POINTER(vp)), ("v_blk", C.POINTER(vp)),
                ("w_lm", vp), ("h_in", vp), ("h_work", vp), ("q", vp), ("attn_out", vp),
                ("logits", vp), ("logits_ld", i64), ("unmask", UnmaskArgs),
                ("timing_events", C.POINTER(vp))]


STRUCTS = [BlockAttnArgs, UnmaskArgs, QkvArgs, OutProjArgs, LmHeadArgs, DenoiseStepArgs,
           LmHeadUnmaskArgs, KvAppendArgs, MaskCorruptArgs, MaskedNllArgs]

ENTRY_POINTS = {
    "twotower_block_attn": (BlockAttnArgs,),
    "twotower_unmask": (UnmaskArgs,),
    "twotower_qkv_projection": (QkvArgs,),
    "twotower_out_projection": (OutProjArgs,),
    "twotower_lm_head": (LmHeadArgs,),
    "twotower_denoise_step": (DenoiseStepArgs,),
    "twotower_lm_head_unmask": (LmHeadUnmaskArgs,),
    "twotower_kv_append": (KvAppendArgs,),
    "twotower_mask_corrupt": (MaskCorruptArgs,),
    "twotower_masked_nll": (MaskedNllArgs,),
}


class LibraryNotBuilt(RuntimeError):
    pass


class TwoTowerError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} returned {status_string(status)} ({status})")


_lib = None


def lib():
    """The loaded library (loaded once)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryNotBuilt(
                f"{LIB_PATH} is missing: build it with `python -m two_tower_cross_amd.build` "
                "(there is no fallback implementation)")
        L = C.CDLL(LIB_PATH)
        for name, (st,) in ENTRY_POINTS.items():
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [C.POINTER(st), vp, C.POINTER(C.c_size_t), vp]
        L.twotower_status_string.restype = C.c_char_p
        L.twotower_status_string.argtypes = [i32]
        L.twotower_abi_version.restype = i32
        L.twotower_abi_version.argtypes = []
        L.twotower_struct_size.restype = i64
        L.twotower_struct_size.argtypes = [i32]
        L.twotower_struct_offset.restype = i64
        L.twotower_struct_offset.argtypes = [i32, i32]
        L.twotower_packed_weight_bytes.restype = C.c_size_t
        L.twotower_packed_weight_bytes.argtypes = [i32, i32]
        L.twotower_pack_weight.restype = i32
        L.twotower_pack_weight.argtypes = [vp, i32, i32, vp, vp]
        L.twotower_block_attn_static.restype = i32
        L.twotower_block_attn_static.argtypes = [C.POINTER(BlockAttnArgs), vp]
        L.twotower_probe_stream_read.restype = i32
        L.twotower_probe_stream_read.argtypes = [vp, C.c_size_t, i32, vp, vp]
        L.twotower_probe_mfma_rate.restype = i32
        L.twotower_probe_mfma_rate.argtypes = [i32, i32, i32, vp, vp]
        if L.twotower_abi_version() != ABI_VERSION:
            raise RuntimeError("libtwotower ABI version mismatch")
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().twotower_status_string(int(status)).decode()


def call(name: str, args, ws, ws_bytes: C.c_size_t, stream) -> int:
    return getattr(lib(), name)(C.byref(args), ws, C.byref(ws_bytes), stream)
