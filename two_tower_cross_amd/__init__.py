"""Thin PyTorch binding of ``libtwotower.so`` (MI355X denoise step of TwoTower block diffusion).

Tensors supply device memory and torch's current stream supplies the HIP stream; every step of
the computation runs in the library's hand-written HIP kernels. The functions here only check
tensor metadata, build the C argument structs and size the workspace. If the shared library
is missing, every call raises ``LibraryNotBuilt`` (there is no fallback).

Layouts follow ``include/twotower.h``:
q [B,S,Hq,D]; k_pages [P,Hkv,page/64,D/8,64,8] (64-token tiles of 8-dimension chunks);
v_pages [P,Hkv,page/64,8,D,8] (64-token tiles of 8-token chunks); k_blk [B,Hkv,S,D];
v_blk [B,Hkv,D,S]; block_table [B,max_pages] int32; ctx_lens [B] int32; logits [B,S,V] fp32.
"""
from __future__ import annotations

import ctypes as C
import math

import torch

from . import _lib
from ._lib import LibraryNotBuilt, TwoTowerError, TT_BF16, TT_FP32  # noqa: F401

__all__ = ["block_attn", "unmask", "qkv_projection", "out_projection", "lm_head",
           "lm_head_unmask", "kv_append", "mask_corrupt", "masked_nll", "DenoiseStep",
           "PackedWeight", "pack_weight", "k_pages_shape", "v_pages_shape", "probe_stream_read",
           "probe_mfma_rate",
           "LibraryNotBuilt", "TwoTowerError", "library_path"]


def library_path() -> str:
    _lib.lib()
    return _lib.LIB_PATH


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TT_BF16
    if t.dtype == torch.float32:
        return TT_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(t: torch.Tensor, name: str, device, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _run(name: str, args, device, workspace=None) -> None:
    n = C.c_size_t(0)
    st = _lib.call(name, args, None, n, None)
    if st != _lib.TT_OK:
        raise TwoTowerError(name, st)
    # ws == NULL always means "query": a call that needs no workspace still gets a buffer.
    if workspace is None:
        ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=device)
    else:
        _check(workspace, "workspace", device, torch.uint8, 1)
        if workspace.numel() < n.value:
            raise ValueError(f"{name} needs a workspace of {n.value} bytes, got {workspace.numel()}")
        ws = workspace
    n = C.c_size_t(ws.numel())
    st = _lib.call(name, args, _p(ws), n, _stream())
    if st != _lib.TT_OK:
        raise TwoTowerError(name, st)


def k_pages_shape(num_pages, num_kv_heads, page_size, head_dim):
    """Shape of a K cache in the library's layout: 64-token tiles of 8-element chunks,
    chunk-major ([..., page_size / 64, head_dim / 8, 64, 8]; see include/twotower.h)."""
    return (num_pages, num_kv_heads, page_size // 64, head_dim // 8, 64, 8)


def v_pages_shape(num_pages, num_kv_heads, page_size, head_dim):
    """Shape of a V cache: 64-token tiles of 8-token chunks ([..., page_size / 64, 8, head_dim,
    8])."""
    return (num_pages, num_kv_heads, page_size // 64, 8, head_dim, 8)


def _cache_dims(k_pages):
    """(num_pages, num_kv_heads, page_size, head_dim) of a K cache tensor."""
    if k_pages.dim() != 6 or tuple(k_pages.shape[4:]) != (64, 8):
        raise ValueError("k_pages must have the shape k_pages_shape(...)")
    P, Hkv, tiles, chunks = k_pages.shape[:4]
    return P, Hkv, tiles * 64, chunks * 8


def _attn_struct(q, k_pages, v_pages, block_table, ctx_lens, k_blk, v_blk, out, lse, scale,
                 max_ctx_len, num_splits):
    B, S, Hq, D = q.shape
    P, Hkv, page, _ = _cache_dims(k_pages)
    a = _lib.BlockAttnArgs()
    a.batch, a.S, a.num_q_heads, a.num_kv_heads, a.head_dim = B, S, Hq, Hkv, D
    a.dtype = _dt(q)
    a.out_dtype = _dt(out) if out is not None else a.dtype
    a.scale = float(scale)
    a.q, a.k_pages, a.v_pages = _p(q), _p(k_pages), _p(v_pages)
    a.num_pages, a.page_size = P, page
    a.max_pages_per_seq = block_table.shape[1]
    a.max_ctx_len = int(max_ctx_len)
    a.block_table, a.ctx_lens = _p(block_table), _p(ctx_lens)
    a.k_blk, a.v_blk = _p(k_blk), _p(v_blk)
    a.out, a.lse = _p(out), _p(lse)
    a.num_splits = int(num_splits)
    return a


def block_attn(q, k_pages, v_pages, block_table, ctx_lens, k_blk, v_blk, *, scale=None,
               max_ctx_len=None, out_dtype=None, return_lse=False, num_splits=0, out=None,
               lse_out=None, timing_events=None, no_alloc=False, workspace=None):
    """Denoiser block attention at one layer; returns ``out`` (and ``lse`` [B,Hq,S] fp32).

    ``max_ctx_len`` bounds ctx_lens (used to plan the context partitions; default: the page
    table's capacity). ``num_splits`` 0 lets the library choose the partition count.
    ``timing_events``: optional 3 hipEvent_t handles (``torch.cuda.Event(...).cuda_event``, or
    events created with hipEventDisableSystemFence), recorded before and after the main kernel and
    after the partition merge; a None entry is not recorded.
    ``no_alloc``: call twotower_block_attn_static (no workspace; the library's per-device scratch);
    nothing is allocated here either, so ``out`` (and ``lse_out`` with ``return_lse``) must be
    given. ``workspace``: a uint8 device tensor used as the call's workspace instead of a new one
    (at least the size the library asks for; its contents need no initialization).
    """
    dev = q.device
    _check(q, "q", dev, ndim=4)
    B, S, Hq, D = q.shape
    _check(k_pages, "k_pages", dev, q.dtype, 6)
    _check(v_pages, "v_pages", dev, q.dtype, 6)
    _check(k_blk, "k_blk", dev, q.dtype, 4)
    _check(v_blk, "v_blk", dev, q.dtype, 4)
    _check(block_table, "block_table", dev, torch.int32, 2)
    _check(ctx_lens, "ctx_lens", dev, torch.int32, 1)
    P, Hkv, page, Dk = _cache_dims(k_pages)
    if (Dk != D or tuple(v_pages.shape) != v_pages_shape(P, Hkv, page, D)
            or tuple(k_blk.shape) != (B, Hkv, S, D) or tuple(v_blk.shape) != (B, Hkv, D, S)
            or block_table.shape[0] != B or ctx_lens.shape[0] != B):
        raise ValueError("inconsistent attention shapes")
    if no_alloc and (out is None or (return_lse and lse_out is None)):
        raise ValueError("no_alloc: pass out (and lse_out to return the log-sum-exp)")
    if out is None:
        od = q.dtype if out_dtype is None else out_dtype
        out = torch.empty((B, S, Hq, D), dtype=od, device=dev)
    else:
        _check(out, "out", dev, None, 4)
    lse = None
    if return_lse:
        if lse_out is None:
            lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
        else:
            _check(lse_out, "lse_out", dev, torch.float32, 3)
            if tuple(lse_out.shape) != (B, Hq, S):
                raise ValueError("lse_out must be [B, Hq, S]")
            lse = lse_out
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_ctx_len is None:
        max_ctx_len = block_table.shape[1] * page
    a = _attn_struct(q, k_pages, v_pages, block_table, ctx_lens, k_blk, v_blk, out, lse, scale,
                     max_ctx_len, num_splits)
    if timing_events is not None:
        if len(timing_events) != 3:
            raise ValueError("timing_events takes 3 events")
        ev = (C.c_void_p * 3)(*timing_events)
        a.timing_events = C.cast(ev, C.POINTER(C.c_void_p))
    if no_alloc:
        st = _lib.lib().twotower_block_attn_static(C.byref(a), _stream())
        if st != _lib.TT_OK:
            raise TwoTowerError("twotower_block_attn_static", st)
    else:
        _run("twotower_block_attn", a, dev, workspace)
    return (out, lse) if return_lse else out


def unmask(logits, masked, tokens, threshold, *, min_commit=False, commit_all=False,
           confidence=None, n_committed=None):
    """Confidence unmasking; updates ``masked`` and ``tokens`` in place.

    Returns (confidence [B,S] fp32, written where masked on entry; n_committed [B] int32), into
    the given ``confidence`` / ``n_committed`` tensors when passed (else new ones, NaN / 0).
    """
    dev = logits.device
    _check(masked, "masked", dev, torch.uint8, 2)
    _check(tokens, "tokens", dev, torch.int32, 2)
    if logits.dtype != torch.float32 or logits.dim() != 3 or logits.stride(2) != 1:
        raise ValueError("logits must be fp32 [B,S,V] with unit vocab stride")
    B, S, V = logits.shape
    if logits.stride(0) != S * logits.stride(1):
        raise ValueError("logits rows must be evenly strided")
    if confidence is None:
        conf = torch.full((B, S), float("nan"), dtype=torch.float32, device=dev)
    else:
        _check(confidence, "confidence", dev, torch.float32, 2)
        conf = confidence
    if n_committed is None:
        ncom = torch.zeros((B,), dtype=torch.int32, device=dev)
    else:
        _check(n_committed, "n_committed", dev, torch.int32, 1)
        ncom = n_committed
    if tuple(conf.shape) != (B, S) or tuple(ncom.shape) != (B,):
        raise ValueError("confidence / n_committed shape mismatch")
    a = _lib.UnmaskArgs()
    a.batch, a.S, a.vocab, a.ld = B, S, V, logits.stride(1)
    a.logits, a.masked, a.tokens = _p(logits), _p(masked), _p(tokens)
    a.confidence, a.n_committed = _p(conf), _p(ncom)
    a.threshold = float(threshold)
    a.min_commit, a.commit_all = int(bool(min_commit)), int(bool(commit_all))
    _run("twotower_unmask", a, dev)
    return conf, ncom


class PackedWeight:
    """A bf16 weight [out_features, in_features] in the library's packed operand layout
    (``include/twotower.h``), written by ``twotower_pack_weight``."""

    def __init__(self, data, out_features, in_features):
        self.data, self.out_features, self.in_features = data, out_features, in_features

    @property
    def shape(self):
        return (self.out_features, self.in_features)

    @property
    def device(self):
        return self.data.device


def pack_weight(w):
    """Pack a row-major bf16 weight [out_features, in_features] (on the GPU) for the projections."""
    if isinstance(w, PackedWeight):
        return w
    _check(w, "w", w.device, torch.bfloat16, 2)
    n, k = w.shape
    nbytes = _lib.lib().twotower_packed_weight_bytes(n, k)
    data = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=w.device)
    st = _lib.lib().twotower_pack_weight(_p(w), n, k, _p(data), _stream())
    if st != _lib.TT_OK:
        raise TwoTowerError("twotower_pack_weight", st)
    return PackedWeight(data, n, k)


def _packed(w, name, device):
    if not isinstance(w, PackedWeight):
        _check(w, name, device, torch.bfloat16, 2)
        w = pack_weight(w)
    elif w.device != device:
        raise ValueError(f"{name} is on {w.device}, expected {device}")
    return w


def qkv_projection(h, w_qkv, num_q_heads, num_kv_heads, head_dim, workspace=None, out=None):
    """[Q | K_blk | V_blk] = H W_qkv^T scattered to q [B,S,Hq,D], k_blk [B,Hkv,S,D],
    v_blk [B,Hkv,D,S] (bf16). ``w_qkv`` is a PackedWeight or a bf16 tensor (packed here).
    ``workspace``: a uint8 device tensor used instead of a new one (at least the size the library
    asks for; any content). ``out``: (q, k_blk, v_blk) tensors to write instead of new ones."""
    dev = h.device
    _check(h, "h", dev, torch.bfloat16, 3)
    w_qkv = _packed(w_qkv, "w_qkv", dev)
    B, S, hidden = h.shape
    if tuple(w_qkv.shape) != ((num_q_heads + 2 * num_kv_heads) * head_dim, hidden):
        raise ValueError("w_qkv shape mismatch")
    shapes = ((B, S, num_q_heads, head_dim), (B, num_kv_heads, S, head_dim),
              (B, num_kv_heads, head_dim, S))
    if out is None:
        q, kb, vb = (torch.empty(sh, dtype=torch.bfloat16, device=dev) for sh in shapes)
    else:
        q, kb, vb = out
        for t, sh, name in zip(out, shapes, ("q", "k_blk", "v_blk")):
            _check(t, name, dev, torch.bfloat16)
            if tuple(t.shape) != sh:
                raise ValueError(f"{name} must be {sh}")
    a = _lib.QkvArgs()
    a.batch, a.S, a.hidden = B, S, hidden
    a.num_q_heads, a.num_kv_heads, a.head_dim = num_q_heads, num_kv_heads, head_dim
    a.h, a.w_qkv, a.q, a.k_blk, a.v_blk = _p(h), _p(w_qkv.data), _p(q), _p(kb), _p(vb)
    _run("twotower_qkv_projection", a, dev, workspace)
    return q, kb, vb


def out_projection(h_in, o, w_o, out=None, workspace=None):
    """H_out = H_in + O W_o^T (bf16). ``o`` is [..., in_features] with the rows of ``h_in``.
    ``workspace``: as for qkv_projection."""
    dev = h_in.device
    _check(h_in, "h_in", dev, torch.bfloat16)
    _check(o, "o", dev, torch.bfloat16)
    w_o = _packed(w_o, "w_o", dev)
    hidden, inf = w_o.shape
    rows = h_in.numel() // hidden
    if h_in.shape[-1] != hidden or o.numel() != rows * inf:
        raise ValueError("out_projection shape mismatch")
    if out is None:
        out = torch.empty_like(h_in)
    a = _lib.OutProjArgs()
    a.rows, a.hidden, a.in_features = rows, hidden, inf
    a.h_in, a.o, a.w_o, a.h_out = _p(h_in), _p(o), _p(w_o.data), _p(out)
    _run("twotower_out_projection", a, dev, workspace)
    return out


def lm_head(h, w_lm, out=None):
    """logits = H W_lm^T in fp32, shape h.shape[:-1] + (vocab,)."""
    dev = h.device
    _check(h, "h", dev, torch.bfloat16)
    w_lm = _packed(w_lm, "w_lm", dev)
    vocab, hidden = w_lm.shape
    rows = h.numel() // hidden
    if out is None:
        out = torch.empty(tuple(h.shape[:-1]) + (vocab,), dtype=torch.float32, device=dev)
    a = _lib.LmHeadArgs()
    a.rows, a.hidden, a.vocab, a.ld = rows, hidden, vocab, vocab
    a.h, a.w_lm, a.logits = _p(h), _p(w_lm.data), _p(out)
    _run("twotower_lm_head", a, dev)
    return out


def lm_head_unmask(h, w_lm, masked, tokens, threshold, *, min_commit=False, commit_all=False,
                   keep_logits=False):
    """lm-head fused with the unmasking (the logits need not reach memory).

    ``h`` is bf16 [B,S,hidden]; updates ``masked`` and ``tokens`` in place. Returns
    (confidence [B,S] fp32, n_committed [B] int32, logits [B,S,V] fp32 or None): the logits are
    stored only when ``keep_logits``.
    """
    dev = h.device
    _check(h, "h", dev, torch.bfloat16, 3)
    _check(masked, "masked", dev, torch.uint8, 2)
    _check(tokens, "tokens", dev, torch.int32, 2)
    w_lm = _packed(w_lm, "w_lm", dev)
    vocab, hidden = w_lm.shape
    B, S, hh = h.shape
    if hh != hidden or tuple(masked.shape) != (B, S) or tuple(tokens.shape) != (B, S):
        raise ValueError("lm_head_unmask shape mismatch")
    logits = (torch.empty((B, S, vocab), dtype=torch.float32, device=dev) if keep_logits
              else None)
    conf = torch.full((B, S), float("nan"), dtype=torch.float32, device=dev)
    ncom = torch.zeros((B,), dtype=torch.int32, device=dev)
    a = _lib.LmHeadUnmaskArgs()
    a.lm.rows, a.lm.hidden, a.lm.vocab, a.lm.ld = B * S, hidden, vocab, vocab
    a.lm.h, a.lm.w_lm, a.lm.logits = _p(h), _p(w_lm.data), _p(logits) if keep_logits else None
    a.unmask.batch, a.unmask.S = B, S
    a.unmask.masked, a.unmask.tokens = _p(masked), _p(tokens)
    a.unmask.confidence, a.unmask.n_committed = _p(conf), _p(ncom)
    a.unmask.threshold = float(threshold)
    a.unmask.min_commit, a.unmask.commit_all = int(bool(min_commit)), int(bool(commit_all))
    _run("twotower_lm_head_unmask", a, dev)
    return conf, ncom, logits


def kv_append(k_pages, v_pages, k_new, v_new, block_table, ctx_lens, free_pages, free_count,
              status):
    """Append the committed block's rows of every layer to the paged context caches.

    k_pages / v_pages / k_new / v_new: lists with one tensor per layer (k_new [B,Hkv,S,D],
    v_new [B,Hkv,D,S]); block_table, ctx_lens, free_count ([1]) and status ([1]) int32 are
    updated in place on the device (no host synchronization).
    """
    dev = block_table.device
    L = len(k_pages)
    if not (len(v_pages) == len(k_new) == len(v_new) == L) or L == 0:
        raise ValueError("one k_pages / v_pages / k_new / v_new tensor per layer")
    P, Hkv, page, D = _cache_dims(k_pages[0])
    B, _, S, _ = k_new[0].shape
    dt = k_pages[0].dtype
    for t in k_pages:
        _check(t, "k_pages", dev, dt, 6)
        if tuple(t.shape) != k_pages_shape(P, Hkv, page, D):
            raise ValueError("k_pages shape mismatch")
    for t in v_pages:
        _check(t, "v_pages", dev, dt, 6)
        if tuple(t.shape) != v_pages_shape(P, Hkv, page, D):
            raise ValueError("v_pages shape mismatch")
    for t in k_new:
        _check(t, "k_new", dev, dt, 4)
        if tuple(t.shape) != (B, Hkv, S, D):
            raise ValueError("k_new shape mismatch")
    for t in v_new:
        _check(t, "v_new", dev, dt, 4)
        if tuple(t.shape) != (B, Hkv, D, S):
            raise ValueError("v_new shape mismatch")
    for t, n in ((block_table, "block_table"), (ctx_lens, "ctx_lens"), (free_pages, "free_pages"),
                 (free_count, "free_count"), (status, "status")):
        _check(t, n, dev, torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(ctx_lens.shape) != (B,):
        raise ValueError("block_table / ctx_lens shape mismatch")

    def arr(ts):
        return (C.c_void_p * L)(*[t.data_ptr() for t in ts])

    keep = [arr(k_pages), arr(v_pages), arr(k_new), arr(v_new)]
    vpp = C.POINTER(C.c_void_p)
    a = _lib.KvAppendArgs()
    a.num_layers, a.batch, a.num_kv_heads, a.head_dim, a.S = L, B, Hkv, D, S
    a.dtype = _dt(k_pages[0])
    a.num_pages, a.page_size, a.max_pages_per_seq = P, page, block_table.shape[1]
    a.k_pages, a.v_pages, a.k_new, a.v_new = [C.cast(x, vpp) for x in keep]
    a.block_table, a.ctx_lens = _p(block_table), _p(ctx_lens)
    a.free_pages, a.free_count, a.status = _p(free_pages), _p(free_count), _p(status)
    _run("twotower_kv_append", a, dev)


def mask_corrupt(clean, u_time, u_mask, mask_id):
    """Linear-schedule [MASK] corruption of clean blocks [B,S] int32 with the caller's uniform
    draws u_time [B], u_mask [B,S] (fp32 in [0, 1)). Returns (noisy int32, masked uint8, t fp32)."""
    dev = clean.device
    _check(clean, "clean", dev, torch.int32, 2)
    _check(u_time, "u_time", dev, torch.float32, 1)
    _check(u_mask, "u_mask", dev, torch.float32, 2)
    B, S = clean.shape
    if tuple(u_time.shape) != (B,) or tuple(u_mask.shape) != (B, S):
        raise ValueError("mask_corrupt shape mismatch")
    noisy = torch.empty_like(clean)
    masked = torch.empty((B, S), dtype=torch.uint8, device=dev)
    t = torch.empty((B,), dtype=torch.float32, device=dev)
    a = _lib.MaskCorruptArgs()
    a.batch, a.S, a.mask_id = B, S, int(mask_id)
    a.clean, a.u_time, a.u_mask = _p(clean), _p(u_time), _p(u_mask)
    a.noisy, a.masked, a.t_out = _p(noisy), _p(masked), _p(t)
    _run("twotower_mask_corrupt", a, dev)
    return noisy, masked, t


def masked_nll(logits, targets, masked):
    """NLL of targets at the masked rows of fp32 logits [B,S,V]. Returns (nll [B,S] fp32, 0 at
    rows not masked; mean over masked rows [1] fp32; number of masked rows [1] int32)."""
    dev = logits.device
    _check(targets, "targets", dev, torch.int32, 2)
    _check(masked, "masked", dev, torch.uint8, 2)
    if logits.dtype != torch.float32 or logits.dim() != 3 or logits.stride(2) != 1:
        raise ValueError("logits must be fp32 [B,S,V] with unit vocab stride")
    B, S, V = logits.shape
    if logits.stride(0) != S * logits.stride(1):
        raise ValueError("logits rows must be evenly strided")
    if tuple(targets.shape) != (B, S) or tuple(masked.shape) != (B, S):
        raise ValueError("masked_nll shape mismatch")
    nll = torch.empty((B, S), dtype=torch.float32, device=dev)
    # zeros: the values of an empty batch (for which the library launches nothing)
    loss = torch.zeros((1,), dtype=torch.float32, device=dev)
    count = torch.zeros((1,), dtype=torch.int32, device=dev)
    a = _lib.MaskedNllArgs()
    a.batch, a.S, a.vocab, a.ld = B, S, V, logits.stride(1)
    a.logits, a.targets, a.masked = _p(logits), _p(targets), _p(masked)
    a.nll, a.loss, a.n_masked = _p(nll), _p(loss), _p(count)
    _run("twotower_masked_nll", a, dev)
    return nll, loss, count


class DenoiseStep:
    """One denoise step of the synthetic attention-only denoiser, reused across steps.

    Holds the per-layer context caches (read only), the packed weights (bf16 tensors given here
    are packed once, at construction) and the block-KV / scratch buffers, so that calling it only
    enqueues kernels on the current stream.
    """

    def __init__(self, *, k_pages, v_pages, w_qkv, w_o, w_lm, block_table, ctx_lens,
                 max_ctx_len, num_q_heads, num_kv_heads, head_dim, batch, S, scale=None,
                 num_splits=0, keep_logits=False):
        dev = w_lm.device
        self.device = dev
        self.L = len(k_pages)
        w_qkv = [_packed(w, "w_qkv", dev) for w in w_qkv]
        w_o = [_packed(w, "w_o", dev) for w in w_o]
        w_lm = _packed(w_lm, "w_lm", dev)
        vocab, hidden = w_lm.shape
        self.hidden, self.vocab = hidden, vocab
        self.B, self.S = batch, S
        self.Hq, self.Hkv, self.D = num_q_heads, num_kv_heads, head_dim
        bf = torch.bfloat16
        self._keep = [list(k_pages), list(v_pages), list(w_qkv), list(w_o), w_lm, block_table,
                      ctx_lens]
        self.k_blk = [torch.empty((batch, num_kv_heads, S, head_dim), dtype=bf, device=dev)
                      for _ in range(self.L)]
        self.v_blk = [torch.empty((batch, num_kv_heads, head_dim, S), dtype=bf, device=dev)
                      for _ in range(self.L)]
        self.q = torch.empty((batch, S, num_q_heads, head_dim), dtype=bf, device=dev)
        self.attn_out = torch.empty_like(self.q)
        self.h_work = torch.empty((batch, S, hidden), dtype=bf, device=dev)
        # the unmasking is fused into the lm-head: the logits are stored only on request
        self.logits = (torch.empty((batch, S, vocab), dtype=torch.float32, device=dev)
                       if keep_logits else None)
        self.confidence = torch.full((batch, S), float("nan"), dtype=torch.float32, device=dev)
        self.n_committed = torch.zeros((batch,), dtype=torch.int32, device=dev)

        def arr(ts):
            a = (C.c_void_p * len(ts))(*[t.data_ptr() for t in ts])
            return a

        self._arrs = [arr(k_pages), arr(v_pages), arr([w.data for w in w_qkv]),
                      arr([w.data for w in w_o]), arr(self.k_blk), arr(self.v_blk)]
        a = _lib.DenoiseStepArgs()
        a.num_layers, a.hidden, a.vocab = self.L, hidden, vocab
        P, _, page, _ = _cache_dims(k_pages[0])
        a.attn.batch, a.attn.S = batch, S
        a.attn.num_q_heads, a.attn.num_kv_heads, a.attn.head_dim = num_q_heads, num_kv_heads, head_dim
        a.attn.dtype = a.attn.out_dtype = TT_BF16
        a.attn.scale = float(1.0 / math.sqrt(head_dim) if scale is None else scale)
        a.attn.num_pages, a.attn.page_size = P, page
        a.attn.max_pages_per_seq = block_table.shape[1]
        a.attn.max_ctx_len = int(max_ctx_len)
        a.attn.block_table, a.attn.ctx_lens = _p(block_table), _p(ctx_lens)
        a.attn.num_splits = int(num_splits)
        vpp = C.POINTER(C.c_void_p)
        a.k_pages, a.v_pages, a.w_qkv, a.w_o, a.k_blk, a.v_blk = [C.cast(x, vpp) for x in self._arrs]
        a.w_lm = _p(w_lm.data)
        a.h_work, a.q, a.attn_out = _p(self.h_work), _p(self.q), _p(self.attn_out)
        a.logits = _p(self.logits) if keep_logits else None
        a.logits_ld = vocab
        a.unmask.confidence, a.unmask.n_committed = _p(self.confidence), _p(self.n_committed)
        self.args = a
        self._ws = None
        self._ws_n = C.c_size_t(0)

    def __call__(self, h_in, masked, tokens, *, threshold, min_commit=True, commit_all=False,
                 timing_events=None, n_committed=None):
        """Enqueue one step; updates masked/tokens in place, fills confidence and the per-sequence
        commit counts (into `n_committed`, an int32 [batch] device tensor, when given, else into
        self.n_committed, which is returned). ``timing_events``: optional 3 * layers hipEvent_t
        handles (None entries skipped), recorded around each layer's attention kernel and after
        its merge."""
        a = self.args
        a.h_in = _p(h_in)
        a.unmask.masked, a.unmask.tokens = _p(masked), _p(tokens)
        if n_committed is None:
            n_committed = self.n_committed
        else:
            _check(n_committed, "n_committed", self.device, torch.int32)
            if n_committed.numel() != self.n_committed.numel() or not n_committed.is_contiguous():
                raise ValueError("n_committed must be a contiguous int32 tensor of batch elements")
        a.unmask.n_committed = _p(n_committed)
        a.unmask.threshold = float(threshold)
        a.unmask.min_commit, a.unmask.commit_all = int(bool(min_commit)), int(bool(commit_all))
        if timing_events is not None:
            if len(timing_events) != 3 * self.L:
                raise ValueError("timing_events takes 3 events per layer")
            self._ev = (C.c_void_p * len(timing_events))(*timing_events)
            a.timing_events = C.cast(self._ev, C.POINTER(C.c_void_p))
        else:
            a.timing_events = None
        if self._ws is None:
            n = C.c_size_t(0)
            st = _lib.call("twotower_denoise_step", a, None, n, None)
            if st != _lib.TT_OK:
                raise TwoTowerError("twotower_denoise_step", st)
            self._ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=self.device)
            self._ws_n = C.c_size_t(self._ws.numel())
        st = _lib.call("twotower_denoise_step", a, _p(self._ws), self._ws_n, _stream())
        if st != _lib.TT_OK:
            raise TwoTowerError("twotower_denoise_step", st)
        return self.confidence, n_committed


def probe_stream_read(src, workgroups, sink):
    """Measurement probe: stream-read the bytes of ``src`` (a contiguous device tensor whose size
    is a multiple of 16 bytes) with ``workgroups`` work-groups; ``sink`` is an int32 device tensor
    of at least ``workgroups`` elements (normally left untouched)."""
    nbytes = src.numel() * src.element_size()
    if not src.is_contiguous() or sink.numel() < workgroups or sink.element_size() != 4:
        raise ValueError("probe_stream_read: contiguous source, sink of >= workgroups words")
    st = _lib.lib().twotower_probe_stream_read(_p(src), nbytes, int(workgroups), _p(sink),
                                                _stream())
    if st != _lib.TT_OK:
        raise TwoTowerError("twotower_probe_stream_read", st)

def probe_mfma_rate(mode, workgroups, iters, sink):
    """Measurement probe: ``workgroups`` x 8 waves x ``iters`` x 16 MFMAs 32x32x16 bf16 (mode bit
    0: A operand read from LDS per MFMA; bit 1: two work-groups per compute unit). ``sink`` is a
    float32 device tensor of at least ``workgroups * 512`` elements (overwritten). Returns the
    flops the call performs."""
    if sink.dtype != torch.float32 or sink.numel() < workgroups * 512 or not sink.is_contiguous():
        raise ValueError("probe_mfma_rate: float32 sink of >= workgroups * 512 elements")
    st = _lib.lib().twotower_probe_mfma_rate(int(mode), int(workgroups), int(iters), _p(sink),
                                              _stream())
    if st != _lib.TT_OK:
        raise TwoTowerError("twotower_probe_mfma_rate", st)
    return int(workgroups) * 8 * int(iters) * 16 * 32768
