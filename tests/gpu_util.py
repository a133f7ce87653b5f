"""Helpers shared by the GPU parity tests: device transfer, library calls, input guards."""
import numpy as np
import torch

import synth
import two_tower_cross_amd as tt
from oracle import unmask as ounmask

DEV = torch.device("cuda", 0)

# Attention tolerances (max-abs against the fp64 oracle): fp32 inputs 1e-5, bf16 inputs 2e-2.
TOL_FP32 = 1e-5
TOL_BF16 = 2e-2


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype)


def dev_case(case):
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    return dict(q=to_dev(case.q, dt), k_pages=to_dev(case.k_pages, dt),
                v_pages=to_dev(case.v_pages, dt),
                block_table=torch.from_numpy(case.block_table).to(DEV),
                ctx_lens=torch.from_numpy(case.ctx_lens).to(DEV),
                k_blk=to_dev(case.k_blk, dt), v_blk=to_dev(case.v_blk, dt))


def gpu_attn(case, d=None, *, out_dtype=torch.float32, num_splits=0, max_ctx_len=None,
             return_lse=True, timing_events=None, **over):
    d = dict(dev_case(case) if d is None else d)
    d.update(over)
    if max_ctx_len is None:
        max_ctx_len = int(case.ctx_lens.max()) if case.B else 0
    r = tt.block_attn(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["ctx_lens"],
                      d["k_blk"], d["v_blk"], scale=case.scale, max_ctx_len=max_ctx_len,
                      out_dtype=out_dtype, return_lse=return_lse, num_splits=num_splits,
                      timing_events=timing_events)
    torch.cuda.synchronize()
    if return_lse:
        out, lse = r
        return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    return r.float().cpu().numpy().astype(np.float64), None


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def guarded_logits(make, threshold, seed, *, margin=1e-3, gap=1e-3, min_commit=False,
                   masked=None, max_iter=64):
    """Logits from ``make(seed)`` [B,S,V], with every row whose oracle confidence lies within
    ``margin`` of ``threshold`` redrawn from later seeds; with ``min_commit``, sequences where the
    fallback fires and the two best confidences are within a relative ``gap`` are redrawn too.
    The decision of the oracle (fp64) and of the GPU (fp32) then cannot differ."""
    x = make(seed)
    B, S, V = x.shape
    for it in range(max_iter):
        conf = np.array([[ounmask.row_confidence(x[b, i])[1] for i in range(S)]
                         for b in range(B)])
        live = np.ones((B, S), bool) if masked is None else masked.astype(bool)
        bad = (np.abs(conf - np.float64(np.float32(threshold))) < margin) & live
        if min_commit:
            for b in range(B):
                cb = np.where(live[b], conf[b], -1.0)
                if live[b].sum() > 1 and not np.any(cb > threshold):
                    c = np.sort(cb)[::-1]
                    if (c[0] - c[1]) < gap * c[0]:
                        bad[b, int(np.argmax(cb))] = True
        if not bad.any():
            return x
        fresh = make(seed + 1000 * (it + 1))
        x[bad] = fresh[bad]
    raise RuntimeError("could not satisfy the confidence guards")
