"""GPU test of twotower_block_attn_static, the attention entry point that allocates nothing (its
split-KV partials live in the library's per-device scratch array), against twotower_block_attn
(caller workspace) on the same inputs: two calls of the no-allocation entry point in a row, the
second with a smaller input, each bit-identical to the workspace entry point (same kernels, same
partition plan) and within the bf16 tolerance of the oracle."""
import numpy as np
import pytest
import torch

import synth
import two_tower_cross_amd as tt
from oracle import attention as oattn
from gpu_util import DEV, TOL_BF16, dev_case, max_abs

pytestmark = pytest.mark.gpu


def _attn(case, d, no_alloc):
    out = torch.empty((case.B, case.S, case.Hq, case.D), dtype=torch.float32, device=DEV)
    lse = torch.empty((case.B, case.Hq, case.S), dtype=torch.float32, device=DEV)
    tt.block_attn(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["ctx_lens"],
                  d["k_blk"], d["v_blk"], scale=case.scale, max_ctx_len=int(case.ctx_lens.max()),
                  out=out, lse_out=lse, return_lse=True, no_alloc=no_alloc)
    return out, lse


def test_static_scratch_entry_matches_the_workspace_entry():
    big = synth.attn_case(90, B=4, S=16, Hq=32, Hkv=2, D=128, ctx_lens=[5000, 3100, 700, 4096],
                          page_size=256, dtype="bf16", spare_frac=0.2)
    small = synth.attn_case(91, B=1, S=16, Hq=16, Hkv=1, D=128, ctx_lens=[1500], dtype="bf16")
    cases = [(c, dev_case(c)) for c in (big, small)]
    refs = [_attn(c, d, no_alloc=False) for c, d in cases]
    torch.cuda.synchronize()
    refs = [(o.cpu().numpy(), l.cpu().numpy()) for o, l in refs]
    # the no-allocation entry point twice in a row: the large input, then the small one
    got = [_attn(c, d, no_alloc=True) for c, d in cases]
    torch.cuda.synchronize()
    for (c, _), (ro, rl), (o, l) in zip(cases, refs, got):
        o, l = o.cpu().numpy(), l.cpu().numpy()
        assert np.array_equal(o, ro), "output differs from the workspace entry point"
        assert np.array_equal(l, rl), "log-sum-exp differs from the workspace entry point"
        oo, ol = oattn.block_attention_case(c)
        assert max_abs(o, oo) <= TOL_BF16
        assert max_abs(l, ol) <= TOL_BF16
