"""Run the block attention at one layer of the 32K block loop a few times, for profilers.

    python -m two_tower_cross_amd.profile_attn [launches]

Batch 8, block size 16, 32 query / 2 KV heads, head_dim 128, context 32768 in one contiguous page
per sequence; seeded N(0,1) bf16 inputs on cuda:0. Prints nothing but a final line.
"""
import math
import sys

import torch

import two_tower_cross_amd as tt


def main(launches: int = 4) -> None:
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev).manual_seed(1)
    B, S, Hq, Hkv, D, L = 8, 16, 32, 2, 128, 32768
    bf = torch.bfloat16
    k = torch.randn(tt.k_pages_shape(B, Hkv, L, D), generator=g, device=dev).to(bf)
    v = torch.randn(tt.v_pages_shape(B, Hkv, L, D), generator=g, device=dev).to(bf)
    q = torch.randn((B, S, Hq, D), generator=g, device=dev).to(bf)
    kb = torch.randn((B, Hkv, S, D), generator=g, device=dev).to(bf)
    vb = torch.randn((B, Hkv, D, S), generator=g, device=dev).to(bf)
    table = torch.arange(B, dtype=torch.int32, device=dev).view(B, 1)
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    for _ in range(launches):
        tt.block_attn(q, k, v, table, lens, kb, vb, scale=1 / math.sqrt(D), max_ctx_len=L,
                      out_dtype=bf)
    torch.cuda.synchronize()
    print(f"profile_attn: {launches} launches done", flush=True)


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 4)
