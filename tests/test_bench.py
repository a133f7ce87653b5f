"""The benchmark's host-side contract (CPU): a multi-GPU request is refused before anything touches
a device, and the algorithmic bytes and flops that the roofline divides by reproduce the closed
forms of the workloads (per context token and KV head: K and V rows of D elements, 2 * D * e
bytes; per query row and key: 4 * D flops for the QK^T and PV products)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (the module only defines functions and constants at import)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_attention_bytes_and_flops_of_the_32k_layer():
    # batch 8 at 32768 tokens, S 16, Hq 32 / Hkv 2, head_dim 128, bf16
    lens = [32768] * 8
    ctx = 8 * 32768 * 2 * 2 * 128 * 2           # K and V of every context token and KV head
    blk = 8 * 2 * 16 * 2 * 128 * 2              # the block's own K and V
    qo = 2 * 8 * 16 * 32 * 128 * 2              # Q read and O written
    assert bench.attn_bytes(lens, 16, 32, 2, 128) == ctx + blk + qo == 270_663_680
    # 256 query rows per KV head (16 heads x 16 positions) against 32768 + 16 keys
    assert bench.attn_flops(lens, 16, 32, 128) == 8 * 32 * 16 * (32768 + 16) * 4 * 128
    assert abs(bench.attn_flops(lens, 16, 32, 128) / 1e9 - 68.75) < 0.01


def test_attention_bytes_of_the_ragged_and_long_workloads():
    # the 131072-token context: one sequence
    assert bench.attn_bytes([131072], 16, 32, 2, 128) == (131072 * 2 * 2 * 128 * 2
                                                         + 2 * 2 * 16 * 128 * 2
                                                         + 2 * 16 * 32 * 128 * 2)
    # ragged lengths add up sequence by sequence; fp32 doubles every term
    lens = [1, 1000, 8192]
    assert bench.attn_bytes(lens, 16, 32, 2, 128, e=4) == 2 * bench.attn_bytes(lens, 16, 32, 2, 128)
    assert bench.attn_bytes([0], 16, 4, 1, 64) == 2 * 1 * 16 * 64 * 2 + 2 * 16 * 4 * 64 * 2
