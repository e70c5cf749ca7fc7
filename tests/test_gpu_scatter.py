"""GPU parity of the reduce-scatter output (every rank's gradient shard)
against the oracle's ring.reduce_scatter, bit for bit: small and ragged
inputs at several N and both dtypes. (The 8 x 1 GiB and 64 x 300M workloads
are compared every element in test_gpu_fullsize.py.)"""

import numpy as np
import pytest
import torch

import ring_all_reduce_ddp_amd as rar
from oracle import ring
from ddp_workloads import host_ring_inputs

from gpu_util import TORCH_DTYPE, to_device, to_host, assert_bit_equal

pytestmark = pytest.mark.gpu


def shard_buffers(count, n, dtype):
    L = -(-count // n)
    out = []
    for c in range(n):
        lo, hi = min(c * L, count), min((c + 1) * L, count)
        out.append(torch.full((hi - lo,), float("nan"), dtype=TORCH_DTYPE[dtype], device="cuda")
                   if hi > lo else None)
    return out


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n,count", [(1, 100), (2, 4096), (3, 7), (5, 12345), (8, 8 * 2048 * 3),
                                     (8, 8 * 4096 + 5), (8, 5), (8, 25), (8, 7 * 4096 + 4093), (9, 100_003),
                                     (16, 16 * 1000 + 8), (64, 64 * 1024),
                                     # 60 ranks and up, equal chunks of whole vectors: the span kernel
                                     # (chunks that start mid-tile, interior and edge spans, one vector)
                                     (64, 64 * 1000), (61, 61 * 8800), (60, 60 * 8), (63, 63 * 2056)])
@pytest.mark.parametrize("mean", [False, True])
def test_shards_against_oracle(dtype, n, count, mean):
    host = host_ring_inputs(n * 7 + count % 13, n, count, dtype, std=1e-2)
    scale = np.float32(1) / np.float32(n) if mean else np.float32(1)
    want = ring.reduce_scatter(host, dtype, scale)
    dev = to_device(host, dtype)
    shards = shard_buffers(count, n, dtype)
    rar.ring_reduce_scatter_fused(dev, shards, float(scale))
    torch.cuda.synchronize()
    for c in range(n):
        if shards[c] is None:
            assert len(want[c]) == 0
            continue
        assert_bit_equal(to_host(shards[c], dtype), want[c], f"n={n} count={count} {dtype} shard {c}")
    for r in range(n):   # inputs are read only
        assert_bit_equal(to_host(dev[r], dtype), host[r], f"input {r} changed")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_unaligned_inputs(dtype):
    n, count = 8, 8 * 3001
    host = host_ring_inputs(77, n, count, dtype)
    want = ring.reduce_scatter(host, dtype, 0.125)
    dev = to_device(host, dtype, pad_front=1)
    shards = shard_buffers(count, n, dtype)
    rar.ring_reduce_scatter_fused(dev, shards, 0.125)
    torch.cuda.synchronize()
    for c in range(n):
        assert_bit_equal(to_host(shards[c], dtype), want[c], f"shard {c}")


def test_overlapping_shard_refused():
    dev = to_device(host_ring_inputs(5, 2, 64, "fp32"), "fp32")
    with pytest.raises(rar.DDPError, match="overlaps bufs"):
        rar.ring_reduce_scatter_fused(dev, [dev[0][:32], dev[1][32:]])
