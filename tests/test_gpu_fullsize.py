"""GPU parity at the workloads' full sizes.

* 8 ranks x 25 MiB fp32 (one DDP bucket): every element against the oracle.
* 8 ranks x 1 GiB (fp32 and bf16) and 64 ranks x 300M fp32 (heavy-tailed):
  inputs are drawn on the GPU; the oracle runs the ring on sampled positions
  (with their chunk ids; every chunk's first and last elements included) read
  back before and after, and the device checks that all ranks agree
  everywhere. The fused kernel is called exactly as the benchmark calls it.
"""

import numpy as np
import pytest
import torch

import ring_all_reduce_ddp_amd as rar
from oracle import ring, rounding
from ddp_workloads import WORKLOADS, host_ring_inputs, device_ring_inputs
from ddp_workloads.gen import elements_for

from gpu_util import to_device, to_host, assert_bit_equal, sample_positions, gather
from test_gpu_ring import run_variant

pytestmark = pytest.mark.gpu

VARIANTS = ["fused", "steps", "persistent"]


@pytest.fixture(scope="module")
def c2_case():
    w = WORKLOADS["ring_n8_25mib"]
    host = host_ring_inputs(w.seed, w.n, w.count, "fp32", std=w.std)
    want = ring.ring_simulate(host, "fp32")["bufs"]
    return host, want


@pytest.mark.parametrize("variant", VARIANTS)
def test_n8_25mib_every_element(c2_case, variant):
    host, want = c2_case
    dev = to_device(host, "fp32")
    run_variant(variant, dev)
    for r in range(len(dev)):
        assert_bit_equal(to_host(dev[r], "fp32"), want[r], f"{variant} rank {r}")


def sampled_check(w, dtype, variant, k_samples):
    count = elements_for(w, dtype)
    bufs = device_ring_inputs(w.seed, w.n, count, dtype, std=w.std, heavy_frac=w.heavy_frac,
                              heavy_mult=w.heavy_mult)
    pos = sample_positions(count, w.n, k_samples, seed=w.seed)
    pos_dev = torch.from_numpy(pos).cuda()
    before = [gather(t, pos_dev, dtype) for t in bufs]
    print(f"[{w.name} {dtype} {variant}] N={w.n} count={count} samples={len(pos)}", flush=True)
    run_variant(variant, bufs)
    after = [gather(t, pos_dev, dtype) for t in bufs]
    mism = torch.zeros(1, dtype=torch.int64, device="cuda")
    rar.ddp_count_mismatches(bufs, mism)
    torch.cuda.synchronize()
    assert int(mism.item()) == 0, "ranks differ after the all-reduce"
    L = ring.chunk_length(count, w.n)
    want = ring.ring_simulate(before, dtype, chunk_of=pos // L)["bufs"]
    for r in range(w.n):
        assert_bit_equal(after[r], want[r], f"{w.name} {dtype} {variant} rank {r}")
    # the result is within the recursive-summation bound of the exact sum
    exact = ring.sum_f64(before, dtype)
    err = np.abs(rounding.to_f64(after[0], dtype) - exact)
    assert np.all(err <= ring.error_bound(before, dtype))
    del bufs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_n8_1gib_sampled(dtype, variant):
    sampled_check(WORKLOADS["ring_n8_1gib"], dtype, variant, k_samples=20000)


@pytest.mark.parametrize("variant", VARIANTS)
def test_n64_300m_sampled(variant):
    sampled_check(WORKLOADS["ring_n64_300m"], "fp32", variant, k_samples=4000)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_span_beyond_cache_sampled(dtype):
    """64 ranks x 2,560,000 elements (328 MB of bf16, 655 MB of fp32: beyond
    the 256 MiB Infinity Cache, so the span kernel streams with non-temporal
    loads), chunks that start mid-tile: the reduce-scatter output and the
    fused all-reduce against the oracle on sampled positions, and all ranks
    equal everywhere after the all-reduce."""
    n, count = 64, 64 * 40_000
    bufs = device_ring_inputs(64, n, count, dtype, std=1e-3)
    pos = sample_positions(count, n, 3000, seed=64)
    pos_dev = torch.from_numpy(pos).cuda()
    before = [gather(t, pos_dev, dtype) for t in bufs]
    print(f"[span {dtype}] N={n} count={count} samples={len(pos)}", flush=True)
    # the reduce-scatter output first (it leaves the inputs as they are): the
    # same k offsets in every chunk form a small ring whose shards the oracle
    # computes
    L = ring.chunk_length(count, n)
    rng = np.random.default_rng(65)
    offs = np.unique(np.concatenate([rng.choice(L, 60, replace=False), [0, 1, L - 2, L - 1]]))
    mini_pos = torch.from_numpy(np.concatenate([c * L + offs for c in range(n)])).cuda()
    mini = [gather(t, mini_pos, dtype) for t in bufs]
    shards = [torch.empty(L, dtype=bufs[0].dtype, device="cuda") for _ in range(n)]
    scale = float(np.float32(1) / np.float32(n))
    rar.ring_reduce_scatter_fused(bufs, shards, scale)
    want_shards = ring.reduce_scatter(mini, dtype, np.float32(scale))
    offs_dev = torch.from_numpy(offs).cuda()
    for c in range(n):
        assert_bit_equal(gather(shards[c], offs_dev, dtype), want_shards[c], f"span {dtype} shard {c}")
    rar.ring_allreduce_fused(bufs)
    after = [gather(t, pos_dev, dtype) for t in bufs]
    mism = torch.zeros(1, dtype=torch.int64, device="cuda")
    rar.ddp_count_mismatches(bufs, mism)
    torch.cuda.synchronize()
    assert int(mism.item()) == 0, "ranks differ after the all-reduce"
    want = ring.ring_simulate(before, dtype, chunk_of=pos // L)["bufs"]
    for r in range(n):
        assert_bit_equal(after[r], want[r], f"span {dtype} rank {r}")
