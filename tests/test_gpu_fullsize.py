"""GPU parity at the workloads' full sizes, every element.

* 8 ranks x 25 MiB fp32 (one DDP bucket): every element of every rank against
  the oracle's hop-by-hop ring.
* 8 ranks x 1 GiB (fp32 and bf16) and 64 ranks x 300M fp32 (heavy-tailed):
  the inputs are drawn on the GPU exactly as the benchmark draws them, and
  the fused kernel runs on those buffers as the benchmark launches it; then
  the step and persistent forms run on the same inputs. On the device, every
  rank must equal rank 0 bit for bit (torch's comparison); rank 0 is then
  compared, every element, with the oracle's closed-form ring-order sum of
  its chunk, computed one chunk column (N ranks x L elements) at a time from
  a pristine copy of the inputs, so host memory stays bounded. The
  reduce-scatter output (every rank's shard, scaled by fl32(1/N)) is checked
  the same way, every element, against the same sums scaled and rounded once.
  Every element also lies within the error bound (N-1) u sum|g_i| of the
  fp64 sum of the inputs (the bound widened by 2^-20 for the fp64 rounding),
  and within the bound of the exact sum on sampled positions.
"""

import os
from concurrent.futures import ThreadPoolExecutor

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
INT_VIEW = {"fp32": torch.int32, "bf16": torch.int16}


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


def oracle_chunk_sum(x, c, dtype):
    """ring.ring_order_sum(x, c, dtype) for an (N, k) chunk column, computed in
    pieces of 2^20 positions on a thread pool: the sum is elementwise, so the
    pieces are independent, and numpy releases the interpreter lock inside
    its loops. Up to 16 threads (the host share of one GPU)."""
    k = x.shape[1]
    piece = 1 << 20
    out = np.empty(k, dtype=x.dtype)

    def run(a):
        b = min(a + piece, k)
        out[a:b] = ring.ring_order_sum(x[:, a:b], c, dtype)

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(run, range(0, k, piece)))
    return out


def bound_holds_everywhere(x, got, dtype):
    """Every element of `got` (an (N, k) chunk column's result) lies within
    (N-1) u sum|g_i| of the sum of the N inputs, with the sum and sum|g_i|
    taken in fp64 (not exactly: their own rounding errors, at most about
    N 2^-53 relative, are covered by widening the bound by a factor 1 + 2^-20,
    far below what a wrong unit roundoff or term count would need). Computed
    in pieces of 2^20 positions on a thread pool, like oracle_chunk_sum."""
    n, k = x.shape
    tol_factor = (n - 1) * rounding.unit_roundoff(dtype) * (1 + 2.0 ** -20)
    piece = 1 << 20

    def run(a):
        b = min(a + piece, k)
        xs = rounding.to_f64(x[:, a:b], dtype)
        err = np.abs(rounding.to_f64(got[a:b], dtype) - xs.sum(axis=0))
        return bool(np.all(err <= tol_factor * np.abs(xs).sum(axis=0)))

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        return all(ex.map(run, range(0, k, piece)))


def every_element_check(w, dtype, variants=VARIANTS):
    n = w.n
    count = elements_for(w, dtype)
    bufs = device_ring_inputs(w.seed, n, count, dtype, std=w.std, heavy_frac=w.heavy_frac,
                              heavy_mult=w.heavy_mult)
    pristine = [b.clone() for b in bufs]
    ivt = INT_VIEW[dtype]
    # the reduce-scatter output first: it reads the inputs and leaves them as they are
    L = ring.chunk_length(count, n)
    scale = float(np.float32(1) / np.float32(n))
    shards = [torch.empty(min(L, count - c * L), dtype=bufs[0].dtype, device="cuda") for c in range(n)]
    print(f"[{w.name} {dtype} reduce-scatter output] N={n} count={count}", flush=True)
    rar.ring_reduce_scatter_fused(bufs, shards, scale)
    torch.cuda.synchronize()
    got_shards = [to_host(t, dtype) for t in shards]
    del shards
    got = {}
    for i, variant in enumerate(variants):
        if i:
            for b, p in zip(bufs, pristine):
                b.copy_(p)
        print(f"[{w.name} {dtype} {variant}] N={n} count={count}", flush=True)
        run_variant(variant, bufs)
        ref = bufs[0].view(ivt)
        for r in range(1, n):
            assert torch.equal(bufs[r].view(ivt), ref), f"{w.name} {dtype} {variant}: rank {r} differs from rank 0"
        got[variant] = to_host(bufs[0], dtype)
    del bufs
    torch.cuda.empty_cache()
    print(f"[{w.name} {dtype}] oracle, {n} chunk columns", flush=True)
    for c in range(n):
        lo, hi = ring.chunk_bounds(count, n, c)
        if lo >= hi:
            continue
        x = np.stack([to_host(p[lo:hi], dtype) for p in pristine])
        want = oracle_chunk_sum(x, c, dtype)
        for variant in variants:
            assert_bit_equal(got[variant][lo:hi], want, f"{w.name} {dtype} {variant} chunk {c}")
        shard = rounding.round_to(rounding.to_f64(want, dtype) * scale, dtype)
        assert_bit_equal(got_shards[c], shard, f"{w.name} {dtype} reduce-scatter shard {c}")
        assert bound_holds_everywhere(x, got[variants[0]][lo:hi], dtype), f"{w.name} {dtype} chunk {c}: error bound"
    # and against the exact sum (an fsum per element) on sampled positions
    pos = sample_positions(count, n, 2000, seed=w.seed)
    pos_dev = torch.from_numpy(pos).cuda()
    before = [gather(p, pos_dev, dtype) for p in pristine]
    err = np.abs(rounding.to_f64(got[variants[0]][pos], dtype) - ring.sum_f64(before, dtype))
    assert np.all(err <= ring.error_bound(before, dtype))
    del pristine
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_n8_1gib_every_element(dtype):
    every_element_check(WORKLOADS["ring_n8_1gib"], dtype)


@pytest.mark.timeout(900)
def test_n64_300m_every_element():
    every_element_check(WORKLOADS["ring_n64_300m"], "fp32")


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
