"""The library's launches captured in a HIP graph (torch.cuda.CUDAGraph on
ROCm) and replayed: the copying DDP sync (pack, fused all-reduce, x1/N,
unpack for every bucket), the in-place sync, the fused all-reduce, the
2(N-1) step launches and the allocation-free persistent all-reduce. Each graph is replayed several times, with the
program's own eager work (restoring the inputs) and a synchronisation
between replays, and every replay must equal the eager result bit for bit.
The first call of a plan on a device makes its device tables, so one eager
call precedes every capture; the launches themselves record no memory set or
copy nodes (buffers that must start at zero are cleared by fill kernels)."""

import numpy as np
import pytest
import torch

import ring_all_reduce_ddp_amd as rar
from ddp_workloads import host_grads, host_ring_inputs, resnet50_param_numels

from gpu_util import to_device, to_host, assert_bit_equal, mean_scale
from test_gpu_ddp import make_arenas, bucket_buffers

pytestmark = pytest.mark.gpu

REPLAYS = 4


def capture(fn):
    """fn() captured on a side stream; returns the graph."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s, capture_error_mode="thread_local"):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def replay_matches_eager(targets, pristine, fn, dtype, what):
    """Eager fn() on pristine inputs gives the expected state; then a captured
    fn() is replayed REPLAYS times, each from restored inputs."""
    for t, p in zip(targets, pristine):
        t.copy_(p)
    fn()
    torch.cuda.synchronize()
    want = [to_host(t, dtype) for t in targets]
    for t, p in zip(targets, pristine):
        t.copy_(p)
    g = capture(fn)
    for k in range(REPLAYS):
        for t, p in zip(targets, pristine):   # eager work between replays
            t.copy_(p)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r, t in enumerate(targets):
            assert_bit_equal(to_host(t, dtype), want[r], f"{what}: replay {k}, rank {r}")


@pytest.mark.parametrize("variant", ["fused", "steps", "view"])
def test_graph_of_resnet50_sync(variant):
    n = 8
    numels = resnet50_param_numels()
    plan = rar.ddp_bucket_plan(numels, "fp32", world_size=n)
    grads = host_grads(33, n, numels)
    arenas, _ = make_arenas(plan, grads, "fp32")
    pristine = [a.clone() for a in arenas]
    buckets = None if variant == "view" else bucket_buffers(plan, n, "fp32")
    print(f"[graph of the ResNet-50 sync, {variant}] buckets={plan.num_buckets}", flush=True)
    replay_matches_eager(arenas, pristine,
                         lambda: rar.ddp_sync(plan, arenas, buckets, variant=variant, scale=mean_scale(n)),
                         "fp32", f"ddp_sync {variant}")
    plan.free()


def test_graph_of_bucket_copies():
    """bucket_pack and bucket_unpack_scale of every bucket, as separate
    launches in one graph."""
    n = 4
    numels = [7, 16, 1, 40, 3, 300, 9, 5000, 33]
    plan = rar.ddp_bucket_plan(numels, "fp32", cap_bytes=4096, first_bucket_bytes=64, world_size=n)
    arenas, _ = make_arenas(plan, host_grads(34, n, numels), "fp32")
    pristine = [a.clone() for a in arenas]
    buckets = bucket_buffers(plan, n, "fp32")

    def copies():
        for b in range(plan.num_buckets):
            rar.bucket_pack(plan, b, arenas, buckets[b])
        for b in range(plan.num_buckets):
            rar.bucket_unpack_scale(plan, b, buckets[b], arenas, 0.5)

    replay_matches_eager(arenas, pristine, copies, "fp32", "pack and unpack")
    plan.free()


@pytest.mark.parametrize("variant", ["fused", "steps"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_graph_of_ring_allreduce(variant, dtype):
    n, count = 8, 8 * 100_000 + 5
    bufs = to_device(host_ring_inputs(35, n, count, dtype, std=1e-2), dtype)
    pristine = [b.clone() for b in bufs]
    fn = (lambda: rar.ring_allreduce_fused(bufs)) if variant == "fused" else \
        (lambda: rar.ring_allreduce_stepwise(bufs))
    replay_matches_eager(bufs, pristine, fn, dtype, f"{variant} {dtype}")


@pytest.mark.parametrize("count", [8 * 100_000 + 5, 8 * 1_000_000], ids=["cached", "tickets"])
def test_graph_of_persistent_noalloc(count):
    """The allocation-free persistent all-reduce (its barrier words cleared by
    a fill kernel in the library's fixed array, then one cooperative launch)
    captured and replayed; 8 x 1M fp32 (32 MiB per rank) exceeds the
    Infinity Cache, so its tiles are handed out by tickets. A barrier time-out
    in any replay would leave a sticky status, which the last call raises."""
    n = 8
    bufs = to_device(host_ring_inputs(36, n, count, "fp32", std=1e-2), "fp32")
    pristine = [b.clone() for b in bufs]
    replay_matches_eager(bufs, pristine, lambda: rar.ring_allreduce_persistent_noalloc(bufs), "fp32",
                         f"persistent without allocation, {count} elements")
    rar.ddp_persistent_status()
