"""GPU parity where one chunk (fused all-reduce, reduce-scatter output) or
one arena (in-place sync) has more tiles than one launch's grid holds (2^22
tiles), so the launcher splits the work over several launches (or, for the
reduce-scatter output, the blocks loop over the tiles beyond). Two ranks,
fp32, 8.6 GB and 4.3 GB per rank; sampled positions, including both sides of
every split, against the oracle. Memory: ~17 GB of HBM for the all-reduce,
~26 GB for the reduce-scatter (inputs and shards), ~9 GB for the in-place
sync."""

import numpy as np
import pytest
import torch

import ring_all_reduce_ddp_amd as rar
from oracle import ring, rounding
from ddp_workloads import device_ring_inputs

from gpu_util import assert_bit_equal, sample_positions, gather

pytestmark = pytest.mark.gpu

MAX_GRID_TILES = 1 << 22   # tiles per launch, at most
TILE_FP32 = 256            # fp32 elements per rank in one tile (64 lanes x 16 bytes)


def with_edges(pos, count, splits):
    extra = np.array([s + d for s in splits for d in (-2, -1, 0, 1)], dtype=np.int64)
    pos = np.concatenate([pos, extra])
    return np.unique(pos[(pos >= 0) & (pos < count)])


@pytest.mark.parametrize("extra", [4096, 4092])
def test_fused_all_reduce_split_over_launches(extra):
    """One chunk needs two launches; with extra = 4096 the chunks are whole
    tiles (the whole-tile kernel), with 4092 they end in a partial tile."""
    n = 2
    L = MAX_GRID_TILES * TILE_FP32 + extra
    count = n * L
    bufs = device_ring_inputs(31, n, count, "fp32", std=1e-3)
    pos = with_edges(sample_positions(count, n, 20000, seed=31), count,
                     [c * L + MAX_GRID_TILES * TILE_FP32 for c in range(n)])
    pos_dev = torch.from_numpy(pos).cuda()
    before = [gather(t, pos_dev, "fp32") for t in bufs]
    print(f"[fused split] N={n} count={count} samples={len(pos)}", flush=True)
    rar.ring_allreduce_fused(bufs)
    torch.cuda.synchronize()
    after = [gather(t, pos_dev, "fp32") for t in bufs]
    want = ring.ring_simulate(before, "fp32", chunk_of=pos // L)["bufs"]
    for r in range(n):
        assert_bit_equal(after[r], want[r], f"rank {r}")


@pytest.mark.parametrize("extra", [4096, 4092])
def test_reduce_scatter_split_over_launches(extra):
    """The reduce-scatter output where one chunk has more tiles than one grid
    holds (the blocks loop over the rest), ending in a whole tile (extra =
    4096) or a partial one (4092): sampled shard positions, scale 1, equal the
    ring's sum at those positions."""
    n = 2
    L = MAX_GRID_TILES * TILE_FP32 + extra
    count = n * L
    bufs = device_ring_inputs(33, n, count, "fp32", std=1e-3)
    pos = with_edges(sample_positions(count, n, 20000, seed=33), count,
                     [c * L + MAX_GRID_TILES * TILE_FP32 for c in range(n)])
    pos_dev = torch.from_numpy(pos).cuda()
    before = [gather(t, pos_dev, "fp32") for t in bufs]
    shards = [torch.empty(L, device="cuda") for _ in range(n)]
    print(f"[reduce-scatter split] N={n} count={count} samples={len(pos)}", flush=True)
    rar.ring_reduce_scatter_fused(bufs, shards, 1.0)
    torch.cuda.synchronize()
    want = ring.ring_simulate(before, "fp32", chunk_of=pos // L)["bufs"][0]
    chunk = pos // L
    got = np.empty(len(pos), np.float32)
    for c in range(n):
        sel = np.nonzero(chunk == c)[0]
        got[sel] = gather(shards[c], torch.from_numpy(pos[sel] - c * L).cuda(), "fp32")
    assert_bit_equal(got, want, "shards")
    del bufs, shards
    torch.cuda.empty_cache()


def test_in_place_sync_split_over_launches():
    n = 2
    numel = MAX_GRID_TILES * TILE_FP32 + 1001   # arena tiles beyond one launch; a ragged last vector
    plan = rar.ddp_bucket_plan([numel], "fp32", cap_bytes=1 << 40, first_bucket_bytes=1 << 40, world_size=n)
    arena_numel, offs = plan.grad_arena()
    assert offs[0] == 0 and arena_numel >= numel
    arenas = device_ring_inputs(32, n, arena_numel, "fp32", std=1e-3)
    padded, _ = plan.bucket(0)
    L = padded // n
    pos = with_edges(sample_positions(numel, n, 20000, seed=32), numel, [MAX_GRID_TILES * TILE_FP32, L])
    pos_dev = torch.from_numpy(pos).cuda()
    before = [gather(t, pos_dev, "fp32") for t in arenas]
    tail = [t[numel:].clone() for t in arenas]   # alignment padding after the member
    print(f"[in-place split] N={n} numel={numel} samples={len(pos)}", flush=True)
    rar.ddp_sync(plan, arenas, None, variant="view", scale=0.5)
    torch.cuda.synchronize()
    after = [gather(t, pos_dev, "fp32") for t in arenas]
    summed = ring.ring_simulate(before, "fp32", chunk_of=pos // L)["bufs"]
    want = rounding.round_to_fp32(rounding.to_f64(summed[0], "fp32") * 0.5)
    for r in range(n):
        assert_bit_equal(after[r], want, f"rank {r}")
        assert torch.equal(arenas[r][numel:], tail[r]), "padding after the member was written"
