"""The oracle's pack / unpack-with-scale / whole-sync functions."""

import numpy as np
import pytest

from oracle import ddp, planner, ring, rounding
from ddp_workloads import host_grads, host_rank_rng


def small_shapes():
    return [7, 16, 1, 40, 3, 300, 9]


def test_pack_unpack_round_trip():
    numels = small_shapes()
    buckets = planner.plan(numels, 4, cap_bytes=512, first_bucket_bytes=64, world_size=3)
    grads = host_grads(11, 1, numels)[0]
    seen = set()
    for b in buckets:
        flat = ddp.pack(grads, b, "fp32")
        covered = np.zeros(b["padded_numel"], bool)
        for p, off, m in b["members"]:
            covered[off:off + m] = True
        assert np.all(flat[~covered] == 0)            # slack and padding are zero
        back = ddp.unpack_scale(flat, b, 1.0, "fp32")
        for p, g in back.items():
            assert np.array_equal(g, grads[p])
            seen.add(p)
    assert seen == set(range(len(numels)))


def test_scale_by_one_eighth_is_exact():
    """fp32(1/8) scaling is exact (a power of two, no underflow at these
    magnitudes): multiplying back by 8 restores the bucket."""
    rng = host_rank_rng(12, 0)
    flat = rng.normal(0, 1e-3, 1024).astype(np.float32)
    b = {"members": [(0, 0, 1024)], "padded_numel": 1024}
    g = ddp.unpack_scale(flat, b, np.float32(0.125), "fp32")[0]
    assert np.array_equal(g * np.float32(8), flat)


def test_scale_rounds_once():
    """x * fl32(1/3) is rounded once to fp32: equal to numpy's float32 multiply."""
    rng = host_rank_rng(13, 0)
    flat = rng.normal(0, 1, 4096).astype(np.float32)
    b = {"members": [(0, 0, 4096)], "padded_numel": 4096}
    s = np.float32(1) / np.float32(3)
    g = ddp.unpack_scale(flat, b, s, "fp32")[0]
    assert np.array_equal(g, flat * s)


@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_ddp_sync_integer_mean(n):
    """Integer gradients: the synced gradient is exactly sum/N for N a power of
    two (sum exact, scaling by 2^-k exact)."""
    numels = small_shapes()
    buckets = planner.plan(numels, 4, cap_bytes=256, first_bucket_bytes=32, world_size=n)
    grads = [[host_rank_rng(14, r).integers(-50, 51, m).astype(np.float32) for m in numels]
             for r in range(n)]
    out = ddp.ddp_sync(grads, buckets, "fp32")
    for p, m in enumerate(numels):
        want = np.sum(np.stack([grads[r][p] for r in range(n)]).astype(np.float64), axis=0) / n
        for r in range(n):
            assert np.array_equal(out[r][p].astype(np.float64), want)


def test_ddp_sync_matches_bucketwise_ring():
    """The whole sync equals, per parameter, the ring-order sum of its
    bucket's chunk, times 1/N, rounded once."""
    n = 4
    numels = small_shapes()
    buckets = planner.plan(numels, 4, cap_bytes=400, first_bucket_bytes=64, world_size=n)
    grads = host_grads(15, n, numels)
    out = ddp.ddp_sync(grads, buckets, "fp32")
    for b in buckets:
        L = b["padded_numel"] // n
        for p, off, m in b["members"]:
            for e in range(m):
                c = (off + e) // L
                x = np.array([[grads[r][p][e]] for r in range(n)], np.float32)
                s = ring.ring_order_sum(x, c, "fp32").astype(np.float64) * 0.25
                assert out[0][p][e] == rounding.round_to_fp32(s)[0]


def test_bf16_compression_pack_rounds_and_unpack_widens():
    """Packing fp32 gradients into a bf16 bucket rounds each to nearest even
    (checked against torch's conversion); unpacking widens exactly and
    rounds the scaled value once to fp32."""
    import torch
    rng = host_rank_rng(16, 0)
    g = rng.normal(0, 1, 1000).astype(np.float32)
    b = planner.plan([1000], 4, world_size=2, vector_elems=8)[0]
    assert b["padded_numel"] % 16 == 0
    flat = ddp.pack([g], b, "bf16", "fp32")
    want = torch.from_numpy(g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(flat[:1000], want)
    back = ddp.unpack_scale(flat, b, np.float32(0.5), "bf16", "fp32")[0]
    assert back.dtype == np.float32
    assert np.array_equal(back, (want.astype(np.uint32) << 16).view(np.float32) * np.float32(0.5))


def test_bf16_compression_integer_sync():
    """Integer gradients in [-8, 8] over 4 ranks: bf16 carries every partial sum
    exactly, so the compressed sync equals the exact mean."""
    n = 4
    numels = [7, 16, 40, 300]
    buckets = planner.plan(numels, 4, cap_bytes=512, first_bucket_bytes=64, world_size=n, vector_elems=8)
    grads = [[host_rank_rng(17, r).integers(-8, 9, m).astype(np.float32) for m in numels] for r in range(n)]
    out = ddp.ddp_sync(grads, buckets, "fp32", comm_dtype="bf16")
    for p in range(len(numels)):
        want = np.sum(np.stack([grads[r][p] for r in range(n)]).astype(np.float64), axis=0) / n
        for r in range(n):
            assert out[r][p].dtype == np.float32
            assert np.array_equal(out[r][p].astype(np.float64), want)


def test_bf16_compression_loses_precision_within_bound():
    """With Gaussian gradients the compressed sync differs from the fp32 sync,
    by at most the bf16 error of N roundings (packing + N-1 hops)."""
    n = 8
    numels = [5000]
    bf = planner.plan(numels, 4, world_size=n, vector_elems=8)
    fp = planner.plan(numels, 4, world_size=n)
    grads = host_grads(18, n, numels)
    comp = ddp.ddp_sync(grads, bf, "fp32", comm_dtype="bf16")
    full = ddp.ddp_sync(grads, fp, "fp32")
    assert not np.array_equal(comp[0][0], full[0][0])
    absum = np.sum(np.stack([np.abs(grads[r][0]).astype(np.float64) for r in range(n)]), axis=0)
    err = np.abs(comp[0][0].astype(np.float64) - full[0][0].astype(np.float64))
    assert np.all(err <= (2 * n) * 2.0 ** -8 * absum / n + 2.0 ** -20 * absum)
