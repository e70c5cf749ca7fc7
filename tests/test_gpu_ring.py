"""GPU parity of the three ring all-reduce forms against the CPU oracle, bit
for bit, on small and ragged inputs (several tiles, short and empty chunks,
unaligned buffers, both dtypes) and hop by hop on the 3-rank example."""

import numpy as np
import pytest
import torch

import ring_all_reduce_ddp_amd as rar
from oracle import ring
from ddp_workloads import WORKLOADS, host_ring_inputs

from gpu_util import to_device, to_host, assert_bit_equal

pytestmark = pytest.mark.gpu

VARIANTS = ["fused", "steps", "persistent"]


def run_variant(variant, bufs, n_steps=None):
    if variant == "fused":
        rar.ring_allreduce_fused(bufs)
    elif variant == "steps":
        n = len(bufs)
        k = 2 * (n - 1) if n_steps is None else n_steps
        for i in range(k):
            phase, s = (rar.DDP_RS, i) if i < n - 1 else (rar.DDP_AG, i - (n - 1))
            rar.ring_allreduce_step(bufs, s, phase)
    elif variant == "persistent":
        rar.ring_allreduce_persistent(bufs, n_steps)
    else:
        raise ValueError(variant)
    torch.cuda.synchronize()
    if variant == "persistent":
        rar.ddp_persistent_status()


def check_against_oracle(n, count, dtype, variant, seed, std=1e-3, pad_front=0, n_steps=None):
    host = host_ring_inputs(seed, n, count, dtype, std=std)
    want = ring.ring_simulate(host, dtype, n_steps=n_steps)["bufs"]
    dev = to_device(host, dtype, pad_front=pad_front)
    run_variant(variant, dev, n_steps)
    for r in range(n):
        assert_bit_equal(to_host(dev[r], dtype), want[r], f"{variant} n={n} count={count} {dtype} rank {r}")


# ---------------------------------------------------------------- the 3-rank, 6-element example

def c1_inputs():
    w = WORKLOADS["ring_n3_6"]
    return host_ring_inputs(w.seed, w.n, w.count, "fp32", dist=w.dist)


@pytest.mark.parametrize("variant", ["steps", "persistent"])
def test_c1_hop_by_hop(variant):
    """State of every rank after each of the 4 steps equals the oracle's."""
    host = c1_inputs()
    states = ring.ring_simulate(host, "fp32", record=True)["states"]
    for k in range(1, 5):
        dev = to_device(host, "fp32")
        run_variant(variant, dev, n_steps=k)
        for r in range(3):
            assert_bit_equal(to_host(dev[r], "fp32"), states[k - 1][2][r], f"{variant} after {k} steps, rank {r}")


def test_c1_fused_and_exact_sum():
    host = c1_inputs()
    dev = to_device(host, "fp32")
    run_variant("fused", dev)
    want = np.sum(np.stack(host).astype(np.int64), axis=0)
    for r in range(3):
        assert np.array_equal(to_host(dev[r], "fp32").astype(np.int64), want)


# ---------------------------------------------------------------- small and ragged

# Chunk lengths that are whole vectors take the chunk-tiled vector kernels.
# Other lengths of at least one tile take the buffer-tiled fused kernel, in
# which a tile may cross a chunk boundary (and, in bf16 with an odd length,
# split a word between two chunks): (5, 12345), (7, 43019), (8, 65541),
# (12, 36017), (33, 8482). Shorter ones take the element-wise kernels.
# (8, 25), (6, 6141), (8, 7 * 4096 + 4093) and (9, 100_003) end in a partial
# vector (and (8, 25) in an empty chunk) on the vector path. Equal chunks of
# whole tiles (64 vectors) take the whole-tile kernel: (2, 4096), (8, 65536),
# (7, 10752) and (13, 13312) in both dtypes, (3, 3840) in fp32. From 60 ranks
# on, equal chunks of whole vectors take the span kernel instead: (64, 65536)
# (whole spans), (64, 64000) (chunks that start mid-tile, so spans at both
# ends are clamped), (61, 61 * 8800) (interior and edge spans), (60, 60 * 8)
# (one vector per chunk in fp32) and (63, 63 * 2056).
SHAPES = [(2, 4096), (3, 6), (3, 7), (4, 3), (5, 12345), (6, 6141), (7, 7 * 2048 * 3 + 11),
          (8, 8 * 4096 * 2), (8, 8 * 4096 * 2 + 5), (8, 5), (8, 25), (8, 7 * 4096 + 4093), (9, 100_003),
          (12, 12 * 3001 + 5), (16, 16 * 1000), (33, 33 * 257 + 1), (64, 64 * 1024),
          (3, 3 * 1280), (7, 7 * 1536), (13, 13 * 1024),
          (64, 64 * 1000), (61, 61 * 8800), (60, 60 * 8), (63, 63 * 2056)]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n,count", SHAPES)
def test_against_oracle(variant, dtype, n, count):
    check_against_oracle(n, count, dtype, variant, seed=n * 1000 + count % 997)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_unaligned_buffers(variant, dtype):
    """Buffers that start off a 16-byte boundary take the element-wise path."""
    check_against_oracle(8, 8 * 3000, dtype, variant, seed=77, pad_front=1)


@pytest.mark.parametrize("variant", ["steps", "persistent"])
@pytest.mark.parametrize("k", [1, 3, 7, 8, 13])
def test_partial_steps_n8(variant, k):
    check_against_oracle(8, 8 * 5000 + 3, "fp32", variant, seed=k, n_steps=k)


@pytest.mark.parametrize("variant", VARIANTS)
def test_noops(variant):
    """count = 0 and N = 1 leave the buffers untouched."""
    one = to_device(host_ring_inputs(3, 1, 1000, "fp32"), "fp32")
    before = to_host(one[0], "fp32")
    if variant != "steps":  # a single rank has no steps to call
        run_variant(variant, one)
    assert_bit_equal(to_host(one[0], "fp32"), before, "N=1")
    two = to_device(host_ring_inputs(3, 4, 10, "fp32"), "fp32")
    snap = [to_host(t, "fp32") for t in two]
    if variant == "fused":
        rar.ring_allreduce_fused(two, count=0)
    elif variant == "persistent":
        rar.ring_allreduce_persistent(two, count=0)
    else:
        rar.ring_allreduce_step(two, 0, rar.DDP_RS, count=0)
    torch.cuda.synchronize()
    for t, s in zip(two, snap):
        assert_bit_equal(to_host(t, "fp32"), s, "count=0")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_special_values(dtype):
    """Subnormals are kept (no flush to zero), infinities propagate, signed
    zeros follow IEEE; NaN positions (not payloads) agree."""
    n, count = 4, 4096
    rng = np.random.default_rng(5)
    host = []
    for r in range(n):
        x = rng.normal(0, 1, count).astype(np.float32)
        tiny = np.float32(2.0 ** -140) if dtype == "fp32" else np.float32(2.0 ** -128)
        x[:1024] = (rng.integers(-3, 4, 1024) * tiny).astype(np.float32)   # subnormals
        x[1024:1030] = [np.inf, -np.inf, 0.0, -0.0, 3e38, -3e38]
        x[1030 + r] = np.nan
        host.append(x)
    if dtype == "bf16":
        from ddp_workloads.gen import to_bf16_bits
        host = [to_bf16_bits(x) for x in host]
    want = ring.ring_simulate(host, dtype)["bufs"]
    for variant in VARIANTS:
        dev = to_device(host, dtype)
        run_variant(variant, dev)
        for r in range(n):
            got = to_host(dev[r], dtype)
            gv = got.view(np.uint32 if dtype == "fp32" else np.uint16)
            wv = want[r].view(np.uint32 if dtype == "fp32" else np.uint16)
            expo = 0x7F800000 if dtype == "fp32" else 0x7F80
            frac = 0x007FFFFF if dtype == "fp32" else 0x007F
            gnan = ((gv & expo) == expo) & ((gv & frac) != 0)
            wnan = ((wv & expo) == expo) & ((wv & frac) != 0)
            assert np.array_equal(gnan, wnan), (variant, r)
            assert np.array_equal(gv[~wnan], wv[~wnan]), (variant, r)


def hip_malloc(nbytes):
    """A device allocation of exactly nbytes, straight from the HIP runtime
    torch uses (torch's allocator rounds sizes up to its own segments)."""
    import ctypes
    import os
    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    p = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(p), ctypes.c_size_t(nbytes)) == 0
    return hip, p.value


def test_errors_on_device_arguments():
    """Ranges past an allocation and overlapping buffers are refused."""
    import ctypes
    hip, p = hip_malloc(4096)
    try:
        with pytest.raises(rar.DDPError, match="past the end"):
            rar.ring_allreduce_fused([p, p + 2048], count=600, dtype="fp32")
        rar.ring_allreduce_fused([p, p + 2048], count=512, dtype="fp32")   # exactly fits
        torch.cuda.synchronize()
    finally:
        hip.hipFree(ctypes.c_void_p(p))
    big = torch.zeros(1000, device="cuda")
    with pytest.raises(rar.DDPError, match="overlap"):
        rar.ring_allreduce_fused([big[:600], big[400:]], count=500)
    with pytest.raises(rar.DDPError, match="not inside a device allocation"):
        host = torch.zeros(100)
        rar.ring_allreduce_fused([host, host.clone()], count=100, dtype="fp32")


def test_mismatch_counter():
    dev = to_device(host_ring_inputs(8, 4, 10000, "fp32"), "fp32")
    out = torch.zeros(1, dtype=torch.int64, device="cuda")
    rar.ddp_count_mismatches(dev, out)
    torch.cuda.synchronize()
    assert int(out.item()) > 9000
    rar.ring_allreduce_fused(dev)
    rar.ddp_count_mismatches(dev, out)
    torch.cuda.synchronize()
    assert int(out.item()) == 0
    dev[2][77] += 1.0
    rar.ddp_count_mismatches(dev, out)
    torch.cuda.synchronize()
    assert int(out.item()) == 1


def test_copy_probe():
    src = torch.randn(1 << 20, device="cuda")
    dst = torch.empty_like(src)
    rar.ddp_copy_probe(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_persistent_grid_leaves_headroom():
    grid, cus = rar.ddp_persistent_grid(8, 268435456, "fp32")
    assert 1 <= grid <= 2 * cus
    small, _ = rar.ddp_persistent_grid(3, 6, "fp32")
    # a tiny buffer is limited by its tiles: 3 transfers x (1 tile + 1 for the
    # tile grid's alignment) per step
    assert small == 6


def test_persistent_timeout_path_exits_and_reports():
    """A barrier told to wait for one block more than the grid has gives up
    after its deadline (20 ms here): every block exits, the status call
    reports the time-out once, and the next launch is unaffected."""
    host = host_ring_inputs(31, 4, 4 * 8192, "fp32")
    dev = to_device(host, "fp32")
    rar.ring_allreduce_persistent_ex(dev, extra_arrivals=1, timeout_us=20_000)
    torch.cuda.synchronize()
    with pytest.raises(rar.DDPError, match="timed out"):
        rar.ddp_persistent_status()
    rar.ddp_persistent_status()          # the flag was cleared
    dev = to_device(host, "fp32")
    run_variant("persistent", dev)
    want = ring.ring_simulate(host, "fp32")["bufs"]
    for r in range(4):
        assert_bit_equal(to_host(dev[r], "fp32"), want[r], f"after a time-out, rank {r}")


@pytest.mark.parametrize("max_blocks", [1, 7, 256, 1000])
def test_persistent_grid_sizes(max_blocks):
    """Any cooperative grid size gives the same bits."""
    host = host_ring_inputs(32, 8, 8 * 40000 + 8, "fp32")
    want = ring.ring_simulate(host, "fp32")["bufs"]
    dev = to_device(host, "fp32")
    rar.ring_allreduce_persistent_ex(dev, max_blocks=max_blocks)
    torch.cuda.synchronize()
    rar.ddp_persistent_status()
    for r in range(8):
        assert_bit_equal(to_host(dev[r], "fp32"), want[r], f"max_blocks={max_blocks} rank {r}")


# Buffers beyond the 256 MiB Infinity Cache take the persistent kernel whose
# tiles are handed out by a ticket counter: 8 ranks x (8 x 1,100,000 + 3)
# fp32 (282 MB; chunk lengths that are not whole vectors, a short last chunk).
BIG_N, BIG_COUNT = 8, 8 * 1_100_000 + 3


@pytest.fixture(scope="module")
def big_inputs():
    return host_ring_inputs(34, BIG_N, BIG_COUNT, "fp32")


@pytest.mark.parametrize("n_steps,max_blocks", [(1, 0), (8, 0), (14, 0), (14, 17), (14, 1000), (13, 61)])
def test_persistent_tickets_beyond_cache(big_inputs, n_steps, max_blocks):
    """Partial and full step counts and several grids on the ticketed path
    give the oracle's state after that many steps, bit for bit."""
    assert BIG_N * BIG_COUNT * 4 > 256 << 20
    want = ring.ring_simulate(big_inputs, "fp32", n_steps=n_steps)["bufs"]
    dev = to_device(big_inputs, "fp32")
    rar.ring_allreduce_persistent_ex(dev, n_steps=n_steps, max_blocks=max_blocks)
    torch.cuda.synchronize()
    rar.ddp_persistent_status()
    for r in range(BIG_N):
        assert_bit_equal(to_host(dev[r], "fp32"), want[r], f"steps={n_steps} max_blocks={max_blocks} rank {r}")


def test_persistent_tickets_timeout_path(big_inputs):
    """The time-out path on the ticketed kernel: every block leaves at the
    barrier it cannot pass, the status call reports it once, and a normal
    launch afterwards is exact."""
    dev = to_device(big_inputs, "fp32")
    rar.ring_allreduce_persistent_ex(dev, extra_arrivals=1, timeout_us=20_000)
    torch.cuda.synchronize()
    with pytest.raises(rar.DDPError, match="timed out"):
        rar.ddp_persistent_status()
    rar.ddp_persistent_status()
    dev = to_device(big_inputs, "fp32")
    run_variant("persistent", dev)
    want = ring.ring_simulate(big_inputs, "fp32")["bufs"]
    for r in range(BIG_N):
        assert_bit_equal(to_host(dev[r], "fp32"), want[r], f"after a time-out, rank {r}")


def test_persistent_slots_reused_across_two_streams():
    """130 persistent launches queued on two streams behind long-running
    kernels, so all are in flight at once and the device's 64 barrier slots
    are each handed out two or three times, alternately to launches on the two
    streams (20 launches on one, then 20 on the other). A slot's next user
    waits for its previous user: every result equals the oracle's."""
    n, count, k = 4, 4 * 2000 + 3, 130
    hosts = [host_ring_inputs(500 + i, n, count, "fp32") for i in range(k)]
    devs = [to_device(h, "fp32") for h in hosts]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    src = [torch.randn(65536, device="cuda") for _ in range(2)]
    dst = [torch.empty_like(t) for t in src]
    torch.cuda.synchronize()
    for st in streams:   # ~10 ms of dependent arithmetic at the head of each stream
        rar.ddp_synthetic_backward(src, dst, work=3_000_000, stream=st)
    for i in range(k):
        rar.ring_allreduce_persistent(devs[i], stream=streams[(i // 20) % 2])
    torch.cuda.synchronize()
    rar.ddp_persistent_status()
    for i in range(k):
        want = ring.ring_simulate(hosts[i], "fp32")["bufs"]
        for r in range(n):
            assert_bit_equal(to_host(devs[i][r], "fp32"), want[r], f"launch {i} rank {r}")
