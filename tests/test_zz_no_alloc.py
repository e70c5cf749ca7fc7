"""ring_allreduce_persistent_noalloc, called through the C ABI, against
ring_allreduce_persistent on the same inputs, bit for bit: three calls in a
row on one stream, each with a smaller input than the last (the
allocation-free scratch keeps the previous call's words, so every call must
clear what it needs). The first input exceeds the Infinity Cache (tiles by
ticket), the second fits in it (a fixed share per block), the third has
chunks that are not whole vectors and is also checked against the oracle's
ring."""

import ctypes

import pytest
import torch

import ring_all_reduce_ddp_amd as rar
from oracle import ring
from ddp_workloads import device_ring_inputs, host_ring_inputs

from gpu_util import to_device, to_host, assert_bit_equal

pytestmark = pytest.mark.gpu

INT_VIEW = {"fp32": torch.int32, "bf16": torch.int16}
CODE = {"fp32": rar.DDP_FP32, "bf16": rar.DDP_BF16}


def noalloc(bufs, dtype, n_steps=None):
    n = len(bufs)
    ptrs = (ctypes.c_void_p * n)(*[b.data_ptr() for b in bufs])
    k = 2 * (n - 1) if n_steps is None else n_steps
    st = rar.lib.ring_allreduce_persistent_noalloc(ptrs, n, bufs[0].numel(), CODE[dtype], k,
                                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == rar.DDP_OK, rar.lib.ddp_last_error().decode()


def compare_with_persistent(n, count, dtype, seed):
    ref = device_ring_inputs(seed, n, count, dtype, std=1e-2)
    got = [t.clone() for t in ref]
    rar.ring_allreduce_persistent(ref)
    noalloc(got, dtype)
    torch.cuda.synchronize()
    rar.ddp_persistent_status()
    for r in range(n):
        assert torch.equal(got[r].view(INT_VIEW[dtype]), ref[r].view(INT_VIEW[dtype])), f"N={n} count={count} rank {r}"
    del ref, got
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_noalloc_matches_persistent_calls_in_a_row(dtype):
    v = 4 if dtype == "fp32" else 8
    # 1: 8 ranks x 1.28 GB in all (beyond the 256 MB Infinity Cache), chunks of
    # whole vectors: tiles handed out by the ticket counter in the scratch
    n, count = 8, 8 * 1_250_000 * v
    print(f"[noalloc {dtype}] call 1: N={n} count={count}", flush=True)
    compare_with_persistent(n, count, dtype, 77)
    # 2: smaller, inside the cache: a fixed share of tiles per block
    n, count = 8, 8 * 25_000 * v
    print(f"[noalloc {dtype}] call 2: N={n} count={count}", flush=True)
    compare_with_persistent(n, count, dtype, 78)
    # 3: smaller still, chunks that are not whole vectors (element by element),
    # all 8 steps and the first 3 alone, also against the oracle
    n, count = 5, 12_345
    print(f"[noalloc {dtype}] call 3: N={n} count={count}", flush=True)
    host = host_ring_inputs(79, n, count, dtype, std=1e-3)
    for n_steps in (None, 3):
        ref = to_device(host, dtype)
        got = to_device(host, dtype)
        rar.ring_allreduce_persistent(ref, n_steps)
        noalloc(got, dtype, n_steps)
        torch.cuda.synchronize()
        rar.ddp_persistent_status()
        want = ring.ring_simulate(host, dtype, n_steps=n_steps)["bufs"]
        for r in range(n):
            assert_bit_equal(to_host(got[r], dtype), to_host(ref[r], dtype), f"call 3 ({n_steps} steps) rank {r}")
            assert_bit_equal(to_host(got[r], dtype), want[r], f"call 3 ({n_steps} steps) rank {r} vs oracle")


def test_noalloc_argument_errors():
    """Bad arguments are refused before anything is launched, as for the
    allocating entry point."""
    lib = rar.lib
    bufs = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    assert lib.ring_allreduce_persistent_noalloc(bufs, 2, 10, 7, 2, None) == rar.DDP_EINVAL
    assert lib.ring_allreduce_persistent_noalloc(bufs, 2, 10, rar.DDP_FP32, 3, None) == rar.DDP_EINVAL
    assert "n_steps" in lib.ddp_last_error().decode()
    assert lib.ring_allreduce_persistent_noalloc(bufs, 2, 10, rar.DDP_FP32, 2, None) == rar.DDP_EINVAL
    assert "device allocation" in lib.ddp_last_error().decode()


def test_noalloc_timeout_is_reported_once():
    """The time-out path of the allocation-free launch, forced from the host
    (every barrier expects one block more than the grid holds, and gives up
    after 20 ms): every block exits, ddp_persistent_status reports it from the
    fixed array's status words once, and the next call is exact."""
    n, count = 4, 4 * 8192
    host = host_ring_inputs(80, n, count, "fp32")
    bufs = to_device(host, "fp32")
    print("[noalloc time-out] forced with the test hook", flush=True)
    rar.ddp_persistent_test_hook(1, 20_000)
    try:
        noalloc(bufs, "fp32")
        torch.cuda.synchronize()
    finally:
        rar.ddp_persistent_test_hook(0, 0)
    with pytest.raises(rar.DDPError, match="timed out"):
        rar.ddp_persistent_status()
    rar.ddp_persistent_status()  # cleared
    bufs = to_device(host, "fp32")
    noalloc(bufs, "fp32")
    torch.cuda.synchronize()
    rar.ddp_persistent_status()
    want = ring.ring_simulate(host, "fp32")["bufs"]
    for r in range(n):
        assert_bit_equal(to_host(bufs[r], "fp32"), want[r], f"after the time-out, rank {r}")
