"""Device memory from the library's allocator (ddp_device_alloc): plain and
physically contiguous buffers hold the ring's rank buffers, and the
all-reduce on them equals the oracle's ring bit for bit. Views of the memory
are torch tensors over the same addresses."""

import numpy as np
import pytest
import torch

import ring_all_reduce_ddp_amd as rar
from ddp_workloads import host_ring_inputs
from oracle import ring

from gpu_util import to_device, to_host, assert_bit_equal

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("contiguous", [True, False])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_ring_on_library_buffers(contiguous, dtype):
    n, count = 8, 8 * 50_000 + 13
    host = host_ring_inputs(41, n, count, dtype, std=1e-2)
    want = ring.ring_simulate(host, dtype)["bufs"]
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    esize = 4 if dtype == "fp32" else 2
    print(f"[library buffers: {n} x {count} {dtype}, contiguous={contiguous}]", flush=True)
    mems = [rar.device_alloc(count * esize + 4096, contiguous=contiguous) for _ in range(n)]
    # rank r's buffer starts r * 16 bytes into its allocation
    bufs = [m.tensor(tdt, count, offset_bytes=16 * r) for r, m in enumerate(mems)]
    for b, src in zip(bufs, to_device(host, dtype)):
        b.copy_(src)
    assert all(b.data_ptr() == m.ptr + 16 * r for r, (b, m) in enumerate(zip(bufs, mems)))
    rar.ring_allreduce_fused(bufs)
    torch.cuda.synchronize()
    for r in range(n):
        assert_bit_equal(to_host(bufs[r], dtype), want[r], f"rank {r}")
    # the step form on the same memory, from the inputs again
    for b, src in zip(bufs, to_device(host, dtype)):
        b.copy_(src)
    rar.ring_allreduce_stepwise(bufs)
    torch.cuda.synchronize()
    for r in range(n):
        assert_bit_equal(to_host(bufs[r], dtype), want[r], f"steps, rank {r}")
    del bufs
    for m in mems:
        m.free()
        assert m.ptr is None
    m.free()  # a second free is a no-op


def test_buffer_views_are_checked():
    m = rar.device_alloc(1024, contiguous=True)
    assert m.tensor(torch.float32).numel() == 256
    assert m.tensor(torch.bfloat16, 100, offset_bytes=824).numel() == 100
    for args in ((torch.float32, 257, 0), (torch.float32, 1, 1024), (torch.float32, 4, 2), (torch.float32, 1, -4)):
        with pytest.raises(ValueError):
            m.tensor(*args)
    # the library checks ranges against the allocation: a buffer that runs past it is refused
    with pytest.raises(rar.DDPError, match="DDP_EINVAL"):
        rar.ring_allreduce_fused([m.ptr, m.ptr + 512], count=200, dtype="fp32")
    m.free()
    with pytest.raises(ValueError):
        m.tensor(torch.float32, 1)
