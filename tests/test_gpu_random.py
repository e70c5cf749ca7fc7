"""Seeded random sweep of the ring entry points against the CPU oracle, bit
for bit: rank counts from 1 to 64; counts from 0 to 500k, half log-uniform
(so short and empty chunks occur) and half uniform over multi-tile sizes;
both dtypes; and per-rank buffer starts that are 16-byte aligned, all off by
the same amount, or mixed (some ranks aligned, some not). Each case is drawn
once from a fixed seed, so a failure names a case that can be rerun alone."""

import os

import numpy as np
import pytest
import torch

import ring_all_reduce_ddp_amd as rar
from oracle import ring
from ddp_workloads import host_ring_inputs

from gpu_util import TORCH_DTYPE, to_host, assert_bit_equal

pytestmark = pytest.mark.gpu

# DDP_RANDOM_SCALE=k draws k times as many cases of each sweep (default 1).
SCALE = max(1, int(os.environ.get("DDP_RANDOM_SCALE", "1")))
N_CASES = 64 * SCALE


def draw_cases(seed=20261202):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(N_CASES):
        n = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 8, 8, 11, 16, 24, 33, 64]))
        u = rng.random()
        if u < 0.05:
            count = 0
        elif u < 0.55:
            count = int(np.exp(rng.uniform(0, np.log(300_000))))
        else:
            count = int(rng.integers(20_000, 500_000))
        count = min(count, 4_000_000 // n)
        dtype = "fp32" if rng.random() < 0.6 else "bf16"
        mode = rng.choice(["aligned", "aligned", "same_offset", "mixed"])
        if mode == "aligned":
            pads = [0] * n
        elif mode == "same_offset":
            pads = [int(rng.integers(1, 8))] * n
        else:
            pads = [int(rng.integers(0, 8)) if rng.random() < 0.5 else 0 for _ in range(n)]
        variant = str(rng.choice(["fused", "steps", "persistent", "reduce_scatter"]))
        cases.append((i, n, count, dtype, tuple(pads), variant))
    return cases


def place(host, dtype, pads):
    """Device views of the host buffers, rank r starting pads[r] elements into
    a 16-byte aligned allocation of its own."""
    out = []
    for a, p in zip(host, pads):
        if dtype == "fp32":
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        else:
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
        big = torch.zeros(len(a) + p + 8, dtype=t.dtype, device="cuda")
        big[p:p + len(a)] = t.cuda()
        out.append(big[p:p + len(a)])
    return out


@pytest.mark.parametrize("case", draw_cases(), ids=lambda c: f"{c[0]}-n{c[1]}-c{c[2]}-{c[3]}-{c[5]}")
def test_random_case(case):
    i, n, count, dtype, pads, variant = case
    print(f"case {i}: n={n} count={count} {dtype} pads={pads} {variant}", flush=True)
    host = host_ring_inputs(1000 + i, n, count, dtype, std=1e-2)
    dev = place(host, dtype, pads)
    if variant == "reduce_scatter":
        want = ring.reduce_scatter(host, dtype, np.float32(1) / np.float32(n))
        L = -(-count // n) if n else 0
        shards = []
        for c in range(n):
            lo, hi = min(c * L, count), min((c + 1) * L, count)
            shards.append(torch.full((hi - lo,), float("nan"), dtype=TORCH_DTYPE[dtype], device="cuda")
                          if hi > lo else None)
        rar.ring_reduce_scatter_fused(dev, shards, float(np.float32(1) / np.float32(n)))
        torch.cuda.synchronize()
        for c in range(n):
            if shards[c] is None:
                assert len(want[c]) == 0
            else:
                assert_bit_equal(to_host(shards[c], dtype), want[c], f"case {i} shard {c}")
        for r in range(n):
            assert_bit_equal(to_host(dev[r], dtype), host[r], f"case {i} input {r} changed")
        return
    want = ring.ring_simulate(host, dtype)["bufs"]
    if variant == "fused":
        rar.ring_allreduce_fused(dev)
    elif variant == "steps":
        if n > 1:
            rar.ring_allreduce_stepwise(dev)
    else:
        rar.ring_allreduce_persistent(dev)
    torch.cuda.synchronize()
    if variant == "persistent":
        rar.ddp_persistent_status()
    for r in range(n):
        assert_bit_equal(to_host(dev[r], dtype), want[r], f"case {i} rank {r}")


# ---------------------------------------------------------------- many ranks, equal chunks

N_SPAN_CASES = 16 * SCALE


def draw_span_cases(seed=20261204):
    """60 to 64 ranks and equal chunks of whole vectors (the span kernels of
    the fused all-reduce and the reduce-scatter output): chunk lengths drawn
    as random multiples of the vector length, so chunk starts fall anywhere
    relative to the 64-vector span grid and spans end anywhere in a chunk."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(N_SPAN_CASES):
        n = int(rng.integers(60, 65))
        dtype = "fp32" if rng.random() < 0.6 else "bf16"
        v = 4 if dtype == "fp32" else 8
        L = v * int(np.exp(rng.uniform(0, np.log(6000))))
        variant = str(rng.choice(["fused", "reduce_scatter"]))
        cases.append((100 + i, n, n * L, dtype, (0,) * n, variant))
    return cases


@pytest.mark.parametrize("case", draw_span_cases(), ids=lambda c: f"{c[0]}-n{c[1]}-c{c[2]}-{c[3]}-{c[5]}")
def test_random_span_case(case):
    test_random_case(case)


# ---------------------------------------------------------------- whole DDP syncs

N_SYNC_CASES = 24 * SCALE


def draw_sync_cases(seed=20261203):
    """Random parameter lists (1 to 40 tensors, sizes log-uniform up to 200k,
    some empty or single-element), bucket capacities from 4 KiB to 25 MiB,
    1 to 13 ranks, fp32 or bf16 gradients or the bf16 compression hook, and
    every sync variant."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(N_SYNC_CASES):
        p = int(rng.integers(1, 41))
        numels = [0 if rng.random() < 0.05 else int(np.exp(rng.uniform(0, np.log(200_000)))) for _ in range(p)]
        cap = int(rng.choice([4096, 65536, 1 << 20, 25 << 20]))
        first = int(rng.choice([256, 4096, 1 << 20]))
        n = int(rng.choice([1, 2, 3, 4, 5, 8, 8, 13]))
        kind = str(rng.choice(["fp32", "bf16", "fp32_to_bf16"]))
        variant = str(rng.choice(["fused", "steps", "persistent", "view"]))
        cases.append((i, numels, cap, first, n, kind, variant))
    return cases


@pytest.mark.parametrize("case", draw_sync_cases(),
                         ids=lambda c: f"{c[0]}-p{len(c[1])}-n{c[4]}-{c[5]}-{c[6]}")
def test_random_sync(case):
    from test_gpu_ddp import sync_case
    i, numels, cap, first, n, kind, variant = case
    print(f"sync case {i}: {len(numels)} params (total {sum(numels)}), cap={cap} first={first} n={n} "
          f"{kind} {variant}", flush=True)
    dtype, comm = ("fp32", "bf16") if kind == "fp32_to_bf16" else (kind, None)
    sync_case(variant, n, dtype, numels, cap, first, seed=3000 + i, comm=comm)
