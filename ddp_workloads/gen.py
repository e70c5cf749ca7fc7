"""Seeded input generators (no arithmetic of the method lives here)."""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int            # workload number k: rank r uses streams (k, r)
    n: int               # virtual ranks
    count: int           # elements per rank buffer (0 for the per-parameter workload)
    dtypes: tuple        # buffer dtypes the workload is run in
    dist: str            # "int8range": uniform integers in [-8, 8]; "normal"
    std: float = 0.0     # standard deviation for "normal"
    heavy_frac: float = 0.0   # fraction of elements multiplied by heavy_mult
    heavy_mult: float = 1.0
    on_device: bool = False   # inputs drawn on the GPU (too large for the host)


WORKLOADS = {
    "ring_n3_6": Workload("ring_n3_6", 1, 3, 6, ("fp32",), "int8range"),
    "ring_n8_25mib": Workload("ring_n8_25mib", 2, 8, 6_553_600, ("fp32",), "normal", 1e-3),
    "ddp_resnet50": Workload("ddp_resnet50", 3, 8, 0, ("fp32",), "normal", 1e-3),
    "ring_n8_1gib": Workload("ring_n8_1gib", 4, 8, 268_435_456, ("fp32", "bf16"), "normal", 1e-2,
                             on_device=True),
    "ring_n64_300m": Workload("ring_n64_300m", 5, 64, 300_000_000, ("fp32",), "normal", 1e-3,
                              heavy_frac=0.01, heavy_mult=1e3, on_device=True),
}


def elements_for(workload, dtype):
    """Elements per rank: the 1 GiB workload holds twice as many bf16 values."""
    if workload.name == "ring_n8_1gib" and dtype == "bf16":
        return 2 * workload.count
    return workload.count


def host_rank_rng(seed, rank):
    """Independent host stream of rank `rank` in workload `seed`."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, rank])))


def _draw_f32(rng, dist, count, std):
    if dist == "int8range":
        return rng.integers(-8, 9, size=count).astype(np.float32)
    if dist == "normal":
        return rng.normal(0.0, std, size=count).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def to_bf16_bits(x32):
    """bf16 bit patterns of float32 inputs, converted by torch on the CPU
    (round to nearest even); used only to make bf16 inputs."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def host_ring_inputs(seed, n, count, dtype="fp32", dist="normal", std=1e-3,
                     heavy_frac=0.0, heavy_mult=1.0):
    """N rank buffers of `count` elements drawn on the host.

    fp32 buffers come back as float32 arrays, bf16 buffers as uint16 bit
    patterns (the fp32 draw rounded to nearest even).
    """
    out = []
    for r in range(n):
        rng = host_rank_rng(seed, r)
        x = _draw_f32(rng, dist, count, std)
        if heavy_frac:
            mask = rng.random(count) < heavy_frac
            x[mask] *= np.float32(heavy_mult)
        out.append(to_bf16_bits(x) if dtype == "bf16" else x)
    return out


def host_grads(seed, n, numels, std=1e-3, dist="normal"):
    """Per-rank, per-parameter fp32 gradients: N lists of 1-D float32 arrays."""
    out = []
    for r in range(n):
        rng = host_rank_rng(seed, r)
        out.append([_draw_f32(rng, dist, int(m), std) for m in numels])
    return out


def device_ring_inputs(seed, n, count, dtype="fp32", std=1e-2, heavy_frac=0.0,
                       heavy_mult=1.0, device="cuda"):
    """N rank buffers drawn on the GPU with torch's generator seeded
    1000 * seed + rank; returns a list of torch tensors (float32 or bfloat16).

    All N buffers are allocated before any is drawn, as a trainer allocates
    its gradient buffers once, so no drawing temporary sits between two of
    them; the draws then go one rank at a time to bound the temporaries.
    (With the temporaries interleaved between the buffers, the 64-rank x 300M
    fused all-reduce ran ~20 % slower on MI355X, although every buffer still
    began on a 2 MiB boundary.)
    """
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = [torch.empty(count, dtype=tdt, device=device) for _ in range(n)]
    for r in range(n):
        g = torch.Generator(device=device)
        g.manual_seed(1000 * seed + r)
        x = torch.randn(count, generator=g, device=device, dtype=torch.float32)
        x.mul_(std)
        if heavy_frac:
            mask = torch.rand(count, generator=g, device=device) < heavy_frac
            x[mask] *= heavy_mult
            del mask
        out[r].copy_(x)  # bf16: rounded to nearest even, as .to(torch.bfloat16)
        del x
    return out
