"""Helpers for the GPU parity tests: moving rank buffers between numpy (the
oracle's representation: float32, or uint16 bf16 bits) and the device."""

import numpy as np
import torch

TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


def to_device(arrs, dtype, pad_front=0):
    """Device tensors holding the numpy rank buffers. pad_front > 0 places each
    buffer `pad_front` elements into a larger allocation (to test unaligned
    starts); the returned tensors are views starting at the data."""
    out = []
    for a in arrs:
        a = np.ascontiguousarray(a)
        if dtype == "fp32":
            t = torch.from_numpy(a.astype(np.float32))
        else:
            t = torch.from_numpy(a.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
        if pad_front:
            big = torch.zeros(len(a) + pad_front, dtype=t.dtype, device="cuda")
            big[pad_front:] = t.cuda()
            out.append(big[pad_front:])
        else:
            out.append(t.cuda())
    return out


def to_host(t, dtype):
    """numpy copy of one device buffer in the oracle's representation."""
    t = t.detach().cpu().contiguous()
    if dtype == "fp32":
        return t.numpy().astype(np.float32)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def mean_scale(n):
    """DDP's divide-by-world-size as the fp32 multiplier fl(1/N) that the
    caller passes to the sync entry points."""
    return float(np.float32(1) / np.float32(n))


def bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def assert_bit_equal(got, want, what=""):
    g, w = bits(got), bits(want)
    if g.shape != w.shape or not np.array_equal(g, w):
        gv = np.ascontiguousarray(got)
        wv = np.ascontiguousarray(want)
        bad = np.nonzero(gv.view(np.uint8).reshape(len(gv), -1).any(axis=1) !=
                         wv.view(np.uint8).reshape(len(wv), -1).any(axis=1))[0] \
            if gv.shape == wv.shape else []
        diff = np.nonzero(gv != wv)[0] if gv.shape == wv.shape else []
        first = int(diff[0]) if len(diff) else -1
        raise AssertionError(f"{what}: {len(diff)} elements differ (first at {first}: "
                             f"got {gv[first] if first >= 0 else None}, want {wv[first] if first >= 0 else None})"
                             if len(diff) or len(bad) else f"{what}: shapes {gv.shape} vs {wv.shape}")


def sample_positions(count, n, k, seed):
    """k random positions plus the first and last element of every chunk."""
    rng = np.random.default_rng(seed)
    L = -(-count // n)
    edges = []
    for c in range(n):
        lo, hi = c * L, min((c + 1) * L, count)
        if lo < hi:
            edges += [lo, lo + 1, hi - 2, hi - 1]
    pos = np.concatenate([rng.integers(0, count, size=k), np.array(edges, dtype=np.int64)])
    pos = pos[(pos >= 0) & (pos < count)]
    return np.unique(pos)


def gather(t, pos_dev, dtype):
    """Values of one device buffer at the given positions, in the oracle's representation."""
    return to_host(t.index_select(0, pos_dev), dtype)
