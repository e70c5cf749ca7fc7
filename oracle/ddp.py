"""Pack, ring all-reduce, scale and unpack: one DDP gradient synchronisation.

TEST INFRASTRUCTURE ONLY: part of the CPU oracle. Only the tests, the smoke
check and the CPU-baseline leg of the benchmark may import this module.

What it follows:
  * page "DDP 与 Ring All-Reduce" (blog.vllbc.top), section 03 (default
    gradient_as_bucket_view=False: gradients are copied into the bucket before
    the all-reduce and the result is copied back into each parameter's .grad)
    and section 05, step 3 (after the all-reduce each rank holds the bucket's
    sum; the reducer divides by the world size);
  * page "Day 17 数据并行 DP/DDP" (blog.ans20xx.com), part "源码阅读路线": after
    each bucket's all-reduce completes, the bucket is divided by the world size
    and copied back into the parameters' gradients.

Readings where the pages leave a step open: the division by N is a multiplication
by the fp32 value scale = fl(1/N), rounded once to the buffer dtype; for N a
power of two this is exactly the division.  Buckets are processed in plan
order, one after the other.
"""

import numpy as np

from . import ring, rounding


def pack(grads, bucket, dtype, grad_dtype=None):
    """Copy one rank's per-parameter gradients into a flat bucket.

    grads      : list of one-dimensional arrays, indexed by parameter.
    bucket     : one entry of planner.plan().
    dtype      : the bucket's dtype.
    grad_dtype : the gradients' dtype (default: the bucket's). fp32 gradients
                 packed into a bf16 bucket are rounded to nearest even: the
                 compression of the bf16 communication hook.
    The positions not covered by a member (alignment slack and the tail
    padding) are zero.
    """
    grad_dtype = dtype if grad_dtype is None else grad_dtype
    out = np.zeros(bucket["padded_numel"], dtype=rounding.storage_dtype(dtype))
    for p, off, numel in bucket["members"]:
        g = np.asarray(grads[p])
        if g.shape != (numel,):
            raise ValueError(f"parameter {p}: expected {numel} elements")
        if grad_dtype == dtype:
            out[off:off + numel] = g
        else:
            out[off:off + numel] = rounding.round_to(rounding.to_f64(g, grad_dtype), dtype)
    return out


def unpack_scale(flat, bucket, scale, dtype, grad_dtype=None):
    """Per-parameter gradients from a reduced bucket, each element multiplied
    by the fp32 value `scale` and rounded once to the gradients' dtype
    (default: the bucket's dtype `dtype`).

    Returns a dict {param_index: array}.
    """
    grad_dtype = dtype if grad_dtype is None else grad_dtype
    s = float(np.float32(scale))
    out = {}
    for p, off, numel in bucket["members"]:
        x = rounding.to_f64(flat[off:off + numel], dtype)
        out[p] = rounding.round_to(x * s, grad_dtype)
    return out


def ddp_sync(grads_per_rank, buckets, dtype, scale=None, comm_dtype=None):
    """One gradient synchronisation over N ranks.

    grads_per_rank : N lists of per-parameter gradient arrays.
    buckets        : planner.plan(...) for these parameters.
    dtype          : the gradients' dtype.
    scale          : multiplier applied on unpack; default fl32(1/N).
    comm_dtype     : the buckets' (communication) dtype, default `dtype`. With
                     fp32 gradients and comm_dtype "bf16" this is the bf16
                     compression hook (page "Day 17 数据并行 DP/DDP", reading
                     list, "PyTorch DDP Communication Hooks": fp16/bf16
                     compression): gradients are rounded to bf16 when packed,
                     the ring adds in bf16 with a rounding per hop, and the
                     copy back widens to fp32, multiplies by `scale` and
                     rounds once to fp32.

    For each bucket in order: pack on every rank, ring all-reduce across the
    ranks, scale and unpack.  Returns N lists of per-parameter gradients.
    """
    n = len(grads_per_rank)
    comm = dtype if comm_dtype is None else comm_dtype
    if scale is None:
        scale = np.float32(1.0) / np.float32(n)
    n_params = len(grads_per_rank[0])
    out = [[None] * n_params for _ in range(n)]
    for bucket in buckets:
        flats = [pack(grads_per_rank[r], bucket, comm, dtype) for r in range(n)]
        reduced = ring.ring_simulate(flats, comm)["bufs"]
        for r in range(n):
            for p, g in unpack_scale(reduced[r], bucket, scale, comm, dtype).items():
                out[r][p] = g
    return out
