"""Hop-by-hop CPU simulation of the two-phase ring all-reduce over N ranks.

TEST INFRASTRUCTURE ONLY: part of the CPU oracle. Only the tests, the smoke
check and the CPU-baseline leg of the benchmark may import this module.

What it follows:
  * page "DDP 与 Ring All-Reduce" (blog.vllbc.top), section 03 "两阶段：先规约，
    再扩散": the buffer of size S is cut into N chunks of S/N; the ranks form a
    ring in which each rank sends only to its right neighbour and receives only
    from its left one; the reduce-scatter phase has N-1 steps, in each of which
    every rank sends one chunk and adds the chunk it receives into its own
    copy; the all-gather phase has N-1 steps that forward reduced chunks and
    overwrite instead of adding;
  * page "DDP 与 Ring-AllReduce" (xuesongtap.github.io), §1.3.1 (2(N-1) steps)
    and the worked example of §1.3.2 (3 GPUs, 6 elements): it fixes which chunk
    each rank sends at each step.  In reduce-scatter step s (counted from 0)
    rank r sends chunk (r-1-s) mod N, so chunk c starts at rank c+1 and ends
    fully reduced on rank c; in all-gather step s rank r sends chunk
    (r-s) mod N.  The section 03 page says every other convention is a global
    shift with the same traffic; parity is defined against this one.

Readings where the pages are silent:
  * chunk length L = ceil(count / N); chunk c covers [c*L, min((c+1)*L, count))
    and may be short or empty when N does not divide count;
  * every hop rounds once to the buffer dtype (see rounding.py);
  * all sends of one step are taken from the state before the step (the
    pages draw the sends of a step as simultaneous).
"""

import numpy as np

from . import rounding


def chunk_length(count, n):
    """L = ceil(count / N) elements per chunk."""
    return -(-count // n) if n > 0 else 0


def chunk_bounds(count, n, c):
    """Element range [lo, hi) of chunk c; empty when lo >= count."""
    L = chunk_length(count, n)
    lo = min(c * L, count)
    hi = min((c + 1) * L, count)
    return lo, hi


def rs_chunk(r, s, n):
    """Chunk that rank r sends to rank r+1 in reduce-scatter step s."""
    return (r - 1 - s) % n


def ag_chunk(r, s, n):
    """Chunk that rank r sends to rank r+1 in all-gather step s."""
    return (r - s) % n


def right_neighbour(r, n):
    """Each rank sends only to its right neighbour in the ring."""
    return (r + 1) % n


def hop_add(received, local, dtype):
    """One reduce-scatter hop: the received partial sum plus the local value,
    rounded once to the buffer dtype (an IEEE add is commutative, so only the
    association fixed by the hops matters)."""
    return rounding.round_to(rounding.to_f64(received, dtype) + rounding.to_f64(local, dtype), dtype)


def hop_copy(received, local, dtype):
    """One all-gather hop: the received reduced chunk replaces the local copy."""
    return received


def _chunk_index(count, n, chunk_of):
    """Element index arrays of every chunk: contiguous ranges by default, or
    the positions whose entry in chunk_of equals c (used to run the ring on a
    sample of elements taken from a larger buffer)."""
    if chunk_of is None:
        return [slice(*chunk_bounds(count, n, c)) for c in range(n)]
    chunk_of = np.asarray(chunk_of)
    if chunk_of.shape != (count,):
        raise ValueError("chunk_of must give one chunk id per element")
    if count and (chunk_of.min() < 0 or chunk_of.max() >= n):
        raise ValueError("chunk ids must lie in [0, N)")
    return [np.nonzero(chunk_of == c)[0] for c in range(n)]


def _size(idx):
    if isinstance(idx, slice):
        return idx.stop - idx.start
    return len(idx)


def ring_simulate(bufs, dtype, n_steps=None, record=False, chunk_of=None):
    """Run the ring all-reduce on N rank buffers, one hop at a time.

    bufs     : sequence of N one-dimensional arrays of equal length (float32 for
               fp32, uint16 bf16 bit patterns for bf16); they are not modified.
    dtype    : "fp32" or "bf16".
    n_steps  : stop after this many of the 2(N-1) steps (reduce-scatter steps
               first, then all-gather steps); None runs all of them.
    record   : when true, also return the state of every rank after each step.
    chunk_of : optional chunk id per element, for running the ring on a
               sample of positions taken from a larger buffer; by default the
               chunks are contiguous ranges of length ceil(count / N).

    Returns a dict with
      "bufs"  : the N final buffers,
      "steps" : the number of steps run,
      "sent"  : elements sent by each rank (received counts are the same),
      "states": list of (phase, step, [N arrays]) after each step (if record).
    """
    n = len(bufs)
    if n < 1:
        raise ValueError("need at least one rank")
    store = rounding.storage_dtype(dtype)
    cur = [np.array(b, dtype=store, copy=True) for b in bufs]
    count = cur[0].shape[0]
    if any(b.shape != (count,) for b in cur):
        raise ValueError("every rank must contribute a buffer of the same length")
    chunks = _chunk_index(count, n, chunk_of)
    total = 2 * (n - 1)
    limit = total if n_steps is None else n_steps
    if not 0 <= limit <= total:
        raise ValueError(f"n_steps must lie in [0, {total}]")
    sent = [0] * n
    states = []
    done = 0

    # Reduce-scatter: N-1 steps, each rank adds what its left neighbour sends.
    for s in range(n - 1):
        if done == limit:
            break
        outgoing = [cur[r][chunks[rs_chunk(r, s, n)]].copy() for r in range(n)]
        for r in range(n):
            c = rs_chunk(r, s, n)
            dst = right_neighbour(r, n)
            cur[dst][chunks[c]] = hop_add(outgoing[r], cur[dst][chunks[c]], dtype)
            sent[r] += _size(chunks[c])
        done += 1
        if record:
            states.append(("rs", s, [b.copy() for b in cur]))

    # All-gather: N-1 steps, each rank overwrites with what its left neighbour sends.
    for s in range(n - 1):
        if done == limit:
            break
        outgoing = [cur[r][chunks[ag_chunk(r, s, n)]].copy() for r in range(n)]
        for r in range(n):
            c = ag_chunk(r, s, n)
            dst = right_neighbour(r, n)
            cur[dst][chunks[c]] = hop_copy(outgoing[r], cur[dst][chunks[c]], dtype)
            sent[r] += _size(chunks[c])
        done += 1
        if record:
            states.append(("ag", s, [b.copy() for b in cur]))

    out = {"bufs": cur, "steps": done, "sent": sent}
    if record:
        out["states"] = states
    return out


def ring_order_sum(x, c, dtype):
    """Closed form of the value the ring leaves in chunk c, per element.

    x is an (N, k) array: the N ranks' values of k elements that all lie in
    chunk c.  Following the reduce-scatter schedule, chunk c's running sum
    starts as rank c+1's value and picks up ranks c+2, c+3, ..., c (indices mod
    N) one hop at a time, with one rounding per hop:
        fl(...fl(fl(x[c+1] + x[c+2]) + x[c+3]) ... + x[c]).
    """
    x = np.asarray(x)
    n = x.shape[0]
    acc = x[(c + 1) % n].copy()
    for k in range(2, n + 1):
        acc = hop_add(acc, x[(c + k) % n], dtype)
    return acc


def reduce_scatter(bufs, dtype, scale=1.0):
    """Reduce-scatter output of the ring: the gradient shard of every rank.

    Runs the reduce-scatter phase (the first N-1 steps; page "DDP 与 Ring
    All-Reduce", blog.vllbc.top, section 03: after it every rank holds one
    chunk reduced over all ranks; page "DDP 与 Ring-AllReduce",
    xuesongtap.github.io, §1.3.2.1: that chunk is chunk r on rank r), then
    returns, for each rank r, its chunk r multiplied by the fp32 value `scale`
    with one rounding to the dtype (scale = 1/N gives the mean, as DDP's
    division by the world size). This is the gradient shard that sharded data
    parallelism keeps (page "DDP 与 Ring All-Reduce", section 07, the part on
    FSDP/ZeRO). Returns a list of N arrays; rank r's has the length of chunk r.
    """
    n = len(bufs)
    after = ring_simulate(bufs, dtype, n_steps=n - 1)["bufs"]
    count = len(after[0])
    s = float(np.float32(scale))
    out = []
    for r in range(n):
        lo, hi = chunk_bounds(count, n, r)
        out.append(rounding.round_to(rounding.to_f64(after[r][lo:hi], dtype) * s, dtype))
    return out


def sum_f64(bufs, dtype):
    """Per-element sum of the exact input values, correctly rounded to float64
    (Python's math.fsum per element; small inputs only)."""
    import math
    x = np.stack([rounding.to_f64(b, dtype) for b in bufs])
    return np.array([math.fsum(col) for col in x.T], dtype=np.float64)


def abs_sum_f64(bufs, dtype):
    """Per-element sum of |g_i| in float64 (used for the error bound)."""
    x = np.stack([np.abs(rounding.to_f64(b, dtype)) for b in bufs])
    return x.sum(axis=0)


def error_bound(bufs, dtype):
    """Per-element bound (N-1) * u * sum_i |g_i| on |ring result - exact sum|,
    with u = 2^-p the unit roundoff of the buffer dtype.

    The ring result is a recursive summation of the N values in one fixed
    order with one round-to-nearest per add; for recursive summation in any
    order the error is at most (n-1) * u * sum |x_i| with no higher-order term
    (C.-P. Jeannerod and S. M. Rump, "Improved error bounds for inner products
    in floating-point arithmetic", SIAM J. Matrix Anal. Appl. 34(2), 2013).
    It holds while no partial sum overflows."""
    n = len(bufs)
    return (n - 1) * rounding.unit_roundoff(dtype) * abs_sum_f64(bufs, dtype)
