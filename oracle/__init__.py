"""CPU oracle for the bucketed ring all-reduce of DDP gradients.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow reference that the
GPU library is checked against. Only `tests/`, `__graft_entry__.smoke()` and
the `cpu_baseline` leg of `bench.py` may import it; the library and its Python
binding never do, and nothing here imports them.

Modules:
  rounding : exact values of fp32/bf16 buffers and rounding of fp64 results
             back to the buffer dtype (nearest, ties to even);
  ring     : hop-by-hop simulation of the two-phase ring all-reduce and the
             closed form of its per-chunk addition order;
  planner  : reverse-order bucket assignment with 1 MiB / 25 MiB capacities;
  ddp      : pack, all-reduce, scale by 1/N and unpack for a whole sync.

Every function cites the passage of the pages it follows in its docstring.
The oracle's checks against what the pages and mathematics fix live in
tests/test_oracle_*.py.  Parity status per function:
  rounding.round_to_fp32 / round_to_bf16 : pinned (library conversions,
      hand-derived halfway cases)
  ring.ring_simulate                     : pinned (worked example, integer
      brute force, association-order fixtures, invariants, error bound)
  ring.ring_order_sum                    : pinned (association-order fixtures)
  ring.error_bound / abs_sum_f64, rounding.unit_roundoff
                                         : pinned (hand-derived bound cases in
      which the bound is reached, numpy's and torch's spacing above 1, fsum)
  ring.reduce_scatter                    : pinned (integer shards, closed-form
      ring-order sums of each chunk)
  planner.plan                           : pinned on constants, invariants and
      hand-derived plans; the exact ResNet-50 split depends on the reading of
      "capacity" and is parity unpinned by the pages
  ddp.pack / unpack_scale / ddp_sync     : pinned (round trips, exact scaling
      by 1/8, integer brute force)
"""

from . import rounding, ring, planner, ddp  # noqa: F401
from .rounding import FP32, BF16  # noqa: F401
