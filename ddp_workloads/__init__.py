"""Seeded synthetic inputs shared by the tests, the smoke check and the
benchmark.

This module holds no arithmetic of the method (no ring, no bucketing, no
scaling): only the shapes and seeded value distributions of the workloads, so
that the GPU library and the CPU oracle can be fed the same bytes while
sharing no code.

Workloads (N = number of virtual ranks):
  ring_n3_6      N=3, 6 fp32 elements per rank (3 chunks of 2), uniform
                 integers in [-8, 8]; the size of the pages' worked example.
  ring_n8_25mib  N=8, one 25 MiB fp32 bucket per rank (6,553,600 elements),
                 N(0, 1e-3).
  ddp_resnet50   N=8, per-rank fp32 gradients with ResNet-50's 161 parameter
                 shapes (25,557,032 elements), N(0, 1e-3).
  ring_n8_1gib   N=8, 1 GiB per rank: 268,435,456 fp32 or 536,870,912 bf16
                 elements, N(0, 1e-2) (bf16 = fp32 draw rounded to nearest even).
  ring_n64_300m  N=64, 300,000,000 fp32 elements per rank, N(0, 1e-3) with 1 %
                 of the elements (Bernoulli per element) multiplied by 1000.

Seeding: workload k uses seed k; rank r draws from
numpy.random.Generator(PCG64(SeedSequence([k, r]))) on the host, or from
torch.Generator('cuda').manual_seed(1000 * k + r) on the device for the two
large workloads.  "N(0, s)" means standard deviation s.
"""

from .shapes import resnet50_param_shapes, resnet50_param_numels  # noqa: F401
from .gen import (WORKLOADS, host_rank_rng, host_ring_inputs, host_grads,  # noqa: F401
                  device_ring_inputs, Workload)
