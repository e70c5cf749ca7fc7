"""Benchmark of the bucketed ring all-reduce on one MI355X.

Headline workload: 8 virtual ranks, 1 GiB of fp32 gradient per rank
(268,435,456 elements, drawn N(0, 1e-2) on the GPU), reduced in place by the
fused ring-order kernel. One step = one complete all-reduce of the 8 buffers.
Reported: bus bandwidth 2(N-1)/N * S / t (the per-rank traffic of a ring
all-reduce), algorithm bandwidth S / t, and the HBM bandwidth of the kernel,
2 * N * S / t, against MI355X's 8 TB/s. The first launch, on the pristine
inputs and outside the timed region, is compared element by element with the
CPU oracle's hop-by-hop ring on the same inputs (`parity`).

Beside it, in the same run: the step-by-step and persistent forms, the
reduce-scatter output alone, the same inputs in one allocation with the ranks
offset by 4 KiB, in separate allocations with rank r starting r * 4 KiB into
its own, and in physically contiguous memory from the library's allocator,
and the bf16 buffers of the same workload, the
launch cost of the pages' 3-rank example, one default-size DDP bucket
(8 x 25 MiB, cache-resident, and again with the cache flushed before each
launch) in all three forms, a copy probe, the whole DDP sync of ResNet-50
gradients (8 ranks; copying, kernel by kernel, in-place, and bf16-compressed
both ways; copying and in place again with the cache flushed before each),
the overlap of that sync with a synthetic
backward over bucket capacities, the 64-rank 300M-element workload, and the
CPU oracle timed on the headline workload's own inputs.

Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W]
      the whole benchmark; prints one JSON line.
  python bench.py --config c1|c2|c3|c4|c5 [--variant V] [--dtype fp32|bf16]
                  [--graph] [--steps K] [--warmup W]
      one workload and one form only (for profiling a single kernel):
        c1  3 ranks x 6 elements    variants: fused, steps, persistent,
                                    persistent-noalloc, step
        c2  8 ranks x 25 MiB        variants: fused, steps, persistent,
                                    persistent-noalloc
        c3  ResNet-50 DDP sync, 8   variants: fused, steps, persistent, view,
                                    pack, unpack, allreduce, bf16-fused,
                                    bf16-view
        c4  8 ranks x 1 GiB         variants: fused, steps, persistent,
                                    persistent-noalloc, reduce-scatter
                                    (--dtype bf16 for bf16)
        c5  64 ranks x 300M fp32    variants: fused, steps, persistent,
                                    persistent-noalloc, reduce-scatter
        probe  the copy probe: 4 GiB read and 4 GiB written (variant: copy),
               the same-run ceiling and the scale for traffic counters
      persistent-noalloc is the allocation-free entry point, which --graph can
      capture; the persistent form itself is timed eagerly.
      K timed steps after W untimed ones (--graph: replays of a HIP graph of
      one step, so no host work sits between its launches); prints one JSON
      line.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ring all-reduce bus GB/s + HBM GB/s (% of MI355X peak), N=8, 1 GiB fp32"
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fused_n8_1gib_fp32.json")
# the sources the fused kernel is built from: its traffic figure is void once any changes
KERNEL_SOURCES = [os.path.join(ROOT, "ring_all_reduce_ddp_amd", "csrc", f)
                  for f in ("fused_kernels.hip", "ring_common.h", "hip_common.h")]

CONFIGS = {"c1": "ring_n3_6", "c2": "ring_n8_25mib", "c3": "ddp_resnet50", "c4": "ring_n8_1gib",
           "c5": "ring_n64_300m", "probe": "copy_probe_4gib"}
VARIANTS = {
    "c1": ("fused", "steps", "persistent", "persistent-noalloc", "step"),
    "c2": ("fused", "steps", "persistent", "persistent-noalloc"),
    "c3": ("fused", "steps", "persistent", "view", "pack", "unpack", "allreduce", "bf16-fused", "bf16-view"),
    "c4": ("fused", "steps", "persistent", "persistent-noalloc", "reduce-scatter"),
    "c5": ("fused", "steps", "persistent", "persistent-noalloc", "reduce-scatter"),
    "probe": ("copy",),
}


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", choices=["all", *CONFIGS], default="all",
                    help="one workload only (default: the whole benchmark)")
    ap.add_argument("--variant", default=None, help="the form to time with --config (default: fused; copy for probe)")
    ap.add_argument("--dtype", choices=["fp32", "bf16"], default="fp32", help="buffer dtype for --config c4")
    ap.add_argument("--graph", action="store_true",
                    help="with --config: time replays of a HIP graph of one step instead of eager calls")
    args = ap.parse_args(argv)
    if args.config == "all":
        if args.variant is not None or args.dtype != "fp32" or args.graph:
            ap.error("--variant, --dtype and --graph need --config")
    else:
        args.variant = args.variant or VARIANTS[args.config][0]
        if args.variant not in VARIANTS[args.config]:
            ap.error(f"--variant {args.variant} is not one of {', '.join(VARIANTS[args.config])} "
                     f"for --config {args.config}")
        if args.dtype == "bf16" and args.config != "c4":
            ap.error("--dtype bf16 is available for --config c4 only")
        if args.graph and args.variant == "persistent":
            ap.error("--graph: the persistent form orders its barrier words with events; time it eagerly "
                     "(or capture persistent-noalloc)")
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")
    return args


def ensure_library():
    from ring_all_reduce_ddp_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()


def time_launches(fn, reps, torch):
    """Mean milliseconds per call of fn() over `reps` calls, measured with HIP
    events on torch's current stream (the stream the library launches on)."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def time_each(fn, reps, torch, between=None):
    """Milliseconds of each of `reps` calls of fn(), each bracketed by its own
    pair of HIP events on torch's current stream; `between()`, if given, runs
    before every call, outside the timed pair. Returns (mean, median, min)."""
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in pairs:
        if between is not None:
            between()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in pairs)
    return sum(t) / reps, t[reps // 2] if reps % 2 else 0.5 * (t[reps // 2 - 1] + t[reps // 2]), t[0]


def gbps(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def graph_of(fn, torch):
    """fn()'s launches captured in a HIP graph (after one eager call, which
    makes a plan's device tables on first use): replaying it runs them back to
    back with no host work between them."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s, capture_error_mode="thread_local"):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def traffic_from_profile():
    """HBM bytes per launch of the fused kernel from the committed counter
    profile, or None if it is missing or was taken on other kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        prof = json.load(f)
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    sha = h.hexdigest()
    if prof.get("kernel_source_sha256") != sha:
        return None
    return prof.get("hbm_bytes_per_launch")


def mean_scale(n, np):
    """DDP's divide-by-world-size as the fp32 multiplier fl(1/N) of the copy back."""
    return float(np.float32(1) / np.float32(n))


# ---------------------------------------------------------------- workloads

def ring_bytes(variant, n, S):
    """Algorithmic HBM bytes of one all-reduce of N buffers of S bytes: the
    fused form reads and writes every rank once (2NS); each of the 2(N-1)
    steps reads 2 chunk-sets and writes 1 (reduce-scatter) or reads and writes
    1 (all-gather), 5(N-1)S in all; the reduce-scatter output reads N*S and
    writes S; one reduce-scatter step reads 2S and writes S."""
    if variant == "fused":
        return 2 * n * S
    if variant in ("steps", "persistent", "persistent-noalloc"):
        return 5 * (n - 1) * S
    if variant == "reduce-scatter":
        return (n + 1) * S
    if variant == "step":
        return 3 * S
    raise ValueError(variant)


def ring_step_fn(rar, variant, bufs, shards=None, scale=1.0):
    if variant == "fused":
        return lambda: rar.ring_allreduce_fused(bufs)
    if variant == "steps":
        return lambda: rar.ring_allreduce_stepwise(bufs)
    if variant == "persistent":
        return lambda: rar.ring_allreduce_persistent(bufs)
    if variant == "persistent-noalloc":
        return lambda: rar.ring_allreduce_persistent_noalloc(bufs)
    if variant == "step":
        return lambda: rar.ring_allreduce_step(bufs, 0, rar.DDP_RS)
    if variant == "reduce-scatter":
        return lambda: rar.ring_reduce_scatter_fused(bufs, shards, scale)
    raise ValueError(variant)


def add_copy_fraction(node, copy_gbps):
    """Adds hbm_frac_of_copy_probe beside every hbm_gbps figure in a nested
    dict of results (the copy probe itself excepted)."""
    if isinstance(node, dict):
        hbm = node.get("hbm_gbps", node.get("hbm_gbps_algorithmic"))
        if isinstance(hbm, (int, float)) and "bytes_moved" not in node:
            node["hbm_frac_of_copy_probe"] = round(hbm / copy_gbps, 4)
        for v in node.values():
            add_copy_fraction(v, copy_gbps)


def contiguous_copies(rar, torch, tensors):
    """Copies of equal-length fp32 tensors in physically contiguous memory
    from the library's allocator, one allocation each: (allocations, views),
    or (None, message) if the memory cannot be had."""
    mems = []
    try:
        for t in tensors:
            mems.append(rar.device_alloc(t.numel() * t.element_size(), contiguous=True))
    except rar.DDPError as e:
        for m in mems:
            m.free()
        return None, str(e)
    views = [m.tensor(t.dtype, t.numel()) for m, t in zip(mems, tensors)]
    for v, t in zip(views, tensors):
        v.copy_(t)
    torch.cuda.synchronize()
    return mems, views


class ResNet50Sync:
    """The ResNet-50 DDP sync over 8 ranks: plan, gradient arenas drawn on the
    GPU, bucket buffers (fp32, and bf16 for the compression hook)."""

    def __init__(self, rar, torch, np):
        from ddp_workloads import WORKLOADS, resnet50_param_numels
        self.rar = rar
        w = WORKLOADS["ddp_resnet50"]
        self.n = w.n
        self.numels = resnet50_param_numels()
        self.plan = rar.ddp_bucket_plan(self.numels, "fp32", world_size=w.n)
        self.inv_n = mean_scale(w.n, np)
        arena_numel, _ = self.plan.grad_arena()
        g = torch.Generator(device="cuda")
        self.arenas = []
        for r in range(w.n):
            g.manual_seed(1000 * w.seed + r)
            self.arenas.append(torch.randn(arena_numel, generator=g, device="cuda") * w.std)
        self.buckets = [[torch.empty(self.plan.bucket(b)[0], device="cuda") for _ in range(w.n)]
                        for b in range(self.plan.num_buckets)]
        self.cplan = rar.ddp_bucket_plan_ex(self.numels, "fp32", "bf16", world_size=w.n)
        self.cbuckets = [[torch.empty(self.cplan.bucket(b)[0], dtype=torch.bfloat16, device="cuda")
                          for _ in range(w.n)] for b in range(self.cplan.num_buckets)]
        self.grad_bytes = sum(self.numels) * 4

    def fn(self, variant):
        rar, plan = self.rar, self.plan
        nb = plan.num_buckets
        if variant in ("fused", "steps", "persistent"):
            return lambda: rar.ddp_sync(plan, self.arenas, self.buckets, variant=variant, scale=self.inv_n)
        if variant == "view":
            return lambda: rar.ddp_sync(plan, self.arenas, None, variant="view", scale=self.inv_n)
        if variant == "pack":
            return lambda: [rar.bucket_pack(plan, b, self.arenas, self.buckets[b]) for b in range(nb)]
        if variant == "unpack":
            return lambda: [rar.bucket_unpack_scale(plan, b, self.buckets[b], self.arenas, self.inv_n)
                            for b in range(nb)]
        if variant == "allreduce":
            return lambda: [rar.ring_allreduce_fused(self.buckets[b]) for b in range(nb)]
        if variant == "bf16-fused":
            return lambda: rar.ddp_sync(self.cplan, self.arenas, self.cbuckets, variant="fused", scale=self.inv_n)
        if variant == "bf16-view":
            return lambda: rar.ddp_sync(self.cplan, self.arenas, None, variant="view", scale=self.inv_n)
        raise ValueError(variant)

    def hbm_bytes(self, variant):
        """Algorithmic bytes of the member elements (bucket padding excluded):
        pack and unpack read and write every gradient once per rank (2NS
        each); the copying sync adds the bucket all-reduce (2NS fused,
        5(N-1)S by steps); the in-place sync reads and writes the gradients
        once (2NS)."""
        n, S = self.n, self.grad_bytes
        return {"fused": 6 * n * S, "steps": 4 * n * S + 5 * (n - 1) * S,
                "persistent": 4 * n * S + 5 * (n - 1) * S, "view": 2 * n * S, "pack": 2 * n * S,
                "unpack": 2 * n * S, "allreduce": 2 * n * S, "bf16-view": 2 * n * S}.get(variant)

    def free(self):
        self.plan.free()
        self.cplan.free()


# ---------------------------------------------------------------- one workload, one form

def run_single(args):
    ensure_library()
    import numpy as np
    import torch
    import ring_all_reduce_ddp_amd as rar
    from ddp_workloads import WORKLOADS, device_ring_inputs, host_ring_inputs
    from ddp_workloads.gen import elements_for

    torch.cuda.set_device(0)
    cfg, variant, dtype = args.config, args.variant, args.dtype
    cfg_info = {"workload": CONFIGS[cfg], "variant": variant}
    w = WORKLOADS.get(CONFIGS[cfg])
    sync = None
    if cfg == "probe":
        src = torch.empty(1 << 30, dtype=torch.float32, device="cuda").normal_()
        dst = torch.empty_like(src)
        n, S = 1, 4 << 30
        fn = lambda: rar.ddp_copy_probe(dst, src)  # noqa: E731
        hbm_bytes = 2 * S
        cfg_info.update({"bytes_read": S, "bytes_written": S})
    elif cfg == "c3":
        sync = ResNet50Sync(rar, torch, np)
        fn = sync.fn(variant)
        n, S = sync.n, sync.grad_bytes
        hbm_bytes = sync.hbm_bytes(variant)
        cfg_info.update({"virtual_ranks": n, "params": len(sync.numels), "grad_bytes_per_rank": S,
                         "buckets": sync.plan.num_buckets})
    else:
        count = elements_for(w, dtype)
        n = w.n
        if cfg == "c1":
            bufs = [torch.from_numpy(x).cuda() for x in host_ring_inputs(w.seed, w.n, w.count, "fp32", dist=w.dist)]
        else:
            print(f"bench: drawing {n} x {count} {dtype}", file=sys.stderr, flush=True)
            bufs = device_ring_inputs(w.seed, n, count, dtype, std=w.std, heavy_frac=w.heavy_frac,
                                      heavy_mult=w.heavy_mult)
        S = count * (4 if dtype == "fp32" else 2)
        shards = None
        if variant == "reduce-scatter":
            shards = [torch.empty(count // n, dtype=bufs[0].dtype, device="cuda") for _ in range(n)]
        fn = ring_step_fn(rar, variant, bufs, shards, mean_scale(n, np))
        hbm_bytes = ring_bytes(variant, n, S)
        cfg_info.update({"virtual_ranks": n, "elements_per_rank": count, "bytes_per_rank": S})
    print(f"bench: {cfg} {variant} {dtype}: {args.warmup} warm-up, {args.steps} timed"
          f"{' (graph replays)' if args.graph else ''}", file=sys.stderr, flush=True)
    if args.graph:
        fn = graph_of(fn, torch).replay
        cfg_info["graph_replay"] = True
    for _ in range(args.warmup):
        fn()
    ms = time_launches(fn, args.steps, torch)
    _, med, lo = time_each(fn, args.steps, torch)
    if variant.startswith("persistent"):
        rar.ddp_persistent_status()
    bus = gbps(2 * (n - 1) / n * S, ms) if cfg != "probe" else gbps(2 * S, ms)
    line = {"metric": METRIC, "value": round(bus, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype, "data": "synthetic (seeded)", "config": cfg_info,
            "algbw_gbps": round(gbps(S, ms), 2), "busbw_gbps": round(bus, 2),
            "ms_per_launch_median": round(med, 4), "ms_per_launch_min": round(lo, 4)}
    if hbm_bytes is not None:
        line["hbm_gbps"] = round(gbps(hbm_bytes, ms), 1)
        line["hbm_frac_of_peak"] = round(gbps(hbm_bytes, ms) / PEAK_HBM_GBPS, 4)
        line["algorithmic_hbm_bytes_per_step"] = hbm_bytes
    print(json.dumps(line), flush=True)
    if sync is not None:
        sync.free()


# ---------------------------------------------------------------- the whole benchmark

def run_all(args):
    ensure_library()
    import numpy as np
    import torch
    import ring_all_reduce_ddp_amd as rar
    from ddp_workloads import WORKLOADS, device_ring_inputs, host_ring_inputs

    torch.cuda.set_device(0)
    extras = {}

    # ------------------------------------------------------------ 64 ranks x 300M fp32
    # Measured first, on two sets of buffers: the first 76.8 GB this process
    # allocates, and a second set allocated while the first is still held.
    # The same kernel on the same values usually ran ~20 % slower on the
    # first set (and on buffers later allocated at its addresses); the step
    # kernels, which touch two ranks per block, ran alike on both.
    print("bench: 64 ranks x 300M fp32", file=sys.stderr, flush=True)
    w5 = WORKLOADS["ring_n64_300m"]
    S5 = w5.count * 4

    def n64_inputs():
        return device_ring_inputs(w5.seed, w5.n, w5.count, "fp32", std=w5.std, heavy_frac=w5.heavy_frac,
                                  heavy_mult=w5.heavy_mult)

    def n64_time(fn, nbytes, launches):
        fn()
        t = time_launches(fn, 5, torch)
        return {"ms": round(t, 3), "bus_gbps": round(gbps(2 * (w5.n - 1) / w5.n * S5, t), 1),
                "hbm_gbps": round(gbps(nbytes, t), 1), "launches": launches}

    first = n64_inputs()
    n64_first = n64_time(lambda: rar.ring_allreduce_fused(first), 2 * w5.n * S5, 1)
    b5 = n64_inputs()
    n64 = {}
    for name, launches in (("fused", 1), ("steps", 2 * (w5.n - 1)), ("persistent", 1)):
        n64[name] = n64_time(ring_step_fn(rar, name, b5), ring_bytes(name, w5.n, S5), launches)
    # reduce-scatter output: every rank's 1/N shard of the sum (reads N*S, writes S)
    shards5 = [torch.empty(w5.count // w5.n, device="cuda") for _ in range(w5.n)]
    n64["reduce_scatter_fused"] = n64_time(lambda: rar.ring_reduce_scatter_fused(b5, shards5, 1.0 / w5.n),
                                           (w5.n + 1) * S5, 1)
    del shards5
    n64["fused_on_first_allocation"] = n64_first
    rar.ddp_persistent_status()
    # The same values in physically contiguous memory from the library's
    # allocator: the slow first-allocation case above spends more time in
    # second-level address translation per request.
    del first
    torch.cuda.empty_cache()
    mems, views = contiguous_copies(rar, torch, b5)
    if mems is None:
        n64["fused_on_contiguous_allocation"] = {"error": views}
    else:
        n64["fused_on_contiguous_allocation"] = n64_time(lambda: rar.ring_allreduce_fused(views),
                                                         2 * w5.n * S5, 1)
        del views
        for m in mems:
            m.free()
    extras["ring_n64_300m"] = n64
    del b5
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ headline: fused, N=8, 1 GiB fp32
    w = WORKLOADS["ring_n8_1gib"]
    n, count = w.n, w.count
    S = count * 4
    bufs = device_ring_inputs(w.seed, n, count, "fp32", std=w.std)
    # the same input, copied to the host for the CPU oracle leg
    host_inputs = [t.cpu().numpy() for t in bufs]

    print("bench: headline fused all-reduce, 8 x 1 GiB fp32", file=sys.stderr, flush=True)
    # The first launch runs on the pristine inputs, outside the timed region;
    # its result is compared with the oracle's at the end.
    rar.ring_allreduce_fused(bufs)
    torch.cuda.synchronize()
    first_result = [t.cpu().numpy() for t in bufs]
    for _ in range(args.warmup):
        rar.ring_allreduce_fused(bufs)
    torch.cuda.synchronize()
    ms = time_launches(lambda: rar.ring_allreduce_fused(bufs), args.steps, torch)
    # the same launches one by one, for the median and the fastest
    _, ms_median, ms_min = time_each(lambda: rar.ring_allreduce_fused(bufs), args.steps, torch)
    mism = torch.zeros(1, dtype=torch.int64, device="cuda")
    rar.ddp_count_mismatches(bufs, mism)
    torch.cuda.synchronize()
    ranks_equal = int(mism.item()) == 0

    bus = gbps(2 * (n - 1) / n * S, ms)
    hbm_bytes = 2 * n * S
    hbm = gbps(hbm_bytes, ms)
    traffic = traffic_from_profile()

    # ------------------------------------------------------------ same workload, other forms
    reps = max(3, args.steps // 4)

    step_bytes = 5 * (n - 1) * S
    for name in ("steps", "persistent"):
        fn = ring_step_fn(rar, name, bufs)
        fn()
        t = time_launches(fn, reps, torch)
        extras[name] = {"ms": round(t, 4), "bus_gbps": round(gbps(2 * (n - 1) / n * S, t), 1),
                        "hbm_gbps": round(gbps(step_bytes, t), 1),
                        "hbm_frac_of_peak": round(gbps(step_bytes, t) / PEAK_HBM_GBPS, 4),
                        "launches": 2 * (n - 1) if name == "steps" else 1}
    rar.ddp_persistent_status()

    # reduce-scatter output (each rank's 1/N shard, scaled by 1/N): reads N*S, writes S
    shards = [torch.empty(count // n, device="cuda") for _ in range(n)]
    rar.ring_reduce_scatter_fused(bufs, shards, 1.0 / n)
    t = time_launches(lambda: rar.ring_reduce_scatter_fused(bufs, shards, 1.0 / n), reps, torch)
    rs_bytes = (n + 1) * S
    extras["reduce_scatter_fused"] = {"ms": round(t, 4), "hbm_gbps": round(gbps(rs_bytes, t), 1),
                                      "hbm_frac_of_peak": round(gbps(rs_bytes, t) / PEAK_HBM_GBPS, 4),
                                      "bus_gbps_rs_phase": round(gbps((n - 1) / n * S, t), 1)}
    del bufs, shards
    torch.cuda.empty_cache()

    # Layout study: the same kernel on the same inputs with the 8 rank buffers
    # carved from one allocation, rank r at byte r * (S + 4 KiB). Separate
    # 1 GiB allocations start 2 MiB apart, so every block's 8 loads of one
    # offset agree in their low 21 address bits; offsets between the ranks
    # that are not multiples of 8 KiB ran faster at this size (multiples of
    # 8 KiB up to 128 KiB did not), which points at DRAM bank conflicts.
    # Reported beside the headline, which keeps the separate allocations a
    # caller would normally hand over.
    pad = 4096 // 4
    arena = torch.empty(n * (count + pad), device="cuda")
    views = [arena[r * (count + pad): r * (count + pad) + count] for r in range(n)]
    for r, src in enumerate(device_ring_inputs(w.seed, n, count, "fp32", std=w.std)):
        views[r].copy_(src)
        del src
    rar.ring_allreduce_fused(views)
    t = time_launches(lambda: rar.ring_allreduce_fused(views), reps, torch)
    extras["layout_one_allocation_4kib_offset"] = {
        "ms": round(t, 4), "hbm_gbps": round(gbps(2 * n * S, t), 1),
        "hbm_frac_of_peak": round(gbps(2 * n * S, t) / PEAK_HBM_GBPS, 4),
        "rank_stride_bytes": (count + pad) * 4}
    # The same inputs in separate allocations from the library's allocator,
    # rank r's buffer starting r * 4 KiB into its own allocation, so that the
    # ranks' same-position accesses differ in their low address bits as in one
    # allocation, without carving the ranks from one block.
    offs = []
    for r in range(n):
        m = rar.device_alloc(S + r * 4096, contiguous=False)
        v = m.tensor(torch.float32, count, offset_bytes=r * 4096)
        v.copy_(views[r])
        offs.append((m, v))
    ov = [v for _, v in offs]
    rar.ring_allreduce_fused(ov)
    t = time_launches(lambda: rar.ring_allreduce_fused(ov), reps, torch)
    extras["layout_rank_offsets_4kib"] = {
        "ms": round(t, 4), "hbm_gbps": round(gbps(2 * n * S, t), 1),
        "hbm_frac_of_peak": round(gbps(2 * n * S, t) / PEAK_HBM_GBPS, 4),
        "buffers": "one allocation per rank (ddp_device_alloc), rank r starting r * 4 KiB into it"}
    del ov
    for m, _ in offs:
        m.free()
    del offs
    # The same inputs again, each rank in physically contiguous memory from the
    # library's allocator (ddp_device_alloc): less second-level address
    # translation per access than torch's allocations.
    mems, cviews = contiguous_copies(rar, torch, views)
    del arena, views
    torch.cuda.empty_cache()
    if mems is None:
        extras["contiguous_allocation"] = {"error": cviews}
    else:
        rar.ring_allreduce_fused(cviews)
        t = time_launches(lambda: rar.ring_allreduce_fused(cviews), reps, torch)
        extras["contiguous_allocation"] = {
            "ms": round(t, 4), "hbm_gbps": round(gbps(2 * n * S, t), 1),
            "hbm_frac_of_peak": round(gbps(2 * n * S, t) / PEAK_HBM_GBPS, 4),
            "buffers": "one physically contiguous allocation per rank (ddp_device_alloc)"}
        del cviews
        for m in mems:
            m.free()

    bb = device_ring_inputs(w.seed, n, 2 * count, "bf16", std=w.std)
    rar.ring_allreduce_fused(bb)
    t = time_launches(lambda: rar.ring_allreduce_fused(bb), reps, torch)
    extras["bf16_fused"] = {"ms": round(t, 4), "bus_gbps": round(gbps(2 * (n - 1) / n * S, t), 1),
                            "hbm_gbps": round(gbps(2 * n * S, t), 1),
                            "hbm_frac_of_peak": round(gbps(2 * n * S, t) / PEAK_HBM_GBPS, 4)}
    del bb
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ 3 ranks x 6 elements: launch cost
    # The four-step example of the pages: latency only (72 bytes in all), so
    # the figure is the time per call as issued from Python, and the kernel
    # time alone from one event pair per call.
    w1 = WORKLOADS["ring_n3_6"]
    b1 = [torch.from_numpy(x).cuda() for x in host_ring_inputs(w1.seed, w1.n, w1.count, "fp32", dist=w1.dist)]
    tiny = {"ranks": w1.n, "elements_per_rank": w1.count}
    for name, key in (("step", "step"), ("steps", "steps_all"), ("persistent", "persistent"), ("fused", "fused")):
        fn = ring_step_fn(rar, name, b1)
        fn()
        per_call = time_launches(fn, 1000, torch)
        _, med, lo = time_each(fn, 200, torch)
        tiny[key] = {"us_per_call_back_to_back": round(per_call * 1e3, 2),
                     "us_gpu_median": round(med * 1e3, 2), "us_gpu_min": round(lo * 1e3, 2)}
    rar.ddp_persistent_status()
    extras["ring_n3_6"] = tiny
    del b1

    # ------------------------------------------------------------ one default-size DDP bucket
    # 8 ranks x 25 MiB fp32 (6,553,600 elements): 200 MiB in all, inside the
    # 256 MB Infinity Cache, so the kernels' loads are cached here.
    w2 = WORKLOADS["ring_n8_25mib"]
    b2 = device_ring_inputs(w2.seed, w2.n, w2.count, "fp32", std=w2.std)
    S2 = w2.count * 4
    bucket = {"bytes_per_rank": S2, "cache_resident": True}
    for name in ("fused", "steps", "persistent"):
        fn = ring_step_fn(rar, name, b2)
        fn()
        t = time_launches(fn, 50, torch)
        bucket[name] = {"ms": round(t, 4), "bus_gbps": round(gbps(2 * (w2.n - 1) / w2.n * S2, t), 1),
                        "algorithm_gbps": round(gbps(S2, t), 1),
                        "hbm_gbps": round(gbps(ring_bytes(name, w2.n, S2), t), 1)}
    rar.ddp_persistent_status()
    # the same bucket with the Infinity Cache flushed before each launch by
    # writing a 512 MiB buffer (outside the timed region): HBM-resident inputs
    flush = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
    cold = {}
    for name in ("fused", "steps"):
        mean, med, lo = time_each(ring_step_fn(rar, name, b2), 20, torch, between=flush.zero_)
        cold[name] = {"ms_median": round(med, 4), "ms_min": round(lo, 4),
                      "bus_gbps": round(gbps(2 * (w2.n - 1) / w2.n * S2, med), 1)}
    bucket["after_cache_flush"] = cold
    del flush
    # the 14 step launches and the fused launch replayed from a HIP graph: no host work between launches
    replayed = {}
    for name in ("fused", "steps"):
        g = graph_of(ring_step_fn(rar, name, b2), torch)
        t = time_launches(g.replay, 50, torch)
        replayed[name] = {"ms": round(t, 4), "bus_gbps": round(gbps(2 * (w2.n - 1) / w2.n * S2, t), 1),
                          "hbm_gbps": round(gbps(ring_bytes(name, w2.n, S2), t), 1)}
        del g
    bucket["graph_replay"] = replayed
    extras["ring_n8_25mib"] = bucket
    del b2
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ copy probe (4 GiB read + 4 GiB written)
    src = torch.empty(1 << 30, dtype=torch.float32, device="cuda").normal_()
    dst = torch.empty_like(src)
    rar.ddp_copy_probe(dst, src)
    t = time_launches(lambda: rar.ddp_copy_probe(dst, src), reps, torch)
    extras["copy_probe"] = {"bytes_moved": 2 * src.numel() * 4, "ms": round(t, 4),
                            "gbps": round(gbps(2 * src.numel() * 4, t), 1)}
    del src, dst
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ whole DDP sync, ResNet-50, N=8
    rs = ResNet50Sync(rar, torch, np)
    wr_n, grad_bytes = rs.n, rs.grad_bytes
    sizes = [rs.plan.bucket(b)[0] * 4 for b in range(rs.plan.num_buckets)]
    sync = {"bucket_sizes": sizes, "params": len(rs.numels), "grad_bytes_per_rank": grad_bytes}
    sync_reps = 50  # a sync takes 0.3-2 ms
    for variant in ("fused", "steps", "persistent", "view"):
        fn = rs.fn(variant)
        fn()
        t = time_launches(fn, sync_reps, torch)
        sync[variant] = {"ms": round(t, 4),
                         "bus_gbps": round(gbps(2 * (wr_n - 1) / wr_n * grad_bytes, t), 1)}
        if variant in ("fused", "view"):
            # pack + fused + unpack move 6*N*S; the in-place sync 2*N*S (padding excluded)
            sync[variant]["hbm_gbps_algorithmic"] = round(gbps(rs.hbm_bytes(variant), t), 1)
    rar.ddp_persistent_status()
    # the copying sync kernel by kernel: all packs, all fused all-reduces, all unpacks
    breakdown = {}
    for name, variant in (("pack", "pack"), ("allreduce_fused", "allreduce"), ("unpack_scale", "unpack")):
        fn = rs.fn(variant)
        fn()
        t = time_launches(fn, sync_reps, torch)
        breakdown[name] = {"ms": round(t, 4), "hbm_gbps_algorithmic": round(gbps(2 * wr_n * grad_bytes, t), 1)}
    sync["fused"]["breakdown"] = breakdown
    # The same syncs replayed from HIP graphs (every launch of the sync captured
    # once): no host work between launches; on this stack a replay is not
    # faster than the eager calls, which already keep the GPU busy.
    replayed = {}
    for variant in ("fused", "view"):
        g = graph_of(rs.fn(variant), torch)
        t = time_launches(g.replay, sync_reps, torch)
        replayed[variant] = {"ms": round(t, 4), "hbm_gbps_algorithmic": round(gbps(rs.hbm_bytes(variant), t), 1)}
        del g
    sync["graph_replay"] = replayed
    # the bf16 compression hook: fp32 gradients through bf16 buckets
    fn = rs.fn("bf16-fused")
    fn()
    t = time_launches(fn, sync_reps, torch)
    sync["bf16_compressed_fused"] = {"ms": round(t, 4),
                                     "bus_gbps_fp32_equivalent": round(gbps(2 * (wr_n - 1) / wr_n * grad_bytes, t), 1)}
    # the same hook in place: bf16 arithmetic on the fp32 gradients, no bf16 bucket (reads and writes 2*N*S)
    fn = rs.fn("bf16-view")
    fn()
    t = time_launches(fn, sync_reps, torch)
    sync["bf16_compressed_view"] = {"ms": round(t, 4),
                                    "bus_gbps_fp32_equivalent": round(gbps(2 * (wr_n - 1) / wr_n * grad_bytes, t), 1),
                                    "hbm_gbps_algorithmic": round(gbps(2 * wr_n * grad_bytes, t), 1)}
    # each sync started with the Infinity Cache flushed (a 512 MiB write outside the timed pair)
    flush = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
    cold = {}
    for variant in ("fused", "view"):
        _, med, lo = time_each(rs.fn(variant), 20, torch, between=flush.zero_)
        cold[variant] = {"ms_median": round(med, 4), "ms_min": round(lo, 4)}
    sync["after_cache_flush"] = cold
    del flush
    extras["ddp_sync_resnet50_n8"] = sync
    arenas, numels, inv_n = rs.arenas, rs.numels, rs.inv_n
    rs.free()
    del rs
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ overlap with a synthetic backward
    # Gradients are produced parameter by parameter in reverse order on one
    # stream (each element copied after `work` dependent FMAs); the reducer
    # syncs each bucket in place on another stream once its last gradient is
    # ready. Swept over bucket capacities, as the pages' tuning experiment.
    print("bench: overlap study", file=sys.stderr, flush=True)
    srcs = [a.clone() for a in arenas]
    compute, comm = torch.cuda.Stream(), torch.cuda.Stream()
    overlap = {"sync": "in place (view)", "params": len(numels), "caps": {}}
    for model, work, lds_kib in (("full_occupancy", 512, 0), ("two_waves_per_simd", 512, 64)):
        rows = {}
        for cap_name, cap, first_cap in (("per_gradient", 1, 1), ("6MiB", 6 << 20, 1 << 20),
                                         ("12MiB", 12 << 20, 1 << 20), ("25MiB", 25 << 20, 1 << 20),
                                         ("50MiB", 50 << 20, 1 << 20)):
            cplan = rar.ddp_bucket_plan(numels, "fp32", cap_bytes=cap, first_bucket_bytes=first_cap,
                                        world_size=wr_n)
            red = rar.Reducer(cplan, arenas, None, variant="view", scale=inv_n, comm_stream=comm)

            def backward(mode):
                rar.ddp_synthetic_backward_pass(cplan, srcs, arenas, work,
                                                red if mode == "overlapped" else None, lds_kib=lds_kib,
                                                stream=compute)
                if mode == "sequential":
                    rar.ddp_sync(cplan, arenas, None, variant="view", scale=inv_n, stream=compute)

            with torch.cuda.stream(compute):
                res = {}
                for mode in ("backward_only", "sequential", "overlapped"):
                    backward(mode)
                    res[mode] = time_launches(lambda: backward(mode), 3, torch)
            torch.cuda.synchronize()
            n_buckets = cplan.num_buckets
            red.free()
            cplan.free()
            rows[cap_name] = {"buckets": n_buckets,
                              "backward_only_ms": round(res["backward_only"], 4),
                              "sequential_ms": round(res["sequential"], 4),
                              "overlapped_ms": round(res["overlapped"], 4),
                              "exposed_comm_ms": round(res["overlapped"] - res["backward_only"], 4),
                              "overlap_gain": round(1 - res["overlapped"] / res["sequential"], 4)}
        overlap["caps"][model] = rows
        overlap["caps"][model]["backward_model"] = {"fma_per_element": work, "reserved_lds_kib_per_block": lds_kib}
    extras["overlap_resnet50_n8"] = overlap
    del arenas, srcs
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ CPU oracle, and the parity of the first launch
    print("bench: CPU oracle on the headline workload", file=sys.stderr, flush=True)
    from oracle import ring as oracle_ring
    t0 = time.perf_counter()
    want = oracle_ring.ring_simulate(host_inputs, "fp32")["bufs"]
    cpu_s = time.perf_counter() - t0
    del host_inputs
    mismatches = sum(int(np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32)))
                     for got, ref in zip(first_result, want))
    parity = {"elements": n * count, "mismatches": mismatches,
              "against": "the CPU oracle's hop-by-hop ring on the same inputs, every element of every rank",
              "launch": "the first fused launch, on the pristine inputs, outside the timed region"}
    del want, first_result
    cpu = {"value": round(gbps(2 * (n - 1) / n * S, cpu_s * 1e3), 4), "unit": "GB/s",
           "cores": 1, "kind": "oracle",
           "sample": (f"the whole workload (8 ranks x {count} fp32, the same bytes the GPU reduced), "
                      f"hop-by-hop numpy simulation with single-threaded ufuncs: {cpu_s:.2f} s"),
           "host_cpus_available": len(os.sched_getaffinity(0))}

    # every other workload's HBM rate also against the same run's copy probe
    add_copy_fraction(extras, extras["copy_probe"]["gbps"])

    line = {
        "metric": METRIC, "value": round(bus, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic (N(0, 1e-2) per rank, seeded on the GPU)",
        "config": {"workload": "ring_n8_1gib", "virtual_ranks": n, "elements_per_rank": count,
                   "bytes_per_rank": S, "variant": "fused", "in_place": True},
        "algbw_gbps": round(gbps(S, ms), 2), "busbw_gbps": round(bus, 2), "hbm_gbps": round(hbm, 1),
        "hbm_frac_of_peak": round(hbm / PEAK_HBM_GBPS, 4),
        "hbm_frac_of_copy_probe": round(hbm / extras["copy_probe"]["gbps"], 4),
        "ms_per_launch_median": round(ms_median, 4), "ms_per_launch_min": round(ms_min, 4),
        "ranks_equal_after": ranks_equal,
        "parity": parity,
        "roofline": {"bound": "hbm", "achieved": round(hbm, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(hbm / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": hbm_bytes},
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: the N ranks are virtual and share one GPU; --gpus {args.gpus} is not "
              "supported (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.config == "all":
        run_all(args)
    else:
        run_single(args)


if __name__ == "__main__":
    main()
