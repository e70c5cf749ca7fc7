"""GPU parity of the bucket pack / unpack-with-scale kernels and of the whole
DDP sync (ResNet-50 gradients, N=8) against the CPU oracle, bit for bit."""

import numpy as np
import pytest
import torch

import ring_all_reduce_ddp_amd as rar
from oracle import ddp, planner, ring
from ddp_workloads import WORKLOADS, host_grads, resnet50_param_numels

from gpu_util import TORCH_DTYPE, to_host, assert_bit_equal, mean_scale

pytestmark = pytest.mark.gpu


def make_arenas(plan, grads, dtype):
    """One device arena per rank holding the rank's gradients at the plan's offsets."""
    arena_numel, offs = plan.grad_arena()
    arenas = []
    for g in grads:
        a = np.zeros(arena_numel, np.float32)
        for p, x in enumerate(g):
            a[offs[p]:offs[p] + len(x)] = x
        t = torch.from_numpy(a).cuda()
        arenas.append(t.to(TORCH_DTYPE[dtype]) if dtype == "bf16" else t)
    return arenas, offs


def read_grads(arenas, offs, numels, dtype):
    out = []
    for a in arenas:
        h = to_host(a, dtype)
        out.append([h[offs[p]:offs[p] + m] for p, m in enumerate(numels)])
    return out


def bucket_buffers(plan, n, dtype, fill=float("nan")):
    bufs = []
    for b in range(plan.num_buckets):
        padded, _ = plan.bucket(b)
        bufs.append([torch.full((padded,), fill, dtype=TORCH_DTYPE[dtype], device="cuda") for _ in range(n)])
    return bufs


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_pack_then_unpack_is_identity(dtype):
    numels = [7, 16, 1, 40, 3, 300, 9, 0, 5000, 33]
    n = 3
    plan = rar.ddp_bucket_plan(numels, dtype, cap_bytes=4096, first_bucket_bytes=64, world_size=n)
    grads = host_grads(21, n, numels)
    if dtype == "bf16":
        from ddp_workloads.gen import to_bf16_bits
        grads = [[to_bf16_bits(x) for x in g] for g in grads]
        grads_f32 = [[(x.astype(np.uint32) << 16).view(np.float32) for x in g] for g in grads]
    else:
        grads_f32 = grads
    arenas, offs = make_arenas(plan, grads_f32, dtype)
    buckets = bucket_buffers(plan, n, dtype)
    oplan = planner.plan(numels, 4 if dtype == "fp32" else 2, 4096, 64, n)
    for b in range(plan.num_buckets):
        rar.bucket_pack(plan, b, arenas, buckets[b])
    torch.cuda.synchronize()
    for b in range(plan.num_buckets):
        for r in range(n):
            assert_bit_equal(to_host(buckets[b][r], dtype), ddp.pack(grads[r], oplan[b], dtype), f"pack b{b} r{r}")
    out = [torch.zeros_like(a) for a in arenas]
    for b in range(plan.num_buckets):
        rar.bucket_unpack_scale(plan, b, buckets[b], out, 1.0)
    torch.cuda.synchronize()
    back = read_grads(out, offs, numels, dtype)
    for r in range(n):
        for p in range(len(numels)):
            assert_bit_equal(back[r][p], grads[r][p], f"unpack r{r} p{p}")


@pytest.mark.parametrize("scale", [0.125, 1.0 / 3.0])
def test_unpack_scale_rounding(scale):
    numels = [1000, 4097]
    n = 2
    plan = rar.ddp_bucket_plan(numels, "fp32", world_size=n)
    grads = host_grads(22, n, numels, std=1.0)
    arenas, offs = make_arenas(plan, grads, "fp32")
    buckets = bucket_buffers(plan, n, "fp32")
    oplan = planner.plan(numels, 4, world_size=n)
    out = [torch.zeros_like(a) for a in arenas]
    for b in range(plan.num_buckets):
        rar.bucket_pack(plan, b, arenas, buckets[b])
        rar.bucket_unpack_scale(plan, b, buckets[b], out, scale)
    torch.cuda.synchronize()
    back = read_grads(out, offs, numels, "fp32")
    for b, bk in enumerate(oplan):
        for r in range(n):
            want = ddp.unpack_scale(ddp.pack(grads[r], bk, "fp32"), bk, np.float32(scale), "fp32")
            for p, w in want.items():
                assert_bit_equal(back[r][p], w, f"scale {scale} r{r} p{p}")


def oracle_sync(grads, numels, n, dtype="fp32"):
    oplan = planner.plan(numels, 4, world_size=n)
    return ddp.ddp_sync(grads, oplan, dtype)


ALL_VARIANTS = ["fused", "steps", "persistent", "view"]


def sync_case(variant, n, dtype, numels, cap, first, seed, scale=None, comm=None):
    """One sync on seeded gradients against the oracle's; comm="bf16" with
    fp32 gradients goes through bf16 buckets (the compression hook)."""
    if comm is None:
        plan = rar.ddp_bucket_plan(numels, dtype, cap_bytes=cap, first_bucket_bytes=first, world_size=n)
    else:
        plan = rar.ddp_bucket_plan_ex(numels, dtype, comm, cap, first, n)
    grads = host_grads(seed, n, numels)
    if dtype == "bf16":
        from ddp_workloads.gen import to_bf16_bits
        grads = [[to_bf16_bits(x) for x in g] for g in grads]
        grads_f32 = [[(x.astype(np.uint32) << 16).view(np.float32) for x in g] for g in grads]
    else:
        grads_f32 = grads
    arenas, offs = make_arenas(plan, grads_f32, dtype)
    buckets = None if variant == "view" else bucket_buffers(plan, n, comm or dtype)
    if scale is None:
        scale = mean_scale(n)
    rar.ddp_sync(plan, arenas, buckets, variant=variant, scale=scale)
    torch.cuda.synchronize()
    if variant == "persistent":
        rar.ddp_persistent_status()
    got = read_grads(arenas, offs, numels, dtype)
    if comm is None:
        oplan = planner.plan(numels, 4 if dtype == "fp32" else 2, cap, first, n)
    else:
        oplan = planner.plan(numels, 4, cap, first, n, vector_elems=8)
    want = ddp.ddp_sync(grads, oplan, dtype, scale=scale, comm_dtype=comm)
    for r in range(n):
        for p in range(len(numels)):
            assert_bit_equal(got[r][p], want[r][p], f"{variant} n={n} {dtype} rank {r} param {p}")


@pytest.mark.parametrize("variant", ALL_VARIANTS)
def test_small_sync_against_oracle(variant):
    numels = [7, 16, 1, 40, 3, 300, 9, 0, 5000, 33, 12345, 2]
    sync_case(variant, 4, "fp32", numels, 8192, 256, seed=23)


@pytest.mark.parametrize("variant", ALL_VARIANTS)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n", [1, 2, 3, 8, 9, 16])
def test_sync_ranks_and_dtypes(variant, dtype, n):
    """Members that straddle ring-chunk boundaries, one-element and empty
    parameters, several buckets; scale = fl(1/N)."""
    numels = [1, 3000, 17, 0, 65, 40000, 2, 129, 7777, 5]
    sync_case(variant, n, dtype, numels, 64 * 1024, 512, seed=40 + n)


@pytest.fixture(scope="module")
def resnet50_case():
    w = WORKLOADS["ddp_resnet50"]
    numels = resnet50_param_numels()
    grads = host_grads(w.seed, w.n, numels, std=w.std)
    want = oracle_sync(grads, numels, w.n)
    return w, numels, grads, want


@pytest.mark.parametrize("variant", ALL_VARIANTS)
def test_resnet50_sync(resnet50_case, variant):
    """The full sync of ResNet-50 gradients over 8 ranks: reverse-order buckets
    (1 MiB first, 25 MiB cap), pack, all-reduce, x1/8, unpack."""
    w, numels, grads, want = resnet50_case
    plan = rar.ddp_bucket_plan(numels, "fp32", world_size=w.n)
    assert plan.num_buckets == 6
    arenas, offs = make_arenas(plan, grads, "fp32")
    buckets = None if variant == "view" else bucket_buffers(plan, w.n, "fp32")
    rar.ddp_sync(plan, arenas, buckets, variant=variant, scale=0.125)
    torch.cuda.synchronize()
    got = read_grads(arenas, offs, numels, "fp32")
    for r in range(w.n):
        for p in range(len(numels)):
            assert_bit_equal(got[r][p], want[r][p], f"{variant} rank {r} param {p}")


@pytest.mark.parametrize("variant", ALL_VARIANTS)
@pytest.mark.parametrize("n", [1, 2, 3, 8, 13, 16, 64])
def test_bf16_compressed_sync(variant, n):
    """fp32 gradients synced through bf16 buckets (the bf16 compression hook),
    or through bf16 arithmetic on the gradients in place (view), equal the
    oracle's compressed sync bit for bit."""
    numels = [1, 3000, 17, 0, 65, 40000, 2, 129, 7777, 5]
    cap, first = 64 * 1024, 512
    plan = rar.ddp_bucket_plan_ex(numels, "fp32", "bf16", cap, first, n)
    grads = host_grads(60 + n, n, numels)
    arenas, offs = make_arenas(plan, grads, "fp32")
    buckets = None if variant == "view" else bucket_buffers(plan, n, "bf16")
    rar.ddp_sync(plan, arenas, buckets, variant=variant, scale=mean_scale(n))
    torch.cuda.synchronize()
    if variant == "persistent":
        rar.ddp_persistent_status()
    got = read_grads(arenas, offs, numels, "fp32")
    oplan = planner.plan(numels, 4, cap, first, n, vector_elems=8)
    want = ddp.ddp_sync(grads, oplan, "fp32", comm_dtype="bf16")
    for r in range(n):
        for p in range(len(numels)):
            assert_bit_equal(got[r][p], want[r][p], f"{variant} n={n} rank {r} param {p}")


@pytest.mark.parametrize("variant", ["fused", "view"])
def test_bf16_compressed_resnet50(variant):
    w = WORKLOADS["ddp_resnet50"]
    numels = resnet50_param_numels()
    grads = host_grads(w.seed, w.n, numels, std=w.std)
    plan = rar.ddp_bucket_plan_ex(numels, "fp32", "bf16", world_size=w.n)
    arenas, offs = make_arenas(plan, grads, "fp32")
    buckets = None if variant == "view" else bucket_buffers(plan, w.n, "bf16")
    rar.ddp_sync(plan, arenas, buckets, variant=variant, scale=0.125)
    torch.cuda.synchronize()
    got = read_grads(arenas, offs, numels, "fp32")
    want = ddp.ddp_sync(grads, planner.plan(numels, 4, world_size=w.n, vector_elems=8), "fp32",
                        scale=0.125, comm_dtype="bf16")
    for r in range(w.n):
        for p in range(len(numels)):
            assert_bit_equal(got[r][p], want[r][p], f"rank {r} param {p}")


@pytest.mark.parametrize("n", [3, 8])
def test_view_compressed_special_values(n):
    """The in-place compressed sync on values whose bf16 rounding matters:
    halfway cases, values that overflow bf16, subnormals and signed zeros,
    against the oracle's compressed sync."""
    rng = np.random.default_rng(90 + n)
    # One sign of the near-maximal value only: sums may overflow to +inf, never meet -inf (inf - inf would
    # give a NaN whose bits differ between processors).
    special = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, -(1.0 + 2.0 ** -8), 3.3895e38,
                        1e-40, -1e-40, 2.0 ** -133, 0.0, -0.0, 65504.0, 1.0 - 2.0 ** -9], dtype=np.float32)
    numels = [37, 1000, 5]
    plan = rar.ddp_bucket_plan_ex(numels, "fp32", "bf16", 4096, 256, n)
    grads = [[rng.choice(special, size=m).astype(np.float32) for m in numels] for _ in range(n)]
    arenas, offs = make_arenas(plan, grads, "fp32")
    rar.ddp_sync(plan, arenas, None, variant="view", scale=mean_scale(n))
    torch.cuda.synchronize()
    got = read_grads(arenas, offs, numels, "fp32")
    want = ddp.ddp_sync(grads, planner.plan(numels, 4, 4096, 256, n, vector_elems=8), "fp32", comm_dtype="bf16")
    for r in range(n):
        for p in range(len(numels)):
            assert_bit_equal(got[r][p], want[r][p], f"rank {r} param {p}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n", [4, 5, 7, 13, 64])
def test_view_sync_more_ranks(dtype, n):
    """The in-place sync at rank counts handled by each kernel form (one wave
    per rank, and eight waves cycling over the ranks above eight, up to 64)."""
    numels = [1, 3000, 17, 0, 65, 40000, 2, 129, 7777, 5]
    sync_case("view", n, dtype, numels, 64 * 1024, 512, seed=140 + n)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_view_sync_leaves_slack_alone(dtype):
    """The in-place sync writes the members' elements only: the arena's
    alignment slack after each member keeps its bits."""
    n = 3
    numels = [5, 1, 30, 7, 1001, 3]
    plan = rar.ddp_bucket_plan(numels, dtype, cap_bytes=256, first_bucket_bytes=64, world_size=n)
    grads = host_grads(44, n, numels)
    arenas, offs = make_arenas(plan, grads, dtype)
    arena_numel = arenas[0].numel()
    slack = np.ones(arena_numel, bool)
    for p, m in enumerate(numels):
        slack[offs[p]:offs[p] + m] = False
    assert slack.any()
    idx = torch.from_numpy(np.nonzero(slack)[0]).cuda()
    for a in arenas:
        a.index_fill_(0, idx, 12345.0)
    before = [to_host(a, dtype)[slack] for a in arenas]
    rar.ddp_sync(plan, arenas, None, variant="view", scale=mean_scale(n))
    torch.cuda.synchronize()
    for r, a in enumerate(arenas):
        assert_bit_equal(to_host(a, dtype)[slack], before[r], f"slack of rank {r}")


def test_bf16_compression_rounding_on_bit_patterns():
    """Packing fp32 gradients into bf16 buckets rounds exactly as the oracle
    does, on 2^22 random fp32 bit patterns (every exponent, subnormals, NaNs,
    infinities) plus hand-picked halfway, overflow and subnormal cases. NaNs
    are compared by position only: the oracle's NaN is canonical, the
    kernel keeps the payload's upper bits with the quiet bit set."""
    edge = np.array([0x00000000, 0x80000000, 0x00000001, 0x00008000, 0x00018000, 0x007fffff,
                     0x00807fff, 0x00808000, 0x00818000, 0x3f808000, 0x3f818000, 0x3f807fff,
                     0x7f7f7fff, 0x7f7f8000, 0x7f7fffff, 0xff7fffff, 0x7f800000, 0xff800000,
                     0x7fc00000, 0x7f800001, 0xffc12345, 0x7fffffff], dtype=np.uint32)
    rng = np.random.default_rng(2024)
    pats = np.concatenate([edge, rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)])
    g = pats.view(np.float32)
    numels = [len(g)]
    plan = rar.ddp_bucket_plan_ex(numels, "fp32", "bf16", world_size=1)
    arenas, offs = make_arenas(plan, [[g]], "fp32")
    padded, _ = plan.bucket(0)
    bucket = [torch.empty(padded, dtype=torch.bfloat16, device="cuda")]
    rar.bucket_pack(plan, 0, arenas, bucket)
    torch.cuda.synchronize()
    got = to_host(bucket[0], "bf16")[:len(g)]
    oplan = planner.plan(numels, 4, world_size=1, vector_elems=8)
    with np.errstate(invalid="ignore", over="ignore"):
        want = ddp.pack([g], oplan[0], "bf16", "fp32")[:len(g)]
    got_nan = (got & 0x7fff) > 0x7f80
    want_nan = (want & 0x7fff) > 0x7f80
    assert np.array_equal(got_nan, want_nan)
    assert np.array_equal(got[~got_nan], want[~want_nan])
    assert got_nan.sum() > 1000   # the sample does hold NaNs


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n", [3, 8, 13])
@pytest.mark.parametrize("order", ["plan", "reversed"])
def test_view_bucket_by_bucket(dtype, n, order):
    """bucket_allreduce_view on one bucket at a time (as the reducer runs it)
    gives the oracle's sync; buckets are disjoint, so their order does not
    matter."""
    numels = [1, 3000, 17, 0, 65, 40000, 2, 129, 7777, 5]
    cap, first = 64 * 1024, 512
    plan = rar.ddp_bucket_plan(numels, dtype, cap_bytes=cap, first_bucket_bytes=first, world_size=n)
    grads = host_grads(170 + n, n, numels)
    if dtype == "bf16":
        from ddp_workloads.gen import to_bf16_bits
        grads = [[to_bf16_bits(x) for x in g] for g in grads]
        grads_f32 = [[(x.astype(np.uint32) << 16).view(np.float32) for x in g] for g in grads]
    else:
        grads_f32 = grads
    arenas, offs = make_arenas(plan, grads_f32, dtype)
    scale = float(np.float32(1) / np.float32(n))
    buckets = list(range(plan.num_buckets))
    if order == "reversed":
        buckets.reverse()
    for b in buckets:
        rar.bucket_allreduce_view(plan, b, arenas, scale)
    torch.cuda.synchronize()
    got = read_grads(arenas, offs, numels, dtype)
    want = ddp.ddp_sync(grads, planner.plan(numels, 4 if dtype == "fp32" else 2, cap, first, n), dtype)
    for r in range(n):
        for p in range(len(numels)):
            assert_bit_equal(got[r][p], want[r][p], f"n={n} {dtype} rank {r} param {p}")


def bucket_space_samples(oplan, offs, n, k, seed):
    """Arena positions to check, drawn in bucket space: the first two and last
    two offsets of every ring chunk of every bucket plus k random offsets, kept
    where they fall inside a member. Returns (arena indices, chunk ids)."""
    rng = np.random.default_rng(seed)
    idx, chunk = [], []
    for bk in oplan:
        padded = bk["padded_numel"]
        L = padded // n
        cand = [rng.integers(0, padded, size=k // len(oplan) + 1)]
        for c in range(n):
            cand.append(np.array([c * L, c * L + 1, (c + 1) * L - 2, (c + 1) * L - 1]))
        cand = np.unique(np.concatenate(cand))
        for p, off, numel in bk["members"]:
            inside = cand[(cand >= off) & (cand < off + numel)]
            idx.append(offs[p] + inside - off)
            chunk.append(inside // L)
    return np.concatenate(idx).astype(np.int64), np.concatenate(chunk).astype(np.int64)


@pytest.mark.parametrize("variant", ALL_VARIANTS)
def test_bf16_resnet50_sampled(variant):
    """bf16 gradients of ResNet-50 over 8 ranks (409 MB of arenas, beyond the
    Infinity Cache, so pack and unpack stream): sampled positions against the
    oracle's ring on those positions, in their chunks' order, then its
    unpack_scale; all ranks equal everywhere."""
    w = WORKLOADS["ddp_resnet50"]
    n = w.n
    numels = resnet50_param_numels()
    plan = rar.ddp_bucket_plan(numels, "bf16", world_size=n)
    arena_numel, offs = plan.grad_arena()
    oplan = planner.plan(numels, 2, world_size=n)
    mask = torch.zeros(arena_numel, dtype=torch.bool, device="cuda")
    for p, m in enumerate(numels):
        mask[offs[p]:offs[p] + m] = True
    g = torch.Generator(device="cuda")
    arenas = []
    for r in range(n):
        g.manual_seed(1000 * w.seed + 500 + r)
        a = (torch.randn(arena_numel, generator=g, device="cuda") * w.std).to(torch.bfloat16)
        arenas.append(torch.where(mask, a, torch.zeros_like(a)))  # slack is zero, as a fresh arena's
    pos, chunk = bucket_space_samples(oplan, offs, n, 20000, seed=7)
    pos_dev = torch.from_numpy(pos).cuda()
    before = [to_host(a.index_select(0, pos_dev), "bf16") for a in arenas]
    print(f"[resnet50 bf16 {variant}] arena={arena_numel} samples={len(pos)}", flush=True)
    buckets = None if variant == "view" else bucket_buffers(plan, n, "bf16")
    rar.ddp_sync(plan, arenas, buckets, variant=variant, scale=mean_scale(n))
    torch.cuda.synchronize()
    if variant == "persistent":
        rar.ddp_persistent_status()
    after = [to_host(a.index_select(0, pos_dev), "bf16") for a in arenas]
    mism = torch.zeros(1, dtype=torch.int64, device="cuda")
    rar.ddp_count_mismatches(arenas, mism)
    torch.cuda.synchronize()
    assert int(mism.item()) == 0, "ranks differ after the sync"
    reduced = ring.ring_simulate(before, "bf16", chunk_of=chunk)["bufs"][0]
    flat = {"members": [(0, 0, len(pos))], "padded_numel": len(pos)}
    want = ddp.unpack_scale(reduced, flat, np.float32(1) / np.float32(n), "bf16")[0]
    for r in range(n):
        assert_bit_equal(after[r], want, f"{variant} rank {r}")


@pytest.mark.parametrize("path", ["ddp_sync", "reducer"])
def test_persistent_timeout_leaves_gradients(path):
    """A persistent all-reduce that gives up at a grid barrier (forced from the
    host: every barrier expects one block more than the grid has, 20 ms
    deadline) is not copied back: every gradient keeps its bits, the status
    call reports the time-out, and a normal sync afterwards equals the
    oracle's."""
    numels = [7, 16, 1, 40, 3, 300, 9, 5000, 33]
    n = 4
    plan = rar.ddp_bucket_plan(numels, "fp32", cap_bytes=4096, first_bucket_bytes=64, world_size=n)
    assert plan.num_buckets > 1
    grads = host_grads(91, n, numels)
    arenas, offs = make_arenas(plan, grads, "fp32")
    buckets = bucket_buffers(plan, n, "fp32")
    before = [to_host(a, "fp32") for a in arenas]
    print(f"[persistent time-out via {path}] buckets={plan.num_buckets}", flush=True)
    rar.ddp_persistent_test_hook(extra_arrivals=1, timeout_us=20_000)
    try:
        if path == "ddp_sync":
            rar.ddp_sync(plan, arenas, buckets, variant="persistent", scale=mean_scale(n))
        else:
            red = rar.Reducer(plan, arenas, buckets, variant="persistent", scale=mean_scale(n),
                              comm_stream=torch.cuda.Stream())
            for p in reversed(range(len(numels))):
                red.mark_ready(p)
            red.finalize()
        torch.cuda.synchronize()
    finally:
        rar.ddp_persistent_test_hook(0, 0)
    with pytest.raises(rar.DDPError, match="timed out"):
        rar.ddp_persistent_status()
    for r in range(n):
        assert_bit_equal(to_host(arenas[r], "fp32"), before[r], f"{path}: rank {r} after the time-out")
    rar.ddp_sync(plan, arenas, buckets, variant="persistent", scale=mean_scale(n))
    torch.cuda.synchronize()
    rar.ddp_persistent_status()
    want = ddp.ddp_sync(grads, planner.plan(numels, 4, 4096, 64, n), "fp32")
    got = read_grads(arenas, offs, numels, "fp32")
    for r in range(n):
        for p in range(len(numels)):
            assert_bit_equal(got[r][p], want[r][p], f"{path}: after recovery, rank {r} param {p}")
