"""The C-ABI library on the CPU: it loads, exports every entry point the header
declares, its host planner agrees with the oracle's, and bad arguments are
refused before anything is launched (no GPU is touched by these calls)."""

import ctypes
import json
import os
import re

import numpy as np
import pytest

from conftest import ROOT

rar = pytest.importorskip("ring_all_reduce_ddp_amd")

from oracle import planner  # noqa: E402
from ddp_workloads import resnet50_param_numels  # noqa: E402

HEADER = os.path.join(ROOT, "include", "ddp_ring.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"if", "sizeof", "defined"})


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ["ddp_bucket_plan", "bucket_pack", "ring_allreduce_step", "ring_allreduce_fused",
                 "ring_allreduce_persistent", "bucket_unpack_scale", "ddp_last_error", "ddp_sync"]:
        assert want in names


def declaration_comments():
    """(function name, the header text between the previous declaration and
    this one) for every declared function: the comment that documents it."""
    text = open(HEADER).read()
    body = text[text.index('extern "C" {'):]
    out, prev = [], 0
    for m in re.finditer(r"^[a-z][^;{}()#]*?\b([a-z_][a-z0-9_]*)\s*\([^;]*\)\s*;", body, flags=re.M | re.S):
        out.append((m.group(1), body[prev:m.start()]))
        prev = m.end()
    return out


def test_every_declaration_cites_its_page():
    """Each entry point's comment names the page passage that defines what it
    computes: [R], [D] or [X] (the three pages listed at the top of the
    header) with a section or part. The one allocation-free variant names,
    instead, the callers it exists for: those that cannot allocate."""
    decls = declaration_comments()
    assert sorted(n for n, _ in decls) == declared_functions()
    cite = re.compile(r"\[(R|D|X)\]\s*(section|§|\"|parts?|reading)")
    flat = {n: re.sub(r"\n\s*\*\s?", " ", comment) for n, comment in decls}   # comment lines joined
    missing = [n for n in flat if not cite.search(flat[n]) and "callers that cannot allocate" not in flat[n]]
    assert [n for n in flat if "cannot allocate" in flat[n]] == ["ring_allreduce_persistent_noalloc"]
    assert missing == []


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(rar.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert missing == []


def test_only_one_hip_runtime_is_mapped():
    maps = open("/proc/self/maps").read()
    paths = set(re.findall(r"\S*libamdhip64\S*", maps))
    assert len(paths) == 1, paths


def as_tuples(buckets):
    return [{"members": [tuple(m) for m in b["members"]], "padded_numel": b["padded_numel"]}
            for b in buckets]


def test_planner_matches_oracle_on_golden_cases(golden_dir):
    with open(os.path.join(golden_dir, "planner_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        p = rar.ddp_bucket_plan(c["numels"], "fp32" if c["elem_bytes"] == 4 else "bf16",
                                c["cap_bytes"], c["first_bucket_bytes"], c["world_size"])
        assert p.buckets() == as_tuples(c["buckets"]), c["name"]


@pytest.mark.parametrize("seed", range(25))
def test_planner_matches_oracle_random(seed):
    rng = np.random.default_rng(1000 + seed)
    numels = [int(x) for x in rng.integers(0, 20000, size=rng.integers(0, 80))]
    dt = ["fp32", "bf16"][seed % 2]
    cap = int(rng.integers(16, 100000))
    first = int(rng.integers(16, 100000))
    n = int(rng.integers(1, 65))
    p = rar.ddp_bucket_plan(numels, dt, cap, first, n)
    want = planner.plan(numels, 4 if dt == "fp32" else 2, cap, first, n)
    assert p.buckets() == as_tuples(want)


def test_planner_resnet50_and_arena():
    numels = resnet50_param_numels()
    p = rar.ddp_bucket_plan(numels, "fp32", world_size=8)
    assert p.buckets() == as_tuples(planner.plan(numels, 4, world_size=8))
    n, offs = p.grad_arena()
    assert offs[0] == 0 and all(o % 4 == 0 for o in offs)
    assert all(offs[i + 1] - offs[i] == -(-numels[i] // 4) * 4 for i in range(len(numels) - 1))
    assert n == offs[-1] + numels[-1]


def expect_status(status, code, fragment):
    assert status == code
    assert fragment in rar.lib.ddp_last_error().decode()


def test_planner_argument_errors():
    lib = rar.lib
    out = ctypes.c_void_p()
    arr = (ctypes.c_int64 * 2)(4, -1)
    expect_status(lib.ddp_bucket_plan(arr, 2, 0, 1024, 1024, 1, ctypes.byref(out)), rar.DDP_EINVAL, "negative")
    arr = (ctypes.c_int64 * 1)(4)
    expect_status(lib.ddp_bucket_plan(arr, 1, 7, 1024, 1024, 1, ctypes.byref(out)), rar.DDP_EINVAL, "dtype")
    expect_status(lib.ddp_bucket_plan(arr, 1, 0, 0, 1024, 1, ctypes.byref(out)), rar.DDP_EINVAL, "capacities")
    expect_status(lib.ddp_bucket_plan(arr, 1, 0, 1024, 1024, 65, ctypes.byref(out)), rar.DDP_EINVAL, "world_size")
    expect_status(lib.ddp_bucket_plan(arr, 1, 0, 1024, 1024, 1, None), rar.DDP_EINVAL, "out")
    p = rar.ddp_bucket_plan([4, 8], "fp32")
    expect_status(lib.ddp_plan_bucket(p.handle, 5, None, None), rar.DDP_EINVAL, "out of range")
    expect_status(lib.ddp_plan_member(p.handle, 0, 9, None, None, None), rar.DDP_EINVAL, "out of range")


def test_zero_count_accepts_null_buffers():
    """count = 0 touches nothing, so NULL rank pointers (what torch reports
    for empty tensors) are accepted and every form returns DDP_OK without a
    launch; the pointer array itself must still exist."""
    lib = rar.lib
    nulls = (ctypes.c_void_p * 4)(None, None, None, None)
    for dt in (rar.DDP_FP32, rar.DDP_BF16):
        assert lib.ring_allreduce_fused(nulls, 4, 0, dt, None) == rar.DDP_OK
        assert lib.ring_allreduce_step(nulls, 4, 0, dt, 1, rar.DDP_AG, None) == rar.DDP_OK
        assert lib.ring_allreduce_persistent(nulls, 4, 0, dt, 6, None) == rar.DDP_OK
        assert lib.ring_reduce_scatter_fused(nulls, nulls, 4, 0, dt, 0.25, None) == rar.DDP_OK
    expect_status(lib.ring_allreduce_fused(None, 4, 0, rar.DDP_FP32, None), rar.DDP_EINVAL, "array is NULL")


def test_ring_argument_errors_before_launch():
    lib = rar.lib
    bufs = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    expect_status(lib.ring_allreduce_fused(bufs, 0, 10, rar.DDP_FP32, None), rar.DDP_EINVAL, "N must")
    expect_status(lib.ring_allreduce_fused(bufs, 65, 10, rar.DDP_FP32, None), rar.DDP_EINVAL, "N must")
    expect_status(lib.ring_allreduce_fused(bufs, 2, 10, 9, None), rar.DDP_EINVAL, "dtype")
    expect_status(lib.ring_allreduce_fused(bufs, 2, -1, rar.DDP_FP32, None), rar.DDP_EINVAL, "count")
    expect_status(lib.ring_allreduce_fused(None, 2, 10, rar.DDP_FP32, None), rar.DDP_EINVAL, "NULL")
    nulls = (ctypes.c_void_p * 2)(0x1000, None)
    expect_status(lib.ring_allreduce_fused(nulls, 2, 10, rar.DDP_FP32, None), rar.DDP_EINVAL, "bufs[1] is NULL")
    odd = (ctypes.c_void_p * 2)(0x1001, 0x2000)
    expect_status(lib.ring_allreduce_fused(odd, 2, 10, rar.DDP_FP32, None), rar.DDP_EINVAL, "aligned")
    expect_status(lib.ring_allreduce_step(bufs, 2, 10, rar.DDP_FP32, 1, rar.DDP_RS, None), rar.DDP_EINVAL, "step")
    expect_status(lib.ring_allreduce_step(bufs, 2, 10, rar.DDP_FP32, -1, rar.DDP_AG, None), rar.DDP_EINVAL, "step")
    expect_status(lib.ring_allreduce_step(bufs, 2, 10, rar.DDP_FP32, 0, 5, None), rar.DDP_EINVAL, "phase")
    expect_status(lib.ring_allreduce_persistent(bufs, 2, 10, rar.DDP_FP32, 3, None), rar.DDP_EINVAL, "n_steps")
    expect_status(lib.ddp_copy_probe(None, None, 15, None), rar.DDP_EINVAL, "multiple of 16")
    p = rar.ddp_bucket_plan([4, 8], "fp32", world_size=2)
    expect_status(lib.bucket_pack(p.handle, 0, bufs, bufs, 3, None), rar.DDP_EINVAL, "world size")
    expect_status(lib.bucket_pack(p.handle, 4, bufs, bufs, 2, None), rar.DDP_EINVAL, "out of range")
    expect_status(lib.ddp_sync(p.handle, bufs, bufs, 2, 9, 0.5, None), rar.DDP_EINVAL, "variant")
    # zero-length work is accepted without touching the device
    assert lib.ring_allreduce_fused(bufs, 2, 0, rar.DDP_FP32, None) == rar.DDP_OK


def test_missing_library_fails_loudly(monkeypatch):
    """Without the built library every entry point raises an ImportError that
    names the build command; nothing falls back to another implementation."""
    monkeypatch.setattr(rar, "LIB_PATH", "/nonexistent/libddp_ring.so")
    monkeypatch.setattr(rar, "_lib", None)
    with pytest.raises(ImportError, match="ring_all_reduce_ddp_amd.build"):
        rar.ddp_bucket_plan([4, 8], "fp32")
    with pytest.raises(ImportError):
        rar.lib


def test_view_sync_argument_errors():
    lib = rar.lib
    p = rar.ddp_bucket_plan([4, 8], "fp32", world_size=2)
    bufs = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    expect_status(lib.bucket_allreduce_view(p.handle, 3, bufs, 2, 0.5, None), rar.DDP_EINVAL, "out of range")
    expect_status(lib.bucket_allreduce_view(p.handle, 0, bufs, 4, 0.5, None), rar.DDP_EINVAL, "world size")
    expect_status(lib.bucket_allreduce_view(None, 0, bufs, 2, 0.5, None), rar.DDP_EINVAL, "plan is NULL")
    odd = (ctypes.c_void_p * 2)(0x1008, 0x2000)
    expect_status(lib.bucket_allreduce_view(p.handle, 0, odd, 2, 0.5, None), rar.DDP_EINVAL, "aligned")
    # the view variant of ddp_sync needs no bucket buffers
    expect_status(lib.ddp_sync(p.handle, odd, None, 2, 3, 0.5, None), rar.DDP_EINVAL, "aligned")
    expect_status(lib.ddp_sync(p.handle, bufs, None, 2, 0, 0.5, None), rar.DDP_EINVAL, "NULL")


def test_reduce_scatter_argument_errors():
    lib = rar.lib
    bufs = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    shards = (ctypes.c_void_p * 2)(0x3000, 0x4000)
    expect_status(lib.ring_reduce_scatter_fused(bufs, None, 2, 0, rar.DDP_FP32, 1.0, None), rar.DDP_EINVAL, "shards")
    expect_status(lib.ring_reduce_scatter_fused(bufs, shards, 0, 10, rar.DDP_FP32, 1.0, None), rar.DDP_EINVAL, "N must")
    odd = (ctypes.c_void_p * 2)(0x3001, 0x4000)
    # empty buffers: nothing to check or launch
    assert lib.ring_reduce_scatter_fused(bufs, odd, 2, 0, rar.DDP_FP32, 1.0, None) == rar.DDP_OK


@pytest.mark.parametrize("seed", range(10))
def test_compressed_plan_matches_oracle(seed):
    """fp32 gradients in bf16 buckets: capacities count fp32 bytes, members and
    padding use bf16 vectors (8 elements)."""
    rng = np.random.default_rng(2000 + seed)
    numels = [int(x) for x in rng.integers(0, 20000, size=rng.integers(1, 60))]
    cap = int(rng.integers(16, 100000))
    first = int(rng.integers(16, 100000))
    n = int(rng.integers(1, 65))
    p = rar.ddp_bucket_plan_ex(numels, "fp32", "bf16", cap, first, n)
    want = planner.plan(numels, 4, cap, first, n, vector_elems=8)
    assert p.buckets() == as_tuples(want)
    arena_numel, offs = p.grad_arena()
    assert all(o % 4 == 0 for o in offs)


def test_compressed_plan_errors():
    lib = rar.lib
    out = ctypes.c_void_p()
    arr = (ctypes.c_int64 * 1)(4)
    expect_status(lib.ddp_bucket_plan_ex(arr, 1, rar.DDP_BF16, rar.DDP_FP32, 1024, 1024, 1, ctypes.byref(out)),
                  rar.DDP_EINVAL, "mixed pair")
    p = rar.ddp_bucket_plan_ex([4, 8], "fp32", "bf16", world_size=2)
    bufs = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    # the in-place sync accepts the compressed plan and checks its fp32 arenas
    expect_status(lib.bucket_allreduce_view(p.handle, 0, bufs, 2, 0.5, None), rar.DDP_EINVAL, "device allocation")


def test_reducer_argument_errors():
    lib = rar.lib
    out = ctypes.c_void_p()
    bufs = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    p = rar.ddp_bucket_plan([4, 8], "fp32", world_size=2)
    expect_status(lib.ddp_reducer_create(None, bufs, None, 2, 3, 0.5, 0, None, ctypes.byref(out)), rar.DDP_EINVAL, "plan")
    expect_status(lib.ddp_reducer_create(p.handle, bufs, None, 3, 3, 0.5, 0, None, ctypes.byref(out)), rar.DDP_EINVAL, "world size")
    expect_status(lib.ddp_reducer_create(p.handle, bufs, None, 2, 0, 0.5, 0, None, ctypes.byref(out)), rar.DDP_EINVAL, "bucket_bufs")
    expect_status(lib.ddp_reducer_create(p.handle, bufs, None, 2, 7, 0.5, 0, None, ctypes.byref(out)), rar.DDP_EINVAL, "variant")
    expect_status(lib.ddp_reducer_create(p.handle, bufs, bufs, 2, 0, 0.5, 64, None, ctypes.byref(out)),
                  rar.DDP_EINVAL, "in-place variant only")
    expect_status(lib.ddp_reducer_create(p.handle, bufs, None, 2, 3, 0.5, -1, None, ctypes.byref(out)),
                  rar.DDP_EINVAL, "comm_max_blocks < 0")
    expect_status(lib.ddp_reducer_mark_ready(None, 0, None), rar.DDP_EINVAL, "NULL")
    expect_status(lib.ddp_synthetic_backward(bufs, bufs, 2, 10, rar.DDP_FP32, -1, 0, None), rar.DDP_EINVAL, "work")
    expect_status(lib.ddp_synthetic_backward(bufs, bufs, 2, 10, rar.DDP_FP32, 1, 65, None), rar.DDP_EINVAL, "lds_kib")


def expected_arena_map(numels, elem_bytes, cap, first, n, bucket_vector_elems=None):
    """The in-place sync's per-vector map, derived from the oracle's plan and
    an arena laid out in registration order on V-element boundaries.
    bucket_vector_elems = 8 with fp32 gradients: the plan of bf16 buckets."""
    v = 16 // elem_bytes
    offs = np.concatenate([[0], np.cumsum([-(-m // v) * v for m in numels])]).astype(np.int64)
    out = np.full(int(offs[-1]) // v, 0xFFFF, dtype=np.uint16)
    for b in planner.plan(numels, elem_bytes, cap, first, n, vector_elems=bucket_vector_elems):
        L = b["padded_numel"] // n
        for p, off, m in b["members"]:
            for e in range(0, m, v):
                out[(offs[p] + e) // v] = ((off + e) // L) | (min(v, m - e) << 8)
    return out


@pytest.mark.parametrize("seed", range(12))
def test_arena_map_matches_oracle_plan(seed):
    """The map the in-place kernels read (chunk and member elements of every
    arena vector) follows from the oracle's bucket plan."""
    rng = np.random.default_rng(2000 + seed)
    numels = [int(x) for x in rng.integers(0, 3000, size=rng.integers(1, 40))]
    dt = ["fp32", "bf16"][seed % 2]
    eb = 4 if dt == "fp32" else 2
    cap = int(rng.integers(64, 20000))
    first = int(rng.integers(64, 20000))
    n = [1, 2, 3, 8, 13, 64][seed % 6]
    p = rar.ddp_bucket_plan(numels, dt, cap, first, n)
    assert np.array_equal(p.arena_map(), expected_arena_map(numels, eb, cap, first, n))


@pytest.mark.parametrize("seed", range(6))
def test_compressed_arena_map_matches_oracle_plan(seed):
    """fp32 gradients in bf16 buckets: one map entry per 4-element fp32 arena
    vector, its chunk taken from the bf16 buckets' layout (8-element vectors),
    so no arena vector straddles a chunk boundary."""
    rng = np.random.default_rng(3000 + seed)
    numels = [int(x) for x in rng.integers(0, 3000, size=rng.integers(1, 40))]
    cap = int(rng.integers(64, 20000))
    first = int(rng.integers(64, 20000))
    n = [1, 2, 3, 8, 13, 64][seed]
    p = rar.ddp_bucket_plan_ex(numels, "fp32", "bf16", cap, first, n)
    assert np.array_equal(p.arena_map(), expected_arena_map(numels, 4, cap, first, n, bucket_vector_elems=8))


def test_arena_map_resnet50():
    numels = resnet50_param_numels()
    p = rar.ddp_bucket_plan(numels, "fp32", world_size=8)
    got = p.arena_map()
    assert np.array_equal(got, expected_arena_map(numels, 4, 25 << 20, 1 << 20, 8))
    assert (got != 0xFFFF).sum() == sum(-(-m // 4) for m in numels)


def test_arena_map_errors():
    lib = rar.lib
    p = rar.ddp_bucket_plan([4, 8], "fp32", world_size=2)
    out = (ctypes.c_uint16 * 4)()
    assert lib.ddp_plan_arena_map(p.handle, out, 3) == rar.DDP_OK   # 4 + 8 fp32 elements: 3 vectors
    expect_status(lib.ddp_plan_arena_map(p.handle, out, 2), rar.DDP_EINVAL, "vector count")
    pc = rar.ddp_bucket_plan_ex([4, 8], "fp32", "bf16", world_size=2)
    assert lib.ddp_plan_arena_map(pc.handle, out, 3) == rar.DDP_OK   # the compressed plan's fp32 arena
    expect_status(lib.ddp_plan_arena_map(pc.handle, out, 4), rar.DDP_EINVAL, "vector count")


def test_device_alloc_argument_errors():
    """ddp_device_alloc refuses a non-positive size, an unknown flag and a
    NULL out before calling the HIP runtime; freeing NULL is a no-op."""
    import ctypes
    lib = rar.lib
    out = ctypes.c_void_p(1234)
    for nbytes, flags, msg in ((0, 0, "nbytes must be positive"), (-16, 1, "nbytes must be positive"),
                               (64, 2, "flags must be 0 or DDP_ALLOC_CONTIGUOUS")):
        assert lib.ddp_device_alloc(nbytes, flags, ctypes.byref(out)) == rar.DDP_EINVAL
        assert msg in lib.ddp_last_error().decode()
        assert out.value is None
    assert lib.ddp_device_alloc(64, 0, None) == rar.DDP_EINVAL
    assert lib.ddp_device_free(None) == rar.DDP_OK
