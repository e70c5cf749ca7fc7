"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer.

csrc/plan.cpp is compiled by g++ for the CPU with -fsanitize=address,undefined
(no GPU code is involved) into a small driver (tests/sanitize/plan_driver.cpp)
that builds plans through the C ABI, reads them back through every accessor,
frees them, and exercises every accessor's error path. The plans it reports
must equal the oracle's (golden cases, random shape lists in both dtypes,
compressed plans, ResNet-50), the arena maps those derived from the oracle's
plan, and the run must end with no sanitizer report and no leak.
"""

import json
import os
import shutil
import subprocess

import numpy as np
import pytest

from conftest import ROOT
from oracle import planner
from ddp_workloads import resnet50_param_numels

from test_abi_cpu import as_tuples, expected_arena_map

CSRC = os.path.join(ROOT, "ring_all_reduce_ddp_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp")
FP32, BF16 = 0, 1


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ is not installed")
    out = str(tmp_path_factory.mktemp("asan") / "plan_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "plan.cpp"), DRIVER, "-o", out]
    subprocess.run(cmd, check=True)
    return out


def run_driver(driver, cases, tmp_path):
    """cases: (grad_dtype, comm_dtype, cap, first, n, numels, want_map).
    Returns the driver's per-case JSON objects and the arena maps."""
    lines, maps = [], []
    for i, (gdt, cdt, cap, first, n, numels, want_map) in enumerate(cases):
        path = str(tmp_path / f"map{i}.bin") if want_map else "-"
        maps.append(path)
        lines.append(" ".join(map(str, ["case", gdt, cdt, cap, first, n, path, len(numels), *numels])))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    proc = subprocess.run([driver], input="\n".join(lines) + "\n", stdout=subprocess.PIPE,
                          stderr=subprocess.PIPE, text=True, env=env, timeout=600)
    assert proc.returncode == 0, proc.stderr[-4000:]
    assert "runtime error" not in proc.stderr and "Sanitizer" not in proc.stderr, proc.stderr[-4000:]
    out = proc.stdout.splitlines()
    assert out[-1] == "errors ok", proc.stderr[-2000:]
    results = [json.loads(x) for x in out[:-1]]
    assert len(results) == len(cases)
    got_maps = [np.fromfile(p, dtype=np.uint16) if p != "-" else None for p in maps]
    return results, got_maps


def golden_cases(golden_dir):
    with open(os.path.join(golden_dir, "planner_cases.json")) as f:
        return json.load(f)["cases"]


def test_planner_under_sanitizers(driver, golden_dir, tmp_path):
    cases, want = [], []
    for c in golden_cases(golden_dir):
        dt = FP32 if c["elem_bytes"] == 4 else BF16
        cases.append((dt, dt, c["cap_bytes"], c["first_bucket_bytes"], c["world_size"], c["numels"], False))
        want.append((as_tuples(c["buckets"]), None))
    rng = np.random.default_rng(4000)
    for k in range(40):
        numels = [int(x) for x in rng.integers(0, 20000, size=rng.integers(0, 80))]
        dt = k % 2
        eb = 4 if dt == FP32 else 2
        cap, first = int(rng.integers(16, 100000)), int(rng.integers(16, 100000))
        n = int(rng.integers(1, 65))
        cases.append((dt, dt, cap, first, n, numels, bool(numels)))
        want.append((as_tuples(planner.plan(numels, eb, cap, first, n)),
                     expected_arena_map(numels, eb, cap, first, n) if numels else None))
    for k in range(12):   # fp32 gradients in bf16 buckets (the compression hook)
        numels = [int(x) for x in rng.integers(0, 20000, size=rng.integers(1, 60))]
        cap, first = int(rng.integers(16, 100000)), int(rng.integers(16, 100000))
        n = int(rng.integers(1, 65))
        cases.append((FP32, BF16, cap, first, n, numels, True))
        want.append((as_tuples(planner.plan(numels, 4, cap, first, n, vector_elems=8)),
                     expected_arena_map(numels, 4, cap, first, n, bucket_vector_elems=8)))
    numels = resnet50_param_numels()
    cases.append((FP32, FP32, 25 << 20, 1 << 20, 8, numels, True))
    want.append((as_tuples(planner.plan(numels, 4, world_size=8)),
                 expected_arena_map(numels, 4, 25 << 20, 1 << 20, 8)))
    cases.append((FP32, FP32, 1024, 1024, 4, [], False))   # no parameters at all
    want.append(([], None))

    results, maps = run_driver(driver, cases, tmp_path)
    for (gdt, cdt, cap, first, n, numels, _), res, (buckets, amap), got_map in zip(cases, results, want, maps):
        assert res["status"] == 0
        assert [{"members": [tuple(m) for m in b["members"]], "padded_numel": b["padded_numel"]}
                for b in res["buckets"]] == buckets, (gdt, cdt, cap, first, n)
        v = 4 if gdt == FP32 else 8
        offs = np.concatenate([[0], np.cumsum([-(-m // v) * v for m in numels])]).astype(np.int64)
        assert res["offsets"] == [int(o) for o in offs[:-1]]
        if amap is not None:
            assert res["map_status"] == 0
            assert np.array_equal(got_map, amap)
