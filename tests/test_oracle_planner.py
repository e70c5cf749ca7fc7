"""The oracle's bucket planner against the pages' constants, hand-derived
plans and the invariants of reverse-order bucketing."""

import json
import os

import numpy as np
import pytest

from oracle import planner
from ddp_workloads import resnet50_param_numels, resnet50_param_shapes


def test_default_capacities():
    """25 MiB regular and 1 MiB first-bucket capacity, computed as MB times
    1024 * 1024 (page "DDP 与 Ring All-Reduce", blog.vllbc.top, section 03, part
    "Bucket"; page "Day 17 数据并行 DP/DDP", part "源码阅读路线")."""
    assert planner.DEFAULT_CAP_BYTES == 26_214_400 == 25 * 1024 * 1024
    assert planner.DEFAULT_FIRST_BUCKET_BYTES == 1_048_576


def load_cases(golden_dir):
    with open(os.path.join(golden_dir, "planner_cases.json")) as f:
        return json.load(f)["cases"]


def as_lists(buckets):
    return [{"members": [list(m) for m in b["members"]], "padded_numel": b["padded_numel"]}
            for b in buckets]


def test_hand_derived_plans(golden_dir):
    cases = load_cases(golden_dir)
    assert len(cases) == 7
    for c in cases:
        got = planner.plan(c["numels"], c["elem_bytes"], c["cap_bytes"],
                           c["first_bucket_bytes"], c["world_size"])
        assert as_lists(got) == c["buckets"], c["name"]


def check_invariants(numels, elem_bytes, cap, first, n, buckets):
    v = 16 // elem_bytes
    order = [m[0] for b in buckets for m in b["members"]]
    # every parameter exactly once, in reverse registration order
    assert order == list(reversed(range(len(numels))))
    for i, b in enumerate(buckets):
        limit = first if i == 0 else cap
        used = 0
        for p, off, numel in b["members"]:
            assert numel == numels[p]
            assert off % v == 0 and off == used        # aligned, packed in order
            used = off + -(-numel // v) * v
        assert b["padded_numel"] % (n * v) == 0 and b["padded_numel"] >= used
        assert b["padded_numel"] - used < n * v
        if len(b["members"]) > 1:
            assert used * elem_bytes <= limit
        if i + 1 < len(buckets):
            # the bucket was closed because the next tensor did not fit
            nxt = buckets[i + 1]["members"][0][2]
            assert (used + -(-nxt // v) * v) * elem_bytes > limit


@pytest.mark.parametrize("seed", range(20))
def test_invariants_random(seed):
    rng = np.random.default_rng(seed)
    numels = list(rng.integers(0, 5000, size=rng.integers(1, 60)))
    elem = [2, 4][seed % 2]
    cap = int(rng.integers(16, 20000))
    first = int(rng.integers(16, 20000))
    n = int(rng.integers(1, 9))
    b = planner.plan(numels, elem, cap, first, n)
    check_invariants([int(x) for x in numels], elem, cap, first, n, b)


def test_resnet50_shapes():
    """161 parameter tensors and 25,557,032 elements (ResNet-50 as defined by
    He et al. 2016, Table 1)."""
    shapes = resnet50_param_shapes()
    numels = resnet50_param_numels()
    assert len(shapes) == 161
    assert sum(numels) == 25_557_032
    assert shapes[-1] == ("fc.bias", (1000,)) and numels[-2] == 2048 * 1000
    assert all(m % 8 == 0 for m in numels)


def test_resnet50_plan():
    """Reverse order with the default capacities: bucket 0 holds fc.bias only
    (fc.weight alone passes 1 MiB); six buckets in all.  The exact split
    depends on the reading of "capacity" (never exceeded) and is not printed
    on the pages; the invariants are."""
    numels = resnet50_param_numels()
    b = planner.plan(numels, 4, world_size=8)
    check_invariants(numels, 4, planner.DEFAULT_CAP_BYTES, planner.DEFAULT_FIRST_BUCKET_BYTES, 8, b)
    assert b[0]["members"] == [(160, 0, 1000)]
    assert b[0]["padded_numel"] == 1024
    used = [m[-1][1] + m[-1][2] for m in (x["members"] for x in b)]
    assert used == [1000, 6_514_688, 4_462_592, 6_300_160, 6_112_256, 2_166_336]


def test_bad_arguments():
    with pytest.raises(ValueError):
        planner.plan([1], 3)
    with pytest.raises(ValueError):
        planner.plan([1], 4, cap_bytes=0)
    with pytest.raises(ValueError):
        planner.plan([-1], 4)
    assert planner.plan([], 4) == []
