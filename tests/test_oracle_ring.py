"""The oracle's ring simulation against what the pages and arithmetic fix:
exact integer sums, the association-order fixtures, the 2(N-1) step count,
the per-rank traffic 2(N-1)/N * S, phase invariants and the error bound."""

import math
import os

import numpy as np
import pytest

from oracle import ring, rounding
from ddp_workloads import host_ring_inputs, host_rank_rng


# ---------------------------------------------------------------- brute force

def int_inputs(n, count, lo, hi, seed, dtype):
    out = []
    for r in range(n):
        x = host_rank_rng(seed, r).integers(lo, hi + 1, size=count).astype(np.float32)
        out.append(rounding.round_to(x.astype(np.float64), dtype))
    return out


@pytest.mark.parametrize("n", range(1, 10))
@pytest.mark.parametrize("extra", [0, 1, 2, 5])
def test_integer_sums_fp32(n, extra):
    """Integer inputs keep every partial sum below 2^24, so any order is exact:
    the all-reduce must give the plain elementwise sum on every rank (page
    "DDP 与 Ring-AllReduce", xuesongtap.github.io, §1.3.2: every GPU ends with
    the sum of the three vectors)."""
    for count in {0, 1, max(n - 1, 0), n, 3 * n + extra, 17 * n + extra}:
        bufs = int_inputs(n, count, -1000, 1000, 100 + n, "fp32")
        want = np.sum(np.stack(bufs).astype(np.int64), axis=0)
        out = ring.ring_simulate(bufs, "fp32")
        for r in range(n):
            assert np.array_equal(out["bufs"][r].astype(np.int64), want), (n, count, r)


@pytest.mark.parametrize("n", [2, 3, 5, 8, 9])
def test_integer_sums_bf16(n):
    """bf16 holds integers up to 256 exactly; inputs in [-8, 8] with N <= 9 keep
    every partial sum exact."""
    count = 7 * n + 3
    bufs = int_inputs(n, count, -8, 8, 200 + n, "bf16")
    want = np.sum(np.stack([rounding.to_f64(b, "bf16") for b in bufs]), axis=0)
    out = ring.ring_simulate(bufs, "bf16")
    for r in range(n):
        assert np.array_equal(rounding.to_f64(out["bufs"][r], "bf16"), want)


# ---------------------------------------------------------------- association order

def parse_order_cases(path):
    cases, cur = [], None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("case "):
                _, dtype, n = line.split()
                cur = {"dtype": dtype, "n": int(n), "ranks": []}
                cases.append(cur)
            elif line.startswith("rank"):
                cur["ranks"].append([float(v) for v in line.split(":", 1)[1].split()])
            elif line.startswith("expect:"):
                cur["expect"] = [float(v) for v in line.split(":", 1)[1].split()]
    return cases


def test_association_order_fixtures(golden_dir):
    cases = parse_order_cases(os.path.join(golden_dir, "ring_order_cases.txt"))
    assert len(cases) == 3
    for case in cases:
        dt, n = case["dtype"], case["n"]
        bufs = [rounding.round_to(np.array(v, dtype=np.float64), dt) for v in case["ranks"]]
        for b, v in zip(bufs, case["ranks"]):   # inputs are exact in the dtype
            assert np.array_equal(rounding.to_f64(b, dt), np.array(v))
        out = ring.ring_simulate(bufs, dt)
        for r in range(n):
            assert list(rounding.to_f64(out["bufs"][r], dt)) == case["expect"], (dt, n, r)
        for c in range(n):   # the closed form agrees element by element
            x = np.stack([b[c:c + 1] for b in bufs])
            got = rounding.to_f64(ring.ring_order_sum(x, c, dt), dt)
            assert got[0] == case["expect"][c]


# ---------------------------------------------------------------- steps and traffic

@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 13])
def test_step_count_and_traffic(n):
    """2(N-1) steps; each rank sends one chunk per step, 2(N-1)/N of the buffer
    in all (page "DDP 与 Ring All-Reduce", blog.vllbc.top, section 04; page "DDP 与
    Ring-AllReduce", xuesongtap.github.io, §1.3.1 and §1.3.3)."""
    count = 6 * n
    bufs = host_ring_inputs(1, n, count, "fp32", std=1.0)
    out = ring.ring_simulate(bufs, "fp32")
    assert out["steps"] == 2 * (n - 1)
    assert out["sent"] == [2 * (n - 1) * count // n] * n


def test_traffic_ratio_8_to_64():
    """Going from 8 to 64 ranks raises the per-rank traffic by 12.5 % and the
    number of steps ninefold (section 04 of the blog.vllbc.top page)."""
    count = 64 * 8
    res = {}
    for n in (8, 64):
        bufs = [np.zeros(count, np.float32) for _ in range(n)]
        out = ring.ring_simulate(bufs, "fp32")
        res[n] = (out["sent"][0], out["steps"])
    assert res[64][0] / res[8][0] == pytest.approx(1.125)
    assert res[64][1] / res[8][1] == 9


@pytest.mark.parametrize("n,count", [(3, 7), (4, 2), (5, 23), (8, 5)])
def test_ragged_total_traffic(n, count):
    """Each chunk is sent by exactly one rank per step, so across ranks every
    step moves the whole buffer once (trailing chunks may be short or empty)."""
    bufs = host_ring_inputs(2, n, count, "fp32", std=1.0)
    out = ring.ring_simulate(bufs, "fp32")
    assert sum(out["sent"]) == 2 * (n - 1) * count


# ---------------------------------------------------------------- phase invariants

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n,count", [(2, 16), (3, 6), (5, 41), (8, 64), (8, 67), (9, 100)])
def test_phase_invariants(dtype, n, count):
    """After the N-1 reduce-scatter steps rank c owns chunk c fully reduced
    (xuesongtap.github.io §1.3.2.1); after all-gather every rank is identical
    (§1.3.2.2) and equals the closed-form ring-order sum."""
    bufs = host_ring_inputs(7, n, count, dtype, std=1e-3)
    rs = ring.ring_simulate(bufs, dtype, n_steps=n - 1)["bufs"]
    full = ring.ring_simulate(bufs, dtype)["bufs"]
    for c in range(n):
        lo, hi = ring.chunk_bounds(count, n, c)
        x = np.stack([b[lo:hi] for b in bufs])
        closed = ring.ring_order_sum(x, c, dtype)
        assert np.array_equal(rs[c][lo:hi].view(np.uint8), closed.view(np.uint8))
        for r in range(n):
            assert np.array_equal(full[r][lo:hi].view(np.uint8), closed.view(np.uint8))


def test_n_steps_prefix_is_consistent():
    """Running k steps and then inspecting equals the k-th recorded state."""
    bufs = host_ring_inputs(3, 4, 20, "fp32", std=1.0)
    rec = ring.ring_simulate(bufs, "fp32", record=True)["states"]
    for k in range(1, 7):
        part = ring.ring_simulate(bufs, "fp32", n_steps=k)["bufs"]
        for r in range(4):
            assert np.array_equal(part[r], rec[k - 1][2][r])
    with pytest.raises(ValueError):
        ring.ring_simulate(bufs, "fp32", n_steps=7)


def test_sampled_positions_match_full_run():
    """Running the ring on a sample of positions (with their chunk ids) gives
    the same values as the full run at those positions."""
    n, count = 8, 800
    bufs = host_ring_inputs(4, n, count, "fp32", std=1e-2)
    full = ring.ring_simulate(bufs, "fp32")["bufs"]
    pos = np.sort(host_rank_rng(9, 0).choice(count, size=57, replace=False))
    L = ring.chunk_length(count, n)
    sampled = ring.ring_simulate([b[pos] for b in bufs], "fp32", chunk_of=pos // L)["bufs"]
    for r in range(n):
        assert np.array_equal(sampled[r], full[r][pos])


# ---------------------------------------------------------------- error bound

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n", [2, 8, 64])
def test_error_bound_against_exact_sum(dtype, n):
    """|ring - exact| <= (N-1) u sum|g_i| per element (recursive summation with
    round-to-nearest), against math.fsum of the exact inputs."""
    count = 4 * n
    bufs = host_ring_inputs(5, n, count, dtype, std=1e-3, heavy_frac=0.05, heavy_mult=1e3)
    out = ring.ring_simulate(bufs, dtype)["bufs"][0]
    exact = ring.sum_f64(bufs, dtype)
    err = np.abs(rounding.to_f64(out, dtype) - exact)
    assert np.all(err <= ring.error_bound(bufs, dtype))


def test_error_bound_is_reached_in_part():
    """The rounding is real: for fp32 Gaussian inputs at N=8 the ring result
    differs from the exact sum somewhere (a ring that kept fp64 partial sums
    would not)."""
    bufs = host_ring_inputs(6, 8, 4000, "fp32", std=1e-3)
    out = ring.ring_simulate(bufs, "fp32")["bufs"][0].astype(np.float64)
    exact = ring.sum_f64(bufs, "fp32")
    assert np.any(out != exact)
    assert np.all(np.abs(out - exact) <= ring.error_bound(bufs, "fp32"))


def parse_bound_cases(path):
    """Cases of tests/golden/error_bound_cases.txt: dtype, N, the per-rank
    inputs and the hand-derived result, exact sum and bound (as floats)."""
    cases, cur = [], None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("case"):
                _, dt, n = line.split()
                cur = {"dtype": dt, "n": int(n)}
                cases.append(cur)
                continue
            key, val = line.split(":", 1)
            val = val.split()
            if key == "ranks":
                cur["ranks"] = [float.fromhex(v) for v in val]
            elif key == "attained":
                cur["attained"] = val[0] == "yes"
            else:
                cur[key] = float.fromhex(val[0])
    return cases


def bound_case_inputs(case):
    dt = case["dtype"]
    return [rounding.round_to(np.array([v], dtype=np.float64), dt) for v in case["ranks"]]


def test_unit_roundoff_is_half_the_spacing_above_one():
    """u is half the distance from 1 to the next value of the format, as numpy
    (binary32) and torch (bfloat16) describe the formats."""
    import torch
    assert rounding.unit_roundoff("fp32") == float(np.finfo(np.float32).eps) / 2
    assert rounding.unit_roundoff("bf16") == torch.finfo(torch.bfloat16).eps / 2


def test_error_bound_golden_cases(golden_dir):
    """Hand-derived values (tests/golden/error_bound_cases.txt): the ring's
    result, the exact sum and the bound (N-1) u sum|g_i|; the error never
    exceeds the bound, and in the cases built for it reaches the bound to
    within a factor 1 + 2^-6, so a constant twice too large would show."""
    cases = parse_bound_cases(os.path.join(golden_dir, "error_bound_cases.txt"))
    assert len(cases) == 5
    for case in cases:
        dt = case["dtype"]
        bufs = bound_case_inputs(case)
        assert len(bufs) == case["n"]
        out = ring.ring_simulate(bufs, dt)["bufs"]
        got = rounding.to_f64(out[0], dt)[0]
        assert got == case["result"], case
        exact = ring.sum_f64(bufs, dt)[0]
        assert exact == case["exact"], case
        bound = ring.error_bound(bufs, dt)[0]
        assert bound == case["bound"], case
        err = abs(got - exact)
        assert err <= bound
        if case["attained"]:
            assert err * (1 + 2.0 ** -6) >= bound, case


def test_fsum_helper_is_exactly_rounded():
    assert ring.sum_f64([np.array([1e8], np.float32), np.array([1.0], np.float32),
                         np.array([-1e8], np.float32)], "fp32")[0] == math.fsum([1e8, 1.0, -1e8])


# ---------------------------------------------------------------- reduce-scatter output

@pytest.mark.parametrize("n,count", [(1, 5), (2, 8), (3, 6), (4, 10), (8, 64), (8, 3), (9, 100)])
def test_reduce_scatter_integer_shards(n, count):
    """Integer inputs: rank r's shard is exactly the sum of chunk r over all
    ranks (times a power-of-two scale, also exact)."""
    bufs = int_inputs(n, count, -1000, 1000, 300 + n, "fp32")
    total = np.sum(np.stack(bufs).astype(np.int64), axis=0)
    for scale, div in ((1.0, 1), (0.25, 4)):
        shards = ring.reduce_scatter(bufs, "fp32", scale)
        assert len(shards) == n
        for r in range(n):
            lo, hi = ring.chunk_bounds(count, n, r)
            assert np.array_equal(shards[r].astype(np.float64), total[lo:hi] / div)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_reduce_scatter_matches_closed_form(dtype):
    """The shards equal the ring-order sum of each chunk, scaled and rounded once."""
    n, count = 5, 5 * 37 + 2
    bufs = host_ring_inputs(12, n, count, dtype, std=1e-2)
    s = np.float32(1) / np.float32(n)
    shards = ring.reduce_scatter(bufs, dtype, s)
    for c in range(n):
        lo, hi = ring.chunk_bounds(count, n, c)
        x = np.stack([b[lo:hi] for b in bufs])
        want = rounding.round_to(rounding.to_f64(ring.ring_order_sum(x, c, dtype), dtype) * float(s), dtype)
        assert np.array_equal(shards[c].view(np.uint8), want.view(np.uint8))
