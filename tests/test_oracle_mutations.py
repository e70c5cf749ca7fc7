"""Plants plausible mistakes in the oracle (on the CPU, through monkeypatch)
and checks that at least one pin fails for each: the pins are discriminating.

Each pin below is a boolean version of a check in test_oracle_*.py.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import ddp, planner, ring, rounding
from ddp_workloads import host_rank_rng, host_grads, resnet50_param_numels

from test_oracle_worked_example import parse_worked_example, label_set, decode
from test_oracle_ring import parse_order_cases, parse_bound_cases, bound_case_inputs
from test_oracle_rounding import parse_cases
from test_oracle_planner import as_lists

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pin_worked_example():
    states, sends = parse_worked_example(os.path.join(GOLDEN, "p3_worked_example.txt"))
    bufs = [np.full(6, 2.0 ** r, dtype=np.float32) for r in range(3)]
    out = ring.ring_simulate(bufs, "fp32", record=True)
    got = [bufs] + [st for _, _, st in out["states"]]
    for state, want in zip(got, states):
        for gpu in range(3):
            for chunk in range(3):
                lo, hi = ring.chunk_bounds(6, 3, chunk)
                for e in range(lo, hi):
                    if decode(state[gpu][e]) != label_set(want["rows"][gpu][chunk], chunk):
                        return False
    for phase, step, labels in sends:
        f = ring.rs_chunk if phase == "rs" else ring.ag_chunk
        if any(f(r, step, 3) != int(lab.split("+")[0][1:]) for r, lab in enumerate(labels)):
            return False
    return True


def pin_integer_sums():
    for n in (2, 3, 5, 8):
        for count in (n, 3 * n + 2, 1):
            bufs = [host_rank_rng(7, r).integers(-100, 101, count).astype(np.float32)
                    for r in range(n)]
            want = np.sum(np.stack(bufs).astype(np.int64), axis=0)
            out = ring.ring_simulate(bufs, "fp32")["bufs"]
            if any(not np.array_equal(b.astype(np.int64), want) for b in out):
                return False
    return True


def pin_order_fixtures():
    for case in parse_order_cases(os.path.join(GOLDEN, "ring_order_cases.txt")):
        dt = case["dtype"]
        bufs = [rounding.round_to(np.array(v, dtype=np.float64), dt) for v in case["ranks"]]
        out = ring.ring_simulate(bufs, dt)["bufs"]
        if any(list(rounding.to_f64(b, dt)) != case["expect"] for b in out):
            return False
        for c in range(case["n"]):
            x = np.stack([b[c:c + 1] for b in bufs])
            if rounding.to_f64(ring.ring_order_sum(x, c, dt), dt)[0] != case["expect"][c]:
                return False
    return True


def pin_traffic():
    for n in (2, 4, 8):
        out = ring.ring_simulate([np.zeros(8 * n, np.float32)] * n, "fp32")
        if out["steps"] != 2 * (n - 1) or out["sent"] != [2 * (n - 1) * 8] * n:
            return False
    return True


def pin_rounding():
    for dtype, value, bits in parse_cases(os.path.join(GOLDEN, "rounding_cases.txt")):
        got = rounding.round_to(np.array([value]), dtype)
        got_bits = int(got.view(np.uint32)[0]) if dtype == "fp32" else int(got[0])
        if got_bits != bits:
            return False
    return True


def pin_planner():
    with open(os.path.join(GOLDEN, "planner_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = planner.plan(c["numels"], c["elem_bytes"], c["cap_bytes"],
                           c["first_bucket_bytes"], c["world_size"])
        if as_lists(got) != c["buckets"]:
            return False
    b = planner.plan(resnet50_param_numels(), 4, world_size=8)
    return b[0]["members"] == [(160, 0, 1000)]


def pin_ddp_mean():
    numels = [7, 16, 1, 40]
    n = 4
    buckets = planner.plan(numels, 4, cap_bytes=128, first_bucket_bytes=32, world_size=n)
    grads = [[host_rank_rng(14, r).integers(-50, 51, m).astype(np.float32) for m in numels]
             for r in range(n)]
    out = ddp.ddp_sync(grads, buckets, "fp32")
    for p in range(len(numels)):
        want = np.sum(np.stack([grads[r][p] for r in range(n)]).astype(np.float64), axis=0) / n
        if any(not np.array_equal(out[r][p].astype(np.float64), want) for r in range(n)):
            return False
    return True


def pin_reduce_scatter():
    for n, count in ((3, 6), (4, 10), (8, 64), (8, 3)):
        bufs = [host_rank_rng(300 + n, r).integers(-1000, 1001, count).astype(np.float32) for r in range(n)]
        total = np.sum(np.stack(bufs).astype(np.int64), axis=0)
        for scale, div in ((1.0, 1), (0.25, 4)):
            shards = ring.reduce_scatter(bufs, "fp32", scale)
            for r in range(n):
                lo, hi = ring.chunk_bounds(count, n, r)
                if len(shards) != n or not np.array_equal(shards[r].astype(np.float64), total[lo:hi] / div):
                    return False
    return True


def pin_compressed_mean():
    n = 4
    numels = [7, 16, 40, 300]
    buckets = planner.plan(numels, 4, cap_bytes=512, first_bucket_bytes=64, world_size=n, vector_elems=8)
    grads = [[host_rank_rng(17, r).integers(-8, 9, m).astype(np.float32) for m in numels] for r in range(n)]
    out = ddp.ddp_sync(grads, buckets, "fp32", comm_dtype="bf16")
    for p in range(len(numels)):
        want = np.sum(np.stack([grads[r][p] for r in range(n)]).astype(np.float64), axis=0) / n
        if any(out[r][p].dtype != np.float32 or not np.array_equal(out[r][p].astype(np.float64), want)
               for r in range(n)):
            return False
    return True


def pin_error_bound():
    import torch
    if rounding.unit_roundoff("fp32") != float(np.finfo(np.float32).eps) / 2:
        return False
    if rounding.unit_roundoff("bf16") != torch.finfo(torch.bfloat16).eps / 2:
        return False
    for case in parse_bound_cases(os.path.join(GOLDEN, "error_bound_cases.txt")):
        dt = case["dtype"]
        bufs = bound_case_inputs(case)
        got = rounding.to_f64(ring.ring_simulate(bufs, dt)["bufs"][0], dt)[0]
        bound = ring.error_bound(bufs, dt)[0]
        err = abs(got - ring.sum_f64(bufs, dt)[0])
        if bound != case["bound"] or err > bound:
            return False
        if case["attained"] and err * (1 + 2.0 ** -6) < bound:
            return False
    return True


PINS = [pin_worked_example, pin_integer_sums, pin_order_fixtures, pin_traffic,
        pin_rounding, pin_planner, pin_ddp_mean, pin_reduce_scatter, pin_compressed_mean,
        pin_error_bound]


def test_all_pins_hold_unmutated():
    assert [p.__name__ for p in PINS if not p()] == []


def _ring_order_from_c(x, c, dtype):
    x = np.asarray(x)
    n = x.shape[0]
    acc = x[c % n].copy()
    for k in range(1, n):
        acc = ring.hop_add(acc, x[(c + k) % n], dtype)
    return acc


def _bf16_truncate(x64):
    x = np.asarray(x64, np.float64).astype(np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _unpack_ignoring_scale(flat, bucket, scale, dtype, grad_dtype=None):
    return {p: rounding.round_to(rounding.to_f64(flat[off:off + m], dtype), grad_dtype or dtype)
            for p, off, m in bucket["members"]}


_reduce_scatter = ring.reduce_scatter


def _reduce_scatter_unscaled(bufs, dtype, scale=1.0):
    return _reduce_scatter(bufs, dtype, 1.0)


def _reduce_scatter_shifted(bufs, dtype, scale=1.0):
    shards = _reduce_scatter(bufs, dtype, scale)
    return shards[1:] + shards[:1]   # rank c receives chunk c+1


_abs_sum = ring.abs_sum_f64


def _abs_of_sum(bufs, dtype):
    return np.abs(np.sum(np.stack([rounding.to_f64(b, dtype) for b in bufs]), axis=0))


def _bound_with_n_terms(bufs, dtype):
    return len(bufs) * rounding.unit_roundoff(dtype) * _abs_sum(bufs, dtype)


MUTATIONS = {
    "rs sends the wrong chunk": (ring, "rs_chunk", lambda r, s, n: (r - s) % n),
    "ag sends the wrong chunk": (ring, "ag_chunk", lambda r, s, n: (r - 1 - s) % n),
    "ring runs leftwards": (ring, "right_neighbour", lambda r, n: (r - 1) % n),
    "rs hop drops the received term": (ring, "hop_add", lambda a, b, d: np.array(b, copy=True)),
    "ag hop adds instead of overwriting": (ring, "hop_copy", lambda a, b, d: ring.hop_add(a, b, d)),
    "chunk length rounds down": (ring, "chunk_length", lambda count, n: count // n),
    "closed form starts at rank c": (ring, "ring_order_sum", _ring_order_from_c),
    "bf16 rounding truncates": (rounding, "round_to_bf16", _bf16_truncate),
    "buckets in forward order": (planner, "bucket_order", lambda n: range(n)),
    "first bucket uses the regular cap": (planner, "bucket_capacity", lambda i, cap, first: cap),
    "unpack ignores the scale": (ddp, "unpack_scale", _unpack_ignoring_scale),
    "reduce-scatter ignores the scale": (ring, "reduce_scatter", _reduce_scatter_unscaled),
    "reduce-scatter gives rank c the next chunk": (ring, "reduce_scatter", _reduce_scatter_shifted),
    "fp32 unit roundoff 2^-23": (rounding, "unit_roundoff", lambda d: 2.0 ** -23 if d == "fp32" else 2.0 ** -8),
    "fp32 unit roundoff 2^-25": (rounding, "unit_roundoff", lambda d: 2.0 ** -25 if d == "fp32" else 2.0 ** -8),
    "bf16 unit roundoff 2^-7": (rounding, "unit_roundoff", lambda d: 2.0 ** -24 if d == "fp32" else 2.0 ** -7),
    "error bound on |sum g| instead of sum |g|": (ring, "abs_sum_f64", _abs_of_sum),
    "error bound with N terms instead of N-1": (ring, "error_bound", _bound_with_n_terms),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    module, attr, fake = MUTATIONS[name]
    monkeypatch.setattr(module, attr, fake)
    failed = []
    for p in PINS:
        try:
            ok = p()
        except Exception:
            ok = False
        if not ok:
            failed.append(p.__name__)
    assert failed, f"no pin catches: {name}"
