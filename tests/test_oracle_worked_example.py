"""The oracle's ring against the pages' worked example (3 GPUs, 6 elements).

Fixture: tests/golden/p3_worked_example.txt, the symbolic state table of page
"DDP 与 Ring-AllReduce" (xuesongtap.github.io), §1.3.2.1 and §1.3.2.2.

Rank r's value is 2^r in every element, so each partial sum in the simulation
decodes exactly into the set of GPUs that contributed to it.
"""

import os

import numpy as np

from oracle import ring

LETTER = {"A": 0, "B": 1, "C": 2}


def parse_worked_example(path):
    states, sends = [], []
    cur = None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("state "):
                cur = {"label": line[6:], "rows": []}
                states.append(cur)
            elif line.startswith("sends "):
                head, body = line.split(":", 1)
                _, phase, step = head.split()
                sends.append((phase, int(step), [t.strip() for t in body.split("|")]))
            else:
                _, body = line.split(":", 1)
                cur["rows"].append([t.strip() for t in body.split("|")])
    return states, sends


def label_set(label, chunk):
    """Contributor set and chunk of a label such as 'A1+C1' or 'S2'."""
    if label.startswith("S"):
        assert int(label[1:]) == chunk
        return {0, 1, 2}
    out = set()
    for term in label.split("+"):
        assert int(term[1:]) == chunk, (label, chunk)
        out.add(LETTER[term[0]])
    return out


def decode(value):
    v = int(value)
    return {r for r in range(3) if v >> r & 1}


def test_fixture_is_consistent(golden_dir):
    states, sends = parse_worked_example(os.path.join(golden_dir, "p3_worked_example.txt"))
    assert [s["label"] for s in states] == ["initial", "rs 0", "rs 1", "ag 0", "ag 1"]
    assert len(sends) == 4
    for s in states:
        assert len(s["rows"]) == 3 and all(len(r) == 3 for r in s["rows"])


def test_states_after_every_step(golden_dir):
    states, _ = parse_worked_example(os.path.join(golden_dir, "p3_worked_example.txt"))
    bufs = [np.full(6, 2.0 ** r, dtype=np.float32) for r in range(3)]
    out = ring.ring_simulate(bufs, "fp32", record=True)
    assert out["steps"] == 4
    got = [("initial", bufs)] + [(f"{ph} {s}", st) for ph, s, st in out["states"]]
    for (label, state), want in zip(got, states):
        assert label == want["label"]
        for gpu in range(3):
            for chunk in range(3):
                expect = label_set(want["rows"][gpu][chunk], chunk)
                lo, hi = ring.chunk_bounds(6, 3, chunk)
                for e in range(lo, hi):
                    assert decode(state[gpu][e]) == expect, (label, gpu, chunk, e)


def test_send_schedule(golden_dir):
    """The chunk each GPU passes right in each step is the one the page shows."""
    _, sends = parse_worked_example(os.path.join(golden_dir, "p3_worked_example.txt"))
    for phase, step, labels in sends:
        for r, lab in enumerate(labels):
            chunk = int(lab.split("+")[0][1:])
            f = ring.rs_chunk if phase == "rs" else ring.ag_chunk
            assert f(r, step, 3) == chunk, (phase, step, r)


def test_rs_ownership_and_ag_equality_symbolic():
    """After reduce-scatter GPU c holds chunk c complete; after all-gather every
    GPU holds every chunk complete (the page's target vector)."""
    bufs = [np.full(6, 2.0 ** r, dtype=np.float32) for r in range(3)]
    rs = ring.ring_simulate(bufs, "fp32", n_steps=2)["bufs"]
    for c in range(3):
        lo, hi = ring.chunk_bounds(6, 3, c)
        assert all(decode(v) == {0, 1, 2} for v in rs[c][lo:hi])
    full = ring.ring_simulate(bufs, "fp32")["bufs"]
    for r in range(3):
        assert all(decode(v) == {0, 1, 2} for v in full[r])
