"""The bookkeeping of the persistent launches' barrier slots (SlotRing in
csrc/barrier_slots.h), on the CPU under ThreadSanitizer: leases of one slot
never overlap, every reuse of a slot makes its stream wait for exactly the
previous lease of that slot, and a failed event creation frees the slot
(tests/sanitize/slot_ring_driver.cpp). Built with g++; no GPU code."""

import os
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "ring_all_reduce_ddp_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "slot_ring_driver.cpp")


def test_slot_ring_under_thread_sanitizer(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path / "slot_ring_driver")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread", "-I", CSRC, DRIVER,
                    "-o", exe], check=True)
    proc = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300,
                          env=dict(os.environ, TSAN_OPTIONS="halt_on_error=1"))
    assert "ThreadSanitizer" not in proc.stderr, proc.stderr[-4000:]
    assert proc.returncode == 0, proc.stderr[-4000:]
    assert proc.stdout.strip() == "slot ring ok"
