"""The benchmark's command line on the CPU: more than one GPU is refused
with a message and exit status 2 before anything touches a GPU, and the
counter-based traffic figure is reported only for the kernel sources it was
taken on."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"],
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert proc.returncode == 2
    assert proc.stdout == ""
    assert "--gpus 8" in proc.stderr and "one GPU" in proc.stderr


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)


def test_single_config_arguments_are_checked_before_any_gpu_work():
    """--config picks one workload and --variant one form of it; a form the
    workload does not have, or --variant without --config, is refused by the
    argument parser (exit status 2) before anything is imported or launched."""
    for argv, msg in ((["--config", "c2", "--variant", "view"], "--variant view is not one of"),
                      (["--variant", "fused"], "need --config"),
                      (["--config", "c5", "--dtype", "bf16"], "c4 only"),
                      (["--config", "c9"], "invalid choice"),
                      (["--config", "c4", "--steps", "0"], "--steps must be"),
                      (["--graph"], "need --config"),
                      (["--config", "c2", "--variant", "persistent", "--graph"], "time it eagerly")):
        proc = run_bench(*argv)
        assert proc.returncode == 2, argv
        assert proc.stdout == ""
        assert msg in proc.stderr, (argv, proc.stderr)


def test_every_config_lists_its_forms():
    sys.path.insert(0, ROOT)
    import bench
    assert set(bench.CONFIGS) == {"c1", "c2", "c3", "c4", "c5", "probe"}
    for cfg in bench.CONFIGS:
        args = bench.parse_args(["--config", cfg])
        assert args.variant == ("copy" if cfg == "probe" else "fused")
        for v in bench.VARIANTS[cfg]:
            assert bench.parse_args(["--config", cfg, "--variant", v]).variant == v
    assert bench.parse_args([]).config == "all"
    # algorithmic bytes: the fused form moves 2NS, the step forms 5(N-1)S
    assert bench.ring_bytes("fused", 8, 1 << 30) == 16 << 30
    assert bench.ring_bytes("steps", 8, 1 << 30) == 35 << 30
    assert bench.ring_bytes("reduce-scatter", 8, 1 << 30) == 9 << 30
    assert bench.ring_bytes("persistent-noalloc", 8, 1 << 30) == bench.ring_bytes("persistent", 8, 1 << 30)
    # the allocation-free persistent entry point is the one form of it that a graph can hold
    for cfg in ("c1", "c2", "c4", "c5"):
        assert bench.parse_args(["--config", cfg, "--variant", "persistent-noalloc", "--graph"]).graph


def test_traffic_figure_follows_the_kernel_sources():
    """bench.py reports the counter-based HBM bytes only while the fused
    kernel's sources hash to the value the counters were taken on."""
    import hashlib
    sys.path.insert(0, ROOT)
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        prof = json.load(f)
    h = hashlib.sha256()
    for src in prof["kernel_sources"]:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    traffic = bench.traffic_from_profile()
    if h.hexdigest() == prof["kernel_source_sha256"]:
        assert traffic == prof["hbm_bytes_per_launch"]
        # within 0.1 % of the headline's algorithmic bytes (2 * 8 ranks * 1 GiB)
        assert prof["algorithmic_bytes_per_launch"] == 2 * 8 * (1 << 30)
        assert abs(traffic / prof["algorithmic_bytes_per_launch"] - 1) < 1e-3
    else:
        assert traffic is None
    assert sorted(os.path.join(ROOT, s) for s in prof["kernel_sources"]) == sorted(bench.KERNEL_SOURCES)


def test_copy_fraction_is_added_beside_every_hbm_rate():
    sys.path.insert(0, ROOT)
    import bench
    extras = {"copy_probe": {"bytes_moved": 8, "ms": 1.0, "gbps": 6000.0, "hbm_gbps": 6000.0},
              "steps": {"hbm_gbps": 6600.0},
              "sync": {"view": {"hbm_gbps_algorithmic": 3000.0}, "plain": {"ms": 1.0}}}
    bench.add_copy_fraction(extras, 6000.0)
    assert extras["steps"]["hbm_frac_of_copy_probe"] == 1.1
    assert extras["sync"]["view"]["hbm_frac_of_copy_probe"] == 0.5
    assert "hbm_frac_of_copy_probe" not in extras["sync"]["plain"]
    assert "hbm_frac_of_copy_probe" not in extras["copy_probe"]
