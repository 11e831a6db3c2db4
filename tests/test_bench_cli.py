"""The benchmark's command-line contract that holds without a GPU: more than
one GPU is refused with a message before anything touches a device, and the
workload list the profiles' commands name is accepted by the parser."""

from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=120):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused_with_a_message():
    for n in ("2", "8"):
        r = run_bench("--gpus", n)
        assert r.returncode == 2, (r.returncode, r.stderr[-500:])
        assert "one GPU" in r.stderr and f"--gpus {n}" in r.stderr
        assert r.stdout.strip() == ""


def test_workload_names_are_accepted():
    r = run_bench("--help")
    assert r.returncode == 0
    for name in ("causal_prefill", "ring_share", "fanout", "fanout_paged", "fanout_prefill", "shard_merge",
                 "merge_scaled", "layouts", "backward", "copy_calibration", "gemm_reference"):
        assert name in r.stdout, name
