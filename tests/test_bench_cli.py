"""bench.py's host-side contract, without a GPU: one GPU only, at least ten
timed batches, and the compact per-path record it prints."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("args", [("--batches", "9"), ("--steps", "0")])
def test_too_few_batches_or_steps_refused(args):
    r = run_bench(*args)
    assert r.returncode == 2


def test_compact_record():
    sys.path.insert(0, ROOT)
    import bench
    full = {"value": 1.0, "unit": "GB/s", "us": 2.0, "sample": "long text",
            "roofline": bench.roofline(4000.0, 8000.0, "GB/s", "hbm", 123, kernel="k"),
            "parity_rel_err": 1e-7, "cpu_baseline": {"value": 0.5, "unit": "GB/s", "cores": 16, "sample": "x"}}
    c = bench.compact(full)
    assert c["frac"] == 0.5 and c["traffic"] == 123 and c["parity_rel_err"] == 1e-7
    assert c["cpu"] == {"value": 0.5, "unit": "GB/s", "cores": 16}
    assert "sample" not in c
