"""bench.py's command-line contract on the CPU (no GPU is touched)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_exits_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_headline_workload():
    sys.path.insert(0, ROOT)
    import workloads
    # T*H*(2R+6) + 8H for the sandwich; reads R partials + residual, writes 2 outputs
    assert workloads.algorithmic_bytes(4, 4096, 5120, epilogue="sandwich") == \
        4096 * 5120 * (2 * 4 + 6) + 8 * 5120
    # finalize: R*(k+1) gathered rows + weights/indices + residual in, 2 outputs
    assert workloads.algorithmic_bytes(8, 64, 6144, epilogue="rmsnorm", k=10) == \
        64 * 6144 * 2 * 8 * 11 + 8 * 64 * 10 + 6 * 64 * 6144 + 4 * 6144


def test_kernel_digest_is_stable_and_matches_stored_traffic_format():
    sys.path.insert(0, ROOT)
    import bench
    d1, d2 = bench.kernel_code_digest(), bench.kernel_code_digest()
    assert d1 == d2 and len(d1) == 64
    # a stored summary for other machine code must read as unknown traffic
    assert bench.stored_traffic("sandwich_h5120_r4", 4096, "0" * 64) is None
