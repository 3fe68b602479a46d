"""bench.py's host-side contract, without a GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_only_for_the_profiled_workload():
    for op in ("fhd", "grid"):
        assert bench.measured_traffic(op, "radial64") is None
    assert bench.measured_traffic("forward", "spiral128") is None


def test_roofline_constants():
    # transcendental-bound: 2 per term at 8 lanes per clock per SIMD
    assert abs(bench.ROOF_TERMS - 256 * 4 * 8 * 2.4e9 / 2) / bench.ROOF_TERMS < 1e-9
    assert bench.ROOF_TERMS < bench.P_FP32 / bench.FLOP_PER_TERM
