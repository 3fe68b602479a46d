"""bench.py's host-side contract, without a GPU."""
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_only_for_the_profiled_workload():
    for op in ("fhd", "grid", "forward"):
        assert bench.measured_traffic(op, "radial64") is None
    assert bench.measured_traffic("normal", "spiral128") is None


def test_roofline_constants():
    # transcendental-bound: 2 per term at 8 lanes per clock per SIMD
    assert abs(bench.ROOF_TERMS - 256 * 4 * 8 * 2.4e9 / 2) / bench.ROOF_TERMS < 1e-9
    assert bench.ROOF_TERMS < bench.P_FP32 / bench.FLOP_PER_TERM


def test_roof_terms_mixes_paths():
    r_direct, r_ramp = bench.ROOF_TERMS, bench.ROOF_TERMS_RAMP
    assert bench.roof_terms([(1.0, r_direct)]) == r_direct
    mixed = bench.roof_terms([(1.0, r_ramp), (1.0, r_direct)])
    assert abs(mixed - 2 / (1 / r_ramp + 1 / r_direct)) < 1e-6 * mixed


def test_issue_ceilings():
    # pure FMA pairs at two per quad-cycle: the FP32 vector peak at 2 FLOP each
    assert abs(bench.issue_terms(1.0, 0.0) * 2 - bench.P_FP32) / bench.P_FP32 < 2e-3
    # transcendentals only: the measured transcendental issue rate
    assert abs(bench.issue_terms(0.0, 1.0) - bench.P_TRANS) / bench.P_TRANS < 1e-12
    # the ramp paths' ceilings lie above the direct-form R
    assert bench.ROOF_TERMS_RAMP > bench.ROOF_TERMS_RAMP_LANE > bench.ROOF_TERMS_RAMP_F > bench.ROOF_TERMS
