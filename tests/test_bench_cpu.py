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
    for (kernel, workload), entry in bench.TRAFFIC.items():
        other = "vdrandom256" if workload != "vdrandom256" else "spiral128"
        if (kernel, other) not in bench.TRAFFIC:
            assert bench.measured_traffic(kernel, other) is None
    assert bench.measured_traffic("fhd_grid_kernel", "spiral128") is None


def test_traffic_follows_the_sources(tmp_path, monkeypatch):
    """A recorded figure holds only for the sources it was taken on."""
    (kernel, workload), entry = next(iter(bench.TRAFFIC.items()))
    src = tmp_path / "csrc"
    src.mkdir()
    for name in entry["sources"]:
        (src / name).write_bytes(open(os.path.join(bench.CSRC, name), "rb").read())
    monkeypatch.setattr(bench, "CSRC", str(src))
    same = bench.measured_traffic(kernel, workload)
    (src / entry["sources"][0]).write_bytes(b"// edited\n" + (src / entry["sources"][0]).read_bytes())
    assert bench.measured_traffic(kernel, workload) is None
    if same is not None:
        assert same == entry["bytes_per_launch"]


def test_alu_kernels_priced_at_their_issue_ceiling():
    r = bench.roofline_for("fhd_gather_kernel<16, true>", 1e12, 50.0, None, (0.0, 1.0, 0.0))
    assert r["bound"] == "alu" and abs(r["frac"] - 1e12 / 0.05 / bench.ROOF_TERMS_RAMP) < 1e-12
    m = bench.roofline_for("fhd_gather_patch_kernel<true, true>", 1e12, 50.0, None)
    assert m["bound"] == "mfma" and m["peak"] == bench.P_MFMA_F16 / 1e12


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
