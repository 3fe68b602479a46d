"""The fp64 oracle against facts fixed by the pages and by mathematics (CPU)."""
import numpy as np
import pytest

import oracle
from non_cartesian_mri_fhd_amd import inputs

from pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(oracle_lib, name):
    PINS[name](oracle_lib)


def test_dense_matrix_brute_force_ragged(oracle_lib):
    """Second implementation: rho = E D with E = exp(i 2 pi X K^T) as a dense
    numpy complex128 matrix, on a ragged off-grid case."""
    c = inputs.random_case(N=97, M=61, seed=17, kmax=30.0)
    X = np.stack([c["x"], c["y"], c["z"]], 1).astype(np.float64)
    K = np.stack([c["kx"], c["ky"], c["kz"]], 1).astype(np.float64)
    E = np.exp(2j * np.pi * (X @ K.T))
    ref = E @ (c["Dr"].astype(np.float64) + 1j * c["Di"].astype(np.float64))
    rr, ri = oracle.fhd(c["kx"], c["ky"], c["kz"], c["Dr"], c["Di"], c["x"], c["y"], c["z"],
                        lib=oracle_lib)
    assert np.max(np.abs(rr + 1j * ri - ref)) < 1e-11


def test_dense_matrix_random16_full(oracle_lib):
    """Dense-matrix brute force over the whole 16^3 x 2048 workload."""
    w = inputs.make_workload("random16")
    X = np.stack([w["x"], w["y"], w["z"]], 1).astype(np.float64)
    K = np.stack([w["kx"], w["ky"], w["kz"]], 1).astype(np.float64)
    ref = np.exp(2j * np.pi * (X @ K.T)) @ (w["Dr"].astype(np.float64)
                                            + 1j * w["Di"].astype(np.float64))
    rr, ri = oracle.fhd(w["kx"], w["ky"], w["kz"], w["Dr"], w["Di"], w["x"], w["y"], w["z"],
                        lib=oracle_lib)
    assert np.linalg.norm(rr + 1j * ri - ref) / np.linalg.norm(ref) < 1e-13


def test_thread_count_independent_bitwise(oracle_lib):
    c = inputs.random_case(N=301, M=77, seed=41)
    outs = [oracle.fhd(c["kx"], c["ky"], c["kz"], c["Dr"], c["Di"], c["x"], c["y"], c["z"],
                       threads=t, lib=oracle_lib) for t in (1, 3, 8, 64)]
    for rr, ri in outs[1:]:
        assert np.array_equal(rr, outs[0][0]) and np.array_equal(ri, outs[0][1])


def test_empty_inputs(oracle_lib):
    c = inputs.random_case(N=5, M=3, seed=1)
    e = np.zeros(0)
    rr, ri = oracle.fhd(e, e, e, e, e, c["x"], c["y"], c["z"], lib=oracle_lib)
    assert np.array_equal(rr, np.zeros(5)) and np.array_equal(ri, np.zeros(5))
    rr, ri = oracle.fhd(c["kx"], c["ky"], c["kz"], c["Dr"], c["Di"], e, e, e, lib=oracle_lib)
    assert rr.size == 0 and ri.size == 0
    Dr, Di = oracle.forward(e, e, e, c["x"], c["y"], c["x"], c["y"], c["z"], lib=oracle_lib)
    assert Dr.size == 0


def test_length_mismatch_rejected(oracle_lib):
    c = inputs.random_case(N=5, M=3, seed=1)
    with pytest.raises(ValueError):
        oracle.fhd(c["kx"][:2], c["ky"], c["kz"], c["Dr"], c["Di"], c["x"], c["y"], c["z"],
                   lib=oracle_lib)


def test_op_count_statement():
    """Page 1 section 17.3 puts 256^3 voxels x 100k samples at about 1.6e12
    terms; the 256^3 workload has that shape."""
    w = inputs.WORKLOADS["vdrandom256"]
    assert w.N == 256 ** 3 and w.M == 100_000
    assert 1.6e12 <= w.terms < 1.7e12
