"""The oracle's fp64 CG (oracle.cg) against facts independent of it (CPU).

* Full integer k-grid over an L^3 voxel grid: F^H F = N I, so one CG step
  from rho = 0 lands exactly on the image whose k-space is D.
* A small over-determined problem: CG on the normal equations reaches the
  least-squares solution that numpy.linalg.lstsq finds from the dense
  forward matrix.
"""
import numpy as np

import oracle
from non_cartesian_mri_fhd_amd import inputs


def test_one_step_on_full_cartesian_grid():
    L = 4
    kx, ky, kz = inputs.cartesian_kgrid(L)
    x, y, z = inputs.grid_coords(L)
    rng = np.random.default_rng(8)
    truth = rng.standard_normal(L ** 3) + 1j * rng.standard_normal(L ** 3)
    Dr, Di = oracle.forward(kx, ky, kz, truth.real, truth.imag, x, y, z)
    rho, res = oracle.cg(kx, ky, kz, Dr, Di, x, y, z, iters=3)
    assert len(res) >= 2 and res[1] < 1e-20 * res[0]
    assert np.max(np.abs(rho - truth)) < 1e-10


def test_reaches_dense_least_squares_solution():
    c = inputs.random_case(N=27, M=200, seed=61, kmax=1.5)
    X = np.stack([c["x"], c["y"], c["z"]], 1).astype(np.float64)
    K = np.stack([c["kx"], c["ky"], c["kz"]], 1).astype(np.float64)
    E = np.exp(-2j * np.pi * (K @ X.T))                      # forward operator, M x N
    D = c["Dr"].astype(np.float64) + 1j * c["Di"].astype(np.float64)
    ls = np.linalg.lstsq(E, D, rcond=None)[0]
    rho, res = oracle.cg(c["kx"], c["ky"], c["kz"], c["Dr"], c["Di"], c["x"], c["y"], c["z"],
                         iters=200, tol=1e-24 * float(np.vdot(E.conj().T @ D, E.conj().T @ D).real))
    assert np.linalg.norm(rho - ls) <= 1e-7 * np.linalg.norm(ls)


def test_zero_iterations_and_zero_data():
    c = inputs.random_case(N=10, M=20, seed=62)
    rho, res = oracle.cg(c["kx"], c["ky"], c["kz"], c["Dr"], c["Di"], c["x"], c["y"], c["z"],
                         iters=0)
    assert np.all(rho == 0) and len(res) == 1
    z0 = np.zeros(20)
    rho, res = oracle.cg(c["kx"], c["ky"], c["kz"], z0, z0, c["x"], c["y"], c["z"], iters=5)
    assert np.all(rho == 0) and res == [0.0]
