"""Pins that tie the fp64 oracle to the pages and to mathematics.

Each pin takes an oracle library handle (so that textual mutants of the
oracle can be run through the same checks) and raises AssertionError when
the oracle disagrees with a fact fixed independently of it:

* hand-worked cases with exact closed-form answers (tests/golden/);
* the single-sample phase ramp and the k = 0 sum (closed forms);
* the Cartesian-grid special case, which reduces to numpy's inverse FFT;
* F^H F = N I on a full integer Cartesian grid (orthogonality of the DFT);
* adjointness <F^H D, rho> = <D, F rho> against the independent forward F;
* conjugation symmetry and linearity (invariants of the definition).

Definitions: page "Case study -- iterative MRI reconstruction", section 17.3
(F^H D equation) and section 17.2 (F maps image to k-space).
"""
from __future__ import annotations

import os

import numpy as np

import oracle
from non_cartesian_mri_fhd_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "fhd_hand_cases.txt")


def _fhd(lib, c, threads=4):
    return oracle.fhd(c["kx"], c["ky"], c["kz"], c["Dr"], c["Di"], c["x"], c["y"], c["z"],
                      threads=threads, lib=lib)


def load_golden(path: str = GOLDEN) -> list[dict]:
    """Parse the hand-worked cases file into dicts of float64 arrays."""
    cases, cur = [], None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "case":
                cur = dict(name=tok[1], op=tok[2], sample=[], voxel=[])
            elif tok[0] in ("sample", "voxel"):
                cur[tok[0]].append([float(t) for t in tok[1:]])
            elif tok[0] == "end":
                cur["sample"] = np.array(cur["sample"], np.float64).reshape(-1, 5)
                cur["voxel"] = np.array(cur["voxel"], np.float64).reshape(-1, 5)
                cases.append(cur)
                cur = None
            else:
                raise ValueError("bad line: %r" % raw)
    return cases


# ---------------------------------------------------------------------------
def pin_golden(lib):
    cases = load_golden()
    assert len(cases) >= 8
    for c in cases:
        s, v = c["sample"], c["voxel"]
        # every input must be exact in fp32, as the GPU path consumes fp32
        for arr in (s[:, :3], v[:, :3]):
            assert np.array_equal(arr.astype(np.float32).astype(np.float64), arr), c["name"]
        if c["op"] == "adjoint":
            rr, ri = oracle.fhd(s[:, 0], s[:, 1], s[:, 2], s[:, 3], s[:, 4],
                                v[:, 0], v[:, 1], v[:, 2], threads=2, lib=lib)
            exp_r, exp_i = v[:, 3], v[:, 4]
        else:
            rr, ri = oracle.forward(s[:, 0], s[:, 1], s[:, 2], v[:, 3], v[:, 4],
                                    v[:, 0], v[:, 1], v[:, 2], threads=2, lib=lib)
            exp_r, exp_i = s[:, 3], s[:, 4]
        err = np.max(np.abs((rr - exp_r) + 1j * (ri - exp_i)))
        assert err < 1e-12, (c["name"], err, rr, ri)


def pin_single_sample_ramp(lib):
    """M = 1: rho_n = D exp(i 2 pi k.x_n): constant modulus |D| and a linear
    phase ramp whose step along axis a of an L-grid is exp(i 2 pi k_a / L)."""
    rng = np.random.default_rng(7)
    L = 8
    x, y, z = inputs.grid_coords(L)
    for trial in range(3):
        k = rng.uniform(-6, 6, 3).astype(np.float32)
        D = rng.standard_normal(2).astype(np.float32)
        rr, ri = oracle.fhd([k[0]], [k[1]], [k[2]], [D[0]], [D[1]], x, y, z, threads=3, lib=lib)
        rho = (rr + 1j * ri).reshape(L, L, L)           # [iz, iy, ix]
        assert np.allclose(np.abs(rho), np.hypot(np.float64(D[0]), np.float64(D[1])),
                           rtol=1e-12, atol=0)
        # the voxel at the grid origin (index L/2 on each axis) has phase 0
        o = L // 2
        assert abs(rho[o, o, o] - (float(D[0]) + 1j * float(D[1]))) < 1e-12
        for axis, ka in ((2, k[0]), (1, k[1]), (0, k[2])):
            step = np.exp(2j * np.pi * np.float64(ka) / L)
            a = np.moveaxis(rho, axis, -1)
            ratio = a[..., 1:] / a[..., :-1]
            assert np.allclose(ratio, step, rtol=0, atol=1e-12), (trial, axis)


def pin_dc_sum(lib):
    """All samples at k = 0: every voxel equals sum_m D_m (no weighting)."""
    rng = np.random.default_rng(11)
    M, N = 33, 17
    Dr, Di = rng.standard_normal(M), rng.standard_normal(M)
    x, y, z = rng.uniform(-0.5, 0.5, (3, N))
    zero = np.zeros(M)
    rr, ri = oracle.fhd(zero, zero, zero, Dr, Di, x, y, z, threads=2, lib=lib)
    assert np.allclose(rr, Dr.sum(), rtol=0, atol=1e-12)
    assert np.allclose(ri, Di.sum(), rtol=0, atol=1e-12)


def cartesian_fft_reference(c: dict) -> np.ndarray:
    """F^H D for a full integer k-grid over an L^3 voxel grid, via numpy.

    With x = (i - L/2)/L per axis, exp(i 2 pi k.x) = exp(i 2 pi k.i / L)
    (-1)^(kx+ky+kz), so rho = N * ifftn(A) where A[kz mod L, ky mod L,
    kx mod L] = D_k (-1)^(kx+ky+kz). Returned flat, voxel n = ix + L(iy + L iz).
    """
    L = c["L"]
    kx, ky, kz = (np.asarray(c[a], np.float64).astype(np.int64) for a in ("kx", "ky", "kz"))
    D = np.asarray(c["Dr"], np.float64) + 1j * np.asarray(c["Di"], np.float64)
    sign = np.where((kx + ky + kz) % 2 == 0, 1.0, -1.0)
    A = np.zeros((L, L, L), np.complex128)
    A[kz % L, ky % L, kx % L] = D * sign
    return (L ** 3 * np.fft.ifftn(A)).reshape(-1)


def pin_cartesian_ifft(lib):
    for L in (4, 8, 16):
        c = inputs.cartesian_case(L, seed=100 + L)
        rr, ri = _fhd(lib, c)
        ref = cartesian_fft_reference(c)
        err = np.linalg.norm(rr + 1j * ri - ref) / np.linalg.norm(ref)
        assert err < 1e-12, (L, err)


def pin_fhf_identity(lib):
    """Full integer k-grid: F^H (F rho) = N rho for any image rho."""
    L = 8
    rng = np.random.default_rng(5)
    kx, ky, kz = inputs.cartesian_kgrid(L)
    x, y, z = inputs.grid_coords(L)
    N = L ** 3
    pr, pi = rng.standard_normal(N), rng.standard_normal(N)
    Dr, Di = oracle.forward(kx, ky, kz, pr, pi, x, y, z, threads=4, lib=lib)
    rr, ri = oracle.fhd(kx, ky, kz, Dr, Di, x, y, z, threads=4, lib=lib)
    err = np.linalg.norm((rr - N * pr) + 1j * (ri - N * pi)) / (N * np.linalg.norm(pr + 1j * pi))
    assert err < 1e-12, err


def pin_adjointness(lib):
    """<F^H D, rho> = <D, F rho> with <u, v> = sum u conj(v), off-grid k and x."""
    c = inputs.random_case(N=211, M=157, seed=3, kmax=20.0)
    rng = np.random.default_rng(9)
    pr, pi = rng.standard_normal(c["N"]), rng.standard_normal(c["N"])
    rr, ri = _fhd(lib, c)
    Fr, Fi = oracle.forward(c["kx"], c["ky"], c["kz"], pr, pi, c["x"], c["y"], c["z"],
                            threads=3, lib=lib)
    lhs = np.vdot(pr + 1j * pi, rr + 1j * ri)          # sum (F^H D) conj(rho)
    D = c["Dr"].astype(np.float64) + 1j * c["Di"].astype(np.float64)
    rhs = np.vdot(Fr + 1j * Fi, D)                     # sum D conj(F rho)
    assert abs(lhs - rhs) <= 1e-12 * abs(lhs), (lhs, rhs)


def pin_conjugation(lib):
    """F^H[conj D](-k) = conj(F^H[D](k))."""
    c = inputs.random_case(N=64, M=48, seed=21)
    rr, ri = _fhd(lib, c)
    m = dict(c, kx=-c["kx"], ky=-c["ky"], kz=-c["kz"], Di=-c["Di"])
    mr, mi = _fhd(lib, m)
    assert np.allclose(mr, rr, rtol=0, atol=1e-12) and np.allclose(mi, -ri, rtol=0, atol=1e-12)


def pin_linearity(lib):
    """F^H (a D1 + b D2) = a F^H D1 + b F^H D2 for complex a, b."""
    rng = np.random.default_rng(13)
    c1 = inputs.random_case(N=50, M=40, seed=31)
    D2r, D2i = rng.standard_normal(40), rng.standard_normal(40)
    a, b = 0.75 - 1.25j, -2.0 + 0.5j
    D1 = c1["Dr"].astype(np.float64) + 1j * c1["Di"].astype(np.float64)
    D = a * D1 + b * (D2r + 1j * D2i)
    r1 = np.add(*[p * w for p, w in zip(_fhd(lib, c1), (1, 1j))])
    r2 = np.add(*[p * w for p, w in zip(_fhd(lib, dict(c1, Dr=D2r, Di=D2i)), (1, 1j))])
    rr, ri = _fhd(lib, dict(c1, Dr=D.real, Di=D.imag))
    assert np.allclose(rr + 1j * ri, a * r1 + b * r2, rtol=0, atol=1e-11)


PINS = {
    "golden": pin_golden,
    "single_sample_ramp": pin_single_sample_ramp,
    "dc_sum": pin_dc_sum,
    "cartesian_ifft": pin_cartesian_ifft,
    "fhf_identity": pin_fhf_identity,
    "adjointness": pin_adjointness,
    "conjugation": pin_conjugation,
    "linearity": pin_linearity,
}


def failing_pins(lib) -> list[str]:
    """Names of the pins that the given oracle library fails."""
    bad = []
    for name, pin in PINS.items():
        try:
            pin(lib)
        except AssertionError:
            bad.append(name)
    return bad
