"""Seeded synthetic inputs for the adjoint non-uniform DFT (F^H D).

This module is shared by the fp64 oracle's tests and by the GPU path's tests
and benchmark. It only *generates* data -- voxel grids, k-space trajectories
and k-space values -- and holds none of the F^H D arithmetic.

Conventions (pages: "Case study -- iterative MRI reconstruction", section
17.3, the F^H D equation; and "Chapter 17: MRI Reconstruction", section 17.2):

* k-space coordinates are in cycles per field of view, voxel coordinates in
  field-of-view units, so the phase of one term is 2*pi*(k . x) radians.
* A voxel grid of side L has per-axis coordinate (i - L/2)/L for i < L, which
  is exact in fp32 (dyadic) and lies in [-0.5, 0.5). Voxel n = ix + L*(iy +
  L*iz): x varies fastest.
* Every array is generated in fp64 with numpy and rounded to fp32 once; the
  GPU path and the oracle both consume these fp32 arrays.

The five named workloads are the benchmark and parity shapes of this project:

=============  =========  ========  ==========================================
name           voxels     samples   trajectory / k-space values
=============  =========  ========  ==========================================
random16       16^3       2,048     k i.i.d. U[-8, 8)^3; D ~ N(0,1) + iN(0,1)
spiral32       32^3       16,384    stack of spirals, 16 planes x 4 x 256
radial64       64^3       65,536    3-D radial kooshball, 256 spokes x 256,
                                    D = analytic FT of 10 Gaussian blobs
spiral128      128^3      100,000   stack of spirals, 25 planes x 8 x 500
vdrandom256    256^3      100,000   variable density k = 128*u*|u|, u ~ U[-1,1)
=============  =========  ========  ==========================================
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

F32 = np.float32


@dataclass(frozen=True)
class Workload:
    """Shape of one named workload."""

    name: str
    L: int          # voxel grid side; N = L**3
    M: int          # number of k-space samples
    seed: int       # numpy default_rng seed of its random draws
    trajectory: str

    @property
    def N(self) -> int:
        return self.L ** 3

    @property
    def terms(self) -> int:
        return self.N * self.M


WORKLOADS = {
    w.name: w
    for w in (
        Workload("random16", 16, 2048, 1001, "uniform random k in [-8,8)^3"),
        Workload("spiral32", 32, 16384, 1002, "stack of spirals 16x4x256"),
        Workload("radial64", 64, 65536, 1003, "3-D radial kooshball 256x256"),
        Workload("spiral128", 128, 100_000, 1004, "stack of spirals 25x8x500"),
        Workload("vdrandom256", 256, 100_000, 1005, "variable-density random"),
    )
}

# Seed of the 4096-voxel subset on which the 256^3 workload is checked.
SUBSET_SEED = 2005
SUBSET_SIZE = 4096


# --------------------------------------------------------------------------
# voxel grids
# --------------------------------------------------------------------------
def grid_axis(L: int) -> np.ndarray:
    """Per-axis voxel coordinates (i - L/2)/L, i < L, in fp64 (exact)."""
    i = np.arange(L, dtype=np.float64)
    return (i - L // 2) / L


def grid_coords(L: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """fp32 x, y, z of an L^3 Cartesian grid, voxel n = ix + L*(iy + L*iz)."""
    a = grid_axis(L).astype(F32)
    z, y, x = np.meshgrid(a, a, a, indexing="ij")
    return (np.ascontiguousarray(x.reshape(-1)),
            np.ascontiguousarray(y.reshape(-1)),
            np.ascontiguousarray(z.reshape(-1)))


def grid_axis_of(L: int) -> tuple[float, ...]:
    """(x0, dx, y0, dy, z0, dz) of the L^3 grid grid_coords(L) lays out."""
    return (-0.5, 1.0 / L) * 3


def coords_from_axis(nx: int, ny: int, nz: int, axis) -> tuple[np.ndarray, ...]:
    """fp32 x, y, z of an nx x ny x nz grid given (x0, dx, y0, dy, z0, dz):
    coordinate c0 + i d in double from the fp32 c0 and d, rounded once to
    fp32; voxel n = ix + nx*(iy + ny*iz)."""
    a = [float(np.float32(v)) for v in axis]
    ax = (a[0] + np.arange(nx, dtype=np.float64) * a[1]).astype(F32)
    ay = (a[2] + np.arange(ny, dtype=np.float64) * a[3]).astype(F32)
    az = (a[4] + np.arange(nz, dtype=np.float64) * a[5]).astype(F32)
    z, y, x = np.meshgrid(az, ay, ax, indexing="ij")
    return (np.ascontiguousarray(x.reshape(-1)), np.ascontiguousarray(y.reshape(-1)),
            np.ascontiguousarray(z.reshape(-1)))


def grid_index(n: np.ndarray, L: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(ix, iy, iz) of voxel indices n on an L^3 grid."""
    n = np.asarray(n, dtype=np.int64)
    return n % L, (n // L) % L, n // (L * L)


# --------------------------------------------------------------------------
# trajectories
# --------------------------------------------------------------------------
def stack_of_spirals(kz_planes: np.ndarray, interleaves: int, samples: int,
                     rmax: float, turns: float) -> tuple[np.ndarray, ...]:
    """Planar Archimedean spirals stacked along kz (fp64).

    Sample m = (p*J + j)*S + s of plane p, interleave j < J, sample s < S has
    t = s/S, radius r = rmax*t, angle theta = 2*pi*(turns*t + j/J) and
    (kx, ky, kz) = (r cos theta, r sin theta, kz_planes[p]).
    """
    P, J, S = len(kz_planes), interleaves, samples
    t = np.arange(S, dtype=np.float64) / S
    j = np.arange(J, dtype=np.float64)
    theta = 2.0 * np.pi * (turns * t[None, :] + j[:, None] / J)   # (J, S)
    r = rmax * t[None, :]
    kx = np.broadcast_to(r * np.cos(theta), (P, J, S)).reshape(-1)
    ky = np.broadcast_to(r * np.sin(theta), (P, J, S)).reshape(-1)
    kz = np.broadcast_to(np.asarray(kz_planes, np.float64)[:, None, None],
                         (P, J, S)).reshape(-1)
    return kx.copy(), ky.copy(), kz.copy()


def fibonacci_directions(count: int) -> np.ndarray:
    """Golden-angle (Fibonacci-sphere) unit vectors, shape (count, 3), fp64.

    Direction i has z = 1 - (2i+1)/count, radius sqrt(1 - z^2) in the xy
    plane and azimuth i*pi*(3 - sqrt(5)).
    """
    i = np.arange(count, dtype=np.float64)
    zc = 1.0 - (2.0 * i + 1.0) / count
    rc = np.sqrt(1.0 - zc * zc)
    phi = i * np.pi * (3.0 - math.sqrt(5.0))
    return np.stack([rc * np.cos(phi), rc * np.sin(phi), zc], axis=1)


def kooshball(spokes: int, samples: int, r0: float, dr: float):
    """3-D radial trajectory: sample m = spoke*S + s at radius r0 + dr*s."""
    d = fibonacci_directions(spokes)                       # (spokes, 3)
    r = r0 + dr * np.arange(samples, dtype=np.float64)     # (S,)
    k = d[:, None, :] * r[None, :, None]                   # (spokes, S, 3)
    k = k.reshape(-1, 3)
    return k[:, 0].copy(), k[:, 1].copy(), k[:, 2].copy()


def gaussian_blob_kspace(kx, ky, kz, amp, centre, sigma):
    """Analytic Fourier transform (forward sign, e^{-i 2 pi k.x}) of a sum of
    isotropic Gaussian blobs A*exp(-|x - c|^2 / (2 sigma^2)), fp64 complex.

    Each blob contributes A (2 pi sigma^2)^{3/2} exp(-2 pi^2 sigma^2 |k|^2)
    exp(-i 2 pi k.c). This only synthesises k-space data; it is not F^H D.
    """
    k2 = kx * kx + ky * ky + kz * kz
    out = np.zeros(kx.shape, np.complex128)
    for a, c, s in zip(amp, centre, sigma):
        env = a * (2.0 * np.pi * s * s) ** 1.5 * np.exp(-2.0 * np.pi ** 2 * s * s * k2)
        out += env * np.exp(-2j * np.pi * (kx * c[0] + ky * c[1] + kz * c[2]))
    return out


# --------------------------------------------------------------------------
# named workloads
# --------------------------------------------------------------------------
def _f32(*arrays):
    return tuple(np.ascontiguousarray(np.asarray(a, np.float64).astype(F32))
                 for a in arrays)


def make_kspace(name: str) -> dict:
    """k-space of a named workload: fp32 kx, ky, kz, Dr, Di (length M)."""
    w = WORKLOADS[name]
    rng = np.random.default_rng(w.seed)
    if name == "random16":
        kx = rng.uniform(-8.0, 8.0, w.M)
        ky = rng.uniform(-8.0, 8.0, w.M)
        kz = rng.uniform(-8.0, 8.0, w.M)
        D = rng.standard_normal(w.M) + 1j * rng.standard_normal(w.M)
    elif name == "spiral32":
        kx, ky, kz = stack_of_spirals(np.arange(-16, 16, 2, dtype=np.float64),
                                      4, 256, 16.0, 8.0)
        D = rng.standard_normal(w.M) + 1j * rng.standard_normal(w.M)
    elif name == "radial64":
        kx, ky, kz = kooshball(256, 256, -32.0, 0.25)
        amp = rng.uniform(0.5, 1.0, 10)
        centre = rng.uniform(-0.3, 0.3, (10, 3))
        sigma = rng.uniform(0.02, 0.08, 10)
        D = gaussian_blob_kspace(kx, ky, kz, amp, centre, sigma)
    elif name == "spiral128":
        kx, ky, kz = stack_of_spirals(-64.0 + 5.12 * np.arange(25, dtype=np.float64),
                                      8, 500, 64.0, 16.0)
        D = rng.standard_normal(w.M) + 1j * rng.standard_normal(w.M)
    elif name == "vdrandom256":
        u = rng.uniform(-1.0, 1.0, (3, w.M))
        k = 128.0 * u * np.abs(u)
        kx, ky, kz = k[0], k[1], k[2]
        D = rng.standard_normal(w.M) + 1j * rng.standard_normal(w.M)
    else:  # pragma: no cover - WORKLOADS lookup above already raised
        raise KeyError(name)
    kx, ky, kz, Dr, Di = _f32(kx, ky, kz, D.real, D.imag)
    assert kx.shape == (w.M,)
    return dict(kx=kx, ky=ky, kz=kz, Dr=Dr, Di=Di)


def make_workload(name: str) -> dict:
    """All fp32 inputs of a named workload: k-space and its voxel grid."""
    w = WORKLOADS[name]
    out = make_kspace(name)
    out["x"], out["y"], out["z"] = grid_coords(w.L)
    out["M"], out["N"], out["L"] = w.M, w.N, w.L
    return out


def voxel_subset(N: int, count: int = SUBSET_SIZE, seed: int = SUBSET_SEED) -> np.ndarray:
    """Sorted seeded subset of voxel indices (without replacement)."""
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(N, size=min(count, N), replace=False)).astype(np.int64)


# --------------------------------------------------------------------------
# small seeded cases for tests
# --------------------------------------------------------------------------
def random_case(N: int, M: int, seed: int, kmax: float = 8.0) -> dict:
    """Off-grid case: voxels U[-0.5,0.5)^3, k U[-kmax,kmax)^3, D ~ CN(0,1)."""
    rng = np.random.default_rng(seed)
    x, y, z = (rng.uniform(-0.5, 0.5, N) for _ in range(3))
    kx, ky, kz = (rng.uniform(-kmax, kmax, M) for _ in range(3))
    Dr, Di = rng.standard_normal(M), rng.standard_normal(M)
    kx, ky, kz, Dr, Di, x, y, z = _f32(kx, ky, kz, Dr, Di, x, y, z)
    return dict(kx=kx, ky=ky, kz=kz, Dr=Dr, Di=Di, x=x, y=y, z=z, M=M, N=N)


def cartesian_kgrid(L: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Integer k-space grid {-L/2, ..., L/2-1}^3 in fp32, kx fastest (M = L^3)."""
    a = (np.arange(L, dtype=np.float64) - L // 2).astype(F32)
    kz, ky, kx = np.meshgrid(a, a, a, indexing="ij")
    return (np.ascontiguousarray(kx.reshape(-1)), np.ascontiguousarray(ky.reshape(-1)),
            np.ascontiguousarray(kz.reshape(-1)))


def cartesian_case(L: int, seed: int) -> dict:
    """Full integer Cartesian k-grid over an L^3 voxel grid, D ~ CN(0,1)."""
    rng = np.random.default_rng(seed)
    kx, ky, kz = cartesian_kgrid(L)
    M = kx.size
    Dr, Di = _f32(rng.standard_normal(M), rng.standard_normal(M))
    x, y, z = grid_coords(L)
    return dict(kx=kx, ky=ky, kz=kz, Dr=Dr, Di=Di, x=x, y=y, z=z, M=M, N=L ** 3, L=L)


def random_image(N: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Seeded complex image, Re and Im i.i.d. N(0,1), as fp32 (re, im)."""
    rng = np.random.default_rng(seed)
    re, im = _f32(rng.standard_normal(N), rng.standard_normal(N))
    return re, im
