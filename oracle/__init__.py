"""fp64 CPU oracle for F^H D and its forward operator F.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check in
``__graft_entry__.py`` and by the CPU-baseline leg of ``bench.py``. The GPU
library and its Python binding never import it, and it shares no code with
them. The arithmetic lives in ``fhd_oracle.c`` (plain C, double precision,
libm sin/cos); this module only compiles and calls it.

Definitions (page "Case study -- iterative MRI reconstruction", section 17.3
F^H D equation, and section 17.2 for F as the image-to-k-space operator):

    F^H D :  rho_n = sum_m D_m  exp(+i 2 pi k_m . x_n)
    F rho :  D_m   = sum_n rho_n exp(-i 2 pi k_m . x_n)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "fhd_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]

_lock = threading.Lock()
_lib = None


def build(source: str = SOURCE, output: str = LIBRARY, extra: list | None = None) -> str:
    """Compile the oracle with gcc into ``output``; returns the path."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *(extra or []), "-o", tmp, source, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, output)
    return output


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    dp = ctypes.POINTER(ctypes.c_double)
    for name in ("oracle_fhd", "oracle_forward"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [dp] * 10 + [ctypes.c_long, ctypes.c_long, ctypes.c_int]
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if absent or stale) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            stale = (not os.path.exists(LIBRARY)
                     or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE))
            if stale:
                build()
            _lib = _bind(ctypes.CDLL(LIBRARY))
        return _lib


def default_threads() -> int:
    """Host threads the oracle uses: the affinity set, capped at 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _d(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def fhd(kx, ky, kz, Dr, Di, x, y, z, threads: int | None = None, lib=None):
    """rho = F^H D in fp64. Inputs of any real dtype are widened exactly.

    Returns (rho_r, rho_i), float64 arrays of length N = len(x).
    """
    kx, ky, kz, Dr, Di, x, y, z = map(_d, (kx, ky, kz, Dr, Di, x, y, z))
    M, N = kx.size, x.size
    if not (ky.size == kz.size == Dr.size == Di.size == M and y.size == z.size == N):
        raise ValueError("inconsistent lengths")
    rr, ri = np.zeros(N), np.zeros(N)
    lib = lib or load()
    rc = lib.oracle_fhd(*map(_ptr, (kx, ky, kz, Dr, Di, x, y, z, rr, ri)), M, N,
                        threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_fhd failed (%d)" % rc)
    return rr, ri


def forward(kx, ky, kz, rho_r, rho_i, x, y, z, threads: int | None = None, lib=None):
    """D = F rho in fp64. Returns (Dr, Di), float64 arrays of length M."""
    kx, ky, kz, rho_r, rho_i, x, y, z = map(_d, (kx, ky, kz, rho_r, rho_i, x, y, z))
    M, N = kx.size, x.size
    if not (ky.size == kz.size == M and rho_r.size == rho_i.size == y.size == z.size == N):
        raise ValueError("inconsistent lengths")
    Dr, Di = np.zeros(M), np.zeros(M)
    lib = lib or load()
    rc = lib.oracle_forward(*map(_ptr, (kx, ky, kz, rho_r, rho_i, x, y, z, Dr, Di)), M, N,
                            threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_forward failed (%d)" % rc)
    return Dr, Di


def fhd_subset(inputs: dict, voxels, threads: int | None = None):
    """F^H D of a workload dict restricted to the given voxel indices."""
    idx = np.asarray(voxels, dtype=np.int64)
    return fhd(inputs["kx"], inputs["ky"], inputs["kz"], inputs["Dr"], inputs["Di"],
               inputs["x"][idx], inputs["y"][idx], inputs["z"][idx], threads=threads)


def cg(kx, ky, kz, Dr, Di, x, y, z, iters: int, tol: float = 0.0, threads: int | None = None):
    """fp64 conjugate gradients on F^H F rho = F^H D from rho = 0.

    The loop the page "Case study -- iterative MRI reconstruction" sketches
    after section 17.3.6, without its unspecified regulariser, applied with
    this module's own F^H (fhd) and F (forward). Inner products are
    Re sum conj(u) v. Stops after `iters` iterations or once ||r||^2 < tol.
    Returns (rho complex128, residuals list of ||r_k||^2 for k = 0..done).
    """
    X = (np.asarray(x, np.float64), np.asarray(y, np.float64), np.asarray(z, np.float64))
    K = (np.asarray(kx, np.float64), np.asarray(ky, np.float64), np.asarray(kz, np.float64))

    def normal_op(v):
        fr, fi = forward(*K, v.real, v.imag, *X, threads=threads)
        hr, hi = fhd(*K, fr, fi, *X, threads=threads)
        return hr + 1j * hi

    br, bi = fhd(*K, Dr, Di, *X, threads=threads)
    r = br + 1j * bi
    rho = np.zeros_like(r)
    p = r.copy()
    rs = float(np.vdot(r, r).real)
    residuals = [rs]
    for _ in range(iters):
        if not rs > 0.0 or rs < tol:
            break
        ap = normal_op(p)
        pap = float(np.vdot(p, ap).real)
        if not pap > 0.0:
            break
        alpha = rs / pap
        rho = rho + alpha * p
        r = r - alpha * ap
        rs_new = float(np.vdot(r, r).real)
        residuals.append(rs_new)
        if rs_new < tol:
            break
        p = r + (rs_new / rs) * p
        rs = rs_new
    return rho, residuals
