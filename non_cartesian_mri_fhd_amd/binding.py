"""Python binding of libfhd.so (the C ABI in include/fhd.h).

Argument marshalling only: every step of F^H D runs in the library's HIP
kernels. torch supplies device memory and the current stream. There is no
CPU fallback: if the library is missing or a tensor is not on the GPU, the
call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from .build import lib_path

FHD_OK = 0
FHD_ERR_INVALID_ARG = -1
FHD_ERR_HIP = -2
FHD_ERR_ALLOC = -3
FHD_GRID_FP32 = 0
FHD_GRID_BF16X3 = 1
FHD_GATHER_ALL = 0
FHD_GATHER_VECTOR = 1
FHD_GATHER_BF16X3 = 2

LIBRARY = lib_path("libfhd.so")

_lock = threading.Lock()
_lib = None


class FhdError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__("%s failed: status %d (%s)" % (where, status, message))
        self.status = status


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libfhd.so; raises FileNotFoundError if it has not been built."""
    global _lib
    with _lock:
        if _lib is None or path is not None:
            p = path or LIBRARY
            if not os.path.exists(p):
                raise FileNotFoundError(
                    "%s is not built; run __graft_entry__.build() or "
                    "python -m non_cartesian_mri_fhd_amd.build" % p)
            lib = ctypes.CDLL(p)
            _declare(lib)
            if path is not None:
                return lib
            _lib = lib
        return _lib


def _declare(lib: ctypes.CDLL) -> None:
    fp, vp, i32, i64 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.fhd_compute.argtypes = [fp] * 10 + [i32, i32, vp]
    lib.fhd_compute.restype = i32
    lib.fhd_compute_paths.argtypes = [fp] * 10 + [i32, i32, i32, vp]
    lib.fhd_compute_paths.restype = i32
    lib.fhd_compute_noalloc.argtypes = [fp] * 10 + [i32, i32, i32, vp]
    lib.fhd_compute_noalloc.restype = i32
    lib.fhd_scatter.argtypes = [fp] * 10 + [i32, i32, vp]
    lib.fhd_scatter.restype = i32
    lib.fhd_packed_bytes.argtypes = [i32]
    lib.fhd_packed_bytes.restype = i64
    lib.fhd_pack.argtypes = [fp] * 5 + [i32, vp, i64, vp]
    lib.fhd_pack.restype = i32
    lib.fhd_gather.argtypes = [vp, i32] + [fp] * 5 + [i32, vp]
    lib.fhd_gather.restype = i32
    lib.fhd_gather_paths.argtypes = [vp, i32] + [fp] * 5 + [i32, i32, vp]
    lib.fhd_gather_paths.restype = i32
    lib.fhd_forward.argtypes = [fp] * 10 + [i32, i32, vp]
    lib.fhd_forward.restype = i32
    lib.fhd_forward_paths.argtypes = [fp] * 10 + [i32, i32, i32, vp]
    lib.fhd_forward_paths.restype = i32
    lib.fhd_forward_pack.argtypes = [fp] * 5 + [i32, vp, i64, vp]
    lib.fhd_forward_pack.restype = i32
    lib.fhd_forward_gather.argtypes = [vp, i32] + [fp] * 5 + [i32, vp]
    lib.fhd_forward_gather.restype = i32
    lib.fhd_normal.argtypes = [fp] * 10 + [i32, i32, vp]
    lib.fhd_normal.restype = i32
    lib.fhd_normal_paths.argtypes = [fp] * 10 + [i32, i32, i32, vp]
    lib.fhd_normal_paths.restype = i32
    lib.fhd_cg.argtypes = [fp] * 10 + [i32, i32, i32, ctypes.c_float,
                                       ctypes.POINTER(ctypes.c_int), ctypes.c_void_p, vp]
    lib.fhd_cg.restype = i32
    lib.fhd_cg_paths.argtypes = [fp] * 10 + [i32, i32, i32, ctypes.c_float,
                                             ctypes.POINTER(ctypes.c_int), ctypes.c_void_p, i32, vp]
    lib.fhd_cg_paths.restype = i32
    lib.fhd_cg_workspace_bytes.argtypes = [i32, i32, i32]
    lib.fhd_cg_workspace_bytes.restype = i64
    fpp = ctypes.POINTER(ctypes.c_float)
    lib.fhd_compute_grid.argtypes = [fp] * 5 + [i32] * 4 + [fpp, i32, fp, fp, vp]
    lib.fhd_compute_grid.restype = i32
    lib.fhd_grid_gather.argtypes = [vp] + [i32] * 4 + [fpp, i32, fp, fp, vp]
    lib.fhd_grid_gather.restype = i32
    lib.fhd_forward_grid.argtypes = [fp] * 3 + [i32] * 4 + [fpp, i32, fp, fp, fp, fp, vp]
    lib.fhd_forward_grid.restype = i32
    lib.fhd_normal_grid.argtypes = [fp] * 3 + [i32] * 4 + [fpp, i32, fp, fp, fp, fp, vp]
    lib.fhd_normal_grid.restype = i32
    lib.fhd_cg_grid.argtypes = ([fp] * 5 + [i32] * 4 + [fpp, i32, fp, fp, i32, ctypes.c_float,
                                                      ctypes.POINTER(ctypes.c_int), fp, vp])
    lib.fhd_cg_grid.restype = i32
    lib.fhd_time_kernel.argtypes = [ctypes.c_char_p, ctypes.c_void_p, i32]
    lib.fhd_time_kernel.restype = i32
    lib.fhd_timed_launches.argtypes = []
    lib.fhd_timed_launches.restype = i32
    lib.fhd_gather_config.argtypes = [ctypes.POINTER(ctypes.c_int)] * 3
    lib.fhd_gather_config.restype = None
    lib.fhd_release_workspaces.argtypes = []
    lib.fhd_release_workspaces.restype = i32
    lib.fhd_status_string.argtypes = [i32]
    lib.fhd_status_string.restype = ctypes.c_char_p
    lib.fhd_last_error.argtypes = []
    lib.fhd_last_error.restype = ctypes.c_char_p


def _check(lib, status: int, where: str) -> None:
    if status != FHD_OK:
        msg = lib.fhd_last_error().decode() or lib.fhd_status_string(status).decode()
        raise FhdError(status, where, msg)


def _vec(t: torch.Tensor, name: str, n: int, device) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU, got %s" % (name, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32, got %s" % (name, t.dtype))
    if not t.is_contiguous() or t.dim() != 1 or t.numel() != n:
        raise ValueError("%s must be a contiguous 1-D tensor of %d elements" % (name, n))
    return t.data_ptr() if n > 0 else 0


def _stream(device, stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def gather_config() -> dict:
    lib = load()
    v, u, b = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    lib.fhd_gather_config(ctypes.byref(v), ctypes.byref(u), ctypes.byref(b))
    return dict(voxels_per_lane=v.value, samples_per_chunk=u.value, block_threads=b.value)


def fhd_packed_bytes(M: int) -> int:
    n = load().fhd_packed_bytes(int(M))
    if n < 0:
        raise ValueError("M must be >= 0")
    return int(n)


def fhd_compute(kx, ky, kz, Dr, Di, x, y, z, rho_r=None, rho_i=None, stream=None,
                paths: int | None = None):
    """rho = F^H D; returns (rho_r, rho_i), float32 tensors on x's device.
    paths=None calls fhd_compute; otherwise fhd_compute_paths with it."""
    lib = load()
    M, N = kx.numel(), x.numel()
    dev = x.device
    if rho_r is None:
        rho_r = torch.empty(N, dtype=torch.float32, device=dev)
    if rho_i is None:
        rho_i = torch.empty(N, dtype=torch.float32, device=dev)
    ptrs = [_vec(t, nm, M, dev) for t, nm in ((kx, "kx"), (ky, "ky"), (kz, "kz"),
                                               (Dr, "Dr"), (Di, "Di"))]
    ptrs += [_vec(t, nm, N, dev) for t, nm in ((x, "x"), (y, "y"), (z, "z"),
                                               (rho_r, "rho_r"), (rho_i, "rho_i"))]
    with torch.cuda.device(dev):
        if paths is None:
            _check(lib, lib.fhd_compute(*ptrs, M, N, _stream(dev, stream)), "fhd_compute")
        else:
            _check(lib, lib.fhd_compute_paths(*ptrs, M, N, int(paths), _stream(dev, stream)),
                   "fhd_compute_paths")
    return rho_r, rho_i


def fhd_release_workspaces() -> None:
    """Free the device buffers the library keeps per stream between calls."""
    lib = load()
    _check(lib, lib.fhd_release_workspaces(), "fhd_release_workspaces")


def fhd_compute_noalloc(kx, ky, kz, Dr, Di, x, y, z, rho_r, rho_i, stream=None,
                        paths: int = FHD_GATHER_ALL):
    """rho = F^H D with no allocation in the library (its static per-GPU
    scratch array holds every temporary); rho_r and rho_i are the caller's
    float32 tensors. Calls that overlap on one GPU race."""
    lib = load()
    M, N = kx.numel(), x.numel()
    dev = x.device
    ptrs = [_vec(t, nm, M, dev) for t, nm in ((kx, "kx"), (ky, "ky"), (kz, "kz"),
                                               (Dr, "Dr"), (Di, "Di"))]
    ptrs += [_vec(t, nm, N, dev) for t, nm in ((x, "x"), (y, "y"), (z, "z"),
                                               (rho_r, "rho_r"), (rho_i, "rho_i"))]
    with torch.cuda.device(dev):
        _check(lib, lib.fhd_compute_noalloc(*ptrs, M, N, int(paths), _stream(dev, stream)),
               "fhd_compute_noalloc")
    return rho_r, rho_i


def fhd_scatter(kx, ky, kz, Dr, Di, x, y, z, rho_r=None, rho_i=None, stream=None):
    """rho = F^H D in the scatter form (a lane per sample, atomic adds into
    rho); the same contract as fhd_compute. Returns (rho_r, rho_i)."""
    lib = load()
    M, N = kx.numel(), x.numel()
    dev = x.device
    if rho_r is None:
        rho_r = torch.empty(N, dtype=torch.float32, device=dev)
    if rho_i is None:
        rho_i = torch.empty(N, dtype=torch.float32, device=dev)
    ptrs = [_vec(t, nm, M, dev) for t, nm in ((kx, "kx"), (ky, "ky"), (kz, "kz"),
                                               (Dr, "Dr"), (Di, "Di"))]
    ptrs += [_vec(t, nm, N, dev) for t, nm in ((x, "x"), (y, "y"), (z, "z"),
                                               (rho_r, "rho_r"), (rho_i, "rho_i"))]
    with torch.cuda.device(dev):
        _check(lib, lib.fhd_scatter(*ptrs, M, N, _stream(dev, stream)), "fhd_scatter")
    return rho_r, rho_i


def fhd_pack(kx, ky, kz, Dr, Di, packed: torch.Tensor, stream=None) -> torch.Tensor:
    """Pre-pass into ``packed`` (a uint8 or float32 device tensor)."""
    lib = load()
    M = kx.numel()
    dev = packed.device
    ptrs = [_vec(t, nm, M, dev) for t, nm in ((kx, "kx"), (ky, "ky"), (kz, "kz"),
                                               (Dr, "Dr"), (Di, "Di"))]
    if packed.device.type != "cuda" or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous GPU tensor")
    nbytes = packed.numel() * packed.element_size()
    with torch.cuda.device(dev):
        _check(lib, lib.fhd_pack(*ptrs, M, packed.data_ptr(), nbytes, _stream(dev, stream)),
               "fhd_pack")
    return packed


def fhd_gather(packed: torch.Tensor, M: int, x, y, z, rho_r=None, rho_i=None, stream=None,
               paths: int | None = None):
    """Gather over a packed k-space of M samples; returns (rho_r, rho_i).
    paths=None calls fhd_gather; FHD_GATHER_ALL, FHD_GATHER_VECTOR or
    FHD_GATHER_BF16X3 calls fhd_gather_paths with it."""
    lib = load()
    N = x.numel()
    dev = x.device
    if rho_r is None:
        rho_r = torch.empty(N, dtype=torch.float32, device=dev)
    if rho_i is None:
        rho_i = torch.empty(N, dtype=torch.float32, device=dev)
    if packed.device != dev or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous tensor on %s" % dev)
    if packed.numel() * packed.element_size() < (fhd_packed_bytes(M) if M > 0 else 0):
        raise ValueError("packed is smaller than fhd_packed_bytes(M)")
    ptrs = [_vec(t, nm, N, dev) for t, nm in ((x, "x"), (y, "y"), (z, "z"),
                                               (rho_r, "rho_r"), (rho_i, "rho_i"))]
    with torch.cuda.device(dev):
        if paths is None:
            _check(lib, lib.fhd_gather(packed.data_ptr(), int(M), *ptrs, N, _stream(dev, stream)),
                   "fhd_gather")
        else:
            _check(lib, lib.fhd_gather_paths(packed.data_ptr(), int(M), *ptrs, N, int(paths),
                                             _stream(dev, stream)), "fhd_gather_paths")
    return rho_r, rho_i


def fhd_forward(kx, ky, kz, x, y, z, rho_r, rho_i, Dr=None, Di=None, stream=None,
                paths: int | None = None):
    """D = F rho; returns (Dr, Di), float32 tensors on kx's device.
    paths=None calls fhd_forward; otherwise fhd_forward_paths with it."""
    lib = load()
    M, N = kx.numel(), x.numel()
    dev = kx.device
    if Dr is None:
        Dr = torch.empty(M, dtype=torch.float32, device=dev)
    if Di is None:
        Di = torch.empty(M, dtype=torch.float32, device=dev)
    ptrs = [_vec(t, nm, M, dev) for t, nm in ((kx, "kx"), (ky, "ky"), (kz, "kz"))]
    ptrs += [_vec(t, nm, N, dev) for t, nm in ((x, "x"), (y, "y"), (z, "z"),
                                               (rho_r, "rho_r"), (rho_i, "rho_i"))]
    ptrs += [_vec(t, nm, M, dev) for t, nm in ((Dr, "Dr"), (Di, "Di"))]
    with torch.cuda.device(dev):
        if paths is None:
            _check(lib, lib.fhd_forward(*ptrs, M, N, _stream(dev, stream)), "fhd_forward")
        else:
            _check(lib, lib.fhd_forward_paths(*ptrs, M, N, int(paths), _stream(dev, stream)),
                   "fhd_forward_paths")
    return Dr, Di


def fhd_forward_pack(x, y, z, rho_r, rho_i, packed: torch.Tensor, stream=None) -> torch.Tensor:
    """Pre-pass of F into ``packed`` (fhd_packed_bytes(N) bytes)."""
    lib = load()
    N = x.numel()
    dev = packed.device
    ptrs = [_vec(t, nm, N, dev) for t, nm in ((x, "x"), (y, "y"), (z, "z"),
                                               (rho_r, "rho_r"), (rho_i, "rho_i"))]
    if packed.device.type != "cuda" or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous GPU tensor")
    nbytes = packed.numel() * packed.element_size()
    with torch.cuda.device(dev):
        _check(lib, lib.fhd_forward_pack(*ptrs, N, packed.data_ptr(), nbytes,
                                         _stream(dev, stream)), "fhd_forward_pack")
    return packed


def fhd_forward_gather(packed: torch.Tensor, N: int, kx, ky, kz, Dr=None, Di=None, stream=None):
    """Gather of F over packed voxels; returns (Dr, Di)."""
    lib = load()
    M = kx.numel()
    dev = kx.device
    if Dr is None:
        Dr = torch.empty(M, dtype=torch.float32, device=dev)
    if Di is None:
        Di = torch.empty(M, dtype=torch.float32, device=dev)
    if packed.device != dev or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous tensor on %s" % dev)
    if packed.numel() * packed.element_size() < (fhd_packed_bytes(N) if N > 0 else 0):
        raise ValueError("packed is smaller than fhd_packed_bytes(N)")
    ptrs = [_vec(t, nm, M, dev) for t, nm in ((kx, "kx"), (ky, "ky"), (kz, "kz"),
                                               (Dr, "Dr"), (Di, "Di"))]
    with torch.cuda.device(dev):
        _check(lib, lib.fhd_forward_gather(packed.data_ptr(), int(N), *ptrs, M,
                                           _stream(dev, stream)), "fhd_forward_gather")
    return Dr, Di


def fhd_normal(kx, ky, kz, x, y, z, p_r, p_i, q_r=None, q_i=None, stream=None,
               paths: int | None = None):
    """q = F^H F p; returns (q_r, q_i), float32 tensors on x's device.
    paths=None calls fhd_normal; otherwise fhd_normal_paths with it."""
    lib = load()
    M, N = kx.numel(), x.numel()
    dev = x.device
    if q_r is None:
        q_r = torch.empty(N, dtype=torch.float32, device=dev)
    if q_i is None:
        q_i = torch.empty(N, dtype=torch.float32, device=dev)
    ptrs = [_vec(t, nm, M, dev) for t, nm in ((kx, "kx"), (ky, "ky"), (kz, "kz"))]
    ptrs += [_vec(t, nm, N, dev) for t, nm in ((x, "x"), (y, "y"), (z, "z"), (p_r, "p_r"),
                                               (p_i, "p_i"), (q_r, "q_r"), (q_i, "q_i"))]
    with torch.cuda.device(dev):
        if paths is None:
            _check(lib, lib.fhd_normal(*ptrs, M, N, _stream(dev, stream)), "fhd_normal")
        else:
            _check(lib, lib.fhd_normal_paths(*ptrs, M, N, int(paths), _stream(dev, stream)),
                   "fhd_normal_paths")
    return q_r, q_i


def fhd_cg(kx, ky, kz, Dr, Di, x, y, z, max_iter: int, tol: float = 0.0,
           rho_r=None, rho_i=None, stream=None, paths: int | None = None):
    """CG on F^H F rho = F^H D from rho = 0 (synchronises the stream).

    Returns (rho_r, rho_i, iterations, residuals) with residuals the numpy
    array of squared residual norms ||r_k||^2, k = 0..iterations.
    paths=None calls fhd_cg; otherwise fhd_cg_paths with it.
    """
    import numpy as np
    lib = load()
    M, N = kx.numel(), x.numel()
    dev = x.device
    if rho_r is None:
        rho_r = torch.empty(N, dtype=torch.float32, device=dev)
    if rho_i is None:
        rho_i = torch.empty(N, dtype=torch.float32, device=dev)
    ptrs = [_vec(t, nm, M, dev) for t, nm in ((kx, "kx"), (ky, "ky"), (kz, "kz"),
                                               (Dr, "Dr"), (Di, "Di"))]
    ptrs += [_vec(t, nm, N, dev) for t, nm in ((x, "x"), (y, "y"), (z, "z"),
                                               (rho_r, "rho_r"), (rho_i, "rho_i"))]
    res = np.zeros(int(max_iter) + 1, dtype=np.float32)
    done = ctypes.c_int(0)
    with torch.cuda.device(dev):
        if paths is None:
            _check(lib, lib.fhd_cg(*ptrs, M, N, int(max_iter), float(tol), ctypes.byref(done),
                                   res.ctypes.data, _stream(dev, stream)), "fhd_cg")
        else:
            _check(lib, lib.fhd_cg_paths(*ptrs, M, N, int(max_iter), float(tol), ctypes.byref(done),
                                         res.ctypes.data, int(paths), _stream(dev, stream)),
                   "fhd_cg_paths")
    return rho_r, rho_i, done.value, res[:done.value + 1].copy()


def _axis(axis):
    a = (ctypes.c_float * 6)(*[float(v) for v in axis])
    if len(axis) != 6:
        raise ValueError("axis must hold x0, dx, y0, dy, z0, dz")
    return a


def fhd_compute_grid(kx, ky, kz, Dr, Di, shape, axis, rho_r=None, rho_i=None, stream=None,
                     precision: int = FHD_GRID_FP32):
    """F^H D on the grid shape = (nx, ny, nz), axis = (x0, dx, y0, dy, z0, dz);
    voxel n = ix + nx*(iy + ny*iz). Returns (rho_r, rho_i) on kx's device."""
    lib = load()
    nx, ny, nz = (int(v) for v in shape)
    M, N = kx.numel(), nx * ny * nz
    dev = kx.device
    if rho_r is None:
        rho_r = torch.empty(N, dtype=torch.float32, device=dev)
    if rho_i is None:
        rho_i = torch.empty(N, dtype=torch.float32, device=dev)
    ptrs = [_vec(t, nm, M, dev) for t, nm in ((kx, "kx"), (ky, "ky"), (kz, "kz"),
                                               (Dr, "Dr"), (Di, "Di"))]
    outs = [_vec(t, nm, N, dev) for t, nm in ((rho_r, "rho_r"), (rho_i, "rho_i"))]
    with torch.cuda.device(dev):
        _check(lib, lib.fhd_compute_grid(*ptrs, M, nx, ny, nz, _axis(axis), int(precision), *outs,
                                         _stream(dev, stream)), "fhd_compute_grid")
    return rho_r, rho_i


def fhd_grid_gather(packed, M: int, shape, axis, rho_r=None, rho_i=None, stream=None,
                    precision: int = FHD_GRID_FP32):
    """Matrix-core gather over k-space packed by fhd_pack; see fhd_compute_grid."""
    lib = load()
    nx, ny, nz = (int(v) for v in shape)
    N = nx * ny * nz
    dev = packed.device
    if rho_r is None:
        rho_r = torch.empty(N, dtype=torch.float32, device=dev)
    if rho_i is None:
        rho_i = torch.empty(N, dtype=torch.float32, device=dev)
    if packed.device.type != "cuda" or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous GPU tensor")
    if packed.numel() * packed.element_size() < (fhd_packed_bytes(M) if M > 0 else 0):
        raise ValueError("packed is smaller than fhd_packed_bytes(M)")
    outs = [_vec(t, nm, N, dev) for t, nm in ((rho_r, "rho_r"), (rho_i, "rho_i"))]
    with torch.cuda.device(dev):
        _check(lib, lib.fhd_grid_gather(packed.data_ptr(), int(M), nx, ny, nz, _axis(axis),
                                        int(precision), *outs, _stream(dev, stream)),
               "fhd_grid_gather")
    return rho_r, rho_i


def fhd_forward_grid(kx, ky, kz, shape, axis, rho_r, rho_i, Dr=None, Di=None, stream=None,
                     precision: int = FHD_GRID_BF16X3):
    """D = F rho for rho on the grid shape = (nx, ny, nz) with axis
    (x0, dx, y0, dy, z0, dz), voxel n = ix + nx*(iy + ny*iz). Returns (Dr, Di)."""
    lib = load()
    nx, ny, nz = (int(v) for v in shape)
    M, N = kx.numel(), nx * ny * nz
    dev = kx.device
    if Dr is None:
        Dr = torch.empty(M, dtype=torch.float32, device=dev)
    if Di is None:
        Di = torch.empty(M, dtype=torch.float32, device=dev)
    ks = [_vec(t, nm, M, dev) for t, nm in ((kx, "kx"), (ky, "ky"), (kz, "kz"))]
    img = [_vec(t, nm, N, dev) for t, nm in ((rho_r, "rho_r"), (rho_i, "rho_i"))]
    outs = [_vec(t, nm, M, dev) for t, nm in ((Dr, "Dr"), (Di, "Di"))]
    with torch.cuda.device(dev):
        _check(lib, lib.fhd_forward_grid(*ks, M, nx, ny, nz, _axis(axis), int(precision), *img, *outs,
                                         _stream(dev, stream)), "fhd_forward_grid")
    return Dr, Di


def fhd_normal_grid(kx, ky, kz, shape, axis, p_r, p_i, q_r=None, q_i=None, stream=None,
                    precision: int = FHD_GRID_BF16X3):
    """q = F^H F p for p on the grid shape = (nx, ny, nz). Returns (q_r, q_i)."""
    lib = load()
    nx, ny, nz = (int(v) for v in shape)
    M, N = kx.numel(), nx * ny * nz
    dev = kx.device
    if q_r is None:
        q_r = torch.empty(N, dtype=torch.float32, device=dev)
    if q_i is None:
        q_i = torch.empty(N, dtype=torch.float32, device=dev)
    ks = [_vec(t, nm, M, dev) for t, nm in ((kx, "kx"), (ky, "ky"), (kz, "kz"))]
    vs = [_vec(t, nm, N, dev) for t, nm in ((p_r, "p_r"), (p_i, "p_i"), (q_r, "q_r"), (q_i, "q_i"))]
    with torch.cuda.device(dev):
        _check(lib, lib.fhd_normal_grid(*ks, M, nx, ny, nz, _axis(axis), int(precision), *vs,
                                        _stream(dev, stream)), "fhd_normal_grid")
    return q_r, q_i


def fhd_cg_grid(kx, ky, kz, Dr, Di, shape, axis, max_iter: int, tol: float = 0.0,
                rho_r=None, rho_i=None, stream=None, precision: int = FHD_GRID_BF16X3):
    """CG on F^H F rho = F^H D with rho on the grid shape = (nx, ny, nz)
    (synchronises the stream). Returns (rho_r, rho_i, iterations, residuals)."""
    import numpy as np
    lib = load()
    nx, ny, nz = (int(v) for v in shape)
    M, N = kx.numel(), nx * ny * nz
    dev = kx.device
    if rho_r is None:
        rho_r = torch.empty(N, dtype=torch.float32, device=dev)
    if rho_i is None:
        rho_i = torch.empty(N, dtype=torch.float32, device=dev)
    ks = [_vec(t, nm, M, dev) for t, nm in ((kx, "kx"), (ky, "ky"), (kz, "kz"), (Dr, "Dr"), (Di, "Di"))]
    outs = [_vec(t, nm, N, dev) for t, nm in ((rho_r, "rho_r"), (rho_i, "rho_i"))]
    done = ctypes.c_int(0)
    res = np.zeros(int(max_iter) + 1, dtype=np.float32)
    with torch.cuda.device(dev):
        _check(lib, lib.fhd_cg_grid(*ks, M, nx, ny, nz, _axis(axis), int(precision), *outs,
                                    int(max_iter), float(tol), ctypes.byref(done), res.ctypes.data,
                                    _stream(dev, stream)), "fhd_cg_grid")
    return rho_r, rho_i, done.value, res[:done.value + 1].copy()


def new_packed(M: int, device) -> torch.Tensor:
    """Device buffer of fhd_packed_bytes(M) bytes for fhd_pack / fhd_gather."""
    return torch.empty(max(fhd_packed_bytes(M), 4), dtype=torch.uint8, device=device)


class KernelTimer:
    """Durations of the next `count` launches of one library kernel, from
    HIP events the library records on the kernel's own stream just before
    and after each launch (fhd_time_kernel). Arm, run the calls, synchronise,
    then read durations_ms(); the hook is thread-local."""

    def __init__(self, kernel: str, count: int, device):
        lib = load()
        self.kernel = kernel
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * count)]
        # torch creates its events lazily: record each once so the handles exist
        s = torch.cuda.current_stream(device)
        for e in self.events:
            e.record(s)
        torch.cuda.synchronize(device)
        handles = (ctypes.c_void_p * max(1, 2 * count))(*[e.cuda_event for e in self.events])
        _check(lib, lib.fhd_time_kernel(kernel.encode(), handles, int(count)), "fhd_time_kernel")

    def durations_ms(self) -> list:
        n = load().fhd_timed_launches()
        return [self.events[2 * i].elapsed_time(self.events[2 * i + 1]) for i in range(n)]

    @staticmethod
    def disarm() -> None:
        load().fhd_time_kernel(None, None, 0)

