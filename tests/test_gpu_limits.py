"""The largest sizes the C ABI accepts (N or M = 2^31 - 1), on the GPU.

Inputs are drawn on the device (seeded) so the host never holds them; the
fp64 oracle checks seeded outputs, always including the first and last
one, so 64-bit indexing and the grid's last workgroup are covered.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
from non_cartesian_mri_fhd_amd import binding, build

from test_gpu_parity import check

pytestmark = pytest.mark.gpu

INT32_MAX = 2 ** 31 - 1


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    build.ensure_built()
    binding.load()
    return torch.device("cuda:0")


def _uniform(n, lo, hi, gen, dev):
    return torch.rand(n, generator=gen, device=dev, dtype=torch.float32) * (hi - lo) + lo


def _picks(n, count, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, count)]))


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def test_adjoint_at_max_voxels(dev):
    """F^H D with N = 2^31 - 1 voxels (5 x 8.6 GB of coordinates and
    output) and a handful of samples."""
    N, M = INT32_MAX, 9
    gen = torch.Generator(device=dev)
    gen.manual_seed(91)
    x, y, z = (_uniform(N, -0.5, 0.5, gen, dev) for _ in range(3))
    rng = np.random.default_rng(92)
    k = [rng.uniform(-20, 20, M).astype(np.float32) for _ in range(3)]
    D = [rng.standard_normal(M).astype(np.float32) for _ in range(2)]
    kt = [torch.from_numpy(a).to(dev) for a in k + D]
    rr, ri = binding.fhd_compute(*kt, x, y, z)
    torch.cuda.synchronize(dev)
    idx = _picks(N, 62, 93)
    it = torch.from_numpy(idx).to(dev)
    xs, ys, zs = (a[it].cpu().numpy() for a in (x, y, z))
    got_r, got_i = rr[it].cpu().numpy(), ri[it].cpu().numpy()
    del x, y, z, rr, ri
    _free()
    ref = oracle.fhd(*k, *D, xs, ys, zs)
    check("F^H D at N = 2^31 - 1", got_r, got_i, *ref)


def test_forward_at_max_samples(dev):
    """F with M = 2^31 - 1 samples and a few voxels."""
    N, M = 17, INT32_MAX
    gen = torch.Generator(device=dev)
    gen.manual_seed(94)
    kx, ky, kz = (_uniform(M, -32.0, 32.0, gen, dev) for _ in range(3))
    rng = np.random.default_rng(95)
    xyz = [rng.uniform(-0.5, 0.5, N).astype(np.float32) for _ in range(3)]
    img = [rng.standard_normal(N).astype(np.float32) for _ in range(2)]
    t = [torch.from_numpy(a).to(dev) for a in xyz + img]
    Dr, Di = binding.fhd_forward(kx, ky, kz, *t)
    torch.cuda.synchronize(dev)
    idx = _picks(M, 62, 96)
    it = torch.from_numpy(idx).to(dev)
    ks = [a[it].cpu().numpy() for a in (kx, ky, kz)]
    got_r, got_i = Dr[it].cpu().numpy(), Di[it].cpu().numpy()
    del kx, ky, kz, Dr, Di
    _free()
    ref = oracle.forward(*ks, *img, *xyz)
    check("F at M = 2^31 - 1", got_r, got_i, *ref)


@pytest.mark.parametrize("precision", [binding.FHD_GRID_FP32, binding.FHD_GRID_BF16X3])
def test_grid_at_max_voxels(dev, precision):
    """The grid form on 2,047 x 1,024 x 1,024 = 2^31 - 2^20 voxels (one
    sample stage, so no split partials)."""
    from non_cartesian_mri_fhd_amd import inputs
    shape = (2047, 1024, 1024)
    N = int(np.prod(shape))
    assert N <= INT32_MAX
    axis = (-0.5, 1.0 / 2048, -0.5, 1.0 / 1024, -0.5, 1.0 / 1024)
    rng = np.random.default_rng(97)
    M = 300
    k = [rng.uniform(-40, 40, M).astype(np.float32) for _ in range(3)]
    D = [rng.standard_normal(M).astype(np.float32) for _ in range(2)]
    kt = [torch.from_numpy(a).to(dev) for a in k + D]
    rr, ri = binding.fhd_compute_grid(*kt, shape, axis, precision=precision)
    torch.cuda.synchronize(dev)
    idx = _picks(N, 62, 98)
    it = torch.from_numpy(idx).to(dev)
    got_r, got_i = rr[it].cpu().numpy(), ri[it].cpu().numpy()
    del rr, ri
    _free()
    ix, iyz = idx % shape[0], idx // shape[0]
    iy, iz = iyz % shape[1], iyz // shape[1]
    a = [float(np.float32(v)) for v in axis]
    xs = (a[0] + ix * a[1]).astype(np.float32)
    ys = (a[2] + iy * a[3]).astype(np.float32)
    zs = (a[4] + iz * a[5]).astype(np.float32)
    ref = oracle.fhd(*k, *D, xs, ys, zs)
    check("grid at N = 2^31 - 2^20, precision %d" % precision, got_r, got_i, *ref)
