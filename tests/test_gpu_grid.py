"""GPU parity of the matrix-core F^H D on a Cartesian voxel grid
(fhd_compute_grid / fhd_grid_gather) against the fp64 oracle, the numpy FFT
on a full integer k-grid, and the direct gather.

The voxel coordinates handed to the oracle are the grid's, built as the
library defines them (c0 + i d in double, rounded once to fp32). Same gate as
the direct path: relative L2 <= 5e-4 and every element within 10x that bound
times the reference's rms magnitude.
"""
import numpy as np
import pytest
import torch

import oracle
from non_cartesian_mri_fhd_amd import binding, build, inputs, metrics

from pins import cartesian_fft_reference
from test_gpu_parity import check

pytestmark = pytest.mark.gpu

ODD_AXIS = (0.3, 0.013, -0.2, 0.021, 0.11, -0.017)
PRECISIONS = [binding.FHD_GRID_FP32, binding.FHD_GRID_BF16X3]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    build.ensure_built()
    binding.load()
    return torch.device("cuda:0")


def t(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gpu_grid(case, shape, axis, dev, out=None, precision=binding.FHD_GRID_FP32):
    k = [t(case[a], dev) for a in ("kx", "ky", "kz", "Dr", "Di")]
    rr, ri = binding.fhd_compute_grid(*k, shape, axis, *(out or (None, None)), precision=precision)
    torch.cuda.synchronize(dev)
    return rr.cpu().numpy(), ri.cpu().numpy()


def oracle_on_grid(case, shape, axis, idx=None):
    x, y, z = inputs.coords_from_axis(*shape, axis)
    if idx is not None:
        x, y, z = x[idx], y[idx], z[idx]
    return oracle.fhd(case["kx"], case["ky"], case["kz"], case["Dr"], case["Di"], x, y, z)


@pytest.mark.parametrize("prec", PRECISIONS)
@pytest.mark.parametrize("name", ["random16", "spiral32"])
def test_grid_workload_all_voxels(dev, name, prec):
    w = inputs.make_workload(name)
    L = inputs.WORKLOADS[name].L
    rr, ri = gpu_grid(w, (L, L, L), inputs.grid_axis_of(L), dev, precision=prec)
    ref = oracle.fhd(w["kx"], w["ky"], w["kz"], w["Dr"], w["Di"], w["x"], w["y"], w["z"])
    check("grid %s precision %d" % (name, prec), rr, ri, *ref)


@pytest.mark.parametrize("prec", PRECISIONS)
@pytest.mark.parametrize("name,count", [("radial64", 8192), ("spiral128", 4096),
                                        ("vdrandom256", inputs.SUBSET_SIZE)])
def test_grid_workload_sampled_voxels(dev, name, count, prec):
    """Full-size run in the benchmark's launch shape; the oracle computes a
    seeded voxel subset."""
    w = inputs.make_workload(name)
    L = inputs.WORKLOADS[name].L
    rr, ri = gpu_grid(w, (L, L, L), inputs.grid_axis_of(L), dev, precision=prec)
    if name == "vdrandom256":
        idx = inputs.voxel_subset(w["N"])
    else:
        idx = inputs.voxel_subset(w["N"], count, seed=inputs.WORKLOADS[name].seed + 1000)
    ref_r, ref_i = oracle.fhd_subset(w, idx)
    check("grid %s precision %d" % (name, prec), rr[idx], ri[idx], ref_r, ref_i)


@pytest.mark.parametrize("prec", PRECISIONS)
@pytest.mark.parametrize("shape,M", [((1, 1, 1), 1), ((70, 5, 27), 1000), ((130, 3, 2), 7),
                                     ((64, 128, 1), 4097), ((33, 17, 9), 513),
                                     ((7, 129, 2), 2049), ((1, 300, 1), 64), ((40, 6, 5), 520),
                                     ((40, 6, 5), 1016)])
def test_grid_ragged(dev, shape, M, prec):
    """Grids whose edges cut the 64-column and 128-row tiles, sample counts
    off the 8-sample chunk and 512-sample stage, non-dyadic axis steps of
    either sign."""
    c = inputs.random_case(1, M, seed=M + shape[0])
    rr, ri = gpu_grid(c, shape, ODD_AXIS, dev, precision=prec)
    check("grid ragged %s M=%d precision %d" % (shape, M, prec), rr, ri,
          *oracle_on_grid(c, shape, ODD_AXIS))


@pytest.mark.parametrize("prec", PRECISIONS)
def test_grid_one_round_no_split(dev, prec):
    """768 workgroups and 2 stages: the unsplit launch (one full round)."""
    shape, M = (64, 384, 256), 600
    c = inputs.random_case(1, M, seed=77)
    rr, ri = gpu_grid(c, shape, ODD_AXIS, dev, precision=prec)
    idx = inputs.voxel_subset(int(np.prod(shape)), 2048, seed=78)
    check("grid unsplit", rr[idx], ri[idx], *oracle_on_grid(c, shape, ODD_AXIS, idx))


@pytest.mark.parametrize("prec", PRECISIONS)
@pytest.mark.parametrize("L", [16, 32])
def test_grid_cartesian_matches_fft(dev, L, prec):
    c = inputs.cartesian_case(L, seed=500 + L)
    rr, ri = gpu_grid(c, (L, L, L), inputs.grid_axis_of(L), dev, precision=prec)
    ref = cartesian_fft_reference(c)
    check("grid cartesian L=%d precision %d" % (L, prec), rr, ri, ref.real, ref.imag)


@pytest.mark.parametrize("prec", PRECISIONS)
def test_grid_no_samples_writes_zeros(dev, prec):
    shape = (40, 9, 3)
    N = int(np.prod(shape))
    out = (torch.full((N,), 7.0, device=dev), torch.full((N,), -7.0, device=dev))
    e = np.zeros(0, np.float32)
    case = dict(kx=e, ky=e, kz=e, Dr=e, Di=e)
    rr, ri = gpu_grid(case, shape, ODD_AXIS, dev, out, precision=prec)
    assert not rr.any() and not ri.any()


def test_grid_empty_grid(dev):
    c = inputs.random_case(1, 64, seed=5)
    for shape in ((0, 2, 2), (3, 0, 5), (4, 4, 0)):
        rr, ri = gpu_grid(c, shape, ODD_AXIS, dev)
        assert rr.shape == (0,) and ri.shape == (0,)


@pytest.mark.parametrize("prec", PRECISIONS)
def test_grid_repeatable_and_two_stage_equal(dev, prec):
    w = inputs.make_workload("spiral32")
    L = inputs.WORKLOADS["spiral32"].L
    axis = inputs.grid_axis_of(L)
    a = gpu_grid(w, (L, L, L), axis, dev, precision=prec)
    b = gpu_grid(w, (L, L, L), axis, dev, precision=prec)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    k = [t(w[n], dev) for n in ("kx", "ky", "kz", "Dr", "Di")]
    packed = binding.new_packed(w["M"], dev)
    binding.fhd_pack(*k, packed)
    rr, ri = binding.fhd_grid_gather(packed, w["M"], (L, L, L), axis, precision=prec)
    torch.cuda.synchronize(dev)
    assert np.array_equal(rr.cpu().numpy(), a[0]) and np.array_equal(ri.cpu().numpy(), a[1])


def test_grid_agrees_with_direct_gather(dev):
    shape = (70, 5, 27)
    c = inputs.random_case(1, 3000, seed=91)
    x, y, z = inputs.coords_from_axis(*shape, ODD_AXIS)
    k = [t(c[n], dev) for n in ("kx", "ky", "kz", "Dr", "Di")]
    dr, di = binding.fhd_compute(*k, t(x, dev), t(y, dev), t(z, dev))
    gr, gi = binding.fhd_compute_grid(*k, shape, ODD_AXIS)
    torch.cuda.synchronize(dev)
    check("grid vs direct", gr.cpu().numpy(), gi.cpu().numpy(),
          dr.cpu().numpy().astype(np.float64), di.cpu().numpy().astype(np.float64))


def test_grid_bf16x3_close_to_fp32(dev):
    """The split-bf16 products differ from the fp32 ones by about 1e-5 of the
    result, well inside the gate; a wide dynamic range of |D| (1e-6 to 1e6)
    stays accurate because bf16 keeps fp32's exponent range."""
    rng = np.random.default_rng(33)
    M = 5000
    c = inputs.random_case(1, M, seed=34)
    scale = (10.0 ** rng.uniform(-6, 6, M)).astype(np.float32)
    c = dict(c, Dr=(c["Dr"] * scale).astype(np.float32), Di=(c["Di"] * scale).astype(np.float32))
    shape = (48, 10, 7)
    a = gpu_grid(c, shape, ODD_AXIS, dev, precision=binding.FHD_GRID_FP32)
    b = gpu_grid(c, shape, ODD_AXIS, dev, precision=binding.FHD_GRID_BF16X3)
    ref = oracle_on_grid(c, shape, ODD_AXIS)
    check("grid wide range fp32", *a, *ref)
    check("grid wide range bf16x3", *b, *ref)
    assert metrics.rel_l2(*b, a[0].astype(np.float64), a[1].astype(np.float64)) < 1e-4


# ---------------------------------------------------------------------------
# forward F on a grid (fhd_forward_grid, split-bf16 products)
# ---------------------------------------------------------------------------
def gpu_forward_grid(case, img, shape, axis, dev):
    k = [t(case[a], dev) for a in ("kx", "ky", "kz")]
    Dr, Di = binding.fhd_forward_grid(*k, shape, axis, t(img[0], dev), t(img[1], dev))
    torch.cuda.synchronize(dev)
    return Dr.cpu().numpy(), Di.cpu().numpy()


def oracle_forward_on_grid(case, img, shape, axis, idx=None):
    x, y, z = inputs.coords_from_axis(*shape, axis)
    kx, ky, kz = case["kx"], case["ky"], case["kz"]
    if idx is not None:
        kx, ky, kz = kx[idx], ky[idx], kz[idx]
    return oracle.forward(kx, ky, kz, img[0], img[1], x, y, z)


@pytest.mark.parametrize("name,samples", [("random16", None), ("spiral32", None),
                                          ("radial64", 1024), ("spiral128", 384)])
def test_forward_grid_workloads(dev, name, samples):
    w = inputs.make_workload(name)
    L = inputs.WORKLOADS[name].L
    img = inputs.random_image(w["N"], seed=inputs.WORKLOADS[name].seed + 7)
    Dr, Di = gpu_forward_grid(w, img, (L, L, L), inputs.grid_axis_of(L), dev)
    idx = (np.arange(w["M"]) if samples is None else
           inputs.voxel_subset(w["M"], samples, seed=inputs.WORKLOADS[name].seed + 3000))
    ref = oracle_forward_on_grid(w, img, (L, L, L), inputs.grid_axis_of(L), idx)
    check("forward grid " + name, Dr[idx], Di[idx], *ref)


@pytest.mark.parametrize("shape,M", [((1, 1, 1), 1), ((70, 5, 27), 1000), ((130, 3, 2), 7),
                                     ((64, 128, 1), 4097), ((33, 17, 9), 513),
                                     ((7, 129, 2), 2049), ((200, 2, 3), 31)])
def test_forward_grid_ragged(dev, shape, M):
    """Grids whose edges cut the 128-row slabs and 64-column groups, sample
    counts off the 32-sample step, non-dyadic axis steps of either sign."""
    c = inputs.random_case(1, M, seed=2 * M + shape[0])
    N = int(np.prod(shape))
    img = inputs.random_image(N, seed=N + 3)
    D = gpu_forward_grid(c, img, shape, ODD_AXIS, dev)
    check("forward grid ragged %s M=%d" % (shape, M), *D,
          *oracle_forward_on_grid(c, img, shape, ODD_AXIS))


def test_forward_grid_adjoint_of_grid_gather(dev):
    """<F^H D, rho> = <D, F rho> with both grid forms on the GPU."""
    shape = (48, 20, 9)
    N = int(np.prod(shape))
    c = inputs.random_case(1, 3000, seed=61, kmax=20.0)
    img = inputs.random_image(N, seed=62)
    rr, ri = gpu_grid(c, shape, ODD_AXIS, dev, precision=binding.FHD_GRID_BF16X3)
    Fr, Fi = gpu_forward_grid(c, img, shape, ODD_AXIS, dev)
    rho = img[0].astype(np.float64) + 1j * img[1].astype(np.float64)
    D = c["Dr"].astype(np.float64) + 1j * c["Di"].astype(np.float64)
    lhs = np.vdot(rho, rr.astype(np.float64) + 1j * ri)
    rhs = np.vdot(Fr.astype(np.float64) + 1j * Fi, D)
    scale = np.linalg.norm(rho) * np.linalg.norm(D) * np.sqrt(3000)
    assert abs(lhs - rhs) <= 1e-5 * scale, (lhs, rhs)


def test_forward_grid_matches_direct_forward(dev):
    w = inputs.make_workload("spiral32")
    L = inputs.WORKLOADS["spiral32"].L
    img = inputs.random_image(w["N"], seed=63)
    g = gpu_forward_grid(w, img, (L, L, L), inputs.grid_axis_of(L), dev)
    d = [t(w[a], dev) for a in ("kx", "ky", "kz", "x", "y", "z")]
    Dr, Di = binding.fhd_forward(*d, t(img[0], dev), t(img[1], dev))
    torch.cuda.synchronize(dev)
    check("forward grid vs direct", *g, Dr.cpu().numpy().astype(np.float64),
          Di.cpu().numpy().astype(np.float64))


def test_forward_grid_repeatable_and_empty(dev):
    c = inputs.random_case(1, 700, seed=64)
    shape = (40, 9, 3)
    img = inputs.random_image(int(np.prod(shape)), seed=65)
    a = gpu_forward_grid(c, img, shape, ODD_AXIS, dev)
    b = gpu_forward_grid(c, img, shape, ODD_AXIS, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    e = np.zeros(0, np.float32)
    k = [t(c[n], dev) for n in ("kx", "ky", "kz")]
    Dr = torch.full((700,), 5.0, device=dev)
    Di = torch.full((700,), 5.0, device=dev)
    binding.fhd_forward_grid(*k, (0, 4, 4), ODD_AXIS, t(e, dev), t(e, dev), Dr, Di)
    torch.cuda.synchronize(dev)
    assert torch.count_nonzero(Dr).item() == 0 and torch.count_nonzero(Di).item() == 0


# ---------------------------------------------------------------------------
# F^H F and CG on a grid (fhd_normal_grid, fhd_cg_grid)
# ---------------------------------------------------------------------------
def test_normal_grid_is_N_identity_on_full_cartesian_grid(dev):
    L = 16
    kx, ky, kz = inputs.cartesian_kgrid(L)
    N = L ** 3
    pr, pi = inputs.random_image(N, seed=81)
    qr, qi = binding.fhd_normal_grid(t(kx, dev), t(ky, dev), t(kz, dev), (L, L, L),
                                     inputs.grid_axis_of(L), t(pr, dev), t(pi, dev))
    torch.cuda.synchronize(dev)
    check("grid F^H F = N I", qr.cpu().numpy(), qi.cpu().numpy(), N * pr.astype(np.float64),
          N * pi.astype(np.float64))


def test_normal_grid_matches_oracle_composition(dev):
    shape = (40, 9, 7)
    N = int(np.prod(shape))
    c = inputs.random_case(1, 2000, seed=82, kmax=12.0)
    pr, pi = inputs.random_image(N, seed=83)
    k = [t(c[a], dev) for a in ("kx", "ky", "kz")]
    qr, qi = binding.fhd_normal_grid(*k, shape, ODD_AXIS, t(pr, dev), t(pi, dev))
    torch.cuda.synchronize(dev)
    x, y, z = inputs.coords_from_axis(*shape, ODD_AXIS)
    Dr, Di = oracle.forward(c["kx"], c["ky"], c["kz"], pr, pi, x, y, z)
    ref = oracle.fhd(c["kx"], c["ky"], c["kz"], Dr, Di, x, y, z)
    check("grid F^H F p", qr.cpu().numpy(), qi.cpu().numpy(), *ref)


def _cg_grid_case():
    L = 8
    rng = np.random.default_rng(72)
    M = 3000
    k = rng.uniform(-3.5, 3.5, (3, M)).astype(np.float32)
    D = rng.standard_normal((2, M)).astype(np.float32)
    x, y, z = inputs.grid_coords(L)
    return L, dict(kx=k[0], ky=k[1], kz=k[2], Dr=D[0], Di=D[1], x=x, y=y, z=z)


@pytest.mark.parametrize("iters", [6, 9])
def test_cg_grid_matches_oracle_cg(dev, iters):
    L, c = _cg_grid_case()
    d = [t(c[a], dev) for a in ("kx", "ky", "kz", "Dr", "Di")]
    rr, ri, done, res = binding.fhd_cg_grid(*d, (L, L, L), inputs.grid_axis_of(L), iters)
    torch.cuda.synchronize(dev)
    ref, ref_res = oracle.cg(c["kx"], c["ky"], c["kz"], c["Dr"], c["Di"], c["x"], c["y"], c["z"],
                             iters=iters)
    assert done == iters == len(ref_res) - 1
    check("grid cg %d iterations" % iters, rr.cpu().numpy(), ri.cpu().numpy(), ref.real, ref.imag)
    assert np.allclose(res, ref_res, rtol=1e-3, atol=0), (res, ref_res)


def test_cg_grid_one_step_on_full_grid(dev):
    L = 16
    kx, ky, kz = inputs.cartesian_kgrid(L)
    x, y, z = inputs.grid_coords(L)
    tr, ti = inputs.random_image(L ** 3, seed=84)
    Dr, Di = oracle.forward(kx, ky, kz, tr, ti, x, y, z)
    rs0 = float(L ** 6 * np.sum(tr.astype(np.float64) ** 2 + ti.astype(np.float64) ** 2))
    d = [t(a, dev) for a in (kx, ky, kz, Dr.astype(np.float32), Di.astype(np.float32))]
    rr, ri, done, res = binding.fhd_cg_grid(*d, (L, L, L), inputs.grid_axis_of(L), 5,
                                            tol=1e-8 * rs0)
    torch.cuda.synchronize(dev)
    assert done == 1, res
    check("grid cg full grid", rr.cpu().numpy(), ri.cpu().numpy(), tr.astype(np.float64),
          ti.astype(np.float64))
