"""GPU parity of the forward operator F and the normal operator F^H F
against the fp64 oracle and against identities that fix them.

Same gate as F^H D: relative L2 <= 5e-4 and every element within 10x that
bound times the reference's rms magnitude.
"""
import numpy as np
import pytest
import torch

import oracle
from non_cartesian_mri_fhd_amd import binding, build, inputs, metrics

from test_gpu_parity import check, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    build.ensure_built()
    binding.load()
    return torch.device("cuda:0")


def t(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def chunk_fractions(x, y, z):
    """Fractions of voxels in 16-voxel ramps and 8-voxel ramp chunks that the
    pre-pass should find, by the package's host-side replica of its test."""
    from non_cartesian_mri_fhd_amd import layout
    return layout.ramp_chunk_fractions(x, y, z)


def gpu_forward(case, img, dev):
    c = to_dev(case, dev)
    Dr, Di = binding.fhd_forward(c["kx"], c["ky"], c["kz"], c["x"], c["y"], c["z"],
                                 t(img[0], dev), t(img[1], dev))
    torch.cuda.synchronize(dev)
    return Dr.cpu().numpy(), Di.cpu().numpy()


@pytest.mark.parametrize("name,samples", [("random16", None), ("spiral32", None),
                                          ("radial64", 1024), ("spiral128", 384),
                                          ("vdrandom256", 32)])
def test_forward_workloads(dev, name, samples):
    w = inputs.make_workload(name)
    img = inputs.random_image(w["N"], seed=inputs.WORKLOADS[name].seed + 7)
    Dr, Di = gpu_forward(w, img, dev)
    idx = (np.arange(w["M"]) if samples is None else
           inputs.voxel_subset(w["M"], samples, seed=inputs.WORKLOADS[name].seed + 3000))
    ref_r, ref_i = oracle.forward(w["kx"][idx], w["ky"][idx], w["kz"][idx], img[0], img[1],
                                  w["x"], w["y"], w["z"])
    check("forward " + name, Dr[idx], Di[idx], ref_r, ref_i)


@pytest.mark.parametrize("N,M", [(1, 1), (9, 1), (8, 63), (7, 2047), (17, 2049), (1001, 4097)])
def test_forward_ragged(dev, N, M):
    c = inputs.random_case(N, M, seed=3 * N + M)
    img = inputs.random_image(N, seed=N + 5)
    Dr, Di = gpu_forward(c, img, dev)
    ref = oracle.forward(c["kx"], c["ky"], c["kz"], img[0], img[1], c["x"], c["y"], c["z"])
    check("forward ragged N=%d M=%d" % (N, M), Dr, Di, *ref)


def test_forward_empty_image_writes_zeros(dev):
    c = inputs.random_case(4, 300, seed=1)
    d = to_dev(c, dev)
    e = torch.empty(0, dtype=torch.float32, device=dev)
    Dr = torch.full((300,), 3.0, device=dev)
    Di = torch.full((300,), 3.0, device=dev)
    binding.fhd_forward(d["kx"], d["ky"], d["kz"], e, e, e, e, e, Dr, Di)
    torch.cuda.synchronize(dev)
    assert torch.count_nonzero(Dr).item() == 0 and torch.count_nonzero(Di).item() == 0


def test_gpu_adjointness(dev):
    """<F^H D, rho> = <D, F rho> with both sides computed by the GPU."""
    c = inputs.random_case(N=5000, M=3000, seed=23, kmax=20.0)
    img = inputs.random_image(5000, seed=24)
    d = to_dev(c, dev)
    rr, ri = binding.fhd_compute(d["kx"], d["ky"], d["kz"], d["Dr"], d["Di"], d["x"], d["y"], d["z"])
    Fr, Fi = binding.fhd_forward(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"],
                                 t(img[0], dev), t(img[1], dev))
    torch.cuda.synchronize(dev)
    rho = img[0].astype(np.float64) + 1j * img[1].astype(np.float64)
    D = c["Dr"].astype(np.float64) + 1j * c["Di"].astype(np.float64)
    lhs = np.vdot(rho, rr.cpu().numpy().astype(np.float64) + 1j * ri.cpu().numpy())
    rhs = np.vdot(Fr.cpu().numpy().astype(np.float64) + 1j * Fi.cpu().numpy(), D)
    scale = np.linalg.norm(rho) * np.linalg.norm(D) * np.sqrt(3000)
    assert abs(lhs - rhs) <= 1e-5 * scale, (lhs, rhs)


def test_normal_is_N_identity_on_full_cartesian_grid(dev):
    """All integer k over an L^3 grid: F^H F p = N p (DFT orthogonality)."""
    L = 16
    kx, ky, kz = inputs.cartesian_kgrid(L)
    x, y, z = inputs.grid_coords(L)
    N = L ** 3
    pr, pi = inputs.random_image(N, seed=31)
    qr, qi = binding.fhd_normal(t(kx, dev), t(ky, dev), t(kz, dev), t(x, dev), t(y, dev),
                                t(z, dev), t(pr, dev), t(pi, dev))
    torch.cuda.synchronize(dev)
    check("F^H F = N I", qr.cpu().numpy(), qi.cpu().numpy(), N * pr.astype(np.float64),
          N * pi.astype(np.float64))


def test_normal_matches_oracle_composition(dev):
    c = inputs.random_case(N=3000, M=2000, seed=41, kmax=12.0)
    pr, pi = inputs.random_image(3000, seed=42)
    d = to_dev(c, dev)
    qr, qi = binding.fhd_normal(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"],
                                t(pr, dev), t(pi, dev))
    torch.cuda.synchronize(dev)
    Dr, Di = oracle.forward(c["kx"], c["ky"], c["kz"], pr, pi, c["x"], c["y"], c["z"])
    ref = oracle.fhd(c["kx"], c["ky"], c["kz"], Dr, Di, c["x"], c["y"], c["z"])
    check("F^H F p", qr.cpu().numpy(), qi.cpu().numpy(), *ref)


def test_normal_without_samples_writes_zeros(dev):
    c = inputs.random_case(100, 4, seed=2)
    d = to_dev(c, dev)
    e = torch.empty(0, dtype=torch.float32, device=dev)
    qr = torch.full((100,), 5.0, device=dev)
    qi = torch.full((100,), 5.0, device=dev)
    binding.fhd_normal(e, e, e, d["x"], d["y"], d["z"], d["x"], d["y"], qr, qi)
    torch.cuda.synchronize(dev)
    assert torch.count_nonzero(qr).item() == 0 and torch.count_nonzero(qi).item() == 0


def test_forward_two_stage_equal_and_repeatable(dev):
    w = inputs.make_workload("spiral32")
    img = inputs.random_image(w["N"], seed=9)
    d = to_dev(w, dev)
    ir, ii = t(img[0], dev), t(img[1], dev)
    a = binding.fhd_forward(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], ir, ii)
    b = binding.fhd_forward(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], ir, ii)
    packed = binding.new_packed(w["N"], dev)
    binding.fhd_forward_pack(d["x"], d["y"], d["z"], ir, ii, packed)
    g = binding.fhd_forward_gather(packed, w["N"], d["kx"], d["ky"], d["kz"])
    torch.cuda.synchronize(dev)
    for u, v in ((a, b), (a, g)):
        assert torch.equal(u[0], v[0]) and torch.equal(u[1], v[1])


def test_forward_shared_kz_and_general_paths_bitwise_equal(dev):
    """Stack-of-spirals samples in plane order (a lane's 8 samples share kz:
    shared path) and interleaved across planes (general path) give bitwise
    identical per-sample results."""
    w = inputs.make_workload("spiral32")
    img = inputs.random_image(w["N"], seed=10)
    # voxels 1 and 2 of every 8 swapped: no chunk is a ramp, so every chunk
    # takes the direct paths under test
    n = np.arange(w["N"])
    swap = n.copy()
    swap[1::8], swap[2::8] = n[2::8], n[1::8]
    w = dict(w, x=w["x"][swap], y=w["y"][swap], z=w["z"][swap])
    img = (img[0][swap], img[1][swap])
    a = gpu_forward(w, img, dev)
    M = w["M"]
    perm = np.arange(M).reshape(16, M // 16).T.reshape(-1)     # plane index fastest
    p = dict(w, kx=w["kx"][perm], ky=w["ky"][perm], kz=w["kz"][perm])
    assert not np.all(p["kz"][:8] == p["kz"][0])
    b = gpu_forward(p, img, dev)
    assert np.array_equal(a[0][perm], b[0]) and np.array_equal(a[1][perm], b[1])


def test_forward_ramp_and_direct_chunks_agree(dev):
    """The same voxels as ramp chunks (x-fastest grid order) and as direct
    chunks (voxels 1 and 2 of every 8 swapped): D is a sum over voxels, so
    both must match the oracle and each other."""
    w = inputs.make_workload("spiral32")
    img = inputs.random_image(w["N"], seed=14)
    n = np.arange(w["N"])
    swap = n.copy()
    swap[1::8], swap[2::8] = n[2::8], n[1::8]
    ramp = gpu_forward(w, img, dev)
    direct = gpu_forward(dict(w, x=w["x"][swap], y=w["y"][swap], z=w["z"][swap]),
                         (img[0][swap], img[1][swap]), dev)
    ref = oracle.forward(w["kx"], w["ky"], w["kz"], img[0], img[1], w["x"], w["y"], w["z"])
    check("forward ramp chunks", *ramp, *ref)
    check("forward direct chunks", *direct, *ref)
    assert metrics.rel_l2(*ramp, direct[0].astype(np.float64), direct[1].astype(np.float64)) < 5e-5


def test_forward_ramp_pairs_and_single_chunks_agree(dev):
    """The same voxels as 16-voxel ramps (x-fastest grid order: every chunk
    pair is one ramp) and as 8-voxel ramp chunks only (the two chunks of
    every pair swapped, so no pair is a ramp but every chunk still is):
    both match the oracle and each other to rounding."""
    w = inputs.make_workload("spiral32")
    img = inputs.random_image(w["N"], seed=24)
    n = np.arange(w["N"]).reshape(-1, 2, 8)[:, ::-1, :].reshape(-1)
    assert chunk_fractions(w["x"], w["y"], w["z"]) == (1.0, 0.0)
    assert chunk_fractions(w["x"][n], w["y"][n], w["z"][n]) == (0.0, 1.0)
    pairs = gpu_forward(w, img, dev)
    single = gpu_forward(dict(w, x=w["x"][n], y=w["y"][n], z=w["z"][n]),
                         (img[0][n], img[1][n]), dev)
    ref = oracle.forward(w["kx"], w["ky"], w["kz"], img[0], img[1], w["x"], w["y"], w["z"])
    check("forward 16-voxel ramps", *pairs, *ref)
    check("forward 8-voxel ramp chunks", *single, *ref)
    assert metrics.rel_l2(*pairs, single[0].astype(np.float64), single[1].astype(np.float64)) < 5e-5


def test_forward_ramp_degenerate_steps_and_partial_chunk(dev):
    """Samples whose x-step phase kx dx is 0, 1/4, 1/2 or -1/2 revolution, on
    an L = 32 grid cut 5 voxels short (the last chunk is partial and takes
    the direct path)."""
    L = 32
    x, y, z = inputs.grid_coords(L)
    N = L ** 3 - 5
    x, y, z = x[:N], y[:N], z[:N]
    rng = np.random.default_rng(15)
    M = 3000
    kx = rng.choice(np.array([0.0, 8.0, 16.0, -16.0, 15.5, -0.25], np.float32), M)
    ky, kz = (rng.uniform(-16, 16, M).astype(np.float32) for _ in range(2))
    c = dict(kx=kx, ky=ky, kz=kz, Dr=kx, Di=kx, x=x, y=y, z=z)
    img = inputs.random_image(N, seed=16)
    D = gpu_forward(c, img, dev)
    ref = oracle.forward(kx, ky, kz, img[0], img[1], x, y, z)
    check("forward ramp degenerate steps", *D, *ref)


def test_forward_mixed_chunks(dev):
    """A grid with some voxels moved off it: their chunks are direct, the
    rest ramp chunks, in one stream."""
    L = 24
    x, y, z = (a.copy() for a in inputs.grid_coords(L))
    rng = np.random.default_rng(17)
    moved = rng.choice(L ** 3, 50, replace=False)
    x[moved] += np.float32(0.002)
    k = inputs.make_kspace("random16")
    c = dict(k, x=x, y=y, z=z)
    img = inputs.random_image(L ** 3, seed=18)
    D = gpu_forward(c, img, dev)
    ref = oracle.forward(k["kx"], k["ky"], k["kz"], img[0], img[1], x, y, z)
    check("forward mixed chunks", *D, *ref)
