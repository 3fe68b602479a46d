"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Gate (per voxel-sample sum, fp32 arithmetic on the GPU): relative L2 error
<= 5e-4 over the compared voxels, and every voxel's error <= 10x that bound
times the rms magnitude of the reference (a Gaussian-like error field with
rel-L2 at the gate would need a >10 sigma outlier to break it). PSNR is
printed, not gated.
"""
import numpy as np
import pytest
import torch

import oracle
from non_cartesian_mri_fhd_amd import binding, build, inputs, metrics

from pins import cartesian_fft_reference

pytestmark = pytest.mark.gpu

REL_L2_TOL = 5e-4
ELEM_TOL = 10 * REL_L2_TOL


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    build.ensure_built()
    binding.load()
    return torch.device("cuda:0")


def to_dev(case, dev):
    return {k: torch.from_numpy(np.ascontiguousarray(case[k])).to(dev)
            for k in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")}


def gpu_fhd(case, dev):
    t = to_dev(case, dev)
    rr, ri = binding.fhd_compute(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"],
                                 t["x"], t["y"], t["z"])
    torch.cuda.synchronize(dev)
    return rr.cpu().numpy(), ri.cpu().numpy()


def check(tag, rr, ri, ref_r, ref_i):
    e = metrics.rel_l2(rr, ri, ref_r, ref_i)
    worst = metrics.max_abs_err(rr, ri, ref_r, ref_i)
    scale = metrics.rms(ref_r, ref_i)
    psnr = metrics.psnr_db(rr, ri, ref_r, ref_i)
    print("%s: rel_l2=%.3e max_err/rms=%.3e psnr=%.1f dB" % (tag, e, worst / scale, psnr),
          flush=True)
    assert np.all(np.isfinite(rr)) and np.all(np.isfinite(ri))
    assert e <= REL_L2_TOL, (tag, e)
    assert worst <= ELEM_TOL * scale, (tag, worst, scale)
    return e


@pytest.mark.parametrize("name", ["random16", "spiral32"])
def test_workload_all_voxels(dev, name):
    w = inputs.make_workload(name)
    rr, ri = gpu_fhd(w, dev)
    ref = oracle.fhd(w["kx"], w["ky"], w["kz"], w["Dr"], w["Di"], w["x"], w["y"], w["z"])
    check(name, rr, ri, *ref)


@pytest.mark.parametrize("name,count", [("radial64", 8192), ("spiral128", 4096),
                                        ("vdrandom256", inputs.SUBSET_SIZE)])
def test_workload_sampled_voxels(dev, name, count):
    """Full-size GPU run, in the launch shape the benchmark times; the oracle
    computes a seeded voxel subset one voxel at a time."""
    w = inputs.make_workload(name)
    rr, ri = gpu_fhd(w, dev)
    if name == "vdrandom256":
        idx = inputs.voxel_subset(w["N"])
    else:
        idx = inputs.voxel_subset(w["N"], count, seed=inputs.WORKLOADS[name].seed + 1000)
    ref_r, ref_i = oracle.fhd_subset(w, idx)
    check(name, rr[idx], ri[idx], ref_r, ref_i)


@pytest.mark.parametrize("name,count", [("radial64", 4096), ("spiral128", 4096),
                                        ("vdrandom256", inputs.SUBSET_SIZE)])
@pytest.mark.parametrize("paths", ["vector", "bf16x3"])
def test_workload_sampled_voxels_other_paths(dev, name, count, paths):
    """The fp32 vector paths (FHD_GATHER_VECTOR) and the opt-in split-bf16
    line form (FHD_GATHER_BF16X3) at full size, in the launch shape the
    benchmark times them in, on seeded voxel subsets."""
    w = inputs.make_workload(name)
    t = to_dev(w, dev)
    code = binding.FHD_GATHER_VECTOR if paths == "vector" else binding.FHD_GATHER_BF16X3
    rr, ri = binding.fhd_compute(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], t["x"], t["y"], t["z"],
                                 paths=code)
    torch.cuda.synchronize(dev)
    rr, ri = rr.cpu().numpy(), ri.cpu().numpy()
    if name == "vdrandom256":
        idx = inputs.voxel_subset(w["N"])
    else:
        idx = inputs.voxel_subset(w["N"], count, seed=inputs.WORKLOADS[name].seed + 1000)
    ref_r, ref_i = oracle.fhd_subset(w, idx)
    check("%s %s" % (name, paths), rr[idx], ri[idx], ref_r, ref_i)


@pytest.mark.parametrize("L", [16, 32, 64])
def test_cartesian_grid_matches_numpy_ifft(dev, L):
    """Full integer k-grid over an L^3 voxel grid reduces to N * ifftn."""
    c = inputs.cartesian_case(L, seed=500 + L)
    rr, ri = gpu_fhd(c, dev)
    ref = cartesian_fft_reference(c)
    check("cartesian L=%d" % L, rr, ri, ref.real, ref.imag)


def test_single_sample_phase_ramp(dev):
    L = 16
    x, y, z = inputs.grid_coords(L)
    k = np.array([3.25, -5.5, 7.125], np.float32)
    D = np.array([0.75, -1.5], np.float32)
    case = dict(kx=k[:1], ky=k[1:2], kz=k[2:], Dr=D[:1], Di=D[1:], x=x, y=y, z=z)
    rr, ri = gpu_fhd(case, dev)
    mod = np.hypot(rr.astype(np.float64), ri.astype(np.float64))
    assert np.allclose(mod, np.hypot(0.75, 1.5), rtol=1e-5)
    ref = oracle.fhd(case["kx"], case["ky"], case["kz"], case["Dr"], case["Di"], x, y, z)
    check("single sample", rr, ri, *ref)


def test_dc_sum(dev):
    rng = np.random.default_rng(3)
    M, N = 1000, 777
    zero = np.zeros(M, np.float32)
    Dr, Di = rng.standard_normal((2, M)).astype(np.float32)
    x, y, z = rng.uniform(-0.5, 0.5, (3, N)).astype(np.float32)
    rr, ri = gpu_fhd(dict(kx=zero, ky=zero, kz=zero, Dr=Dr, Di=Di, x=x, y=y, z=z), dev)
    s = Dr.astype(np.float64).sum() + 1j * Di.astype(np.float64).sum()
    err = np.abs(rr + 1j * ri - s)
    assert err.max() <= 1e-5 * np.sqrt(M) * 4, err.max()
    assert np.ptp(rr) == 0 and np.ptp(ri) == 0     # every voxel sums identically


@pytest.mark.parametrize("N,M", [(1, 1), (1, 9), (63, 8), (2047, 7), (2049, 17),
                                 (4097, 1001), (5000, 123)])
def test_ragged_sizes(dev, N, M):
    c = inputs.random_case(N, M, seed=N * 7 + M)
    rr, ri = gpu_fhd(c, dev)
    ref = oracle.fhd(c["kx"], c["ky"], c["kz"], c["Dr"], c["Di"], c["x"], c["y"], c["z"])
    check("ragged N=%d M=%d" % (N, M), rr, ri, *ref)


def test_zero_samples_writes_zeros(dev):
    c = inputs.random_case(300, 4, seed=1)
    t = to_dev(c, dev)
    e = torch.empty(0, dtype=torch.float32, device=dev)
    rho_r = torch.full((300,), 7.0, device=dev)
    rho_i = torch.full((300,), 7.0, device=dev)
    binding.fhd_compute(e, e, e, e, e, t["x"], t["y"], t["z"], rho_r, rho_i)
    torch.cuda.synchronize(dev)
    assert torch.count_nonzero(rho_r).item() == 0 and torch.count_nonzero(rho_i).item() == 0


def test_zero_voxels_is_a_no_op(dev):
    c = inputs.random_case(4, 10, seed=2)
    t = to_dev(c, dev)
    e = torch.empty(0, dtype=torch.float32, device=dev)
    rr, ri = binding.fhd_compute(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], e, e, e)
    torch.cuda.synchronize(dev)
    assert rr.numel() == 0 and ri.numel() == 0


def test_bitwise_repeatable_and_two_stage_equal(dev):
    c = inputs.random_case(10000, 3001, seed=77, kmax=40.0)
    t = to_dev(c, dev)
    a = binding.fhd_compute(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], t["x"], t["y"], t["z"])
    b = binding.fhd_compute(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], t["x"], t["y"], t["z"])
    packed = binding.new_packed(c["M"], dev)
    binding.fhd_pack(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], packed)
    g = binding.fhd_gather(packed, c["M"], t["x"], t["y"], t["z"])
    torch.cuda.synchronize(dev)
    for u, v in ((a, b), (a, g)):
        assert torch.equal(u[0], v[0]) and torch.equal(u[1], v[1])


@pytest.mark.parametrize("paths", ["all", "bf16x3"])
def test_full_size_line_form_repeatable(dev, paths):
    """At 128^3 x 100,000, in the launch shape the benchmark times (the
    long-line instance with its B table, three sample splits), four calls
    in a row give bitwise identical results. The workgroups' waves share
    each step's copies into LDS, so a missing wait between them would show
    up as differences from run to run."""
    w = inputs.make_workload("spiral128")
    t = to_dev(w, dev)
    code = binding.FHD_GATHER_ALL if paths == "all" else binding.FHD_GATHER_BF16X3
    runs = [binding.fhd_compute(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], t["x"], t["y"], t["z"],
                                paths=code) for _ in range(4)]
    torch.cuda.synchronize(dev)
    for r in runs[1:]:
        assert torch.equal(r[0], runs[0][0]) and torch.equal(r[1], runs[0][1])


def test_side_stream(dev):
    """Work is enqueued on the caller's stream."""
    c = inputs.random_case(3000, 500, seed=8)
    t = to_dev(c, dev)
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        rr, ri = binding.fhd_compute(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"],
                                     t["x"], t["y"], t["z"])
    s.synchronize()
    ref = oracle.fhd(c["kx"], c["ky"], c["kz"], c["Dr"], c["Di"], c["x"], c["y"], c["z"])
    check("side stream", rr.cpu().numpy(), ri.cpu().numpy(), *ref)


def test_binding_rejects_host_tensors(dev):
    c = inputs.random_case(10, 10, seed=4)
    t = {k: torch.from_numpy(c[k]) for k in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")}
    with pytest.raises(ValueError):
        binding.fhd_compute(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], t["x"], t["y"], t["z"])


def test_c_abi_rejects_overlap_and_short_pack_buffer(dev):
    lib = binding.load()
    c = inputs.random_case(64, 16, seed=5)
    t = to_dev(c, dev)
    out = torch.empty(64, device=dev)
    # rho_r aliases x
    rc = lib.fhd_compute(*[t[k].data_ptr() for k in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")],
                         t["x"].data_ptr(), out.data_ptr(), 16, 64, None)
    assert rc == binding.FHD_ERR_INVALID_ARG
    small = torch.empty(8, dtype=torch.uint8, device=dev)
    rc = lib.fhd_pack(*[t[k].data_ptr() for k in ("kx", "ky", "kz", "Dr", "Di")], 16,
                      small.data_ptr(), 8, None)
    assert rc == binding.FHD_ERR_INVALID_ARG


def test_large_exact_phases_closed_form(dev):
    """Phases of up to ~1e5 revolutions that are exact in fp32 (integer k,
    dyadic x): rho must equal the closed form sum D_m e^{i 2 pi frac(k.x)}.
    Pins that the hardware sine/cosine reduce huge revolution counts exactly
    (the kernel applies no explicit range reduction)."""
    rng = np.random.default_rng(12)
    M, N = 64, 4096
    kx, ky, kz = (rng.integers(-40000, 40000, M).astype(np.float32) for _ in range(3))
    # D on the axes (a, -a, i a, -i a): arg(D) / 2 pi is 0, 1/2 or +-1/4, so
    # the kernel's phase (k.x plus that offset) stays an exact multiple of 1/8
    a = rng.uniform(0.5, 2.0, M)
    axis = rng.integers(0, 4, M)
    Dr = np.where(axis == 0, a, np.where(axis == 1, -a, 0.0)).astype(np.float32)
    Di = np.where(axis == 2, a, np.where(axis == 3, -a, 0.0)).astype(np.float32)
    # multiples of 1/8 in [-1, 1): every k.x is an exact multiple of 1/8
    x, y, z = (rng.integers(-8, 8, N).astype(np.float32) / 8 for _ in range(3))
    rr, ri = gpu_fhd(dict(kx=kx, ky=ky, kz=kz, Dr=Dr, Di=Di, x=x, y=y, z=z), dev)
    ph = (np.outer(x, kx).astype(np.float64) + np.outer(y, ky) + np.outer(z, kz))
    assert np.abs(ph).max() > 3e4
    frac8 = np.mod(np.rint(ph * 8).astype(np.int64), 8)        # phase in 1/8 turns
    e = np.exp(2j * np.pi * frac8 / 8.0)
    ref = e @ (Dr.astype(np.float64) + 1j * Di.astype(np.float64))
    check("large exact phases", rr, ri, ref.real, ref.imag)
    assert metrics.rel_l2(rr, ri, ref.real, ref.imag) < 1e-5


def test_ramp_shared_and_general_paths(dev):
    """One grid, three voxel orders. x fastest: each lane's 16 voxels share y
    and z and are equally spaced in x (the ramp path). The same with voxels
    1 and 2 of every 8 swapped: y, z still shared, x no longer a ramp (the
    shared-phase path). z fastest: nothing shared (the general path). The
    shared and general paths give bitwise identical per-voxel results; the
    ramp path meets the oracle gate and agrees with them to rounding."""
    L = 32
    k = inputs.make_kspace("spiral32")
    x, y, z = inputs.grid_coords(L)
    n = np.arange(L ** 3)
    swap = n.copy()
    swap[1::8], swap[2::8] = n[2::8], n[1::8]
    zfast = n.reshape(L, L, L).transpose(2, 1, 0).reshape(-1)
    ramp = gpu_fhd(dict(k, x=x, y=y, z=z), dev)
    shared = gpu_fhd(dict(k, x=x[swap], y=y[swap], z=z[swap]), dev)
    general = gpu_fhd(dict(k, x=x[zfast], y=y[zfast], z=z[zfast]), dev)
    assert not np.array_equal(z[zfast][:8], np.full(8, z[zfast][0]))   # z varies within a lane
    sh = (np.empty_like(shared[0]), np.empty_like(shared[1]))
    sh[0][swap], sh[1][swap] = shared
    assert np.array_equal(sh[0][zfast], general[0]) and np.array_equal(sh[1][zfast], general[1])
    ref = oracle.fhd(k["kx"], k["ky"], k["kz"], k["Dr"], k["Di"], x, y, z)
    check("ramp path", *ramp, *ref)
    check("shared path", *sh, *ref)
    assert metrics.rel_l2(*ramp, sh[0].astype(np.float64), sh[1].astype(np.float64)) < 5e-5


def test_ramp_path_odd_spacing(dev):
    """A grid whose fp32 x steps are not all equal (non-dyadic origin and
    step, negative step in z): lanes whose voxels are not an exact ramp fall
    back; everything meets the oracle gate."""
    shape, axis = (72, 5, 27), (0.3, 0.013, -0.2, 0.021, 0.11, -0.017)
    x, y, z = inputs.coords_from_axis(*shape, axis)
    c = inputs.random_case(1, 3000, seed=91)
    w = dict(c, x=x, y=y, z=z)
    rr, ri = gpu_fhd(w, dev)
    ref = oracle.fhd(c["kx"], c["ky"], c["kz"], c["Dr"], c["Di"], x, y, z)
    check("odd spacing", rr, ri, *ref)


def test_ramp_path_nyquist_and_zero_steps(dev):
    """Samples whose x-step phase kx dx is 0, 1/4, 1/2 or -1/2 revolution (the
    recurrence's degenerate points) on an L = 32 grid."""
    L = 32
    x, y, z = inputs.grid_coords(L)
    rng = np.random.default_rng(12)
    M = 4096
    kx = rng.choice(np.array([0.0, 8.0, 16.0, -16.0, 15.5, -0.25], np.float32), M)
    ky, kz = (rng.uniform(-16, 16, M).astype(np.float32) for _ in range(2))
    Dr, Di = (rng.standard_normal(M).astype(np.float32) for _ in range(2))
    w = dict(kx=kx, ky=ky, kz=kz, Dr=Dr, Di=Di, x=x, y=y, z=z)
    rr, ri = gpu_fhd(w, dev)
    ref = oracle.fhd(kx, ky, kz, Dr, Di, x, y, z)
    check("ramp degenerate steps", rr, ri, *ref)


def test_ramp_path_per_lane_steps(dev):
    """Lanes whose 16 voxels are exact ramps, in two layouts of two
    workgroups each. A: every lane steps by 1/128 (the ramp path with one
    step per workgroup, half-step values formed once per sample in LDS).
    B: the same voxels, except that one lane of the second workgroup steps
    by 3/256, so that workgroup forms the half-step values per lane. Both
    meet the oracle gate, and the second workgroup's other voxels agree
    between A and B to rounding (the shared-step form folds the amplitude
    and the centre offset into its sample records, one rounding each)."""
    V, lanes = 16, 256
    groups = 2 * lanes
    rng = np.random.default_rng(31)
    k = inputs.make_kspace("spiral32")
    x0 = (rng.integers(-64, 44, groups) / 128.0).astype(np.float32)
    yz = [np.repeat(rng.uniform(-0.5, 0.5, groups).astype(np.float32), V) for _ in range(2)]
    steps = np.full(groups, 1.0 / 128, np.float32)
    odd = lanes + 5
    out = []
    for layout in ("A", "B"):
        st = steps.copy()
        if layout == "B":
            st[odd] = np.float32(3.0 / 256)
        x = (x0[:, None] + np.arange(V, dtype=np.float32)[None, :] * st[:, None]).reshape(-1)
        x = x.astype(np.float32)
        # exact ramps: x0 + v step is a multiple of 1/256 below 1 in magnitude
        assert np.array_equal(x, (x0[:, None].astype(np.float64) + np.arange(V)[None, :] * st[:, None].astype(np.float64)).reshape(-1))
        rr, ri = gpu_fhd(dict(k, x=x, y=yz[0], z=yz[1]), dev)
        ref = oracle.fhd(k["kx"], k["ky"], k["kz"], k["Dr"], k["Di"], x, yz[0], yz[1])
        check("ramp steps, layout " + layout, rr, ri, *ref)
        out.append((rr, ri))
    keep = np.ones(groups * V, bool)
    keep[:lanes * V] = False                      # first workgroup: one step in both
    keep[odd * V:(odd + 1) * V] = False           # the lane that differs
    a, b = out
    diff = metrics.rel_l2(a[0][keep], a[1][keep], b[0][keep].astype(np.float64),
                          b[1][keep].astype(np.float64))
    print("shared-step vs per-lane form: rel diff %.2e" % diff)
    assert 0 < diff < 2e-6


def test_mixed_waves(dev):
    """A grid with a few voxels moved off the grid: the waves holding them
    take the general path, the rest the shared one; all match the oracle."""
    L = 24
    k = inputs.make_kspace("random16")
    x, y, z = (a.copy() for a in inputs.grid_coords(L))
    rng = np.random.default_rng(4)
    moved = rng.choice(L ** 3, 40, replace=False)
    y[moved] += np.float32(0.001)
    w = dict(k, x=x, y=y, z=z)
    rr, ri = gpu_fhd(w, dev)
    ref = oracle.fhd(w["kx"], w["ky"], w["kz"], w["Dr"], w["Di"], x, y, z)
    check("mixed waves", rr, ri, *ref)


def test_c_abi_rejects_misaligned_packed(dev):
    lib = binding.load()
    c = inputs.random_case(64, 16, seed=6)
    t = to_dev(c, dev)
    buf = torch.empty(binding.fhd_packed_bytes(16) + 64, dtype=torch.uint8, device=dev)
    rc = lib.fhd_pack(*[t[k].data_ptr() for k in ("kx", "ky", "kz", "Dr", "Di")], 16,
                      buf.data_ptr() + 4, binding.fhd_packed_bytes(16), None)
    assert rc == binding.FHD_ERR_INVALID_ARG
    assert b"aligned" in lib.fhd_last_error()
