"""GPU parity of F^H D's matrix-core instance (units whose aligned 64-voxel
runs are lines along x with one step) against the fp64 oracle.

Gate as in test_gpu_parity: relative L2 error <= 5e-4 over the compared
voxels and every voxel's error <= 10x that times the reference's rms. The
instance computes in split bf16 (three bf16 products per fp32 product,
fp32 accumulation), about 1e-5 relative.
"""
import numpy as np
import pytest
import torch

from non_cartesian_mri_fhd_amd import layout
import oracle
from non_cartesian_mri_fhd_amd import binding, build, inputs, metrics

pytestmark = pytest.mark.gpu

REL_L2_TOL = 5e-4
ELEM_TOL = 10 * REL_L2_TOL
AX64 = (-0.5, 1.0 / 64, -0.5, 1.0 / 16, -0.25, 1.0 / 32)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    build.ensure_built()
    binding.load()
    return torch.device("cuda:0")


def gpu_fhd(case, dev):
    t = {k: torch.from_numpy(np.ascontiguousarray(case[k])).to(dev)
         for k in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")}
    rr, ri = binding.fhd_compute(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"],
                                 t["x"], t["y"], t["z"])
    torch.cuda.synchronize(dev)
    return rr.cpu().numpy(), ri.cpu().numpy()


def check(tag, case, rr, ri):
    ref_r, ref_i = oracle.fhd(case["kx"], case["ky"], case["kz"], case["Dr"], case["Di"],
                              case["x"], case["y"], case["z"])
    e = metrics.rel_l2(rr, ri, ref_r, ref_i)
    worst = metrics.max_abs_err(rr, ri, ref_r, ref_i)
    scale = metrics.rms(ref_r, ref_i)
    print("%s: rel_l2=%.3e max_err/rms=%.3e psnr=%.1f dB"
          % (tag, e, worst / scale, metrics.psnr_db(rr, ri, ref_r, ref_i)), flush=True)
    assert np.all(np.isfinite(rr)) and np.all(np.isfinite(ri))
    assert e <= REL_L2_TOL, (tag, e)
    assert worst <= ELEM_TOL * scale, (tag, worst, scale)
    return e


def classes(case):
    return layout.gather_unit_classes(case["x"], case["y"], case["z"])[0].tolist()


@pytest.mark.parametrize("shape,axis,M,cls", [
    ((64, 16, 8), AX64, 3000, [2, 2]),                                     # lines = rows
    ((128, 16, 4), (-0.5, 1.0 / 128, -0.5, 1.0 / 16, 0.0, 0.25), 1009, [3, 3]),   # tail of 3 chunks
    ((64, 32, 6), (0.25, -1.0 / 64, -0.5, 1.0 / 32, -0.5, 1.0 / 8), 5, [2, 2, 2]),  # negative step, one chunk
    ((256, 8, 4), (-0.5, 1.0 / 256, -0.5, 1.0 / 8, -0.5, 0.25), 1537, [3, 3]),    # half rows, 3 stages + 1
    ((128, 32, 3), (-0.5, 1.0 / 128, -0.5, 1.0 / 32, 0.0, 0.25), 272, [3, 3, 2]),  # lone last unit, tail of 2
    ((384, 8, 4), (-0.75, 1.0 / 256, -0.5, 1.0 / 8, -0.5, 0.25), 2000, [3, 3, 2]),
])
def test_lines_grids(dev, shape, axis, M, cls):
    x, y, z = inputs.coords_from_axis(*shape, axis)
    c = dict(inputs.random_case(1, M, seed=sum(shape) + M, kmax=min(shape[0], 256) / 2.0), x=x, y=y, z=z)
    assert classes(c) == cls
    rr, ri = gpu_fhd(c, dev)
    check("lines %s M=%d" % (shape, M), c, rr, ri)


def test_long_lines_against_lines(dev):
    """Rows of 128 (the long-line instance, unit pairs) and the same voxels
    with the two halves of every row swapped (64-voxel lines only: the
    single-unit matrix-core instance) meet the oracle gate and agree to
    rounding, not bitwise."""
    k = inputs.make_kspace("spiral32")
    x, y, z = inputs.coords_from_axis(128, 16, 4, (-0.5, 1.0 / 128, -0.5, 1.0 / 16, 0.0, 0.25))
    perm = np.arange(x.size).reshape(-1, 2, 64)[:, ::-1, :].reshape(-1)
    a = dict(k, x=x, y=y, z=z)
    b = dict(k, x=x[perm], y=y[perm], z=z[perm])
    assert classes(a) == [3, 3] and classes(b) == [2, 2]
    ra = gpu_fhd(a, dev)
    rb = gpu_fhd(b, dev)
    check("long lines", a, *ra)
    check("64-voxel lines", b, *rb)
    back = (np.empty_like(rb[0]), np.empty_like(rb[1]))
    back[0][perm], back[1][perm] = rb
    diff = metrics.rel_l2(ra[0], ra[1], back[0].astype(np.float64), back[1].astype(np.float64))
    print("long lines vs 64-voxel lines: rel diff %.2e" % diff)
    assert 0 < diff < 1e-4


def test_lines_spiral_kspace_and_ragged_tail(dev):
    """Stack-of-spirals samples on a 64 x 16 x 9 grid: two whole units of
    lines and a partial last unit on the VALU paths."""
    k = inputs.make_kspace("spiral32")
    x, y, z = inputs.coords_from_axis(64, 16, 9, AX64)
    c = dict(k, x=x, y=y, z=z)
    assert classes(c) == [2, 2, 0]
    rr, ri = gpu_fhd(c, dev)
    check("lines + tail", c, rr, ri)


def test_lines_against_one_step_form(dev):
    """The same voxels in two orders: rows of 64 (the matrix-core instance)
    and each 64-run made of 16-voxel pieces of four rows (the one-step ramp
    path). Both meet the oracle gate and agree to the split-bf16 rounding,
    but not bitwise (so the matrix-core instance did run)."""
    k = inputs.make_kspace("spiral32")
    x, y, z = inputs.coords_from_axis(64, 16, 8, AX64)
    perm = np.arange(x.size).reshape(-1, 4, 4, 16).transpose(0, 2, 1, 3).reshape(-1)
    a = dict(k, x=x, y=y, z=z)
    b = dict(k, x=x[perm], y=y[perm], z=z[perm])
    assert classes(a) == [2, 2] and classes(b) == [1, 1]
    ra = gpu_fhd(a, dev)
    rb = gpu_fhd(b, dev)
    check("lines order", a, *ra)
    check("one-step order", b, *rb)
    back = (np.empty_like(rb[0]), np.empty_like(rb[1]))
    back[0][perm], back[1][perm] = rb
    diff = metrics.rel_l2(ra[0], ra[1], back[0].astype(np.float64), back[1].astype(np.float64))
    print("lines vs one-step: rel diff %.2e" % diff)
    assert 0 < diff < 1e-4


def test_lines_units_of_different_steps(dev):
    """Unit 0: rows of 64 at step 1/64; unit 1: rows of 128 at 1/128 (each
    unit one step); unit 2: like unit 0 with one line at twice the step
    (not a lines unit: per-lane ramps); then 1000 random voxels."""
    xa, ya, za = inputs.coords_from_axis(64, 8, 8, AX64)
    xb, yb, zb = inputs.coords_from_axis(128, 8, 4, (-0.5, 1.0 / 128, -0.5, 1.0 / 8, 0.0, 0.125))
    xc, yc, zc = (a.copy() for a in inputs.coords_from_axis(64, 8, 8, (-0.375, 1.0 / 64, -0.5, 1.0 / 8, 0.25, 1.0 / 16)))
    xc[64 * 3:64 * 4] = (xc[64 * 3] + np.arange(64) * (2.0 / 64)).astype(np.float32)
    rng = np.random.default_rng(8)
    xr, yr, zr = rng.uniform(-0.5, 0.5, (3, 1000)).astype(np.float32)
    x, y, z = (np.concatenate(t) for t in ((xa, xb, xc, xr), (ya, yb, yc, yr), (za, zb, zc, zr)))
    c = dict(inputs.make_kspace("random16"), x=x, y=y, z=z)
    assert classes(c) == [2, 2, 0, 0]
    rr, ri = gpu_fhd(c, dev)
    check("mixed units", c, rr, ri)


def test_lines_zero_step_and_degenerate_angles(dev):
    """A step of zero (every voxel of a line at one x: all its voxels equal)
    and samples whose half-step angle kx dx / 2 is 0, 1/8, 1/4 or 1/2
    revolution (factors of exactly 0 and +-1)."""
    rng = np.random.default_rng(5)
    M = 2000
    kx = rng.choice(np.array([0.0, 16.0, 32.0, -32.0, 64.0, -0.5], np.float32), M)
    ky, kz = (rng.uniform(-16, 16, M).astype(np.float32) for _ in range(2))
    Dr, Di = (rng.standard_normal(M).astype(np.float32) for _ in range(2))
    x, y, z = inputs.coords_from_axis(64, 16, 8, AX64)
    c = dict(kx=kx, ky=ky, kz=kz, Dr=Dr, Di=Di, x=x, y=y, z=z)
    check("degenerate angles", c, *gpu_fhd(c, dev))
    # two units whose lines pair up (the 64-voxel line-pair instance): the
    # voxels of a line are equal in exact arithmetic; the two halves of a
    # line come from pair columns at +d/2 and -d/2, so they agree to
    # rounding only
    c0 = dict(c, x=np.full_like(x, np.float32(0.125)))
    assert classes(c0) == [2, 2]
    assert layout.line_pair64_pairs(c0["x"], c0["y"], c0["z"]).tolist() == [True]
    rr, ri = gpu_fhd(c0, dev)
    check("zero step, line pairs", c0, rr, ri)
    scale = np.sqrt(np.mean(rr.astype(np.float64) ** 2 + ri.astype(np.float64) ** 2))
    assert np.max(np.abs(rr.reshape(-1, 64) - rr.reshape(-1, 64)[:, :1])) <= 1e-5 * scale
    assert np.max(np.abs(ri.reshape(-1, 64) - ri.reshape(-1, 64)[:, :1])) <= 1e-5 * scale
    # four units in four-line groups (the line-pair instance's 64-voxel
    # form): likewise equal to rounding
    xg, yg, zg = inputs.coords_from_axis(64, 32, 8, AX64)
    cg = dict(c, x=np.full_like(xg, np.float32(0.125)), y=yg, z=zg)
    assert classes(cg) == [2, 2, 2, 2]
    assert layout.line_group64_quads(cg["x"], cg["y"], cg["z"]).tolist() == [True]
    rr, ri = gpu_fhd(cg, dev)
    check("zero step, four-line groups", cg, rr, ri)
    scale = np.sqrt(np.mean(rr.astype(np.float64) ** 2 + ri.astype(np.float64) ** 2))
    assert np.max(np.abs(rr.reshape(-1, 64) - rr.reshape(-1, 64)[:, :1])) <= 1e-5 * scale
    assert np.max(np.abs(ri.reshape(-1, 64) - ri.reshape(-1, 64)[:, :1])) <= 1e-5 * scale
    # one unit (the 64-voxel line instance): every pair column has the same
    # operands, so a line's voxels are equal bit for bit
    xs, ys, zs = inputs.coords_from_axis(64, 16, 4, AX64)
    c1 = dict(c, x=np.full_like(xs, np.float32(0.125)), y=ys, z=zs)
    assert classes(c1) == [2]
    rr, ri = gpu_fhd(c1, dev)
    check("zero step, single unit", c1, rr, ri)
    assert np.all(rr.reshape(-1, 64) == rr.reshape(-1, 64)[:, :1])
    assert np.all(ri.reshape(-1, 64) == ri.reshape(-1, 64)[:, :1])


def test_lines_zero_samples_and_repeatable(dev):
    x, y, z = inputs.coords_from_axis(64, 16, 8, AX64)
    empty = np.zeros(0, np.float32)
    c = dict(kx=empty, ky=empty, kz=empty, Dr=empty, Di=empty, x=x, y=y, z=z)
    rr, ri = gpu_fhd(c, dev)
    assert not np.any(rr) and not np.any(ri)
    c = dict(inputs.make_kspace("spiral32"), x=x, y=y, z=z)
    a = gpu_fhd(c, dev)
    b = gpu_fhd(c, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def gather_paths(case, dev, paths):
    t = {k: torch.from_numpy(np.ascontiguousarray(case[k])).to(dev)
         for k in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")}
    M = t["kx"].numel()
    packed = binding.new_packed(M, dev)
    binding.fhd_pack(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], packed)
    rr, ri = binding.fhd_gather(packed, M, t["x"], t["y"], t["z"], paths=paths)
    torch.cuda.synchronize(dev)
    return rr.cpu().numpy(), ri.cpu().numpy()


def test_vector_paths_option(dev):
    """fhd_gather_paths: FHD_GATHER_ALL is fhd_gather bitwise; with
    FHD_GATHER_VECTOR the rows-of-64 order takes the one-step ramp path,
    bitwise equal to the same lanes in the order whose units are one-step
    anyway, and differs from the matrix-core result only by rounding."""
    k = inputs.make_kspace("spiral32")
    x, y, z = inputs.coords_from_axis(64, 16, 8, AX64)
    perm = np.arange(x.size).reshape(-1, 4, 4, 16).transpose(0, 2, 1, 3).reshape(-1)
    a = dict(k, x=x, y=y, z=z)
    b = dict(k, x=x[perm], y=y[perm], z=z[perm])
    full = gpu_fhd(a, dev)
    every = gather_paths(a, dev, binding.FHD_GATHER_ALL)
    assert np.array_equal(full[0], every[0]) and np.array_equal(full[1], every[1])
    vec = gather_paths(a, dev, binding.FHD_GATHER_VECTOR)
    check("vector paths", a, *vec)
    one = gather_paths(b, dev, binding.FHD_GATHER_ALL)
    back = (np.empty_like(one[0]), np.empty_like(one[1]))
    back[0][perm], back[1][perm] = one
    assert np.array_equal(vec[0], back[0]) and np.array_equal(vec[1], back[1])
    diff = metrics.rel_l2(full[0], full[1], vec[0].astype(np.float64), vec[1].astype(np.float64))
    assert 0 < diff < 1e-4


def test_gather_paths_rejects_unknown_mode(dev):
    import ctypes
    lib = binding.load()
    x, y, z = (torch.from_numpy(a).to(dev) for a in inputs.coords_from_axis(64, 8, 8, AX64))
    out = [torch.empty(x.numel(), device=dev) for _ in range(2)]
    packed = binding.new_packed(8, dev)
    rc = lib.fhd_gather_paths(packed.data_ptr(), 8, x.data_ptr(), y.data_ptr(), z.data_ptr(),
                              out[0].data_ptr(), out[1].data_ptr(), x.numel(), 3, None)
    assert rc == binding.FHD_ERR_INVALID_ARG
    assert b"paths" in ctypes.string_at(lib.fhd_last_error())


def test_long_lines_table_and_in_kernel_factors_agree_bitwise(dev):
    """The long-line instance takes its B factors from a table formed once
    per call for the first pair's step, and forms them itself in pairs of
    another step: the same arithmetic either way. Two pairs of units (steps
    1/128 and 1/256) in both orders: each pair's result is bitwise the same
    whichever way its factors were formed."""
    ga = inputs.coords_from_axis(128, 16, 4, (-0.5, 1.0 / 128, -0.5, 1.0 / 16, 0.0, 0.25))
    gb = inputs.coords_from_axis(128, 16, 4, (-0.25, 1.0 / 256, -0.5, 1.0 / 16, 0.125, 0.25))
    k = inputs.make_kspace("spiral32")
    one = dict(k, **{n: np.concatenate((a, b)) for n, a, b in zip("xyz", ga, gb)})
    two = dict(k, **{n: np.concatenate((b, a)) for n, a, b in zip("xyz", ga, gb)})
    assert classes(one) == [3, 3, 3, 3] and classes(two) == [3, 3, 3, 3]
    r1 = gpu_fhd(one, dev)
    r2 = gpu_fhd(two, dev)
    check("two steps", one, *r1)
    h = ga[0].size
    for p in range(2):
        assert np.array_equal(r1[p][:h], r2[p][h:]) and np.array_equal(r1[p][h:], r2[p][:h])


def test_long_pairs_then_a_ragged_partial_unit(dev):
    """Two long-line pairs followed by 100 random voxels (a partial third
    pair's first unit): the partial unit takes a vector path, the pairs the
    long-line form; the whole result meets the oracle gate."""
    g = inputs.coords_from_axis(128, 32, 4, (-0.5, 1.0 / 128, -0.5, 1.0 / 32, 0.0, 0.25))
    r = inputs.random_case(100, 1, seed=77)
    x, y, z = (np.concatenate((a, r[n])) for a, n in zip(g, ("x", "y", "z")))
    c = dict(inputs.random_case(1, 700, seed=78, kmax=64.0), x=x, y=y, z=z)
    assert classes(c)[:4] == [3, 3, 3, 3] and classes(c)[4] != 3
    rr, ri = gpu_fhd(c, dev)
    check("long pairs + ragged unit", c, rr, ri)
