"""GPU parity of the forward operator F in its matrix-core forms against
the fp64 oracle, against each other and the vector form on the same
voxels, and through adjointness with F^H D. The line form takes F when
every aligned pair of 4096-voxel units is lines of 128 voxels along x with
one step; the line-pair form when, beyond that, the lines 2i + 1 are the
lines 2i moved by one common offset (rows one step apart, or the halves of
rows of 256), and also when the units are 64-voxel lines in four-line
groups at 0, d, e and e + d (rows y .. y + 3 of a grid with rows of 64).
Swapping the rows two by two keeps the line form's rule and breaks the
line-pair form's.

Gate as in test_gpu_parity: relative L2 <= 5e-4 and every element within
10x that bound times the reference's rms. Both forms compute in split
fp16 by default (three fp16 products per fp32 product, fp32
accumulation).
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
AX128 = (-0.5, 1.0 / 128, -0.5, 1.0 / 16, 0.0, 0.25)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    build.ensure_built()
    binding.load()
    return torch.device("cuda:0")


def t(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gpu_forward(k, x, y, z, img, dev):
    Dr, Di = binding.fhd_forward(t(k["kx"], dev), t(k["ky"], dev), t(k["kz"], dev), t(x, dev), t(y, dev),
                                 t(z, dev), t(img[0], dev), t(img[1], dev))
    torch.cuda.synchronize(dev)
    return Dr.cpu().numpy(), Di.cpu().numpy()


def check(tag, k, x, y, z, img, Dr, Di):
    ref_r, ref_i = oracle.forward(k["kx"], k["ky"], k["kz"], img[0], img[1], x, y, z)
    e = metrics.rel_l2(Dr, Di, ref_r, ref_i)
    worst = metrics.max_abs_err(Dr, Di, ref_r, ref_i)
    scale = metrics.rms(ref_r, ref_i)
    print("%s: rel_l2=%.3e max_err/rms=%.3e" % (tag, e, worst / scale), flush=True)
    assert np.all(np.isfinite(Dr)) and np.all(np.isfinite(Di))
    assert e <= REL_L2_TOL, (tag, e)
    assert worst <= ELEM_TOL * scale, (tag, worst, scale)
    return e


def all_long_pairs(x, y, z):
    cls = layout.gather_unit_classes(x, y, z)[0]
    return cls.size > 0 and bool(np.all(cls == 3))


def swap_rows(n):
    """Voxel order with the 128-voxel rows swapped two by two (rows 0, 1,
    3, 2, 4, 5, 7, 6, ...): line pairs (2i, 2i + 1) then alternate between
    two offsets."""
    rows = np.arange(n // 128)
    rows[2::4], rows[3::4] = rows[3::4].copy(), rows[2::4].copy()
    return (rows[:, None] * 128 + np.arange(128)).reshape(-1)


@pytest.mark.parametrize("form", ["pairs", "lines"])
@pytest.mark.parametrize("shape,axis,M", [
    ((128, 16, 4), AX128, 3000),                                           # one pair of units
    ((256, 16, 6), (-0.5, 1.0 / 256, -0.5, 1.0 / 16, -0.5, 1.0 / 6), 1000),   # 3 pairs, half rows
    ((128, 32, 2), (0.25, -1.0 / 128, -0.5, 1.0 / 32, 0.0, 0.5), 129),      # negative step, ragged M
    ((128, 16, 4), AX128, 1),
])
def test_forward_lines_grids(dev, shape, axis, M, form):
    x, y, z = inputs.coords_from_axis(*shape, axis)
    if form == "lines":
        perm = swap_rows(x.size)
        x, y, z = x[perm], y[perm], z[perm]
    assert all_long_pairs(x, y, z)
    assert layout.forward_pairs_form(x, y, z) == (form == "pairs")
    k = inputs.random_case(1, M, seed=sum(shape) + M, kmax=shape[0] / 2.0)
    img = inputs.random_image(x.size, seed=M + 5)
    check("forward %s %s M=%d" % (form, shape, M), k, x, y, z, img, *gpu_forward(k, x, y, z, img, dev))


@pytest.mark.parametrize("shape,M", [((64, 32, 4), 3000),   # one unit pair of groups
                                     ((64, 64, 8), 1500),   # four unit pairs
                                     ((64, 2, 64), 777)])   # groups across two slices
def test_forward_groups_of_64_voxel_lines(dev, shape, M):
    axis = (-0.5, 1.0 / shape[0], -0.5, 1.0 / shape[1], -0.5, 1.0 / shape[2])
    x, y, z = inputs.coords_from_axis(*shape, axis)
    assert np.all(layout.gather_unit_classes(x, y, z)[0] == 2)
    assert layout.forward_pairs_form(x, y, z) and not layout.forward_lines_form(x, y, z)
    k = inputs.random_case(1, M, seed=sum(shape) + M, kmax=shape[0] / 2.0)
    img = inputs.random_image(x.size, seed=M + 7)
    check("forward groups %s M=%d" % (shape, M), k, x, y, z, img, *gpu_forward(k, x, y, z, img, dev))


def test_forward_groups_against_vector_form(dev):
    """Rows of 64 in four-line groups (the line-pair form) and the same
    voxels with one group's second line pair moved apart from the rest in
    the order (groups broken: the vector form) give the same D to
    rounding; a grid whose groups differ from pair 0's takes the vector
    form too."""
    k = inputs.make_kspace("spiral32")
    x, y, z = inputs.coords_from_axis(64, 32, 8, (-0.5, 1.0 / 64, -0.5, 1.0 / 32, -0.5, 0.125))
    img = inputs.random_image(x.size, seed=35)
    # lines 2, 3 after lines 4 .. 7: the first two groups' e are then +4
    # and -4 rows
    perm = np.arange(x.size).reshape(-1, 64)
    perm = np.concatenate([perm[:2], perm[4:8], perm[2:4], perm[8:]]).reshape(-1)
    assert layout.forward_pairs_form(x, y, z)
    assert not layout.forward_pairs_form(x[perm], y[perm], z[perm])
    a = gpu_forward(k, x, y, z, img, dev)
    b = gpu_forward(k, x[perm], y[perm], z[perm], (img[0][perm], img[1][perm]), dev)
    check("groups", k, x, y, z, img, *a)
    check("groups broken", k, x[perm], y[perm], z[perm], (img[0][perm], img[1][perm]), *b)
    diff = metrics.rel_l2(a[0], a[1], b[0].astype(np.float64), b[1].astype(np.float64))
    print("groups vs vector form: rel diff %.2e" % diff)
    assert 0 < diff < 2e-5


def test_forward_pairs_against_line_form(dev):
    """The same voxels and image in row order (the line-pair form) and with
    the rows swapped two by two (the line form) give the same D to
    rounding, not bitwise (one phasor per line pair against one per line)."""
    k = inputs.make_kspace("spiral32")
    x, y, z = inputs.coords_from_axis(128, 32, 4, (-0.5, 1.0 / 128, -0.5, 1.0 / 32, -0.5, 0.25))
    img = inputs.random_image(x.size, seed=33)
    perm = swap_rows(x.size)
    assert layout.forward_pairs_form(x, y, z)
    assert layout.forward_lines_form(x[perm], y[perm], z[perm])
    assert not layout.forward_pairs_form(x[perm], y[perm], z[perm])
    a = gpu_forward(k, x, y, z, img, dev)
    b = gpu_forward(k, x[perm], y[perm], z[perm], (img[0][perm], img[1][perm]), dev)
    check("line-pair form", k, x, y, z, img, *a)
    diff = metrics.rel_l2(a[0], a[1], b[0].astype(np.float64), b[1].astype(np.float64))
    print("line-pair vs line form: rel diff %.2e" % diff)
    assert 0 < diff < 2e-5


def test_forward_lines_against_vector_form(dev):
    """Rows of 128 (the line-pair form) and the same voxels with the two
    halves of every row swapped (64-voxel lines only: the vector form) meet
    the oracle gate and agree to rounding, not bitwise."""
    k = inputs.make_kspace("spiral32")
    x, y, z = inputs.coords_from_axis(128, 16, 4, AX128)
    perm = np.arange(x.size).reshape(-1, 2, 64)[:, ::-1, :].reshape(-1)
    img = inputs.random_image(x.size, seed=31)
    pimg = (img[0][perm], img[1][perm])
    assert all_long_pairs(x, y, z) and not all_long_pairs(x[perm], y[perm], z[perm])
    a = gpu_forward(k, x, y, z, img, dev)
    b = gpu_forward(k, x[perm], y[perm], z[perm], pimg, dev)
    check("line-pair form", k, x, y, z, img, *a)
    check("vector form", k, x[perm], y[perm], z[perm], pimg, *b)
    diff = metrics.rel_l2(a[0], a[1], b[0].astype(np.float64), b[1].astype(np.float64))
    print("line-pair vs vector form: rel diff %.2e" % diff)
    assert 0 < diff < 1e-4


def test_forward_lines_fall_back_on_a_second_step(dev):
    """Two pairs of units of different steps: not one step throughout, so
    the vector form takes F (bitwise the two-stage vector entry points)."""
    ga = inputs.coords_from_axis(128, 16, 4, AX128)
    gb = inputs.coords_from_axis(128, 16, 4, (-0.25, 1.0 / 256, -0.5, 1.0 / 16, 0.125, 0.25))
    x, y, z = (np.concatenate((a, b)) for a, b in zip(ga, gb))
    assert all_long_pairs(x, y, z)
    k = inputs.make_kspace("random16")
    img = inputs.random_image(x.size, seed=8)
    a = gpu_forward(k, x, y, z, img, dev)
    check("two steps", k, x, y, z, img, *a)
    packed = binding.new_packed(x.size, dev)
    binding.fhd_forward_pack(t(x, dev), t(y, dev), t(z, dev), t(img[0], dev), t(img[1], dev), packed)
    g = binding.fhd_forward_gather(packed, x.size, t(k["kx"], dev), t(k["ky"], dev), t(k["kz"], dev))
    torch.cuda.synchronize(dev)
    assert np.array_equal(a[0], g[0].cpu().numpy()) and np.array_equal(a[1], g[1].cpu().numpy())


def test_forward_lines_adjointness_and_normal(dev):
    """<F^H D, rho> = <D, F rho> with both operators in their line forms
    (F in its line-pair form), and F^H F p against the oracle's
    composition."""
    x, y, z = inputs.coords_from_axis(128, 16, 4, AX128)
    c = inputs.random_case(1, 2000, seed=41, kmax=32.0)
    img = inputs.random_image(x.size, seed=42)
    d = {n: t(c[n], dev) for n in ("kx", "ky", "kz", "Dr", "Di")}
    X, Y, Z = t(x, dev), t(y, dev), t(z, dev)
    rr, ri = binding.fhd_compute(d["kx"], d["ky"], d["kz"], d["Dr"], d["Di"], X, Y, Z)
    Fr, Fi = binding.fhd_forward(d["kx"], d["ky"], d["kz"], X, Y, Z, t(img[0], dev), t(img[1], dev))
    qr, qi = binding.fhd_normal(d["kx"], d["ky"], d["kz"], X, Y, Z, t(img[0], dev), t(img[1], dev))
    torch.cuda.synchronize(dev)
    rho = img[0].astype(np.float64) + 1j * img[1].astype(np.float64)
    D = c["Dr"].astype(np.float64) + 1j * c["Di"].astype(np.float64)
    lhs = np.vdot(rho, rr.cpu().numpy().astype(np.float64) + 1j * ri.cpu().numpy())
    rhs = np.vdot(Fr.cpu().numpy().astype(np.float64) + 1j * Fi.cpu().numpy(), D)
    scale = np.linalg.norm(rho) * np.linalg.norm(D) * np.sqrt(2000)
    assert abs(lhs - rhs) <= 1e-4 * scale, (lhs, rhs)
    Dr_ref, Di_ref = oracle.forward(c["kx"], c["ky"], c["kz"], img[0], img[1], x, y, z)
    q_ref = oracle.fhd(c["kx"], c["ky"], c["kz"], Dr_ref.astype(np.float32), Di_ref.astype(np.float32), x, y, z)
    e = metrics.rel_l2(qr.cpu().numpy(), qi.cpu().numpy(), *q_ref)
    print("normal, line forms: rel_l2=%.3e" % e)
    assert e <= REL_L2_TOL


def test_forward_lines_zero_image_and_repeatable(dev):
    x, y, z = inputs.coords_from_axis(128, 16, 4, AX128)
    k = inputs.make_kspace("spiral32")
    zero = (np.zeros(x.size, np.float32), np.zeros(x.size, np.float32))
    Dr, Di = gpu_forward(k, x, y, z, zero, dev)
    assert not np.any(Dr) and not np.any(Di)
    img = inputs.random_image(x.size, seed=3)
    a = gpu_forward(k, x, y, z, img, dev)
    b = gpu_forward(k, x, y, z, img, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
