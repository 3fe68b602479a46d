"""The arithmetic of the matrix-core line forms, through the C ABI.

The default paths (FHD_GATHER_ALL) sum lines of voxels along x on the matrix
cores with each fp32 operand split into an fp16 part and an fp16 remainder
(three products per fp32 product): fp32-class products. FHD_GATHER_BF16X3
is the same form with bf16 parts (16 significant bits), FHD_GATHER_VECTOR
the fp32 vector-ALU paths.

On inputs whose phases are exact in fp32 (integer k, dyadic voxel
coordinates, D on the real and imaginary axes) the fp32 phase rounding,
which dominates every path's error on the benchmark workloads, is absent,
so what is left is the arithmetic of the products and the hardware
sine/cosine: there the default path must be as accurate as the fp32 vector
paths (within 2x of their error), while the split-bf16 form is measurably
worse. Power-of-two scaling of D (or of the image, for F) must scale the
result exactly, since the fp16 form rescales by powers of two.
"""
import numpy as np
import pytest
import torch

import oracle
from non_cartesian_mri_fhd_amd import binding, build, inputs, layout, metrics

pytestmark = pytest.mark.gpu

REL_L2_TOL = 5e-4
# 128 x 16 x 4 voxels: one aligned pair of 4096-voxel units whose rows are
# lines of 128 (the long-line instance), x = (i - 64) / 128 exactly
LINES128 = ((128, 16, 4), (-0.5, 1.0 / 128, -0.5, 1.0 / 16, -0.5, 0.25))
# 64 x 16 x 8: two units of 64-voxel lines (the 64-voxel instance)
LINES64 = ((64, 16, 8), (-0.5, 1.0 / 64, -0.5, 1.0 / 16, -0.5, 0.125))
# four units of 64-voxel lines in four-line groups (rows y .. y + 3: the
# line-pair instance's 64-voxel form)
GROUPS64 = ((64, 32, 8), (-0.5, 1.0 / 64, -0.5, 1.0 / 32, -0.5, 0.125))
# one unit of 64-voxel lines, no pair (the 64-voxel line instance)
LINES64_SOLO = ((64, 16, 4), (-0.5, 1.0 / 64, -0.5, 1.0 / 16, -0.5, 0.25))
# one quad of four units whose lines pair up (the line-pair instance):
# rows of 128 one step apart along y, and rows of 256 (halves along x)
PAIRS_Y = ((128, 32, 4), (-0.5, 1.0 / 128, -0.5, 1.0 / 32, -0.5, 0.25))
PAIRS_X = ((256, 16, 4), (-0.5, 1.0 / 256, -0.5, 1.0 / 16, -0.5, 0.25))
PATHS = {"all": binding.FHD_GATHER_ALL, "vector": binding.FHD_GATHER_VECTOR,
         "bf16x3": binding.FHD_GATHER_BF16X3}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    build.ensure_built()
    binding.load()
    return torch.device("cuda:0")


def exact_phase_case(grid, M, seed):
    """Integer k inside the grid's Nyquist box and D on the axes: every
    phase k.x + arg(D)/2pi, and every pair factor's argument, is an exact
    fp32 value (a multiple of 1/256 below 2^8 in magnitude)."""
    shape, axis = grid
    x, y, z = inputs.coords_from_axis(*shape, axis)
    rng = np.random.default_rng(seed)
    kx, ky, kz = (rng.integers(-n // 2, n // 2, M).astype(np.float32) for n in shape)
    a = rng.uniform(0.5, 2.0, M)
    which = rng.integers(0, 4, M)
    Dr = np.where(which == 0, a, np.where(which == 1, -a, 0.0)).astype(np.float32)
    Di = np.where(which == 2, a, np.where(which == 3, -a, 0.0)).astype(np.float32)
    return dict(kx=kx, ky=ky, kz=kz, Dr=Dr, Di=Di, x=x, y=y, z=z)


def to_dev(case, dev):
    return {k: torch.from_numpy(np.ascontiguousarray(case[k])).to(dev)
            for k in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")}


def fhd(case, dev, paths):
    d = to_dev(case, dev)
    rr, ri = binding.fhd_compute(d["kx"], d["ky"], d["kz"], d["Dr"], d["Di"], d["x"], d["y"], d["z"],
                                 paths=PATHS[paths])
    torch.cuda.synchronize(dev)
    return rr.cpu().numpy(), ri.cpu().numpy()


def forward(case, img, dev, paths):
    d = to_dev(case, dev)
    ir, ii = (torch.from_numpy(a).to(dev) for a in img)
    Dr, Di = binding.fhd_forward(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], ir, ii,
                                 paths=PATHS[paths])
    torch.cuda.synchronize(dev)
    return Dr.cpu().numpy(), Di.cpu().numpy()


@pytest.mark.parametrize("grid,cls,quads,pairs64", [(LINES128, [3, 3], [], [False]),
                                                    (LINES64, [2, 2], [], [True]),
                                                    (GROUPS64, [2, 2, 2, 2], [False], [False, False]),
                                                    (LINES64_SOLO, [2], [], []),
                                                    (PAIRS_Y, [3, 3, 3, 3], [True], [False, False]),
                                                    (PAIRS_X, [3, 3, 3, 3], [True], [False, False])])
def test_adjoint_line_form_is_fp32_class(dev, grid, cls, quads, pairs64):
    c = exact_phase_case(grid, 3001, seed=910)
    assert layout.gather_unit_classes(c["x"], c["y"], c["z"])[0].tolist() == cls
    assert layout.line_pair_quads(c["x"], c["y"], c["z"]).tolist() == quads
    assert layout.line_pair64_pairs(c["x"], c["y"], c["z"]).tolist() == pairs64
    groups = layout.line_group64_quads(c["x"], c["y"], c["z"]).tolist()
    assert groups == ([True] if grid is GROUPS64 else [False] * len(groups))
    ref = oracle.fhd(c["kx"], c["ky"], c["kz"], c["Dr"], c["Di"], c["x"], c["y"], c["z"])
    err = {}
    for p in PATHS:
        rr, ri = fhd(c, dev, p)
        err[p] = metrics.rel_l2(rr, ri, *ref)
    print("exact phases, F^H D on %s voxels: rel-L2 %s" % (grid[0], err), flush=True)
    assert max(err.values()) <= REL_L2_TOL
    assert err["all"] <= 2.0 * err["vector"], err
    # the opt-in split-bf16 form carries 16-bit operands: the test tells
    # the two splits apart
    assert err["bf16x3"] > 2.0 * err["vector"], err


@pytest.mark.parametrize("form", ["pairs", "lines", "groups"])
def test_forward_line_form_is_fp32_class(dev, form):
    c = exact_phase_case(GROUPS64 if form == "groups" else LINES128, 2003, seed=911)
    if form == "lines":
        # rows swapped two by two: the line form (the line-pair form's
        # common offset broken)
        rows = np.arange(c["x"].size // 128)
        rows[2::4], rows[3::4] = rows[3::4].copy(), rows[2::4].copy()
        perm = (rows[:, None] * 128 + np.arange(128)).reshape(-1)
        c = dict(c, x=c["x"][perm], y=c["y"][perm], z=c["z"][perm])
    assert layout.forward_lines_form(c["x"], c["y"], c["z"]) == (form != "groups")
    assert layout.forward_pairs_form(c["x"], c["y"], c["z"]) == (form != "lines")
    # an image of dyadic values: rho enters the sums exactly
    rng = np.random.default_rng(912)
    img = tuple((rng.integers(-512, 512, c["x"].size) / 256.0).astype(np.float32) for _ in range(2))
    ref = oracle.forward(c["kx"], c["ky"], c["kz"], img[0], img[1], c["x"], c["y"], c["z"])
    err = {}
    for p in PATHS:
        Dr, Di = forward(c, img, dev, p)
        err[p] = metrics.rel_l2(Dr, Di, *ref)
    print("exact phases, F on 128-voxel lines (%s form): rel-L2 %s" % (form, err), flush=True)
    assert max(err.values()) <= REL_L2_TOL
    assert err["all"] <= 2.0 * err["vector"], err
    assert err["bf16x3"] > 2.0 * err["vector"], err


@pytest.mark.parametrize("grid", [LINES128, LINES64, LINES64_SOLO, PAIRS_Y, GROUPS64])
def test_amplitude_scaling_is_exact(dev, grid):
    """F^H (2^e D) = 2^e F^H D bit for bit on every path, for scales that
    move the largest |D| far outside fp16's range in both directions."""
    c = inputs.random_case(1, 1500, seed=913, kmax=grid[0][0] / 2.0)
    x, y, z = inputs.coords_from_axis(*grid[0], grid[1])
    c = dict(c, x=x, y=y, z=z)
    for p in PATHS:
        base = fhd(c, dev, p)
        for e in (-100, -20, 40, 90):
            s = np.float32(2.0 ** e)
            got = fhd(dict(c, Dr=c["Dr"] * s, Di=c["Di"] * s), dev, p)
            assert np.array_equal(got[0], base[0] * s) and np.array_equal(got[1], base[1] * s), (p, e)


def test_forward_image_scaling_is_exact(dev):
    """F (2^e rho) = 2^e F rho bit for bit (each line's own power-of-two
    scale), also when one line's values are 2^60 times the others'."""
    c = inputs.random_case(1, 700, seed=914, kmax=8.0)
    x, y, z = inputs.coords_from_axis(*LINES128[0], LINES128[1])
    c = dict(c, x=x, y=y, z=z)
    img = inputs.random_image(x.size, seed=915)
    for p in PATHS:
        base = forward(c, img, dev, p)
        for e in (-90, 70):
            s = np.float32(2.0 ** e)
            got = forward(c, (img[0] * s, img[1] * s), dev, p)
            assert np.array_equal(got[0], base[0] * s) and np.array_equal(got[1], base[1] * s), (p, e)
    loud = (img[0].copy(), img[1].copy())
    loud[0][128 * 7:128 * 8] *= np.float32(2.0 ** 60)
    loud[1][128 * 7:128 * 8] *= np.float32(2.0 ** 60)
    ref = oracle.forward(c["kx"], c["ky"], c["kz"], loud[0], loud[1], x, y, z)
    got = forward(c, loud, dev, "all")
    assert metrics.rel_l2(*got, *ref) <= REL_L2_TOL


def test_adjoint_wide_dynamic_range_and_tiny_amplitudes(dev):
    """Samples whose |D| spans 2^-60 .. 2^40 of each other, and a k-space of
    amplitudes around 1e-30 (far below fp16's range): the fp16 form's one
    power-of-two scale per call keeps every term's error at fp32 level
    relative to the largest amplitude."""
    shape, axis = LINES128
    x, y, z = inputs.coords_from_axis(*shape, axis)
    c = inputs.random_case(1, 2000, seed=916, kmax=32.0)
    rng = np.random.default_rng(917)
    mag = (2.0 ** rng.uniform(-60, 40, 2000)).astype(np.float32)
    wide = dict(c, Dr=c["Dr"] * mag, Di=c["Di"] * mag, x=x, y=y, z=z)
    tiny = dict(c, Dr=c["Dr"] * np.float32(1e-30), Di=c["Di"] * np.float32(1e-30), x=x, y=y, z=z)
    for case in (wide, tiny):
        ref = oracle.fhd(case["kx"], case["ky"], case["kz"], case["Dr"], case["Di"], x, y, z)
        for p in ("all", "vector"):
            got = fhd(case, dev, p)
            e = metrics.rel_l2(*got, *ref)
            print("dynamic range case, %s: rel-L2 %.3e" % (p, e), flush=True)
            assert e <= REL_L2_TOL, (p, e)


def test_zero_and_single_nonzero_amplitude(dev):
    """All-zero D gives exact zeros; one non-zero sample gives its pure phase
    ramp, |rho_n| = |D| everywhere, on the line form."""
    shape, axis = LINES128
    x, y, z = inputs.coords_from_axis(*shape, axis)
    c = inputs.random_case(1, 777, seed=918, kmax=16.0)
    zero = dict(c, Dr=np.zeros_like(c["Dr"]), Di=np.zeros_like(c["Di"]), x=x, y=y, z=z)
    for p in PATHS:
        rr, ri = fhd(zero, dev, p)
        assert not rr.any() and not ri.any(), p
    one = dict(zero, Dr=zero["Dr"].copy(), Di=zero["Di"].copy())
    one["Dr"][400], one["Di"][400] = np.float32(3.0), np.float32(-4.0)
    rr, ri = fhd(one, dev, "all")
    assert np.allclose(np.hypot(rr.astype(np.float64), ri), 5.0, rtol=2e-6)
    ref = oracle.fhd(one["kx"], one["ky"], one["kz"], one["Dr"], one["Di"], x, y, z)
    assert metrics.rel_l2(rr, ri, *ref) <= 1e-5
