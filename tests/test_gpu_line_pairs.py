"""The line-pair matrix-core instances of F^H D, through the C ABI.

Quads of four units whose lines of 128 voxels, two by two, are one line and
the same line moved by a common offset d (rows of a grid along y, or the
two halves of rows of 256 along x) are summed about each line pair's
centre; so are quads of 64-voxel lines in groups of four at 0, d, e and
e + d (rows of 64: rows y .. y + 3), about each group's centre, and unit
pairs whose lines of 64 voxels only pair up. Each case states which quads
or pairs the instances take (the host mirror of the classification,
layout.line_pair_quads / line_group64_quads / line_pair64_pairs) and
checks every voxel against the oracle; groups that break the structure
fall back to the long-line (or 64-voxel line-pair, or 64-voxel line)
instance.
fhd_compute_noalloc forms the B operands itself and takes every group with
the structure: where both forms take the same groups its output is
bitwise fhd_compute's.
"""
import numpy as np
import pytest
import torch

import oracle
from non_cartesian_mri_fhd_amd import binding, build, inputs, layout, metrics

pytestmark = pytest.mark.gpu

TOL = 5e-4


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    build.ensure_built()
    binding.load()
    return torch.device("cuda:0")


def grid_case(shape, M, seed, kmax=None):
    nx, ny, nz = shape
    x, y, z = inputs.coords_from_axis(nx, ny, nz, (-0.5, 1.0 / nx, -0.5, 1.0 / ny, -0.5, 1.0 / nz))
    rng = np.random.default_rng(seed)
    km = kmax if kmax is not None else min(shape) / 2.0
    kx, ky, kz = (rng.uniform(-km, km, M).astype(np.float32) for _ in range(3))
    Dr, Di = (rng.standard_normal(M).astype(np.float32) for _ in range(2))
    return dict(kx=kx, ky=ky, kz=kz, Dr=Dr, Di=Di, x=x, y=y, z=z)


def run(case, dev, paths=binding.FHD_GATHER_ALL, noalloc=False):
    t = [torch.from_numpy(np.ascontiguousarray(case[k])).to(dev)
         for k in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")]
    N = t[5].numel()
    if noalloc:
        rr, ri = torch.empty(N, device=dev), torch.empty(N, device=dev)
        binding.fhd_compute_noalloc(*t, rr, ri, paths=paths)
    else:
        rr, ri = binding.fhd_compute(*t, paths=paths)
    torch.cuda.synchronize(dev)
    return rr.cpu().numpy(), ri.cpu().numpy()


def bend_rows(case, first_line, count, amount, line=128):
    """Moves lines first_line .. first_line + count - 1 (of `line` voxels)
    by `amount` along y, breaking the common line-pair offset there (or,
    moving a whole line pair, only the four-line groups' second offset)."""
    y = case["y"].copy()
    for ln in range(first_line, first_line + count):
        y[ln * line:(ln + 1) * line] += np.float32(amount)
    case["y"] = y
    return case


def cases64():
    # 64-voxel lines: (name, case, four-line groups taken by quad, in the
    # table form and formed; unit pairs taken by the 64-voxel line-pair
    # instance, in the table form and formed). One unit pair (no quad);
    # one quad; two quads; the second quad's first pair bent in one line
    # (its other pair goes to the 64-voxel line-pair instance in the formed
    # form; in the table form that instance's pair 0, inside a group, takes
    # no table, so the line instance takes both); the first quad so bent
    # (no group and no pair in the table forms; quad 1 and pair 1 in the
    # formed ones); one group's second pair moved together (its quad's
    # records flag 2 only: the 64-voxel line-pair instance takes both pairs)
    yield "64x32x4", grid_case((64, 32, 4), 3001, 970), [], [], [True], [True]
    yield "64x64x4", grid_case((64, 64, 4), 2048, 971), [True], [True], [False, False], [False, False]
    yield ("64x64x8", grid_case((64, 64, 8), 2048, 974), [True, True], [True, True],
           [False] * 4, [False] * 4)
    c = bend_rows(grid_case((64, 64, 8), 2048, 972), 256 + 1, 1, 1.0 / 512, line=64)
    yield "second quad bent", c, [True, False], [True, False], [False] * 4, [False, False, False, True]
    c = bend_rows(grid_case((64, 64, 8), 2048, 973), 3, 1, 1.0 / 512, line=64)
    yield "first quad bent", c, [False, False], [False, True], [False] * 4, [False, True, False, False]
    c = bend_rows(grid_case((64, 64, 4), 2048, 975), 2, 2, 1.0 / 512, line=64)
    yield "second offset broken", c, [False], [False], [True, True], [True, True]


def cases():
    # one quad of rows along y; one quad of 256-voxel rows (d along x); two
    # quads; two quads, the second bent (long lines there); the first bent
    # (no quad in the table form, the second in the formed one)
    yield "128x32x4", grid_case((128, 32, 4), 3001, 960), [True], [True]
    yield "256x16x4", grid_case((256, 16, 4), 2999, 961), [True], [True]
    yield "128x64x4", grid_case((128, 64, 4), 2048, 962), [True, True], [True, True]
    c = bend_rows(grid_case((128, 64, 4), 2048, 963), 128 + 1, 1, 1.0 / 512)
    yield "second quad bent", c, [True, False], [True, False]
    c = bend_rows(grid_case((128, 64, 4), 2048, 964), 3, 1, 1.0 / 512)
    yield "first quad bent", c, [False, False], [False, True]


@pytest.mark.parametrize("name,case,taken,formed", list(cases()), ids=[c[0] for c in cases()])
def test_line_pairs_match_the_oracle(dev, name, case, taken, formed):
    cls = layout.gather_unit_classes(case["x"], case["y"], case["z"])[0]
    assert np.all(cls == 3), (name, cls)
    assert layout.line_pair_quads(case["x"], case["y"], case["z"], cls).tolist() == taken, name
    assert layout.line_pair_quads(case["x"], case["y"], case["z"], cls, formed=True).tolist() == formed, name
    ref = oracle.fhd(case["kx"], case["ky"], case["kz"], case["Dr"], case["Di"], case["x"], case["y"], case["z"])
    print("line pairs: %s" % name, flush=True)
    got = run(case, dev)
    e = metrics.rel_l2(*got, *ref)
    vec = metrics.rel_l2(*run(case, dev, binding.FHD_GATHER_VECTOR), *ref)
    na = run(case, dev, noalloc=True)
    e_na = metrics.rel_l2(*na, *ref)
    print("  rel-L2 default %.3g, vector %.3g, noalloc %.3g" % (e, vec, e_na), flush=True)
    assert e <= TOL and e_na <= TOL and vec <= TOL
    if taken == formed:
        assert np.array_equal(got[0], na[0]) and np.array_equal(got[1], na[1]), name


def test_line_pairs_split_sums_repeatable(dev):
    """The same call twice on a grid large enough for several sample
    splits per quad gives the same bits (fixed-order sums, no races)."""
    case = grid_case((128, 128, 8), 20000, 965, kmax=32.0)
    assert layout.line_pair_quads(case["x"], case["y"], case["z"]).all()
    a = run(case, dev)
    b = run(case, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    idx = inputs.voxel_subset(case["x"].size, 600, seed=966)
    ref = oracle.fhd(case["kx"], case["ky"], case["kz"], case["Dr"], case["Di"],
                     case["x"][idx], case["y"][idx], case["z"][idx])
    assert metrics.rel_l2(a[0][idx], a[1][idx], *ref) <= TOL


@pytest.mark.parametrize("name,case,groups,groups_f,pairs,pairs_f", list(cases64()),
                         ids=[c[0] for c in cases64()])
def test_64_voxel_line_groups_and_pairs_match_the_oracle(dev, name, case, groups, groups_f, pairs, pairs_f):
    cls = layout.gather_unit_classes(case["x"], case["y"], case["z"])[0]
    assert np.all(cls == 2), (name, cls)
    assert layout.line_group64_quads(case["x"], case["y"], case["z"], cls).tolist() == groups, name
    assert layout.line_group64_quads(case["x"], case["y"], case["z"], cls, formed=True).tolist() == groups_f, name
    assert layout.line_pair64_pairs(case["x"], case["y"], case["z"], cls).tolist() == pairs, name
    assert layout.line_pair64_pairs(case["x"], case["y"], case["z"], cls, formed=True).tolist() == pairs_f, name
    ref = oracle.fhd(case["kx"], case["ky"], case["kz"], case["Dr"], case["Di"], case["x"], case["y"], case["z"])
    print("64-voxel lines: %s" % name, flush=True)
    got = run(case, dev)
    e = metrics.rel_l2(*got, *ref)
    bf = metrics.rel_l2(*run(case, dev, binding.FHD_GATHER_BF16X3), *ref)
    na = run(case, dev, noalloc=True)
    e_na = metrics.rel_l2(*na, *ref)
    print("  rel-L2 default %.3g, bf16x3 %.3g, noalloc %.3g" % (e, bf, e_na), flush=True)
    assert e <= TOL and e_na <= TOL and bf <= TOL
    if groups == groups_f and pairs == pairs_f:
        assert np.array_equal(got[0], na[0]) and np.array_equal(got[1], na[1]), name


def test_64_voxel_line_groups_split_sums_repeatable(dev):
    """Four-line groups over several sample splits: the same call twice
    gives the same bits, and sampled voxels match the oracle."""
    case = grid_case((64, 64, 32), 20000, 976, kmax=32.0)
    assert layout.line_group64_quads(case["x"], case["y"], case["z"]).all()
    a = run(case, dev)
    b = run(case, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    idx = inputs.voxel_subset(case["x"].size, 600, seed=977)
    ref = oracle.fhd(case["kx"], case["ky"], case["kz"], case["Dr"], case["Di"],
                     case["x"][idx], case["y"][idx], case["z"][idx])
    assert metrics.rel_l2(a[0][idx], a[1][idx], *ref) <= TOL


def test_mixed_quad_kinds_in_one_call(dev):
    """A quad of 128-voxel line pairs followed by a quad of four-line
    groups of 64-voxel lines: in the table form the table serves quad 0's
    kind, so the groups fall to the 64-voxel line instance (pair 0, a long
    pair, opens no 64-voxel pair table); fhd_compute_noalloc forms both
    kinds in the one line-pair launch, each with its own split count. Both
    match the oracle, and so does F (pair 0's kind fails for the second
    quad: the vector form)."""
    a = grid_case((128, 32, 4), 10, 980)
    b = grid_case((64, 64, 4), 10, 981)
    rng = np.random.default_rng(982)
    M = 2500
    k = {n: rng.uniform(-16, 16, M).astype(np.float32) for n in ("kx", "ky", "kz")}
    D = {n: rng.standard_normal(M).astype(np.float32) for n in ("Dr", "Di")}
    case = dict(k, **D, **{n: np.concatenate((a[n], b[n])) for n in ("x", "y", "z")})
    x, y, z = case["x"], case["y"], case["z"]
    cls = layout.gather_unit_classes(x, y, z)[0]
    assert cls.tolist() == [3, 3, 3, 3, 2, 2, 2, 2]
    assert layout.line_pair_quads(x, y, z, cls).tolist() == [True, False]
    assert layout.line_group64_quads(x, y, z, cls).tolist() == [False, False]
    assert layout.line_group64_quads(x, y, z, cls, formed=True).tolist() == [False, True]
    assert layout.line_pair64_pairs(x, y, z, cls).tolist() == [False] * 4
    ref = oracle.fhd(case["kx"], case["ky"], case["kz"], case["Dr"], case["Di"], x, y, z)
    got = run(case, dev)
    na = run(case, dev, noalloc=True)
    e, e_na = metrics.rel_l2(*got, *ref), metrics.rel_l2(*na, *ref)
    print("mixed quad kinds: rel-L2 default %.3g, noalloc %.3g" % (e, e_na), flush=True)
    assert e <= TOL and e_na <= TOL
    img = inputs.random_image(x.size, seed=983)
    assert not layout.forward_pairs_form(x, y, z) and not layout.forward_lines_form(x, y, z)
    t = [torch.from_numpy(np.ascontiguousarray(v)).to(dev)
         for v in (case["kx"], case["ky"], case["kz"], x, y, z, img[0], img[1])]
    Dr, Di = binding.fhd_forward(*t)
    torch.cuda.synchronize(dev)
    fr = oracle.forward(case["kx"], case["ky"], case["kz"], img[0], img[1], x, y, z)
    ef = metrics.rel_l2(Dr.cpu().numpy(), Di.cpu().numpy(), *fr)
    print("mixed quad kinds, F: rel-L2 %.3g" % ef, flush=True)
    assert ef <= TOL
