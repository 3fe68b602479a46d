"""The host-side mirror of the kernels' voxel-layout tests (package module
layout), without a GPU."""
import numpy as np

from non_cartesian_mri_fhd_amd import layout


def test_ramp_fraction_mirrors_the_kernel_test():
    from non_cartesian_mri_fhd_amd import inputs
    L = 32
    x, y, z = inputs.grid_coords(L)
    assert layout.ramp_voxel_fraction(x, y, z) == 1.0
    n = np.arange(L ** 3)
    zfast = n.reshape(L, L, L).transpose(2, 1, 0).reshape(-1)
    assert layout.ramp_voxel_fraction(x[zfast], y[zfast], z[zfast]) == 0.0
    swap = n.copy()
    swap[1::8], swap[2::8] = n[2::8], n[1::8]
    assert layout.ramp_voxel_fraction(x[swap], y[swap], z[swap]) == 0.0
    # one voxel off the grid spoils its unit only (4096 voxels of 32768)
    x2 = x.copy()
    x2[5000] += np.float32(1e-3)
    assert layout.ramp_voxel_fraction(x2, y, z) == 1.0 - 4096 / L ** 3
    # a partial last unit takes a direct path
    m = L ** 3 - 8
    assert layout.ramp_voxel_fraction(x[:m], y[:m], z[:m]) == (L ** 3 - 4096) / m


def test_ramp_fractions_split_by_step():
    """A workgroup whose lanes are ramps with different x steps counts as
    per-lane steps; workgroups sharing one step count as one step."""
    vox, block = 16, 256
    lanes = 2 * block
    rng = np.random.default_rng(3)
    x0 = (rng.integers(-64, 44, lanes) / 128.0).astype(np.float32)
    steps = np.full(lanes, 1.0 / 128, np.float32)
    steps[block + 7] = np.float32(3.0 / 256)
    x = (x0[:, None] + np.arange(vox, dtype=np.float32)[None, :] * steps[:, None]).reshape(-1)
    y, z = (np.repeat(rng.uniform(-0.5, 0.5, lanes).astype(np.float32), vox) for _ in range(2))
    assert layout.ramp_voxel_fractions(x, y, z, block, vox) == (0.0, 0.5, 0.5)
    assert layout.ramp_voxel_fraction(x, y, z, block, vox) == 1.0
    steps[block + 7] = np.float32(1.0 / 128)
    x = (x0[:, None] + np.arange(vox, dtype=np.float32)[None, :] * steps[:, None]).reshape(-1)
    assert layout.ramp_voxel_fractions(x, y, z, block, vox) == (0.0, 1.0, 0.0)


def test_gather_unit_classes_lines():
    """Units of 4096 voxels whose aligned 64-voxel runs are lines along x
    with one step take the matrix-core class (2); the same voxels with each
    64-run made of 16-voxel pieces of four rows are one-step ramps (1); a
    unit with one line of another step, a partial last unit and a z-fastest
    order are class 0 (the first still all per-lane ramps)."""
    from non_cartesian_mri_fhd_amd import inputs
    ax = (-0.5, 1.0 / 64, -0.5, 1.0 / 16, -0.25, 1.0 / 32)
    x, y, z = inputs.coords_from_axis(64, 16, 8, ax)
    cls, all_ramp, counts = layout.gather_unit_classes(x, y, z)
    assert cls.tolist() == [2, 2] and counts.tolist() == [4096, 4096]
    # rows of 128: pairs of units of 128-voxel lines
    x2, y2, z2 = inputs.coords_from_axis(128, 16, 4, (-0.5, 1.0 / 128, -0.5, 1.0 / 16, 0.0, 0.25))
    assert layout.gather_unit_classes(x2, y2, z2)[0].tolist() == [3, 3]
    # ... but not a pair whose units step differently, nor a lone last unit
    x3, y3, z3 = inputs.coords_from_axis(128, 8, 4, (-0.5, 1.0 / 64, -0.5, 1.0 / 8, 0.0, 0.25))
    xx, yy, zz = (np.concatenate(t) for t in ((x2[:4096], x3, x2), (y2[:4096], y3, y2), (z2[:4096], z3, z2)))
    assert layout.gather_unit_classes(xx, yy, zz)[0].tolist() == [2, 2, 3, 3]
    x4, y4, z4 = inputs.coords_from_axis(128, 32, 3, (-0.5, 1.0 / 128, -0.5, 1.0 / 32, 0.0, 0.25))
    assert layout.gather_unit_classes(x4, y4, z4)[0].tolist() == [3, 3, 2]
    assert layout.ramp_voxel_fractions(xx, yy, zz) == (1.0, 0.0, 0.0)
    # 64-runs of four rows' 16-voxel pieces
    perm = np.arange(x.size).reshape(-1, 4, 4, 16).transpose(0, 2, 1, 3).reshape(-1)
    assert layout.gather_unit_classes(x[perm], y[perm], z[perm])[0].tolist() == [1, 1]
    assert layout.ramp_voxel_fractions(x[perm], y[perm], z[perm]) == (0.0, 1.0, 0.0)
    # one line of the second unit at twice the step
    xs = x.copy()
    first = 4096 + 64 * 5
    xs[first:first + 64] = (xs[first] + np.arange(64) * (2.0 / 64)).astype(np.float32)
    cls, all_ramp, _ = layout.gather_unit_classes(xs, y, z)
    assert cls.tolist() == [2, 0] and all_ramp.tolist() == [True, True]
    assert layout.ramp_voxel_fractions(xs, y, z) == (0.5, 0.0, 0.5)
    # a step of zero is a line too
    x0 = np.full_like(x, np.float32(0.125))
    assert layout.gather_unit_classes(x0, y, z)[0].tolist() == [2, 2]
    # partial last unit
    x3, y3, z3 = inputs.coords_from_axis(64, 16, 9, ax)
    cls, all_ramp, counts = layout.gather_unit_classes(x3, y3, z3)
    assert cls.tolist() == [2, 2, 0] and counts.tolist() == [4096, 4096, 1024]
    assert not all_ramp[2]
    # z fastest
    n = np.arange(x.size).reshape(8, 16, 64).transpose(2, 1, 0).reshape(-1)
    assert layout.gather_unit_classes(x[n], y[n], z[n])[0].tolist() == [0, 0]


def test_ramp_chunk_fractions_pairs_and_chunks():
    """16-voxel ramps count once; a disturbed voxel demotes its pair to two
    chunks of which the untouched one is still an 8-voxel ramp."""
    from non_cartesian_mri_fhd_amd import inputs
    L = 16
    x, y, z = inputs.grid_coords(L)
    assert layout.ramp_chunk_fractions(x, y, z) == (1.0, 0.0)
    x2 = x.copy()
    x2[21] += np.float32(1e-3)   # voxel 5 of the pair (16..31): its chunk 16..23 fails
    f16, f8 = layout.ramp_chunk_fractions(x2, y, z)
    assert f16 == 1.0 - 16 / L ** 3 and f8 == 8 / L ** 3


def test_ramp_chunk_fraction():
    from non_cartesian_mri_fhd_amd import inputs
    L = 16
    x, y, z = inputs.grid_coords(L)
    assert layout.ramp_chunk_fraction(x, y, z) == 1.0
    x2 = x.copy()
    x2[[3, 100]] += np.float32(1e-3)          # spoils 2 chunks of 8
    assert layout.ramp_chunk_fraction(x2, y, z) == 1.0 - 16 / L ** 3
    m = L ** 3 - 3                            # partial last chunk
    assert layout.ramp_chunk_fraction(x[:m], y[:m], z[:m]) == (L ** 3 - 8) / m


def test_forward_lines_form_mirror():
    """fhd_forward's line form: whole unit pairs of 128-voxel lines with one
    step throughout; rows of 64, a second step or a partial pair fall back."""
    from non_cartesian_mri_fhd_amd import inputs
    ax = (-0.5, 1.0 / 128, -0.5, 1.0 / 16, 0.0, 0.25)
    x, y, z = inputs.coords_from_axis(128, 16, 4, ax)
    assert layout.forward_lines_form(x, y, z)
    x2, y2, z2 = inputs.coords_from_axis(64, 16, 8, (-0.5, 1.0 / 64, -0.5, 1.0 / 16, 0.0, 0.25))
    assert not layout.forward_lines_form(x2, y2, z2)
    gb = inputs.coords_from_axis(128, 16, 4, (-0.25, 1.0 / 256, -0.5, 1.0 / 16, 0.125, 0.25))
    xx, yy, zz = (np.concatenate((a, b)) for a, b in zip((x, y, z), gb))
    assert not layout.forward_lines_form(xx, yy, zz)
    assert not layout.forward_lines_form(x[:4096], y[:4096], z[:4096])


def test_forward_pairs_form_mirror():
    """fhd_forward's line-pair form: the line form, and lines 2i + 1 the
    lines 2i moved by one offset throughout (rows one step apart along y,
    or the halves of rows of 256); rows swapped two by two, a bent row or a
    second offset fall back to the line form."""
    from non_cartesian_mri_fhd_amd import inputs
    ax = (-0.5, 1.0 / 128, -0.5, 1.0 / 16, 0.0, 0.25)
    x, y, z = inputs.coords_from_axis(128, 16, 4, ax)
    assert layout.forward_pairs_form(x, y, z)
    h = inputs.coords_from_axis(256, 16, 2, (-0.5, 1.0 / 256, -0.5, 1.0 / 16, 0.0, 0.5))
    assert layout.forward_pairs_form(*h)
    rows = np.arange(x.size // 128)
    rows[2::4], rows[3::4] = rows[3::4].copy(), rows[2::4].copy()
    perm = (rows[:, None] * 128 + np.arange(128)).reshape(-1)
    xs, ys, zs = x[perm], y[perm], z[perm]
    assert layout.forward_lines_form(xs, ys, zs) and not layout.forward_pairs_form(xs, ys, zs)
    yb = y.copy()
    yb[5 * 128:6 * 128] += np.float32(1.0 / 512)
    assert layout.forward_lines_form(x, yb, z) and not layout.forward_pairs_form(x, yb, z)
    g2 = inputs.coords_from_axis(128, 16, 4, (-0.5, 1.0 / 128, -0.5, 1.0 / 32, 0.0, 0.25))
    xx, yy, zz = (np.concatenate((a, b)) for a, b in zip((x, y, z), g2))
    assert layout.forward_lines_form(xx, yy, zz) and not layout.forward_pairs_form(xx, yy, zz)


def test_line_group64_mirror():
    """Four-line groups of 64-voxel lines: rows y .. y + 3 of a grid with
    rows of 64 (or two rows by two slices); a line moved in one group
    breaks its quad (its unit pairs then pair up or not), a pair of lines
    moved together keeps the pairs but breaks the group."""
    from non_cartesian_mri_fhd_amd import inputs
    ax = (-0.5, 1.0 / 64, -0.5, 1.0 / 64, -0.5, 0.25)
    x, y, z = inputs.coords_from_axis(64, 64, 8, ax)
    assert layout.line_group64_quads(x, y, z).tolist() == [True, True]
    assert layout.line_pair64_pairs(x, y, z).tolist() == [False] * 4
    x2, y2, z2 = inputs.coords_from_axis(64, 2, 128, (-0.5, 1.0 / 64, -0.5, 0.5, -0.5, 1.0 / 128))
    assert layout.line_group64_quads(x2, y2, z2).tolist() == [True]
    yb = y.copy()
    yb[2 * 64:4 * 64] += np.float32(1.0 / 512)          # lines 2, 3 together
    assert layout.line_group64_quads(x, yb, z).tolist() == [False, False]
    assert layout.line_group64_quads(x, yb, z, formed=True).tolist() == [False, True]
    # in the table form no quad is a group (quad 0 is not), so every pair
    # with pair 0's step and d is the 64-voxel line-pair instance's
    assert layout.line_pair64_pairs(x, yb, z).tolist() == [True] * 4
    assert layout.line_pair64_pairs(x, yb, z, formed=True).tolist() == [True, True, False, False]
    yc = y.copy()
    yc[3 * 64:4 * 64] += np.float32(1.0 / 512)          # line 3 alone
    assert layout.line_pair64_pairs(x, yc, z, formed=True).tolist() == [False, True, False, False]
    assert layout.line_group64_quads(x[:8192], y[:8192], z[:8192]).tolist() == []
