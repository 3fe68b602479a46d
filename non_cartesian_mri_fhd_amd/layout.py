"""Host-side mirror of the voxel-layout tests the F^H D and F kernels run on
the device: which path each unit of voxels takes.

The gathers classify their voxels on the GPU (fhd.hip: fhd_classify_kernel;
fhd_forward.hip: the forward pre-pass's ramp test). The functions below
repeat those tests in numpy, bit for bit on the same fp32 coordinates, so a
benchmark can price each voxel at its path's ceiling and a test can assert
which path it exercised. No F^H D arithmetic happens here.
"""
from __future__ import annotations

import numpy as np


def _lane_ramps(x, y, z, vox: int = 8):
    """Per group of `vox` consecutive voxels (the last partial group
    dropped): do they share y and z bitwise and sit at x_0 + v (x_1 - x_0)
    rounded once to fp32 -- the gathers' ramp test -- and that step."""
    x, y, z = (np.asarray(a, np.float32) for a in (x, y, z))
    full = x.size // vox * vox
    lanes = full // vox
    if lanes == 0:
        return np.zeros(0, bool), np.zeros(0, np.float32)
    X, Y, Z = (a[:full].reshape(lanes, vox) for a in (x, y, z))
    same = (np.all(Y.view(np.uint32) == Y[:, :1].view(np.uint32), axis=1)
            & np.all(Z.view(np.uint32) == Z[:, :1].view(np.uint32), axis=1))
    dx = (X[:, 1] - X[:, 0]).astype(np.float32)
    v = np.arange(vox, dtype=np.float64)
    ramp_x = (X[:, :1].astype(np.float64) + v * dx[:, None].astype(np.float64)).astype(np.float32)
    return same & np.isfinite(dx) & np.all(ramp_x == X, axis=1), dx


def ramp_chunk_fraction(x, y, z, vox: int = 8) -> float:
    """Fraction of voxels that F's pre-pass writes as ramp chunks of `vox`."""
    n = np.asarray(x).size
    return float(np.sum(_lane_ramps(x, y, z, vox)[0]) * vox / n) if n else 0.0


def ramp_chunk_fractions(x, y, z) -> tuple[float, float]:
    """Fractions of voxels that F's pre-pass writes as 16-voxel ramps (chunk
    pairs) and as 8-voxel ramp chunks (the other chunks)."""
    n = np.asarray(x).size
    if n == 0:
        return 0.0, 0.0
    ok16 = _lane_ramps(x, y, z, 16)[0]
    ok8 = _lane_ramps(x, y, z, 8)[0]
    both8 = ok8[:2 * ok16.size].reshape(-1, 2)
    # chunks of a 16-voxel ramp are 8-voxel ramps too: count them once
    single = int(np.sum(ok8)) - 2 * int(np.sum(ok16 & both8.all(axis=1)))
    return float(np.sum(ok16) * 16 / n), float(single * 8 / n)


def gather_unit_classes(x, y, z, block: int = 256, vox: int = 16, line: int = 64,
                        long_line: int = 128, allow_lines: bool = True):
    """Per unit of block*vox consecutive voxels (one workgroup of the F^H D
    gather's single-unit instances), the class its classify kernel gives
    it, by the same tests (a line: see _lane_ramps): 3 when the unit and
    the other unit of its aligned pair are whole and all their aligned runs
    of `long_line` voxels are lines with one step for the pair (the
    long-line matrix-core instance); else 2 when the unit is whole and its
    aligned runs of `line` voxels are lines with one step (the matrix-core
    instance); else 1 when every lane's `vox` voxels are such a ramp, all
    with one step (the ramp path with sample records); else 0. Returned
    with, per unit, whether all its lanes are ramps (the per-lane ramp path
    when the class is 0) and its voxel count. allow_lines=False mirrors
    FHD_GATHER_VECTOR (no unit takes a matrix-core class)."""
    x, y, z = (np.asarray(a, np.float32) for a in (x, y, z))
    N = x.size
    unit = block * vox
    units = (N + unit - 1) // unit
    counts = np.minimum(unit, N - np.arange(units) * unit)

    def per_unit(per):
        # groups of `per` voxels past N (a partial last unit) stay False;
        # returns (all groups qualify, ... with one step, that step)
        ok, dx = _lane_ramps(x, y, z, per)
        n = units * (unit // per)
        o = np.zeros(n, bool)
        o[:ok.size] = ok
        st = np.zeros(n, np.float32)
        st[:dx.size] = dx
        o = o.reshape(units, -1)
        S = st.view(np.uint32).reshape(units, -1)
        every = o.all(axis=1)
        return every, every & np.all(S == S[:, :1], axis=1), S[:, 0]

    whole = counts == unit
    all_ramp, one, _ = per_unit(vox)
    _, lines, _ = per_unit(line)
    _, longl, step = per_unit(long_line)
    lines &= whole & allow_lines
    longl &= whole & allow_lines
    pair = np.zeros(units, bool)
    both = units // 2 * 2
    if both:
        ok = (longl[0:both:2] & longl[1:both:2] & (step[0:both:2] == step[1:both:2]))
        pair[0:both:2] = ok
        pair[1:both:2] = ok
    cls = np.where(pair, 3, np.where(lines, 2, np.where(one, 1, 0)))
    return cls, all_ramp, counts


def line_pair_quads(x, y, z, cls=None, block: int = 256, vox: int = 16, long_line: int = 128,
                    formed: bool = False):
    """Per quad of four units (units 4q .. 4q + 3, all present), whether
    the F^H D line-pair instance takes it, by the classify kernel's
    line-pair record: both unit pairs of the quad of class 3, in each the
    lines 2i + 1 the lines 2i moved by one common offset d (bitwise equal
    fp32 differences of their first voxels' x, y, z, all finite; d from
    the pair's lines 0 and 1), the same step and d in both pairs; and,
    unless `formed` (the instance forming its own B operands, as in
    fhd_compute_noalloc), quad 0 so too with the quad's step and d."""
    x, y, z = (np.asarray(a, np.float32) for a in (x, y, z))
    unit = block * vox
    if cls is None:
        cls = gather_unit_classes(x, y, z, block, vox)[0]
    quads = x.size // (4 * unit)
    if quads == 0:
        return np.zeros(0, bool)
    nl = 4 * unit // long_line                     # lines per quad
    first = np.arange(quads * nl) * long_line      # every line's first voxel
    fx, fy, fz = x[first], y[first], z[first]
    step = (x[first + 1] - fx).astype(np.float32)
    sx = (fx[1::2] - fx[0::2]).astype(np.float32)  # per line pair
    sy = (fy[1::2] - fy[0::2]).astype(np.float32)
    sz = (fz[1::2] - fz[0::2]).astype(np.float32)
    lp_per_pair = nl // 4                          # line pairs per unit pair
    P = quads * 2

    def bits(a):
        return a.view(np.uint32).reshape(P, lp_per_pair)

    SX, SY, SZ = bits(sx), bits(sy), bits(sz)
    fin = (np.isfinite(sx) & np.isfinite(sy) & np.isfinite(sz)).reshape(P, lp_per_pair)
    shifted = (fin.all(axis=1) & np.all(SX == SX[:, :1], axis=1) & np.all(SY == SY[:, :1], axis=1)
               & np.all(SZ == SZ[:, :1], axis=1))
    long_pair = cls[0:4 * quads:2] == 3
    rec_ok = long_pair & shifted
    pstep = step.view(np.uint32).reshape(P, 2 * lp_per_pair)[:, 0]
    key = np.stack([pstep, SX[:, 0], SY[:, 0], SZ[:, 0]], axis=1)
    quad = rec_ok[0::2] & rec_ok[1::2] & np.all(key[0::2] == key[1::2], axis=1)
    if formed:
        return quad
    if not quad[0]:
        return np.zeros(quads, bool)
    return quad & np.all(key[0::2] == key[0], axis=1)


def _pair64_records(x, y, z, cls, block: int, vox: int, line: int):
    """Per unit pair, the classify kernel's 64-voxel records as the host
    sees them: (flag 2 or 3, flag 3, key = step, d and e bits). Flag 2:
    both units of class 2 with one step for the pair (bitwise), the lines
    2i + 1 the lines 2i moved by one common offset d (bitwise equal fp32
    differences of their first voxels' x, y, z, all finite; d from the
    pair's lines 0 and 1). Flag 3: beyond that, the lines 4i + 2 the lines
    4i moved by one common offset e (e from the pair's lines 0 and 2)."""
    unit = block * vox
    pairs = cls.size // 2
    nl = 2 * unit // line                          # lines per unit pair
    first = np.arange(pairs * nl) * line
    if pairs == 0 or not (first + 1 < x.size).all():
        z0 = np.zeros(pairs, bool)
        return z0, z0, np.zeros((pairs, 7), np.uint32)
    fx, fy, fz = x[first], y[first], z[first]
    step = (x[first + 1] - fx).astype(np.float32).view(np.uint32).reshape(pairs, nl)

    def offsets(k, per):
        # line (per i + k) minus line (per i), per group of `per` lines
        out = []
        for a in (fx, fy, fz):
            g = a.reshape(-1, per)
            out.append((g[:, k] - g[:, 0]).astype(np.float32))
        fin = np.isfinite(out[0]) & np.isfinite(out[1]) & np.isfinite(out[2])
        bits = [o.view(np.uint32).reshape(pairs, nl // per) for o in out]
        same = fin.reshape(pairs, -1).all(axis=1)
        for b in bits:
            same &= np.all(b == b[:, :1], axis=1)
        return same, [b[:, 0] for b in bits]

    shifted, d = offsets(1, 2)
    grouped, e = offsets(2, 4)
    both = (cls[0:2 * pairs:2] == 2) & (cls[1:2 * pairs:2] == 2)
    # one step for the pair: the two units' first lines (each unit's lines
    # share its step, as class 2 says)
    common = step[:, 0] == step[:, nl // 2]
    ok = both & common & shifted
    key = np.stack([step[:, 0], *d, *e], axis=1)
    return ok, ok & grouped, key


def line_group64_quads(x, y, z, cls=None, block: int = 256, vox: int = 16, line: int = 64,
                       formed: bool = False):
    """Per quad of four units (all present), whether the F^H D line-pair
    instance takes it as four-line groups of 64-voxel lines: both unit
    pairs' records flag 3 (see _pair64_records) with the same step, d and
    e; and, unless `formed`, quad 0 so too with the same step and
    offsets."""
    x, y, z = (np.asarray(a, np.float32) for a in (x, y, z))
    if cls is None:
        cls = gather_unit_classes(x, y, z, block, vox)[0]
    quads = cls.size // 4
    if quads == 0:
        return np.zeros(0, bool)
    _, grp, key = _pair64_records(x, y, z, cls, block, vox, line)
    grp, key = grp[:2 * quads], key[:2 * quads]
    quad = grp[0::2] & grp[1::2] & np.all(key[0::2] == key[1::2], axis=1)
    if formed:
        return quad
    if not quad[0]:
        return np.zeros(quads, bool)
    return quad & np.all(key[0::2] == key[0], axis=1)


def line_pair64_pairs(x, y, z, cls=None, block: int = 256, vox: int = 16, line: int = 64,
                      formed: bool = False):
    """Per unit pair (units 2p, 2p + 1, both present), whether the F^H D
    64-voxel line-pair instance takes it: its record is flag 2 or 3 (see
    _pair64_records), its quad is not taken as four-line groups (in the
    same mode, line_group64_quads); and, unless `formed`, pair 0 so too
    with the same step and d."""
    x, y, z = (np.asarray(a, np.float32) for a in (x, y, z))
    if cls is None:
        cls = gather_unit_classes(x, y, z, block, vox)[0]
    pairs = cls.size // 2
    if pairs == 0:
        return np.zeros(0, bool)
    ok, _, key = _pair64_records(x, y, z, cls, block, vox, line)
    groups = line_group64_quads(x, y, z, cls, block, vox, line, formed)
    in_group = np.zeros(pairs, bool)
    in_group[:2 * groups.size] = np.repeat(groups, 2)
    ok = ok & ~in_group
    if formed:
        return ok
    if not ok[0]:
        return np.zeros(pairs, bool)
    return ok & np.all(key[:, :4] == key[0, :4], axis=1)


def ramp_voxel_fractions(x, y, z, block: int = 256, vox: int = 16,
                         allow_lines: bool = True) -> tuple[float, float, float]:
    """Fractions of voxels by the F^H D gather path their unit takes (see
    gather_unit_classes): (lines on the matrix cores, either instance; ramps
    with one step for the workgroup; ramps with per-lane steps); the rest
    is direct."""
    N = np.asarray(x).size
    if N == 0:
        return 0.0, 0.0, 0.0
    cls, all_ramp, counts = gather_unit_classes(x, y, z, block, vox, allow_lines=allow_lines)
    return (float(np.sum(counts[cls >= 2]) / N), float(np.sum(counts[cls == 1]) / N),
            float(np.sum(counts[(cls == 0) & all_ramp]) / N))


def forward_lines_form(x, y, z, block: int = 256, vox: int = 16, long_line: int = 128) -> bool:
    """Whether fhd_forward takes its matrix-core line form, by the same
    rule: a whole number of unit pairs, every unit of class 3, and one step
    for every line of `long_line` voxels."""
    N = np.asarray(x).size
    if N == 0 or N % (2 * block * vox) != 0:
        return False
    cls = gather_unit_classes(x, y, z, block, vox)[0]
    ok, dx = _lane_ramps(x, y, z, long_line)
    return bool(np.all(cls == 3) and dx.size and np.all(dx.view(np.uint32) == dx.view(np.uint32)[0]))


def forward_pairs_form(x, y, z, block: int = 256, vox: int = 16, long_line: int = 128,
                       line: int = 64) -> bool:
    """Whether fhd_forward takes its matrix-core line-pair form: either the
    line form's rule and, in every unit pair, the lines 2i + 1 the lines
    2i moved by one offset d (bitwise equal fp32 differences of their first
    voxels' x, y, z, all finite), with pair 0's step and d throughout (the
    classify kernel's records, flag 1); or every unit of class 2, a whole
    number of unit pairs, and every pair's 64-voxel lines in four-line
    groups with pair 0's step, d and e (flag 3, see _pair64_records)."""
    x, y, z = (np.asarray(a, np.float32) for a in (x, y, z))
    N = x.size
    if N == 0 or N % (2 * block * vox) != 0:
        return False
    if forward_lines_form(x, y, z, block, vox, long_line):
        pairs = N // (2 * block * vox)
        nl = 2 * block * vox // long_line              # lines per unit pair
        first = np.arange(pairs * nl) * long_line
        fx, fy, fz = x[first], y[first], z[first]
        d = [(a[1::2] - a[0::2]).astype(np.float32) for a in (fx, fy, fz)]
        if not all(np.all(np.isfinite(a)) for a in d):
            return False
        bits = [a.view(np.uint32).reshape(pairs, nl // 2) for a in d]
        # within each pair (the record), then pair 0's throughout (the step
        # is one throughout by the line form's rule)
        return bool(all(np.all(b == b[0, 0]) for b in bits))
    cls = gather_unit_classes(x, y, z, block, vox)[0]
    if not np.all(cls == 2):
        return False
    _, grp, key = _pair64_records(x, y, z, cls, block, vox, line)
    return bool(grp.all() and np.all(key == key[0]))


def ramp_voxel_fraction(x, y, z, block: int = 256, vox: int = 16) -> float:
    """Fraction of voxels on a ramp path, any form (lines included)."""
    return sum(ramp_voxel_fractions(x, y, z, block, vox))
