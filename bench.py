"""Benchmark of the F^H D hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input: the
loop-fission pre-pass (fhd_pack) and the gather kernel (fhd_gather) through
the C ABI, on the 128^3-voxel x 100,000-sample stack-of-spirals workload by
default, with every input already resident in device memory.

Prints one JSON line (rank 0, N = 1) with the throughput in voxel-sample
terms per second, the gather kernel's ALU roofline figures (per-launch HIP
event timing on the launch stream), the sampled parity against the fp64
oracle and the oracle's own CPU throughput on that sample.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--op fhd|forward|normal|cg|grid|grid_bf16x3|forward_grid|
                           normal_grid|cg_grid]

--op selects the operator timed (default fhd, the headline F^H D):
forward = D = F rho; normal = F^H F rho (2 N M terms per step); cg = a
3-iteration conjugate-gradient reconstruction (F^H D, then per iteration
F^H F, two inner products and the vector updates; 7 N M terms per step);
grid = F^H D with the voxels on the workload's Cartesian grid, as a
complex matrix product on the fp32 matrix cores (fhd_pack +
fhd_grid_gather; N M terms per step, priced against the fp32 MFMA peak);
grid_bf16x3 = the same product with each fp32 operand split into two bf16
parts and three bf16 products per real product (priced as 24 FLOP per
term against the 2.5 PFLOP/s dense bf16 peak); forward_grid = D = F rho
with rho on the workload's grid, split-bf16 matrix products (same
pricing); normal_grid, cg_grid = F^H F and the 3-iteration CG with both
operators in that grid form.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "F^H D voxel-sample terms/s at 128^3 x 100k; % of FP32 VALU/trans roofline"

# gfx950 ALU ceilings of the gathers, from unit counts and clock: 256 CUs
# x 4 SIMDs at 2.4 GHz. FP32 vector peak 157.3 TFLOP/s (AMD's figure:
# two FP32 FMA instructions per SIMD issue quad-cycle). v_sin_f32 /
# v_cos_f32 issue one wave64 instruction per 8 SIMD cycles, i.e. 8 lanes
# per cycle per SIMD (measured by the issue-rate micro-benchmarks), so the
# transcendental peak is 256 * 4 * 8 * 2.4e9 = 1.97e13 /s. A term counts
# 13 FLOP (the fixed convention) and every ceiling is quoted as 13 x
# terms/s.
#   direct evaluation (sin and cos of every term): R = min(P_fp32 / 13,
#     P_trans / 2) = 9.83e12 terms/s, transcendental-bound;
#   ramp evaluation (F^H D, 16 voxels per lane in 8 symmetric pairs, one
#     x step for the whole workgroup, as on any grid): one lane per sample
#     writes an LDS record of the pairs' sample-only factors, and every
#     lane spends per sample 2 transcendentals and 35 other VALU
#     instructions (centre phase 3, 8 x 4 accumulating FMAs) on 16 terms;
#     the records cost about 40 VALU and 2 transcendentals per sample and
#     workgroup of 4096 voxels, which is left out. The 13-FLOP convention
#     no longer bounds it, the issue port does: at best two VALU
#     instructions per quad-cycle and two quad-cycles per transcendental,
#     i.e. 4 (35/2 + 2 x 2) / 16 = 5.4 clk per wave-term, 2.93e13 terms/s
#     (a workgroup whose lanes step differently forms everything per lane:
#     55 VALU and 4 transcendentals, 1.77e13);
#   F's ramp chunks (Horner): per sample and chunk of 8 voxels 4
#     transcendentals and 36 VALU (phase 3, step 1, Horner 28, finish 4):
#     13 clk per wave-term, 1.21e13 terms/s; F's 16-voxel ramps (voxel
#     pairs about the centre, a chunk pair, the pairs' real factors kept
#     per lane while the step repeats): per sample 2 transcendentals and 40
#     VALU (centre phase 4, pair sums 32, finish 4) for 16 terms: 6.0 clk
#     per wave-term, 2.62e13 terms/s.
CUS, SIMDS_PER_CU, TRANS_LANES_PER_CYCLE, CLOCK_HZ = 256, 4, 8, 2.4e9
P_FP32 = 157.3e12
P_TRANS = CUS * SIMDS_PER_CU * TRANS_LANES_PER_CYCLE * CLOCK_HZ
FLOP_PER_TERM = 13
# the separable grid form: one complex multiply-add (4 real FMAs) per term
# on the matrix cores, whose dense fp32 peak is 157.3 TFLOP/s
MFMA_FLOP_PER_TERM = 8
P_MFMA_FP32 = 157.3e12
P_MFMA_BF16 = 2.5e15
TRANS_PER_TERM_DIRECT = 2.0
ROOF_TERMS = min(P_FP32 / FLOP_PER_TERM, P_TRANS / TRANS_PER_TERM_DIRECT)


def issue_terms(valu: float, trans: float) -> float:
    """Terms/s when each wave64 term needs `valu` VALU instructions (two per
    quad-cycle at best) and `trans` transcendentals (two quad-cycles each)
    on every SIMD of the chip."""
    clk_per_wave_term = 4.0 * (valu / 2.0 + 2.0 * trans)
    return CUS * SIMDS_PER_CU * CLOCK_HZ * 64 / clk_per_wave_term


ROOF_TERMS_RAMP = issue_terms(35.0 / 16, 2.0 / 16)
ROOF_TERMS_RAMP_LANE = issue_terms(55.0 / 16, 4.0 / 16)
ROOF_TERMS_RAMP_F = issue_terms(36.0 / 8, 4.0 / 8)
ROOF_TERMS_RAMP_F16 = issue_terms(40.0 / 16, 2.0 / 16)
# F^H D on lines of 64 voxels along x with one step per unit of 4096 (any
# x-fastest grid with rows of a multiple of 64 voxels): the voxels pair up
# about each line's centre and the sum becomes four real matrix products
# (lines x samples by samples x pairs), each as three bf16 products of
# split fp32 operands on the matrix cores: 6 bf16 multiply-adds = 12 FLOP
# per term against the 2.5 PFLOP/s dense bf16 peak
LINES_FLOP_PER_TERM = 12
ROOF_TERMS_LINES = P_MFMA_BF16 / LINES_FLOP_PER_TERM


def roof_terms(parts) -> float:
    """Terms/s ceiling of work made of (terms, ceiling terms/s) parts run
    one after another: total terms over the sum of each part's time."""
    total = sum(n for n, _ in parts)
    t_min = sum(n / r for n, r in parts if n > 0)
    return total / t_min if t_min > 0 else ROOF_TERMS


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


def ramp_voxel_fraction(x, y, z, block: int = 256, vox: int = 16) -> float:
    """Fraction of voxels on a ramp path, any form (lines included)."""
    return sum(ramp_voxel_fractions(x, y, z, block, vox))


# HBM bytes per launch of each operator's dominant kernel at 128^3 x 100k,
# from rocprofv3 FETCH_SIZE and WRITE_SIZE passes scaled by a 1 GiB copy's
# readings (factors 2.0 and 1.0). Valid only for the sources they were taken
# on (SHA-256 over the listed files, in order); any later edit reports null
# until the counters are taken again.
#   fhd  (fhd_gather_long_lines_kernel): 414.4 MiB read (the 48.8 MiB B
#        table about once per XCD L2, the packed samples, x, y, z) + 48.1
#        MiB written (3 split partial sums of rho)
#   grid (fhd_grid_kernel):   15.4 MiB read (packed samples once per XCD L2)
#        + 48.0 MiB written (3 split partial sums of rho)
#   forward (fhd_forward_lines_kernel): 146.6 MiB read (the 17 MB of line
#        operand tiles about once per XCD L2, k) + 8.4 MiB written (the
#        split partial sums of D)
CSRC = os.path.join(ROOT, "non_cartesian_mri_fhd_amd", "csrc")
TRAFFIC = {
    "fhd": {"workload": "spiral128", "sources": ["fhd.hip", "fhd_internal.h"],
            "sha256": "700209e517e5110bf56990065da5d5492a2c683198a4c0d50e0f2352043cd72e",
            "bytes_per_launch": (213337.7 * 2.0 + 49224.3 * 1.0) * 1024},
    "grid": {"workload": "spiral128", "sources": ["fhd_grid.hip", "fhd_internal.h"],
             "sha256": "b1b1479f1a3565e78aa09c4f94013be3f4790b1f2dfc96d2775dd1407cc3389f",
             "bytes_per_launch": (7881.0 * 2.0 + 49152.0 * 1.0) * 1024},
    "forward": {"workload": "spiral128", "sources": ["fhd_forward.hip", "fhd_internal.h"],
                "sha256": "9d2169da1eeef71dd5922037a019fdccd37625bf2540d492141f3ceaed2a8aa1",
                "bytes_per_launch": (75065.7 * 2.0 + 8594.0 * 1.0) * 1024},
}


def measured_traffic(op: str, workload: str):
    import hashlib
    entry = TRAFFIC.get(op)
    if entry is None or workload != entry["workload"]:
        return None
    h = hashlib.sha256()
    for name in entry["sources"]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return entry["bytes_per_launch"] if h.hexdigest() == entry["sha256"] else None


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="spiral128")
    ap.add_argument("--op", default="fhd", choices=["fhd", "forward", "normal", "cg", "grid", "grid_bf16x3",
                                                       "forward_grid", "normal_grid", "cg_grid", "scatter"],
                    help="scatter: fhd_scatter (a lane per sample, atomic adds), timed beside "
                         "fhd_compute on the same workload; use a small workload (spiral32)")
    ap.add_argument("--paths", default="all", choices=["all", "vector"],
                    help="paths (--op fhd): all (fhd_gather: lines on the matrix cores) or vector "
                         "(fhd_gather_paths with FHD_GATHER_VECTOR: the fp32 VALU paths only); "
                         "--op forward --paths vector times fhd_forward_pack + fhd_forward_gather, "
                         "the vector form of F")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    return ap.parse_args(argv)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w: dict, name: str, target_s: float, rho_r, rho_i) -> tuple[dict, dict]:
    """Time the fp64 oracle on a seeded voxel sample of the full workload
    and compare the GPU result on the same voxels."""
    import oracle
    from non_cartesian_mri_fhd_amd import inputs, metrics
    threads = oracle.default_threads()
    N, M = w["N"], w["M"]
    probe = inputs.voxel_subset(N, 1024, seed=4242)
    t0 = time.perf_counter()
    oracle.fhd_subset(w, probe, threads=threads)
    rate = probe.size * M / (time.perf_counter() - t0)
    count = int(np.clip(target_s * rate / M, 256, min(N, 262144)))
    idx = inputs.voxel_subset(N, count, seed=inputs.WORKLOADS[name].seed + 2000
                              if name in inputs.WORKLOADS else 2000)
    t0 = time.perf_counter()
    ref_r, ref_i = oracle.fhd_subset(w, idx, threads=threads)
    dt = time.perf_counter() - t0
    g_r, g_i = rho_r[idx], rho_i[idx]
    parity = dict(voxels=int(idx.size), rel_l2=metrics.rel_l2(g_r, g_i, ref_r, ref_i),
                  psnr_db=metrics.psnr_db(g_r, g_i, ref_r, ref_i), tolerance=5e-4)
    base = dict(value=idx.size * M / dt, unit="terms/s", cores=threads, kind="oracle",
                sample="%d seeded voxels x all %d samples of %s (%.1f s, fp64, %s)"
                       % (idx.size, M, name, dt, cpu_model()))
    return base, parity


def main(argv=None) -> int:
    args = parse(argv)
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the F^H D path shards over voxels "
              "with no exchange, and this build measures one GPU's share only "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        return 2

    if args.op != "fhd":
        return bench_other(args)

    import torch
    from non_cartesian_mri_fhd_amd import binding, build, inputs

    build.ensure_built()
    binding.load()
    assert torch.cuda.is_available(), "no GPU visible"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = inputs.make_workload(args.workload)
    N, M = w["N"], w["M"]
    t = {k: torch.from_numpy(w[k]).to(dev) for k in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")}
    packed = binding.new_packed(M, dev)
    rho_r = torch.empty(N, dtype=torch.float32, device=dev)
    rho_i = torch.empty(N, dtype=torch.float32, device=dev)

    paths = None if args.paths == "all" else binding.FHD_GATHER_VECTOR
    other = binding.FHD_GATHER_VECTOR if args.paths == "all" else binding.FHD_GATHER_ALL

    def step():
        binding.fhd_pack(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], packed)
        binding.fhd_gather(packed, M, t["x"], t["y"], t["z"], rho_r, rho_i, paths=paths)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(stream)
        binding.fhd_pack(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], packed)
        e[1].record(stream)
        binding.fhd_gather(packed, M, t["x"], t["y"], t["z"], rho_r, rho_i, paths=paths)
        e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_step = wall * 1e3 / args.steps
    gather_all = np.array([e[1].elapsed_time(e[2]) for e in ev])

    # the same gather with the other choice of paths, timed beside it: by
    # default the vector-ALU fp32 paths (FHD_GATHER_VECTOR), the evidence
    # that the matrix-core form of lines beats the VALU form here
    alt_r = torch.empty_like(rho_r)
    alt_i = torch.empty_like(rho_i)
    binding.fhd_gather(packed, M, t["x"], t["y"], t["z"], alt_r, alt_i, paths=other)
    vev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(3)]
    for e in vev:
        e[0].record(stream)
        binding.fhd_gather(packed, M, t["x"], t["y"], t["z"], alt_r, alt_i, paths=other)
        e[1].record(stream)
    torch.cuda.synchronize()
    alt_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in vev]))
    gather_ms = float(np.mean(gather_all))
    pack_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    terms = float(N) * float(M)
    value = terms / (ms_step * 1e-3)
    cfg = binding.gather_config()

    # the ceiling for the paths this voxel layout takes (the x-fastest
    # grids of the workloads: the ramp path throughout)
    def ceiling(allow_lines):
        fr = ramp_voxel_fractions(w["x"], w["y"], w["z"], cfg["block_threads"], cfg["voxels_per_lane"],
                                  allow_lines=allow_lines)
        ln, on, la = fr
        return fr, roof_terms([(terms * ln, ROOF_TERMS_LINES), (terms * on, ROOF_TERMS_RAMP),
                               (terms * la, ROOF_TERMS_RAMP_LANE),
                               (terms * (1 - ln - on - la), ROOF_TERMS)])

    (lines, one, lane), roof = ceiling(args.paths == "all")
    dominant_kernel = "fhd_gather_long_lines_kernel" if lines == 1.0 else "fhd_gather_kernel"
    _, alt_roof = ceiling(args.paths != "all")
    rate = terms / (gather_ms * 1e-3)
    if lines == 1.0:
        # every unit on the matrix cores: bf16 FLOP against the bf16 peak
        roofline = {"bound": "mfma", "achieved": LINES_FLOP_PER_TERM * rate / 1e12,
                    "peak": P_MFMA_BF16 / 1e12}
    else:
        roofline = {"bound": "alu", "achieved": FLOP_PER_TERM * rate / 1e12,
                    "peak": FLOP_PER_TERM * roof / 1e12}
    roofline.update(unit="TFLOP/s", frac=rate / roof, traffic=measured_traffic("fhd", args.workload))
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "terms/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "%s: F^H D over %d^3 voxels x %d samples (%s)"
                        % (args.workload, w["L"], M, inputs.WORKLOADS[args.workload].trajectory),
            "N": N, "M": M, "terms": terms, "lines_voxel_fraction": lines,
            "one_step_voxel_fraction": one, "per_lane_ramp_voxel_fraction": lane, **cfg,
        },
        "roofline": roofline,
        "roofline_direct_form": {
            "note": "R for 2 transcendentals per term, the pages' direct evaluation",
            "peak": FLOP_PER_TERM * ROOF_TERMS / 1e12, "unit": "TFLOP/s",
            "frac": FLOP_PER_TERM * terms / (gather_ms * 1e-3) / (FLOP_PER_TERM * ROOF_TERMS)},
        # HIP events around each fhd_gather call: its classify, B-table,
        # gather and reduce kernels, of which the dominant one takes ~97 %
        "kernel_ms": {"timed": "fhd_gather call", "dominant": dominant_kernel, "mean": gather_ms,
                      "median": float(np.median(gather_all)), "min": float(np.min(gather_all)),
                      "fhd_pack_call": pack_ms},
        "gflops_13_per_term": FLOP_PER_TERM * value / 1e9,
        ("vector_paths_only" if args.paths == "all" else "all_paths"): {
            "note": ("fhd_gather_paths(FHD_GATHER_VECTOR): every unit on the fp32 VALU paths"
                     if args.paths == "all" else "fhd_gather: lines on the matrix cores"),
            "gather_ms": alt_ms, "terms_per_s": terms / (alt_ms * 1e-3),
            "speedup_of_the_timed_paths": alt_ms / gather_ms,
            "frac_of_its_ceiling": terms / (alt_ms * 1e-3) / alt_roof},
    }
    out["config"]["paths"] = args.paths
    if not args.no_cpu_baseline:
        base, parity = cpu_baseline(w, args.workload, args.cpu_seconds,
                                    rho_r.cpu().numpy(), rho_i.cpu().numpy())
        out["cpu_baseline"] = base
        out["parity"] = parity
    print(json.dumps(out), flush=True)
    return 0


def oracle_forward_sample(w: dict, name: str, target_s: float, Dr, Di, img):
    """Time the fp64 oracle's F on a seeded subset of the samples (all
    voxels each) and compare the GPU's D on those samples."""
    import oracle
    from non_cartesian_mri_fhd_amd import inputs, metrics
    threads = oracle.default_threads()
    N, M = w["N"], w["M"]
    probe = inputs.voxel_subset(M, 128, seed=4243)
    t0 = time.perf_counter()
    oracle.forward(w["kx"][probe], w["ky"][probe], w["kz"][probe], img[0], img[1],
                   w["x"], w["y"], w["z"], threads=threads)
    rate = probe.size * N / (time.perf_counter() - t0)
    count = int(np.clip(target_s * rate / N, 64, min(M, 65536)))
    seed = inputs.WORKLOADS[name].seed + 3000 if name in inputs.WORKLOADS else 3000
    idx = inputs.voxel_subset(M, count, seed=seed)
    t0 = time.perf_counter()
    ref_r, ref_i = oracle.forward(w["kx"][idx], w["ky"][idx], w["kz"][idx], img[0], img[1],
                                  w["x"], w["y"], w["z"], threads=threads)
    dt = time.perf_counter() - t0
    parity = dict(samples=int(idx.size), rel_l2=metrics.rel_l2(Dr[idx], Di[idx], ref_r, ref_i),
                  psnr_db=metrics.psnr_db(Dr[idx], Di[idx], ref_r, ref_i), tolerance=5e-4)
    base = dict(value=idx.size * N / dt, unit="terms/s", cores=threads, kind="oracle",
                sample="%d seeded samples x all %d voxels of %s (%.1f s, fp64, %s)"
                       % (idx.size, N, name, dt, cpu_model()))
    return base, parity


def bench_other(args) -> int:
    """Times F, F^H F, a CG reconstruction or the grid form of F^H D on the
    workload (one JSON line)."""
    import torch
    from non_cartesian_mri_fhd_amd import binding, build, inputs
    build.ensure_built()
    binding.load()
    assert torch.cuda.is_available(), "no GPU visible"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    w = inputs.make_workload(args.workload)
    N, M = w["N"], w["M"]
    t = {k: torch.from_numpy(w[k]).to(dev) for k in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")}
    img_np = inputs.random_image(N, seed=77)
    img = [torch.from_numpy(a).to(dev) for a in img_np]
    # step(): the whole operator; timed(): the same with HIP events on the
    # launch stream around its dominant kernel (None where one call covers it)
    dominant = None
    k_iters = 3
    if args.op == "forward" and args.paths == "vector":
        # the two-stage entry points, which are always the vector form
        Dr = torch.empty(M, device=dev)
        Di = torch.empty(M, device=dev)
        vox = binding.new_packed(N, dev)

        def pre():
            binding.fhd_forward_pack(t["x"], t["y"], t["z"], img[0], img[1], vox)

        def main_kernel():
            binding.fhd_forward_gather(vox, N, t["kx"], t["ky"], t["kz"], Dr, Di)
        dominant = "fhd_forward_gather_kernel"
        terms_per_step = float(N) * M
    elif args.op == "forward":
        Dr = torch.empty(M, device=dev)
        Di = torch.empty(M, device=dev)

        def pre():
            pass

        def main_kernel():
            binding.fhd_forward(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], img[0], img[1], Dr, Di)
        terms_per_step = float(N) * M
    elif args.op in ("grid", "grid_bf16x3"):
        precision = binding.FHD_GRID_BF16X3 if args.op == "grid_bf16x3" else binding.FHD_GRID_FP32
        L = inputs.WORKLOADS[args.workload].L
        axis = inputs.grid_axis_of(L)
        packed = binding.new_packed(M, dev)
        rr = torch.empty(N, device=dev)
        ri = torch.empty(N, device=dev)

        def pre():
            binding.fhd_pack(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], packed)

        def main_kernel():
            binding.fhd_grid_gather(packed, M, (L, L, L), axis, rr, ri, precision=precision)
        dominant = ("fhd_grid_bf16x3_kernel" if args.op == "grid_bf16x3" else "fhd_grid_kernel") + \
            " + reduce_splits_kernel"
        terms_per_step = float(N) * M
    elif args.op == "forward_grid":
        L = inputs.WORKLOADS[args.workload].L
        axis = inputs.grid_axis_of(L)
        Dr = torch.empty(M, device=dev)
        Di = torch.empty(M, device=dev)

        def pre():
            pass

        def main_kernel():
            binding.fhd_forward_grid(t["kx"], t["ky"], t["kz"], (L, L, L), axis, img[0], img[1], Dr, Di)
        dominant = "fhd_forward_grid_bf16x3_kernel + reduce_splits_kernel"
        terms_per_step = float(N) * M
    elif args.op == "normal_grid":
        L = inputs.WORKLOADS[args.workload].L
        axis = inputs.grid_axis_of(L)
        qr = torch.empty(N, device=dev)
        qi = torch.empty(N, device=dev)

        def pre():
            pass

        def main_kernel():
            binding.fhd_normal_grid(t["kx"], t["ky"], t["kz"], (L, L, L), axis, img[0], img[1], qr, qi)
        terms_per_step = 2.0 * N * M
    elif args.op == "cg_grid":
        L = inputs.WORKLOADS[args.workload].L
        axis = inputs.grid_axis_of(L)
        rr = torch.empty(N, device=dev)
        ri = torch.empty(N, device=dev)

        def pre():
            pass

        def main_kernel():
            binding.fhd_cg_grid(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], (L, L, L), axis, k_iters,
                                0.0, rr, ri)
        terms_per_step = float(N) * M * (1 + 2 * k_iters)
    elif args.op == "scatter":
        rr = torch.empty(N, device=dev)
        ri = torch.empty(N, device=dev)

        def pre():
            pass

        def main_kernel():
            binding.fhd_scatter(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], t["x"], t["y"], t["z"],
                                rr, ri)
        terms_per_step = float(N) * M
    elif args.op == "normal":
        qr = torch.empty(N, device=dev)
        qi = torch.empty(N, device=dev)

        def pre():
            pass

        def main_kernel():
            binding.fhd_normal(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], img[0], img[1],
                               qr, qi)
        terms_per_step = 2.0 * N * M
    else:
        rr = torch.empty(N, device=dev)
        ri = torch.empty(N, device=dev)

        def pre():
            pass

        def main_kernel():
            binding.fhd_cg(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], t["x"], t["y"], t["z"],
                           k_iters, 0.0, rr, ri)
        # F^H D once plus k_iters applications of F^H F
        terms_per_step = float(N) * M * (1 + 2 * k_iters)
    for _ in range(args.warmup):
        pre()
        main_kernel()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        pre()
        e[0].record(stream)
        main_kernel()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    value = terms_per_step / (ms * 1e-3)
    k_rate = terms_per_step / (float(np.mean(kms)) * 1e-3)
    # ceiling: F^H terms at the adjoint gather's path mix, F terms direct
    NM = float(N) * M
    gcfg = binding.gather_config()
    lines, one, lane = ramp_voxel_fractions(w["x"], w["y"], w["z"], gcfg["block_threads"],
                                            gcfg["voxels_per_lane"])
    ramp_f16, ramp_f = ramp_chunk_fractions(w["x"], w["y"], w["z"])
    adjoint = {"normal": 1, "cg": 1 + k_iters}.get(args.op, 0)
    forward_terms = {"forward": 1, "normal": 1, "cg": k_iters}.get(args.op, 0)
    f_lines = 1.0 if args.paths == "all" and forward_lines_form(w["x"], w["y"], w["z"]) else 0.0
    roof = roof_terms([(adjoint * NM * lines, ROOF_TERMS_LINES),
                       (adjoint * NM * one, ROOF_TERMS_RAMP),
                       (adjoint * NM * lane, ROOF_TERMS_RAMP_LANE),
                       (adjoint * NM * (1 - lines - one - lane), ROOF_TERMS),
                       (forward_terms * NM * f_lines, ROOF_TERMS_LINES),
                       (forward_terms * NM * (1 - f_lines) * ramp_f16, ROOF_TERMS_RAMP_F16),
                       (forward_terms * NM * (1 - f_lines) * ramp_f, ROOF_TERMS_RAMP_F),
                       (forward_terms * NM * (1 - f_lines) * (1 - ramp_f16 - ramp_f), ROOF_TERMS)])
    out = {
        "metric": "%s voxel-sample terms/s (%s)" % (args.op, args.workload),
        "value": value, "unit": "terms/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "op": args.op, "N": N, "M": M,
                   "terms_per_step": terms_per_step},
        "roofline": {"bound": "alu", "achieved": FLOP_PER_TERM * k_rate / 1e12,
                     "peak": FLOP_PER_TERM * roof / 1e12, "unit": "TFLOP/s",
                     "frac": k_rate / roof, "traffic": None},
        "kernel_ms": {"timed": dominant or "whole call", "mean": float(np.mean(kms)),
                      "median": float(np.median(kms)), "min": float(np.min(kms))},
    }
    if args.op in ("forward", "normal", "cg") and (adjoint == 0 or lines == 1.0) and \
            (forward_terms == 0 or f_lines == 1.0):
        # every term on the bf16 matrix cores (both operators in line form)
        out["roofline"] = {"bound": "mfma", "achieved": LINES_FLOP_PER_TERM * k_rate / 1e12,
                           "peak": P_MFMA_BF16 / 1e12, "unit": "TFLOP/s",
                           "frac": k_rate / roof,
                           "traffic": measured_traffic("forward", args.workload) if args.op == "forward" else None}
        out["dtype"] = "bf16x3 (fp32 accumulation)"
    if args.op == "grid":
        # one complex multiply-add per term on the fp32 matrix cores
        achieved = MFMA_FLOP_PER_TERM * k_rate
        out["roofline"] = {"bound": "mfma", "achieved": achieved / 1e12,
                           "peak": P_MFMA_FP32 / 1e12, "unit": "TFLOP/s",
                           "frac": achieved / P_MFMA_FP32,
                           "traffic": measured_traffic("grid", args.workload)}
    elif args.op in ("grid_bf16x3", "forward_grid", "normal_grid", "cg_grid"):
        # three bf16 products per real product: 3 x 8 FLOP per term on the
        # bf16 matrix cores (2.5 PFLOP/s dense)
        achieved = 3 * MFMA_FLOP_PER_TERM * k_rate
        out["dtype"] = "bf16x3 (fp32 accumulation)"
        out["roofline"] = {"bound": "mfma", "achieved": achieved / 1e12,
                           "peak": P_MFMA_BF16 / 1e12, "unit": "TFLOP/s",
                           "frac": achieved / P_MFMA_BF16, "traffic": None}
    if args.op == "scatter":
        # the gather form on the same workload, timed the same way
        gr = torch.empty(N, device=dev)
        gi = torch.empty(N, device=dev)
        args_g = [t[n] for n in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")]
        binding.fhd_compute(*args_g, gr, gi)
        gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(3)]
        for e in gev:
            e[0].record(stream)
            binding.fhd_compute(*args_g, gr, gi)
            e[1].record(stream)
        torch.cuda.synchronize()
        g_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in gev]))
        out["roofline"] = {"bound": "alu", "achieved": FLOP_PER_TERM * k_rate / 1e12,
                           "peak": FLOP_PER_TERM * ROOF_TERMS / 1e12, "unit": "TFLOP/s",
                           "frac": k_rate / ROOF_TERMS, "traffic": None,
                           "note": "direct-form ceiling R (2 transcendentals per term)"}
        out["gather_form"] = {"call": "fhd_compute", "ms": g_ms, "terms_per_s": terms_per_step / (g_ms * 1e-3),
                              "scatter_over_gather_time": float(np.mean(kms)) / g_ms,
                              "rel_l2_scatter_vs_gather": float(
                                  np.linalg.norm((rr - gr).double().cpu().numpy() + 1j * (ri - gi).double().cpu().numpy())
                                  / np.linalg.norm(gr.double().cpu().numpy() + 1j * gi.double().cpu().numpy()))}
    if not args.no_cpu_baseline:
        if args.op in ("grid", "grid_bf16x3", "scatter"):
            base, parity = cpu_baseline(w, args.workload, args.cpu_seconds,
                                        rr.cpu().numpy(), ri.cpu().numpy())
        elif args.op in ("forward", "forward_grid"):
            base, parity = oracle_forward_sample(w, args.workload, args.cpu_seconds,
                                                 Dr.cpu().numpy(), Di.cpu().numpy(), img_np)
        else:
            # F^H F and CG run F then F^H: the oracle's rate for one term of
            # each, timed on bounded samples, gives its rate per term here
            half = args.cpu_seconds / 2
            g = binding.fhd_compute(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"],
                                    t["x"], t["y"], t["z"])
            b_adj, parity = cpu_baseline(w, args.workload, half,
                                         g[0].cpu().numpy(), g[1].cpu().numpy())
            Dr_, Di_ = binding.fhd_forward(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"],
                                           img[0], img[1])
            b_fwd, _ = oracle_forward_sample(w, args.workload, half, Dr_.cpu().numpy(),
                                             Di_.cpu().numpy(), img_np)
            rate = 2.0 / (1.0 / b_adj["value"] + 1.0 / b_fwd["value"])
            base = dict(value=rate, unit="terms/s", cores=b_adj["cores"], kind="oracle",
                        sample="F^H: %s; F: %s" % (b_adj["sample"], b_fwd["sample"]))
            parity = {"F^H D": parity}
        out["cpu_baseline"] = base
        out["parity"] = parity
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
