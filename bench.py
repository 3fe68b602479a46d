"""Benchmark of the F^H D hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input: the
loop-fission pre-pass (fhd_pack) and the gather (fhd_gather_paths) through
the C ABI, on the 128^3-voxel x 100,000-sample stack-of-spirals workload by
default, with every input already resident in device memory.

Prints one JSON line with the throughput in voxel-sample terms per second;
the dominant kernel's roofline figures, from its own launch durations (HIP
events the library records on the kernel's stream around each launch,
fhd_time_kernel); the arithmetic the timed path computes in (`dtype`,
derived from the paths that ran); the sampled parity of every path timed
against the fp64 oracle; and the oracle's own CPU throughput on that sample.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--paths P]
                    [--op OP] [--iters K] [--no-cpu-baseline] [--cpu-seconds S]

--paths (F^H D, F, F^H F and CG): all (the default: lines of voxels along x
on the matrix cores with fp32-class split-fp16 products, other voxels on the
vector ALUs in fp32), vector (fp32 vector ALUs only) or bf16x3 (the line
form in split bf16, 16 significant bits per operand). With --op fhd the two
other paths are timed beside the chosen one and reported under
"other_paths", each with its own parity.

--op selects the operator: fhd (the headline F^H D), forward (D = F rho),
normal (F^H F rho, 2NM terms per step), cg (--iters CG iterations: F^H D,
then per iteration F^H F, two inner products and the vector updates; (1 + 2
iters) N M terms per step), grid / grid_bf16x3 (F^H D for the voxels of the
workload's Cartesian grid as a complex matrix product on the fp32 matrix
cores, or split bf16), forward_grid, normal_grid, cg_grid (the grid forms of
F, F^H F and CG, split bf16) and scatter (the scatter form, a lane per
sample with atomic adds, timed beside the gather; use a small workload).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "F^H D G voxel-sample terms/s at 128^3 x 100k; % of FP32 VALU/trans roofline"

# gfx950 ceilings from unit counts and clock: 256 CUs x 4 SIMDs at 2.4 GHz.
# FP32 vector peak 157.3 TFLOP/s (AMD's figure: two FP32 FMA instructions
# per SIMD issue quad-cycle). v_sin_f32 / v_cos_f32 issue one wave64
# instruction per 8 SIMD cycles, i.e. 8 lanes per cycle per SIMD (measured
# by the issue-rate micro-benchmarks), so the transcendental peak is
# 256 * 4 * 8 * 2.4e9 = 1.97e13 /s. A term counts 13 FLOP (the fixed
# convention: phase 3 mul + 2 add, complex MAC 4 mul + 4 add).
#   direct evaluation (sin and cos of every term): R = min(P_fp32 / 13,
#     P_trans / 2) = 9.83e12 terms/s, transcendental-bound;
#   ramp evaluation (F^H D on the vector ALUs, 16 voxels per lane in 8
#     symmetric pairs, one x step for the workgroup, as on any grid): per
#     sample and lane 2 transcendentals and 35 other VALU instructions for
#     16 terms (the per-sample LDS records are left out): at best two VALU
#     instructions per quad-cycle and two quad-cycles per transcendental,
#     4 (35/2 + 2 x 2) / 16 = 5.4 clk per wave-term, 2.93e13 terms/s (lanes
#     with their own steps: 55 VALU + 4 transcendentals, 1.77e13);
#   F's ramp chunks (Horner over 8 voxels): 4 transcendentals and 36 VALU
#     per sample, 1.21e13 terms/s; F's 16-voxel ramps with the pair factors
#     kept per lane: 2 transcendentals and 40 VALU per 16 terms, 2.62e13.
CUS, SIMDS_PER_CU, TRANS_LANES_PER_CYCLE, CLOCK_HZ = 256, 4, 8, 2.4e9
P_FP32 = 157.3e12
P_TRANS = CUS * SIMDS_PER_CU * TRANS_LANES_PER_CYCLE * CLOCK_HZ
FLOP_PER_TERM = 13
TRANS_PER_TERM_DIRECT = 2.0
ROOF_TERMS = min(P_FP32 / FLOP_PER_TERM, P_TRANS / TRANS_PER_TERM_DIRECT)
# dense matrix-core peaks of MI355X (AMD's published figures, no sparsity)
P_MFMA_FP32 = 157.3e12
P_MFMA_F16 = 2.5e15     # fp16 and bf16 alike
# The separable grid form: one complex multiply-add (4 real FMAs, 8 FLOP)
# per term on the fp32 matrix cores; its split-bf16 mode does three bf16
# products per real product (24 FLOP per term).
MFMA_FLOP_PER_TERM = 8
# The line form (F^H D and F on lines of voxels along x): per voxel pair
# four real products (lines x samples by samples x pairs), each as three
# products of split operands (fp16 parts by default, bf16 parts opt-in):
# 12 executed FLOP per term on the matrix cores.
LINES_EXEC_FLOP_PER_TERM = 12
ROOF_TERMS_LINES = P_MFMA_F16 / LINES_EXEC_FLOP_PER_TERM


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


def roof_terms(parts) -> float:
    """Terms/s ceiling of work made of (terms, ceiling terms/s) parts run
    one after another: total terms over the sum of each part's time."""
    total = sum(n for n, _ in parts)
    t_min = sum(n / r for n, r in parts if n > 0)
    return total / t_min if t_min > 0 else ROOF_TERMS


# The arithmetic each choice of paths computes its matrix-core terms in
# (vector-ALU terms are fp32 on every choice).
PATH_DTYPE = {
    "all": "f16x3: fp32 operands split into fp16 hi + lo, 3 fp16 products per fp32 product, "
           "fp32 accumulation (fp32-class, within 2^-21 per product)",
    "bf16x3": "bf16x3: fp32 operands split into bf16 hi + lo, 3 bf16 products per fp32 product, "
              "fp32 accumulation (16-bit operands, ~2^-16 per product)",
    "vector": "f32",
}

# HBM bytes per launch of a kernel on one workload, from rocprofv3
# FETCH_SIZE and WRITE_SIZE passes (KiB per dispatch, the mean of the
# call's full launches) scaled by a 1 GiB copy's readings (factors 2.0 and
# 1.0; copycal.py). Valid only for the sources they were taken on
# (SHA-256 over the listed files, in order): any later edit reports null
# until the counters are taken again.
CSRC = os.path.join(ROOT, "non_cartesian_mri_fhd_amd", "csrc")
_GATHER_SRC = ["fhd.hip", "fhd_internal.h"]
_GATHER_SHA = "6292fa24e0e3bd5b1a8145097191074396175d6a7e2047eef0ccc084b8aa300c"
_FORWARD_SRC = ["fhd_forward.hip", "fhd_internal.h"]
_FORWARD_SHA = "e1130f81255b284b83e9650dfa21ccf7cec954127d270b614c092c7775cee3ed"
TRAFFIC = {
    ("fhd_gather_patch_kernel<true, true>", "spiral128"): {
        "sources": _GATHER_SRC, "sha256": _GATHER_SHA,
        "bytes_per_launch": (108288.0 * 2.0 + 65710.3 * 1.0) * 1024},
    ("fhd_gather_kernel<16, true>", "spiral128"): {
        "sources": _GATHER_SRC, "sha256": _GATHER_SHA,
        "bytes_per_launch": (52924.4 * 2.0 + 87040.0 * 1.0) * 1024},
    ("fhd_gather_patch_kernel<true, true>", "radial64"): {
        "sources": _GATHER_SRC, "sha256": _GATHER_SHA,
        "bytes_per_launch": (35071.0 * 2.0 + 69234.4 * 1.0) * 1024},
    ("fhd_forward_pairs_kernel<true>", "spiral128"): {
        "sources": _FORWARD_SRC, "sha256": _FORWARD_SHA,
        "bytes_per_launch": (75520.6 * 2.0 + 10156.2 * 1.0) * 1024},
    ("fhd_forward_pairs_kernel<true>", "radial64"): {
        "sources": _FORWARD_SRC, "sha256": _FORWARD_SHA,
        "bytes_per_launch": (8734.5 * 2.0 + 512.0 * 1.0) * 1024},
}


def measured_traffic(kernel: str, workload: str):
    """Measured HBM bytes per launch of `kernel` on `workload`, when the
    counters were taken on the current sources (else None)."""
    entry = TRAFFIC.get((kernel, workload))
    if entry is None:
        return None
    h = hashlib.sha256()
    for name in entry["sources"]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return entry["bytes_per_launch"] if h.hexdigest() == entry["sha256"] else None


def line_instance_masks(w: dict, cls: np.ndarray, paths: str):
    """The quads the line-pair instance takes (128-voxel line pairs or
    four-line groups of 64-voxel lines) and the unit pairs the 64-voxel
    line-pair instance takes, as the layout mirror gives them."""
    from non_cartesian_mri_fhd_amd import layout
    if paths == "vector":
        return None, None
    q128 = layout.line_pair_quads(w["x"], w["y"], w["z"], cls)
    q64 = layout.line_group64_quads(w["x"], w["y"], w["z"], cls)
    n = min(q128.size, q64.size) if q64.size else q128.size
    quads = q128[:n] | (q64[:n] if q64.size else False)
    return quads, layout.line_pair64_pairs(w["x"], w["y"], w["z"], cls)


def adjoint_kernel(cls: np.ndarray, counts: np.ndarray, paths: str, quads=None,
                   pairs64=None) -> tuple[str, float]:
    """The F^H D kernel that takes most voxels, for unit classes as the
    layout mirror gives them (and the quads and unit pairs the line-pair
    instances take), and the fraction of voxels it takes."""
    split = "false" if paths == "bf16x3" else "true"
    names = {5: "fhd_gather_patch64_kernel<%s, true>" % split, 4: "fhd_gather_patch_kernel<%s, true>" % split,
             3: "fhd_gather_long_lines_kernel<%s>" % split, 2: "fhd_gather_lines_kernel<%s>" % split,
             1: "fhd_gather_kernel<16, true>", 0: "fhd_gather_kernel<16, false>"}
    cls = np.array(cls)
    if quads is not None and quads.size:
        taken = np.zeros(cls.size, bool)
        taken[:4 * quads.size] = np.repeat(quads, 4)
        cls[taken] = 4
    if pairs64 is not None and pairs64.size:
        taken = np.zeros(cls.size, bool)
        taken[:2 * pairs64.size] = np.repeat(pairs64, 2)
        cls[taken & (cls == 2)] = 5
    total = float(np.sum(counts)) or 1.0
    share = {c: float(np.sum(counts[cls == c])) / total for c in names}
    best = max(share, key=share.get)
    return names[best], share[best]


def adjoint_ceiling(w: dict, allow_lines: bool) -> tuple[tuple[float, float, float], float]:
    """Voxel fractions (lines, one-step ramps, per-lane ramps) and the
    terms/s ceiling of F^H D's path mix on this layout."""
    from non_cartesian_mri_fhd_amd import layout
    fr = layout.ramp_voxel_fractions(w["x"], w["y"], w["z"], allow_lines=allow_lines)
    ln, on, la = fr
    return fr, roof_terms([(ln, ROOF_TERMS_LINES), (on, ROOF_TERMS_RAMP), (la, ROOF_TERMS_RAMP_LANE),
                           (1 - ln - on - la, ROOF_TERMS)])


def path_dtype(paths: str, lines_fraction: float) -> str:
    """The arithmetic a timed path ran in, from the voxels' layout."""
    if paths == "vector" or lines_fraction == 0.0:
        return PATH_DTYPE["vector"]
    if lines_fraction == 1.0:
        return PATH_DTYPE[paths]
    return "mixed: %.3f of voxels %s; the rest f32" % (lines_fraction, PATH_DTYPE[paths])


def alu_ceiling(kernel: str, fractions=None) -> float:
    """Terms/s issue ceiling of a vector-ALU kernel: the one-step ramp
    instance at ROOF_TERMS_RAMP, the general instance at its mix of per-lane
    ramps and direct evaluation (fractions = the layout's voxel fractions
    (lines, one-step, per-lane ramps)), F's vector gather at its ramp-chunk
    ceiling on ramp layouts, else direct evaluation R."""
    if kernel == "fhd_gather_kernel<16, true>":
        return ROOF_TERMS_RAMP
    if kernel == "fhd_gather_kernel<16, false>" and fractions is not None:
        ln, on, la = fractions
        return roof_terms([(la, ROOF_TERMS_RAMP_LANE), (max(0.0, 1.0 - ln - on - la), ROOF_TERMS)])
    if kernel.startswith("fhd_forward_gather_kernel") and fractions is not None and sum(fractions[1:]) > 0.5:
        return ROOF_TERMS_RAMP_F
    return ROOF_TERMS


def roofline_for(kernel: str, terms: float, kernel_ms: float, traffic, fractions=None) -> dict:
    """Roofline figures of one launch of `kernel` over `terms` voxel-sample
    terms taking kernel_ms: achieved = 13 FLOP per term over the launch's
    duration. The line forms are held against the dense fp16/bf16
    matrix-core peak (with their executed-FLOP utilisation beside); the
    vector-ALU kernels against their own issue ceiling (alu_ceiling, from
    the instruction counts per term and the chip's SIMD count and clock),
    expressed at 13 FLOP per term, since their ramp recurrences reach a
    13-FLOP term with fewer operations than 13."""
    rate = terms / (kernel_ms * 1e-3)
    out = {"kernel": kernel, "achieved": FLOP_PER_TERM * rate / 1e12, "unit": "TFLOP/s",
           "traffic": traffic, "flop_per_term": FLOP_PER_TERM}
    if "lines" in kernel or "patch" in kernel or "pairs" in kernel:
        out.update(bound="mfma", peak=P_MFMA_F16 / 1e12,
                   executed={"flop_per_term": LINES_EXEC_FLOP_PER_TERM,
                             "tflops": LINES_EXEC_FLOP_PER_TERM * rate / 1e12,
                             "frac": LINES_EXEC_FLOP_PER_TERM * rate / P_MFMA_F16})
    else:
        ceiling = alu_ceiling(kernel, fractions)
        out.update(bound="alu", peak=FLOP_PER_TERM * ceiling / 1e12, ceiling_terms_per_s=ceiling,
                   fp32_vector_peak=P_FP32 / 1e12,
                   note="peak: this kernel's VALU + transcendental issue ceiling in terms/s "
                        "(256 CUs x 4 SIMDs x 2.4 GHz) at 13 FLOP per term")
    out["frac"] = out["achieved"] / out["peak"]
    return out


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: 20, or 3 for the multi-call cg, cg_grid and "
                         "scatter steps): after an idle spell the shader clock settles over about ten "
                         "calls of the 128^3 operators")
    ap.add_argument("--workload", default="spiral128")
    ap.add_argument("--op", default="fhd", choices=["fhd", "forward", "normal", "cg", "grid", "grid_bf16x3",
                                                       "forward_grid", "normal_grid", "cg_grid", "scatter"])
    ap.add_argument("--paths", default="all", choices=["all", "vector", "bf16x3"])
    ap.add_argument("--iters", type=int, default=3, help="CG iterations per step (--op cg, cg_grid)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    args = ap.parse_args(argv)
    if args.warmup is None:
        args.warmup = 3 if args.op in ("cg", "cg_grid", "scatter") else 20
    return args


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_adjoint_sample(w: dict, name: str, target_s: float):
    """The fp64 oracle's F^H D on a seeded voxel sample of the full workload
    sized to about target_s seconds of CPU time: (voxel indices, reference
    real and imaginary parts, cpu_baseline record)."""
    import oracle
    from non_cartesian_mri_fhd_amd import inputs
    threads = oracle.default_threads()
    N, M = w["N"], w["M"]
    probe = inputs.voxel_subset(N, 1024, seed=4242)
    t0 = time.perf_counter()
    oracle.fhd_subset(w, probe, threads=threads)
    rate = probe.size * M / (time.perf_counter() - t0)
    count = int(np.clip(target_s * rate / M, 256, min(N, 262144)))
    seed = inputs.WORKLOADS[name].seed + 2000 if name in inputs.WORKLOADS else 2000
    idx = inputs.voxel_subset(N, count, seed=seed)
    t0 = time.perf_counter()
    ref_r, ref_i = oracle.fhd_subset(w, idx, threads=threads)
    dt = time.perf_counter() - t0
    base = dict(value=idx.size * M / dt, unit="terms/s", cores=threads, kind="oracle",
                sample="%d seeded voxels x all %d samples of %s (%.1f s, fp64, %s)"
                       % (idx.size, M, name, dt, cpu_model()))
    return idx, ref_r, ref_i, base


def oracle_forward_sample(w: dict, name: str, target_s: float, img):
    """The fp64 oracle's F on a seeded sample of the samples (all voxels
    each): (sample indices, reference parts, cpu_baseline record)."""
    import oracle
    from non_cartesian_mri_fhd_amd import inputs
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
    base = dict(value=idx.size * N / dt, unit="terms/s", cores=threads, kind="oracle",
                sample="%d seeded samples x all %d voxels of %s (%.1f s, fp64, %s)"
                       % (idx.size, N, name, dt, cpu_model()))
    return idx, ref_r, ref_i, base


def parity(got_r, got_i, ref_r, ref_i, what: str, count: int) -> dict:
    from non_cartesian_mri_fhd_amd import metrics
    return {what: int(count), "rel_l2": metrics.rel_l2(got_r, got_i, ref_r, ref_i),
            "psnr_db": metrics.psnr_db(got_r, got_i, ref_r, ref_i), "tolerance": 5e-4}


def summary(ms) -> dict:
    a = np.asarray(ms, dtype=np.float64)
    if a.size == 0:
        return {"count": 0}
    return {"mean": float(a.mean()), "median": float(np.median(a)), "min": float(a.min()),
            "count": int(a.size)}


def timed_calls(call, n: int, stream, kernel, launches_per_call: int, device):
    """Runs call() n times with HIP events on `stream` around each call and,
    when `kernel` is named, the library's events around each of its
    launches. Returns (per-call ms, per-launch ms of the kernel)."""
    import torch
    from non_cartesian_mri_fhd_amd import binding
    timer = binding.KernelTimer(kernel, n * launches_per_call, device) if kernel else None
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize(device)
    call_ms = [a.elapsed_time(b) for a, b in ev]
    kernel_ms = timer.durations_ms() if timer else []
    binding.KernelTimer.disarm()
    return call_ms, kernel_ms


def main(argv=None) -> int:
    args = parse(argv)
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the F^H D path shards over voxels "
              "with no exchange, and this benchmark measures one GPU's share only "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        return 2
    if args.op != "fhd":
        return bench_other(args)

    import torch
    from non_cartesian_mri_fhd_amd import binding, build, inputs, layout

    build.ensure_built()
    binding.load()
    assert torch.cuda.is_available(), "no GPU visible"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    PATHS = {"all": binding.FHD_GATHER_ALL, "vector": binding.FHD_GATHER_VECTOR,
             "bf16x3": binding.FHD_GATHER_BF16X3}

    w = inputs.make_workload(args.workload)
    N, M = w["N"], w["M"]
    terms = float(N) * float(M)
    t = {k: torch.from_numpy(w[k]).to(dev) for k in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")}
    packed = binding.new_packed(M, dev)
    rho = {p: (torch.empty(N, dtype=torch.float32, device=dev), torch.empty(N, dtype=torch.float32, device=dev))
           for p in PATHS}

    def pack():
        binding.fhd_pack(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], packed)

    def gather(p):
        binding.fhd_gather(packed, M, t["x"], t["y"], t["z"], *rho[p], paths=PATHS[p])

    # the host's mirror of the kernels' path tests (seconds of CPU work at
    # 128^3) runs before the warm-up, so the GPU goes from the warm-up
    # straight into the timed steps
    cls, _, counts = layout.gather_unit_classes(w["x"], w["y"], w["z"], allow_lines=args.paths != "vector")
    lp, lp64 = line_instance_masks(w, cls, args.paths)
    kernel, kernel_share = adjoint_kernel(cls, counts, args.paths, lp, lp64)

    # the other choices of paths on the same packed k-space first, each
    # after its own warm-up (the evidence for the default; each with its
    # own parity below): the GPU then comes to the default path's warm-up
    # busy, not from the idle spell in which the workload was built
    pack()
    other_runs = {}
    for p in PATHS:
        if p == args.paths:
            continue
        c2, _, n2 = layout.gather_unit_classes(w["x"], w["y"], w["z"], allow_lines=p != "vector")
        lp2, lq2 = line_instance_masks(w, c2, p)
        k2, share2 = adjoint_kernel(c2, n2, p, lp2, lq2)
        other_runs[p] = (k2, share2)
    for p, (k2, share2) in other_runs.items():
        for _ in range(args.warmup):
            gather(p)
        torch.cuda.synchronize()
        call_ms, kms = timed_calls(lambda: gather(p), 5, stream, k2, 1, dev)
        other_runs[p] = (k2, share2, call_ms, kms)

    for _ in range(args.warmup):
        pack()
        gather(args.paths)
    torch.cuda.synchronize()

    timer = binding.KernelTimer(kernel, args.steps, dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(stream)
        pack()
        e[1].record(stream)
        gather(args.paths)
        e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = timer.durations_ms()
    binding.KernelTimer.disarm()

    ms_step = wall * 1e3 / args.steps
    value = terms / (ms_step * 1e-3)
    gather_ms = [e[1].elapsed_time(e[2]) for e in ev]
    pack_ms = [e[0].elapsed_time(e[1]) for e in ev]
    (lines, one, lane), roof = adjoint_ceiling(w, args.paths != "vector")
    k_ms = summary(kernel_ms)["mean"]
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
        "dtype": path_dtype(args.paths, lines),
        "data": "synthetic",
        "config": {
            "workload": "%s: F^H D over %d^3 voxels x %d samples (%s)"
                        % (args.workload, w["L"], M, inputs.WORKLOADS[args.workload].trajectory),
            "N": N, "M": M, "terms": terms, "paths": args.paths, "lines_voxel_fraction": lines,
            "one_step_voxel_fraction": one, "per_lane_ramp_voxel_fraction": lane,
            **binding.gather_config(),
        },
        "roofline": roofline_for(kernel, terms * kernel_share, k_ms, measured_traffic(kernel, args.workload),
                                 (lines, one, lane)),
        "roofline_direct_form": {
            "note": "R = 9.83e12 terms/s: the pages' direct evaluation, 2 transcendentals per term "
                    "on the vector ALUs; fraction of the whole fhd_gather call",
            "peak": FLOP_PER_TERM * ROOF_TERMS / 1e12, "unit": "TFLOP/s",
            "frac": terms / (np.mean(gather_ms) * 1e-3) / ROOF_TERMS},
        "path_ceiling": {"note": "terms/s ceiling of this layout's path mix (lines at the executed "
                                 "matrix-core FLOP, ramps at their issue ceilings), against the "
                                 "dominant kernel's time",
                         "terms_per_s": roof, "frac": terms * kernel_share / (k_ms * 1e-3) / roof},
        "kernel_ms": {"kernel": kernel, "voxel_share": kernel_share, **summary(kernel_ms),
                      "fhd_gather_call": summary(gather_ms), "fhd_pack_call": summary(pack_ms)},
        "gflops_13_per_term": FLOP_PER_TERM * value / 1e9,
    }

    others = {}
    for p, (k2, share2, call_ms, kms) in other_runs.items():
        fr2, _ = adjoint_ceiling(w, p != "vector")
        others[p] = {"dtype": path_dtype(p, fr2[0]), "fhd_gather_call": summary(call_ms),
                     "kernel_ms": {"kernel": k2, **summary(kms)},
                     "terms_per_s": terms / (np.mean(call_ms) * 1e-3),
                     "roofline": roofline_for(k2, terms * share2, summary(kms)["mean"],
                                              measured_traffic(k2, args.workload), fr2),
                     "time_over_timed_path": float(np.mean(call_ms) / np.mean(gather_ms))}
    out["other_paths"] = others

    if not args.no_cpu_baseline:
        idx, ref_r, ref_i, base = oracle_adjoint_sample(w, args.workload, args.cpu_seconds)
        out["cpu_baseline"] = base
        got = {p: (rho[p][0].cpu().numpy()[idx], rho[p][1].cpu().numpy()[idx]) for p in PATHS}
        out["parity"] = parity(*got[args.paths], ref_r, ref_i, "voxels", idx.size)
        for p in others:
            others[p]["parity"] = parity(*got[p], ref_r, ref_i, "voxels", idx.size)
    print(json.dumps(out), flush=True)
    return 0


def bench_other(args) -> int:
    """Times F, F^H F, a CG reconstruction, the grid forms or the scatter
    form on the workload (one JSON line)."""
    import torch
    from non_cartesian_mri_fhd_amd import binding, build, inputs, layout
    build.ensure_built()
    binding.load()
    assert torch.cuda.is_available(), "no GPU visible"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    PATHS = {"all": binding.FHD_GATHER_ALL, "vector": binding.FHD_GATHER_VECTOR,
             "bf16x3": binding.FHD_GATHER_BF16X3}
    paths = PATHS[args.paths]
    w = inputs.make_workload(args.workload)
    N, M = w["N"], w["M"]
    NM = float(N) * M
    t = {k: torch.from_numpy(w[k]).to(dev) for k in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")}
    img_np = inputs.random_image(N, seed=77)
    img = [torch.from_numpy(a).to(dev) for a in img_np]
    k_iters = args.iters
    L = inputs.WORKLOADS[args.workload].L
    axis = inputs.grid_axis_of(L)
    split = "false" if args.paths == "bf16x3" else "true"
    f_lines = args.paths != "vector" and layout.forward_lines_form(w["x"], w["y"], w["z"])
    f_pairs = args.paths != "vector" and layout.forward_pairs_form(w["x"], w["y"], w["z"])
    cls, _, counts = layout.gather_unit_classes(w["x"], w["y"], w["z"], allow_lines=args.paths != "vector")
    lp, lp64 = line_instance_masks(w, cls, args.paths)
    adj_kernel, adj_share = adjoint_kernel(cls, counts, args.paths, lp, lp64)
    fwd_kernel = ("fhd_forward_pairs_kernel<%s>" % split if f_pairs else
                  "fhd_forward_lines_kernel<%s>" % split if f_lines else "fhd_forward_gather_kernel<2>")
    out_r = torch.empty(max(N, M), device=dev)
    out_i = torch.empty(max(N, M), device=dev)
    grid_op = args.op in ("grid", "grid_bf16x3", "forward_grid", "normal_grid", "cg_grid")
    # per op: the call, its terms per step, the kernel timed and its
    # launches per call, the numbers of F^H and F applications per call
    if args.op == "forward":
        def call():
            binding.fhd_forward(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], img[0], img[1],
                                out_r[:M], out_i[:M], paths=paths)
        terms_per_step, kernel, launches, n_adj, n_fwd = NM, fwd_kernel, 1, 0, 1
    elif args.op == "normal":
        def call():
            binding.fhd_normal(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], img[0], img[1],
                               out_r[:N], out_i[:N], paths=paths)
        terms_per_step, kernel, launches, n_adj, n_fwd = 2 * NM, adj_kernel, 1, 1, 1
    elif args.op == "cg":
        def call():
            binding.fhd_cg(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], t["x"], t["y"], t["z"], k_iters, 0.0,
                           out_r[:N], out_i[:N], paths=paths)
        terms_per_step, kernel, launches = NM * (1 + 2 * k_iters), adj_kernel, 1 + k_iters
        n_adj, n_fwd = 1 + k_iters, k_iters
    elif args.op in ("grid", "grid_bf16x3"):
        precision = binding.FHD_GRID_BF16X3 if args.op == "grid_bf16x3" else binding.FHD_GRID_FP32
        packed = binding.new_packed(M, dev)
        binding.fhd_pack(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], packed)

        def call():
            binding.fhd_grid_gather(packed, M, (L, L, L), axis, out_r[:N], out_i[:N], precision=precision)
        tiles = 2 if L <= 64 else 4
        kernel = "fhd_grid_bf16x3_kernel<%d>" % tiles if args.op == "grid_bf16x3" else "fhd_grid_kernel"
        terms_per_step, launches, n_adj, n_fwd = NM, 1, 1, 0
    elif args.op == "forward_grid":
        def call():
            binding.fhd_forward_grid(t["kx"], t["ky"], t["kz"], (L, L, L), axis, img[0], img[1],
                                     out_r[:M], out_i[:M])
        terms_per_step, kernel, launches, n_adj, n_fwd = NM, "fhd_forward_grid_bf16x3_kernel", 1, 0, 1
    elif args.op == "normal_grid":
        def call():
            binding.fhd_normal_grid(t["kx"], t["ky"], t["kz"], (L, L, L), axis, img[0], img[1],
                                    out_r[:N], out_i[:N])
        terms_per_step, kernel, launches, n_adj, n_fwd = 2 * NM, "fhd_forward_grid_bf16x3_kernel", 1, 1, 1
    elif args.op == "cg_grid":
        def call():
            binding.fhd_cg_grid(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], (L, L, L), axis, k_iters, 0.0,
                                out_r[:N], out_i[:N])
        terms_per_step, kernel, launches = NM * (1 + 2 * k_iters), "fhd_forward_grid_bf16x3_kernel", k_iters
        n_adj, n_fwd = 1 + k_iters, k_iters
    else:   # scatter
        def call():
            binding.fhd_scatter(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], t["x"], t["y"], t["z"],
                                out_r[:N], out_i[:N])
        terms_per_step, kernel, launches, n_adj, n_fwd = NM, None, 1, 1, 0

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    call_ms, kernel_ms = timed_calls(call, args.steps, stream, kernel, launches, dev)
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    value = terms_per_step / (ms * 1e-3)
    if grid_op:
        dtype = "f32" if args.op == "grid" else PATH_DTYPE["bf16x3"]
    elif args.op == "scatter":
        dtype = "f32"
    else:
        lines_adj = float(np.sum(counts[cls >= 2])) / N if args.paths != "vector" else 0.0
        parts = []
        if n_adj:
            parts.append("F^H: " + path_dtype(args.paths, lines_adj))
        if n_fwd:
            parts.append("F: " + path_dtype(args.paths, 1.0 if f_lines or f_pairs else 0.0))
        dtype = "; ".join(parts)
    out = {
        "metric": "%s voxel-sample terms/s (%s)" % (args.op, args.workload),
        "value": value, "unit": "terms/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": args.workload, "op": args.op, "paths": args.paths, "N": N, "M": M,
                   "terms_per_step": terms_per_step, **({"iters": k_iters} if "cg" in args.op else {})},
        "call_ms": summary(call_ms),
    }
    if kernel and kernel_ms:
        km = summary(kernel_ms)
        # terms one launch of the timed kernel covers
        per_launch = NM * adj_share if kernel.startswith("fhd_gather") else NM
        if grid_op:
            exec_flop = MFMA_FLOP_PER_TERM * (1 if args.op == "grid" else 3)
            peak = P_MFMA_FP32 if args.op == "grid" else P_MFMA_F16
            rate = per_launch / (km["mean"] * 1e-3)
            out["roofline"] = {"kernel": kernel, "bound": "mfma", "unit": "TFLOP/s",
                               "achieved": exec_flop * rate / 1e12, "peak": peak / 1e12,
                               "frac": exec_flop * rate / peak, "flop_per_term": exec_flop,
                               "traffic": measured_traffic(kernel, args.workload)}
        else:
            # F's vector gather sees the voxels' ramps whatever the paths
            fr, _ = adjoint_ceiling(w, args.paths != "vector" and not kernel.startswith("fhd_forward_gather"))
            out["roofline"] = roofline_for(kernel, per_launch, km["mean"], measured_traffic(kernel, args.workload),
                                           fr)
        out["kernel_ms"] = {"kernel": kernel, "launches_per_call": launches, **km}
    if args.op == "scatter":
        gr = torch.empty(N, device=dev)
        gi = torch.empty(N, device=dev)
        args_g = [t[n] for n in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")]
        # the gather's first call sets up its workspace: one untimed call
        binding.fhd_compute(*args_g, gr, gi)
        g_ms, _ = timed_calls(lambda: binding.fhd_compute(*args_g, gr, gi), 5, stream, None, 1, dev)
        out["roofline"] = {"bound": "alu", "achieved": FLOP_PER_TERM * value / 1e12,
                           "peak": FLOP_PER_TERM * ROOF_TERMS / 1e12, "unit": "TFLOP/s",
                           "frac": value / ROOF_TERMS, "traffic": None,
                           "note": "whole call against the direct-form ceiling R"}
        out["gather_form"] = {"call": "fhd_compute", **summary(g_ms),
                              "scatter_over_gather_time": float(np.median(call_ms) / np.median(g_ms))}
    if not args.no_cpu_baseline:
        if args.op in ("forward", "forward_grid"):
            idx, ref_r, ref_i, base = oracle_forward_sample(w, args.workload, args.cpu_seconds, img_np)
            out["parity"] = parity(out_r[:M].cpu().numpy()[idx], out_i[:M].cpu().numpy()[idx],
                                   ref_r, ref_i, "samples", idx.size)
        elif args.op in ("grid", "grid_bf16x3", "scatter"):
            idx, ref_r, ref_i, base = oracle_adjoint_sample(w, args.workload, args.cpu_seconds)
            out["parity"] = parity(out_r[:N].cpu().numpy()[idx], out_i[:N].cpu().numpy()[idx],
                                   ref_r, ref_i, "voxels", idx.size)
        else:
            # F^H F and CG apply F then F^H: the oracle's rate for one term of
            # each, timed on bounded samples, gives its rate per term here;
            # parity is that of the operators they are made of, F^H D and F
            half = args.cpu_seconds / 2
            g = binding.fhd_compute(t["kx"], t["ky"], t["kz"], t["Dr"], t["Di"], t["x"], t["y"], t["z"],
                                    paths=paths)
            idx, ref_r, ref_i, b_adj = oracle_adjoint_sample(w, args.workload, half)
            par = {"F^H D": parity(g[0].cpu().numpy()[idx], g[1].cpu().numpy()[idx], ref_r, ref_i,
                                   "voxels", idx.size)}
            if not grid_op:
                Dr_, Di_ = binding.fhd_forward(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], img[0], img[1],
                                               paths=paths)
                fidx, fr, fi, b_fwd = oracle_forward_sample(w, args.workload, half, img_np)
                par["F"] = parity(Dr_.cpu().numpy()[fidx], Di_.cpu().numpy()[fidx], fr, fi, "samples",
                                  fidx.size)
                rate = 2.0 / (1.0 / b_adj["value"] + 1.0 / b_fwd["value"])
                base = dict(value=rate, unit="terms/s", cores=b_adj["cores"], kind="oracle",
                            sample="F^H: %s; F: %s" % (b_adj["sample"], b_fwd["sample"]))
            else:
                base = b_adj
            out["parity"] = par
        out["cpu_baseline"] = base
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
