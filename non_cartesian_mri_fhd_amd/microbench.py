"""Issue-rate micro-benchmarks (libfhd_microbench.so) and their reading.

``python -m non_cartesian_mri_fhd_amd.microbench [--iters K]`` prints one
JSON line per measurement:

* ``mix`` lines: A plain fp32 FMAs and B transcendentals per stream-
  iteration, with the measured SIMD cycles per wave64 unit next to two issue
  models, blocking (A*fma + B*trans) and side-by-side (max of the two);
* ``form`` lines: one exact VALU instruction form (inline assembly, eight
  independent chains), as SIMD cycles per wave64 instruction, both at the
  clock the kernel measured and at the 2.4 GHz peak clock;
* the ``lds_read_b128`` form also as LDS bytes per clock and CU (conflict-
  free 16-byte reads, eight in flight per wave);
* ``mfma_form`` lines: v_mfma_f32_16x16x32_f16 alone and each followed by
  independent vector instructions or an LDS read, at one and two waves per
  SIMD, as SIMD cycles per MFMA;
* a ``summary`` line: fma_cycles (VGPR FMA), sgpr_fma_cycles, trans_cycles,
  lds_bytes_per_clk_per_cu.

Cycle counts are per SIMD: elapsed time x clock x SIMDs / wave64
instructions. Each launch keeps every SIMD at 8 resident waves.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import sys

from .build import lib_path

STREAMS = 8
BLOCK = 256
PEAK_CLOCK_HZ = 2.4e9


def load():
    lib = ctypes.CDLL(lib_path("libfhd_microbench.so"))
    dp = ctypes.POINTER(ctypes.c_double)
    lib.fhdmb_mix.argtypes = [ctypes.c_int] * 4 + [dp] * 3
    lib.fhdmb_mix.restype = ctypes.c_int
    lib.fhdmb_mix_pair.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                   ctypes.POINTER(ctypes.c_int)]
    lib.fhdmb_form.argtypes = [ctypes.c_int] * 3 + [dp] * 3
    lib.fhdmb_form.restype = ctypes.c_int
    lib.fhdmb_form_name.argtypes = [ctypes.c_int]
    lib.fhdmb_form_name.restype = ctypes.c_char_p
    lib.fhdmb_form_instrs.argtypes = [ctypes.c_int]
    return lib


def _time(fn, *args):
    ms, mhz, chk = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    rc = fn(*args, ctypes.byref(ms), ctypes.byref(mhz), ctypes.byref(chk))
    if rc != 0:
        raise RuntimeError("micro-benchmark launch failed: %d" % rc)
    return ms.value, mhz.value, chk.value


def run_mixes(lib, cus: int, iters: int, blocks_per_cu: int = 32) -> list[dict]:
    blocks = cus * blocks_per_cu
    simds = cus * 4
    waves = blocks * BLOCK // 64
    rows = []
    for i in range(lib.fhdmb_mix_count()):
        a, b = ctypes.c_int(), ctypes.c_int()
        lib.fhdmb_mix_pair(i, ctypes.byref(a), ctypes.byref(b))
        ms, mhz, chk = _time(lib.fhdmb_mix, a.value, b.value, blocks, iters)
        units = waves * iters * STREAMS          # wave64 stream-iterations
        rows.append(dict(kind="mix", a=a.value, b=b.value, ms=ms, sclk_mhz=mhz,
                         cycles_per_wave_unit=ms * 1e-3 * mhz * 1e6 * simds / units,
                         checksum=chk))
    by = {(r["a"], r["b"]): r for r in rows}
    fma = by[(8, 0)]["cycles_per_wave_unit"] / 8.0
    trans = by[(0, 2)]["cycles_per_wave_unit"] / 2.0
    for r in rows:
        r["model_blocking"] = r["a"] * fma + r["b"] * trans
        r["model_side_by_side"] = max(r["a"] * fma, r["b"] * trans)
    return rows


def run_forms(lib, cus: int, iters: int, waves_per_simd: int = 8) -> list[dict]:
    blocks = cus * waves_per_simd       # 4 waves per block: one per SIMD
    rows = []
    for i in range(lib.fhdmb_form_count()):
        ms, mhz, chk = _time(lib.fhdmb_form, i, blocks, iters)
        per_simd = waves_per_simd * iters * 4 * lib.fhdmb_form_instrs(i)
        row = dict(kind="form", form=lib.fhdmb_form_name(i).decode(), ms=ms, sclk_mhz=mhz,
                   cycles_per_instr=ms * 1e-3 * mhz * 1e6 / per_simd,
                   cycles_per_instr_at_peak_clock=ms * 1e-3 * PEAK_CLOCK_HZ / per_simd,
                   checksum=chk)
        if row["form"] == "lds_read_b128":
            # 1 KB per wave64 read, four SIMDs per CU
            per_cu = 4 * per_simd * 1024.0
            row["lds_bytes_per_clk_per_cu"] = per_cu / (ms * 1e-3 * mhz * 1e6)
        rows.append(row)
    return rows


MFMA_FORMS = ("mfma_f16_16x16x32", "mfma_f16_plus_4fma", "mfma_f16_plus_sin_fma",
              "mfma_f16_plus_lds_read_b128")


def run_mfma_forms(lib, cus: int, iters: int) -> list[dict]:
    """The matrix-core forms at one and two waves per SIMD: cycles per
    MFMA (with its vector instructions) per SIMD."""
    names = [lib.fhdmb_form_name(i).decode() for i in range(lib.fhdmb_form_count())]
    rows = []
    for waves in (1, 2):
        for name in MFMA_FORMS:
            i = names.index(name)
            ms, mhz, chk = _time(lib.fhdmb_form, i, cus * waves, iters)
            per_simd = waves * iters * 4 * lib.fhdmb_form_instrs(i)
            rows.append(dict(kind="mfma_form", form=name, waves_per_simd=waves, ms=ms, sclk_mhz=mhz,
                             cycles_per_mfma=ms * 1e-3 * mhz * 1e6 / per_simd, checksum=chk))
    return rows


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--iters", type=int, default=20000, help="form-kernel iterations")
    ap.add_argument("--mix-iters", type=int, default=2000)
    ap.add_argument("--forms-only", action="store_true")
    args = ap.parse_args(sys.argv[1:] if argv is None else argv)
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    lib = load()
    rows = [] if args.forms_only else run_mixes(lib, cus, args.mix_iters)
    rows += run_forms(lib, cus, args.iters)
    rows += run_mfma_forms(lib, cus, args.iters)
    for r in rows:
        print(json.dumps(r), flush=True)
    forms = {r["form"]: r for r in rows if r["kind"] == "form"}
    summary = dict(
        cus=cus,
        fma_cycles=forms["fmac_vop2_vgpr"]["cycles_per_instr"],
        sgpr_fma_cycles=forms["fmac_vop2_sgpr"]["cycles_per_instr"],
        trans_cycles=forms["sin"]["cycles_per_instr"],
        fract_cycles=forms["fract"]["cycles_per_instr"],
        lds_bytes_per_clk_per_cu=forms["lds_read_b128"]["lds_bytes_per_clk_per_cu"],
    )
    print(json.dumps({"summary": summary}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
