"""Issue-rate micro-benchmarks (libfhd_microbench.so) and their reading.

``python -m non_cartesian_mri_fhd_amd.microbench`` times every (A, B) mix of
A plain fp32 FMAs and B transcendentals per stream-iteration and prints one
JSON line per mix plus a summary line with:

* ``fma_cycles``   -- SIMD cycles per wave64 FMA (A = 8, B = 0);
* ``trans_cycles`` -- SIMD cycles per wave64 v_sin/v_cos (A = 0);
* for each mix, the measured cycles per wave64 unit next to the two issue
  models: blocking (A*fma + B*trans) and side-by-side (max of the two).
"""
from __future__ import annotations

import ctypes
import json
import sys

from .build import lib_path

STREAMS = 8
BLOCK = 256


def load():
    lib = ctypes.CDLL(lib_path("libfhd_microbench.so"))
    lib.fhdmb_mix.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_double)] * 3
    lib.fhdmb_mix.restype = ctypes.c_int
    lib.fhdmb_mix_pair.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                   ctypes.POINTER(ctypes.c_int)]
    return lib


def pairs(lib):
    out = []
    for i in range(lib.fhdmb_mix_count()):
        a, b = ctypes.c_int(), ctypes.c_int()
        lib.fhdmb_mix_pair(i, ctypes.byref(a), ctypes.byref(b))
        out.append((a.value, b.value))
    return out


def run(cus: int, blocks_per_cu: int = 32, iters: int = 2000) -> list[dict]:
    lib = load()
    blocks = cus * blocks_per_cu
    simds = cus * 4
    waves = blocks * BLOCK // 64
    rows = []
    for a, b in pairs(lib):
        ms, mhz, chk = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        rc = lib.fhdmb_mix(a, b, blocks, iters, ctypes.byref(ms), ctypes.byref(mhz),
                           ctypes.byref(chk))
        if rc != 0:
            raise RuntimeError("fhdmb_mix(%d, %d) failed: %d" % (a, b, rc))
        units = waves * iters * STREAMS          # wave64 stream-iterations
        cycles = ms.value * 1e-3 * mhz.value * 1e6 * simds / units
        rows.append(dict(a=a, b=b, ms=ms.value, sclk_mhz=mhz.value,
                         cycles_per_wave_unit=cycles, checksum=chk.value))
    by = {(r["a"], r["b"]): r for r in rows}
    fma = by[(8, 0)]["cycles_per_wave_unit"] / 8.0
    trans = by[(0, 2)]["cycles_per_wave_unit"] / 2.0
    for r in rows:
        r["model_blocking"] = r["a"] * fma + r["b"] * trans
        r["model_side_by_side"] = max(r["a"] * fma, r["b"] * trans)
    return rows


def main(argv=None) -> int:
    import torch
    argv = sys.argv[1:] if argv is None else argv
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = run(cus)
    for r in rows:
        print(json.dumps(r), flush=True)
    by = {(r["a"], r["b"]): r for r in rows}
    summary = dict(
        cus=cus,
        fma_cycles=by[(8, 0)]["cycles_per_wave_unit"] / 8.0,
        sin_only_cycles=by[(0, 1)]["cycles_per_wave_unit"],
        trans_cycles=by[(0, 2)]["cycles_per_wave_unit"] / 2.0,
        sclk_mhz=sum(r["sclk_mhz"] for r in rows) / len(rows),
    )
    print(json.dumps({"summary": summary}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
