"""Compile the HIP sources of this package into in-tree shared libraries.

``python -m non_cartesian_mri_fhd_amd.build`` (or ``build_all()``) runs hipcc
for gfx950 on every source below. It needs no GPU: hipcc cross-compiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE,
]

# library name -> source files
LIBRARIES = {
    "libfhd.so": ["fhd.hip", "fhd_forward.hip", "fhd_cg.hip", "fhd_grid.hip", "fhd_scatter.hip",
                  "fhd_noalloc.hip", "fhd_workspace.hip", "abi_checks.hip"],
    "libfhd_microbench.so": ["microbench.hip"],
}


def lib_path(name: str) -> str:
    return os.path.join(PKG, name)


def build_library(name: str, verbose: bool = False) -> str:
    out = lib_path(name)
    srcs = [os.path.join(CSRC, s) for s in LIBRARIES[name]]
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *HIP_FLAGS, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (name, res.stdout, res.stderr))
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list[str]:
    return [build_library(n, verbose) for n in LIBRARIES]


def sources_of(name: str) -> list[str]:
    """Every file a library is built from: its sources, the package's
    private headers and the public headers."""
    files = [os.path.join(CSRC, s) for s in LIBRARIES[name]]
    files += [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".h")]
    files += [os.path.join(INCLUDE, f) for f in sorted(os.listdir(INCLUDE)) if f.endswith(".h")]
    return files


def is_stale(name: str) -> bool:
    """Whether the library is missing or older than any file it is built from."""
    out = lib_path(name)
    if not os.path.exists(out):
        return True
    built = os.path.getmtime(out)
    return any(os.path.getmtime(f) > built for f in sources_of(name))


def ensure_built() -> None:
    """Build the libraries that are missing or older than their sources."""
    for n in LIBRARIES:
        if is_stale(n):
            build_library(n)


if __name__ == "__main__":
    for p in build_all(verbose="-v" in sys.argv):
        print(p)
