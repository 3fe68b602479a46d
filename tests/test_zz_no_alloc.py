"""fhd_compute_noalloc through the C ABI: the same results as
fhd_compute_paths, bit for bit, with no allocation.

Two calls and more in a row on one stream, each smaller than the one
before (the library's scratch array keeps the last call's contents), on
every choice of paths; a size beyond the scratch array is refused.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from non_cartesian_mri_fhd_amd import binding, build, inputs, metrics

pytestmark = pytest.mark.gpu

PATHS = {"all": binding.FHD_GATHER_ALL, "vector": binding.FHD_GATHER_VECTOR,
         "bf16x3": binding.FHD_GATHER_BF16X3}


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    build.ensure_built()
    lib = binding.load()
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.fhd_compute_noalloc.argtypes = [vp] * 10 + [i32, i32, i32, vp]
    lib.fhd_compute_noalloc.restype = i32
    return lib


def device_case(case, dev):
    return [torch.from_numpy(np.ascontiguousarray(case[k])).to(dev)
            for k in ("kx", "ky", "kz", "Dr", "Di", "x", "y", "z")]


def noalloc(lib, t, paths, dev):
    M, N = t[0].numel(), t[5].numel()
    rr = torch.full((N,), float("nan"), device=dev)
    ri = torch.full((N,), float("nan"), device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.fhd_compute_noalloc(*[a.data_ptr() for a in t], rr.data_ptr(), ri.data_ptr(), M, N,
                                 PATHS[paths], stream)
    assert rc == binding.FHD_OK, lib.fhd_last_error()
    return rr, ri


@pytest.mark.parametrize("paths", ["all", "vector", "bf16x3"])
def test_noalloc_matches_compute_on_calls_of_shrinking_size(lib, paths):
    """128^3 x 100,000 (about 70 MiB of workspace on the line forms, whose
    line-pair workgroups form their B operands themselves here; 86 MB on
    the vector paths), then smaller calls on the same scratch: 64^3 x
    65,536 (four-line groups of 64-voxel lines, formed here too), 32^3 and
    a ragged case."""
    dev = torch.device("cuda:0")
    first = "spiral128"
    cases = [(first, inputs.make_workload(first)),
             ("radial64", inputs.make_workload("radial64")),
             ("spiral32", inputs.make_workload("spiral32")),
             ("ragged 5000 x 123", inputs.random_case(5000, 123, seed=931))]
    for name, c in cases:
        t = device_case(c, dev)
        print("noalloc %s, paths %s" % (name, paths), flush=True)
        got = noalloc(lib, t, paths, dev)
        want = binding.fhd_compute(*t, paths=PATHS[paths])
        torch.cuda.synchronize(dev)
        assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1]), (name, paths)
        # and the parity bar against the oracle on a seeded voxel sample
        idx = inputs.voxel_subset(c["x"].size, min(1024, c["x"].size), seed=932)
        ref = oracle.fhd(c["kx"], c["ky"], c["kz"], c["Dr"], c["Di"], c["x"][idx], c["y"][idx], c["z"][idx])
        e = metrics.rel_l2(got[0].cpu().numpy()[idx], got[1].cpu().numpy()[idx], *ref)
        assert e <= 5e-4, (name, paths, e)


def test_noalloc_refuses_a_workspace_beyond_its_scratch(lib):
    """Eight million samples need 160 MB of packed k-space alone, more than
    the 128 MiB scratch: FHD_ERR_INVALID_ARG, saying what was needed."""
    dev = torch.device("cuda:0")
    M, N = 8_000_000, 4096
    k = torch.zeros(M, device=dev)
    v = torch.zeros(N, device=dev)
    out = [torch.empty(N, device=dev) for _ in range(2)]
    rc = lib.fhd_compute_noalloc(k.data_ptr(), k.data_ptr(), k.data_ptr(), k.data_ptr(), k.data_ptr(),
                                 v.data_ptr(), v.data_ptr(), v.data_ptr(), out[0].data_ptr(), out[1].data_ptr(),
                                 M, N, binding.FHD_GATHER_ALL, None)
    assert rc == binding.FHD_ERR_INVALID_ARG
    assert b"needs" in lib.fhd_last_error() and str(128 * 1024 * 1024).encode() in lib.fhd_last_error()


def test_noalloc_empty_sizes(lib):
    dev = torch.device("cuda:0")
    c = inputs.random_case(700, 1, seed=933)
    t = device_case(c, dev)

    rr = torch.full((700,), 7.0, device=dev)
    ri = torch.full((700,), 7.0, device=dev)
    rc = lib.fhd_compute_noalloc(*[0] * 5, *[a.data_ptr() for a in t[5:]], rr.data_ptr(), ri.data_ptr(), 0, 700,
                                 binding.FHD_GATHER_ALL, None)
    torch.cuda.synchronize(dev)
    assert rc == binding.FHD_OK and not rr.any() and not ri.any()
    rc = lib.fhd_compute_noalloc(*[a.data_ptr() for a in t[:5]], *[0] * 5, 1, 0, binding.FHD_GATHER_ALL, None)
    assert rc == binding.FHD_OK
