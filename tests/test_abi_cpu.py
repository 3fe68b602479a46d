"""The C ABI without a GPU: exports, sizes and argument checks.

Every case here fails (or returns) before the library makes any HIP call,
so it runs on a host with no device.
"""
import ctypes
import os
import re

import pytest

from non_cartesian_mri_fhd_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fhd.h")

FHD_OK, FHD_ERR_INVALID_ARG = 0, -1


@pytest.fixture(scope="module")
def lib():
    build.ensure_built()
    lib = ctypes.CDLL(build.lib_path("libfhd.so"))
    vp = ctypes.c_void_p
    lib.fhd_compute.argtypes = [vp] * 10 + [ctypes.c_int, ctypes.c_int, vp]
    lib.fhd_scatter.argtypes = [vp] * 10 + [ctypes.c_int, ctypes.c_int, vp]
    lib.fhd_pack.argtypes = [vp] * 5 + [ctypes.c_int, vp, ctypes.c_int64, vp]
    lib.fhd_gather.argtypes = [vp, ctypes.c_int] + [vp] * 5 + [ctypes.c_int, vp]
    lib.fhd_packed_bytes.argtypes = [ctypes.c_int]
    lib.fhd_packed_bytes.restype = ctypes.c_int64
    lib.fhd_cg.argtypes = [vp] * 10 + [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                       vp, vp, vp]
    lib.fhd_cg_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.fhd_cg_workspace_bytes.restype = ctypes.c_int64
    lib.fhd_forward.argtypes = [vp] * 10 + [ctypes.c_int, ctypes.c_int, vp]
    lib.fhd_normal.argtypes = [vp] * 10 + [ctypes.c_int, ctypes.c_int, vp]
    lib.fhd_compute_grid.argtypes = [vp] * 5 + [ctypes.c_int] * 4 + [vp, ctypes.c_int] + [vp] * 3
    lib.fhd_grid_gather.argtypes = [vp] + [ctypes.c_int] * 4 + [vp, ctypes.c_int] + [vp] * 3
    lib.fhd_forward_grid.argtypes = [vp] * 3 + [ctypes.c_int] * 4 + [vp, ctypes.c_int] + [vp] * 5
    lib.fhd_normal_grid.argtypes = [vp] * 3 + [ctypes.c_int] * 4 + [vp, ctypes.c_int] + [vp] * 5
    lib.fhd_cg_grid.argtypes = ([vp] * 5 + [ctypes.c_int] * 4 + [vp, ctypes.c_int] + [vp] * 2 +
                                [ctypes.c_int, ctypes.c_float, vp, vp, vp])
    lib.fhd_last_error.restype = ctypes.c_char_p
    lib.fhd_status_string.restype = ctypes.c_char_p
    return lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fhd_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fhd_compute", "fhd_pack", "fhd_gather", "fhd_packed_bytes",
              "fhd_status_string", "fhd_last_error", "fhd_gather_config",
              "fhd_forward", "fhd_forward_pack", "fhd_forward_gather", "fhd_normal",
              "fhd_cg", "fhd_cg_workspace_bytes", "fhd_compute_grid", "fhd_grid_gather", "fhd_forward_grid",
              "fhd_normal_grid", "fhd_cg_grid", "fhd_compute_paths", "fhd_gather_paths",
              "fhd_forward_paths", "fhd_normal_paths", "fhd_cg_paths", "fhd_time_kernel",
              "fhd_timed_launches"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_microbench_library_loads():
    build.ensure_built()
    mb = ctypes.CDLL(build.lib_path("libfhd_microbench.so"))
    assert mb.fhdmb_mix_count() >= 8


def test_packed_bytes(lib):
    assert lib.fhd_packed_bytes(-1) == -1
    assert lib.fhd_packed_bytes(0) == 0
    # chunks of 8 samples x 5 fp32 fields
    assert lib.fhd_packed_bytes(1) == 8 * 5 * 4
    assert lib.fhd_packed_bytes(8) == 8 * 5 * 4
    assert lib.fhd_packed_bytes(9) == 2 * 8 * 5 * 4
    assert lib.fhd_packed_bytes(100_000) == 100_000 * 20
    assert lib.fhd_packed_bytes(2 ** 31 - 1) == ((2 ** 31 - 1 + 7) // 8) * 160


def test_status_strings(lib):
    for s in (0, -1, -2, -3, 7):
        assert lib.fhd_status_string(s)
    assert b"INVALID" in lib.fhd_status_string(-1)


def _last(lib):
    return lib.fhd_last_error().decode()


def test_negative_sizes_rejected(lib):
    assert lib.fhd_compute(*[None] * 10, -1, 4, None) == FHD_ERR_INVALID_ARG
    assert "M < 0" in _last(lib)
    assert lib.fhd_compute(*[None] * 10, 4, -1, None) == FHD_ERR_INVALID_ARG
    assert "N < 0" in _last(lib)
    assert lib.fhd_gather(None, -3, *[None] * 5, 4, None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_pack(*[None] * 5, -2, None, 0, None) == FHD_ERR_INVALID_ARG


def test_empty_calls_succeed_without_device(lib):
    # N = 0: nothing to do; M = 0 pack: nothing to do
    assert lib.fhd_compute(*[None] * 10, 5, 0, None) == FHD_OK
    assert lib.fhd_gather(None, 5, *[None] * 5, 0, None) == FHD_OK
    assert lib.fhd_pack(*[None] * 5, 0, None, 0, None) == FHD_OK


def test_null_pointers_rejected(lib):
    fake = [0x10000 * (i + 1) for i in range(10)]
    for i, name in enumerate(["kx", "ky", "kz", "Dr", "Di", "x", "y", "z", "rho_r", "rho_i"]):
        args = list(fake)
        args[i] = None
        assert lib.fhd_compute(*args, 16, 16, None) == FHD_ERR_INVALID_ARG
        assert name in _last(lib)


def test_misaligned_rejected(lib):
    fake = [0x100000 * (i + 1) for i in range(10)]
    fake[6] += 2
    assert lib.fhd_compute(*fake, 16, 16, None) == FHD_ERR_INVALID_ARG
    assert "aligned" in _last(lib)


def test_overlapping_output_rejected(lib):
    fake = [0x100000 * (i + 1) for i in range(10)]
    fake[9] = fake[8] + 8            # rho_i overlaps rho_r
    assert lib.fhd_compute(*fake, 16, 16, None) == FHD_ERR_INVALID_ARG
    assert "overlaps" in _last(lib)
    fake = [0x100000 * (i + 1) for i in range(10)]
    fake[8] = fake[5]                # rho_r aliases x
    assert lib.fhd_compute(*fake, 16, 16, None) == FHD_ERR_INVALID_ARG


def test_packed_buffer_alignment(lib):
    fake = [0x100000 * (i + 1) for i in range(6)]
    assert lib.fhd_pack(*fake[:5], 8, fake[5] + 4, 160, None) == FHD_ERR_INVALID_ARG
    assert "16-byte" in _last(lib)
    assert lib.fhd_gather(fake[5] + 8, 8, *fake[:5], 16, None) == FHD_ERR_INVALID_ARG


def test_pack_buffer_too_small_rejected(lib):
    fake = [0x100000 * (i + 1) for i in range(6)]
    assert lib.fhd_pack(*fake[:5], 9, fake[5], 160, None) == FHD_ERR_INVALID_ARG
    assert "packed_bytes" in _last(lib)


def test_binding_fails_loudly_without_library(tmp_path):
    from non_cartesian_mri_fhd_amd import binding
    with pytest.raises(FileNotFoundError):
        binding.load(str(tmp_path / "libfhd.so"))


def test_forward_and_normal_argument_checks(lib):
    fake = [0x100000 * (i + 1) for i in range(10)]
    assert lib.fhd_forward(*[None] * 10, -1, 3, None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_forward(*[None] * 10, 0, 3, None) == FHD_OK          # no samples: nothing
    args = list(fake)
    args[8] = fake[6]                                                  # Dr aliases rho_r
    assert lib.fhd_forward(*args, 16, 16, None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_normal(*[None] * 10, 3, -1, None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_normal(*[None] * 10, 3, 0, None) == FHD_OK          # no voxels: nothing
    args = list(fake)
    args[3] = None                                                     # x
    assert lib.fhd_normal(*args, 16, 16, None) == FHD_ERR_INVALID_ARG


def test_cg_argument_checks(lib):
    done = ctypes.c_int(7)
    fake = [0x100000 * (i + 1) for i in range(10)]
    assert lib.fhd_cg(*fake, 16, 16, 3, 0.0, None, None, None) == FHD_ERR_INVALID_ARG
    assert "iters_done" in _last(lib)
    assert lib.fhd_cg(*fake, 16, 16, -1, 0.0, ctypes.addressof(done), None, None) == \
        FHD_ERR_INVALID_ARG
    assert lib.fhd_cg(*fake, 16, 16, 3, -1.0, ctypes.addressof(done), None, None) == \
        FHD_ERR_INVALID_ARG
    assert lib.fhd_cg(*fake, 16, 16, 3, float("nan"), ctypes.addressof(done), None, None) == \
        FHD_ERR_INVALID_ARG
    assert lib.fhd_cg(*[None] * 10, 16, 0, 3, 0.0, ctypes.addressof(done), None, None) == FHD_OK
    assert done.value == 0
    assert lib.fhd_cg_workspace_bytes(-1, 4, 3) == -1
    assert lib.fhd_cg_workspace_bytes(4, 4, -3) == -1
    assert lib.fhd_cg_workspace_bytes(100, 1000, 50) >= 6 * 4000 + 2 * 400 + 51 * 8
    assert lib.fhd_cg_workspace_bytes(100, 1000, 1000) > lib.fhd_cg_workspace_bytes(100, 1000, 50)


def test_grid_argument_checks(lib):
    axis = (ctypes.c_float * 6)(-0.5, 1 / 16, -0.5, 1 / 16, -0.5, 1 / 16)
    ax = ctypes.addressof(axis)
    fake = [0x100000 * (i + 1) for i in range(7)]
    assert lib.fhd_compute_grid(*fake[:5], -1, 4, 4, 4, ax, 0, *fake[5:], None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_compute_grid(*fake[:5], 8, 4, -4, 4, ax, 0, *fake[5:], None) == FHD_ERR_INVALID_ARG
    assert "negative" in _last(lib)
    assert lib.fhd_compute_grid(*fake[:5], 8, 2048, 2048, 1024, ax, 0, *fake[5:], None) == \
        FHD_ERR_INVALID_ARG
    assert "2^31" in _last(lib)
    assert lib.fhd_compute_grid(*fake[:5], 8, 4, 4, 4, None, 0, *fake[5:], None) == FHD_ERR_INVALID_ARG
    assert "axis" in _last(lib)
    bad = (ctypes.c_float * 6)(-0.5, float("inf"), -0.5, 0.1, -0.5, 0.1)
    assert lib.fhd_compute_grid(*fake[:5], 8, 4, 4, 4, ctypes.addressof(bad), 0, *fake[5:], None) == \
        FHD_ERR_INVALID_ARG
    assert "finite" in _last(lib)
    # an empty grid does nothing, even with NULL buffers
    assert lib.fhd_compute_grid(*[None] * 5, 8, 0, 4, 4, ax, 0, None, None, None) == FHD_OK
    assert lib.fhd_grid_gather(None, 8, 4, 4, 0, ax, 0, None, None, None) == FHD_OK
    args = list(fake)
    args[2] = None                                                     # kz
    assert lib.fhd_compute_grid(*args[:5], 8, 4, 4, 4, ax, 0, *args[5:], None) == FHD_ERR_INVALID_ARG
    assert "kz" in _last(lib)
    args = list(fake)
    args[6] = args[5] + 16                                             # rho_i overlaps rho_r
    assert lib.fhd_compute_grid(*args[:5], 8, 4, 4, 4, ax, 0, *args[5:], None) == FHD_ERR_INVALID_ARG
    assert "overlaps" in _last(lib)
    assert lib.fhd_grid_gather(fake[0] + 8, 8, 4, 4, 4, ax, 0, fake[5], fake[6], None) == \
        FHD_ERR_INVALID_ARG
    assert "16-byte" in _last(lib)
    assert lib.fhd_grid_gather(fake[0], -8, 4, 4, 4, ax, 0, fake[5], fake[6], None) == \
        FHD_ERR_INVALID_ARG
    for bad_precision in (-1, 2, 7):
        assert lib.fhd_grid_gather(fake[0], 8, 4, 4, 4, ax, bad_precision, fake[5], fake[6],
                                   None) == FHD_ERR_INVALID_ARG
        assert "precision" in _last(lib)


def test_forward_grid_argument_checks(lib):
    axis = (ctypes.c_float * 6)(-0.5, 1 / 16, -0.5, 1 / 16, -0.5, 1 / 16)
    ax = ctypes.addressof(axis)
    fake = [0x100000 * (i + 1) for i in range(7)]
    k, img, out = fake[:3], fake[3:5], fake[5:]
    assert lib.fhd_forward_grid(*k, -1, 4, 4, 4, ax, 1, *img, *out, None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_forward_grid(*k, 8, 4, -1, 4, ax, 1, *img, *out, None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_forward_grid(*k, 8, 4, 4, 4, None, 1, *img, *out, None) == FHD_ERR_INVALID_ARG
    # only the split-bf16 mode exists for F on a grid
    assert lib.fhd_forward_grid(*k, 8, 4, 4, 4, ax, 0, *img, *out, None) == FHD_ERR_INVALID_ARG
    assert "BF16X3" in _last(lib)
    assert lib.fhd_forward_grid(*k, 8, 4, 4, 4, ax, 5, *img, *out, None) == FHD_ERR_INVALID_ARG
    # no samples: nothing to do
    assert lib.fhd_forward_grid(None, None, None, 0, 4, 4, 4, ax, 1, None, None, None, None,
                                None) == FHD_OK
    bad = list(out)
    bad[1] = img[0]                                                    # Di aliases rho_r
    assert lib.fhd_forward_grid(*k, 8, 4, 4, 4, ax, 1, *img, *bad, None) == FHD_ERR_INVALID_ARG
    assert "overlaps" in _last(lib)


def test_normal_and_cg_grid_argument_checks(lib):
    axis = (ctypes.c_float * 6)(-0.5, 1 / 16, -0.5, 1 / 16, -0.5, 1 / 16)
    ax = ctypes.addressof(axis)
    done = ctypes.c_int(9)
    d = ctypes.addressof(done)
    fake = [0x100000 * (i + 1) for i in range(7)]
    assert lib.fhd_normal_grid(*fake[:3], 8, 4, 4, 4, ax, 0, *fake[3:], None) == FHD_ERR_INVALID_ARG
    assert "BF16X3" in _last(lib)
    assert lib.fhd_normal_grid(*fake[:3], -1, 4, 4, 4, ax, 1, *fake[3:], None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_normal_grid(*fake[:3], 8, 0, 4, 4, ax, 1, *fake[3:], None) == FHD_OK
    bad = list(fake)
    bad[5] = bad[3]                                                    # q_r aliases p_r
    assert lib.fhd_normal_grid(*bad[:3], 8, 4, 4, 4, ax, 1, *bad[3:], None) == FHD_ERR_INVALID_ARG
    args = fake[:5]
    assert lib.fhd_cg_grid(*args, 8, 4, 4, 4, ax, 1, fake[5], fake[6], 3, 0.0, None, None,
                           None) == FHD_ERR_INVALID_ARG
    assert "iters_done" in _last(lib)
    assert lib.fhd_cg_grid(*args, 8, 4, 4, 4, ax, 1, fake[5], fake[6], -1, 0.0, d, None,
                           None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_cg_grid(*args, 8, 4, 4, 4, ax, 1, fake[5], fake[6], 3, float("nan"), d, None,
                           None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_cg_grid(*args, 8, 4, 4, 4, ax, 0, fake[5], fake[6], 3, 0.0, d, None,
                           None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_cg_grid(*args, 8, 4, 0, 4, ax, 1, None, None, 3, 0.0, d, None, None) == FHD_OK
    assert done.value == 0


def test_scatter_argument_checks(lib):
    """fhd_scatter shares fhd_compute's contract: sizes, NULLs, alignment and
    overlap are rejected on the host before any HIP call."""
    assert lib.fhd_scatter(*[None] * 10, -1, 4, None) == FHD_ERR_INVALID_ARG
    assert "M < 0" in _last(lib)
    assert lib.fhd_scatter(*[None] * 10, 4, -1, None) == FHD_ERR_INVALID_ARG
    assert "N < 0" in _last(lib)
    assert lib.fhd_scatter(*[None] * 10, 5, 0, None) == FHD_OK
    fake = [0x100000 * (i + 1) for i in range(10)]
    args = list(fake)
    args[3] = None
    assert lib.fhd_scatter(*args, 16, 16, None) == FHD_ERR_INVALID_ARG
    assert "Dr" in _last(lib)
    args = list(fake)
    args[7] += 2
    assert lib.fhd_scatter(*args, 16, 16, None) == FHD_ERR_INVALID_ARG
    assert "aligned" in _last(lib)
    args = list(fake)
    args[9] = args[8] + 8
    assert lib.fhd_scatter(*args, 16, 16, None) == FHD_ERR_INVALID_ARG
    assert "overlaps" in _last(lib)


def test_unknown_paths_rejected_before_any_device_call(lib):
    """Every *_paths entry point refuses a paths value other than
    FHD_GATHER_ALL (0), FHD_GATHER_VECTOR (1) and FHD_GATHER_BF16X3 (2),
    with sizes that would otherwise do nothing."""
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.fhd_compute_paths.argtypes = [vp] * 10 + [i32, i32, i32, vp]
    lib.fhd_gather_paths.argtypes = [vp, i32] + [vp] * 5 + [i32, i32, vp]
    lib.fhd_forward_paths.argtypes = [vp] * 10 + [i32, i32, i32, vp]
    lib.fhd_normal_paths.argtypes = [vp] * 10 + [i32, i32, i32, vp]
    lib.fhd_cg_paths.argtypes = [vp] * 10 + [i32, i32, i32, ctypes.c_float, vp, vp, i32, vp]
    done = ctypes.c_int(0)
    for bad in (-1, 3, 7):
        assert lib.fhd_compute_paths(*[None] * 10, 0, 0, bad, None) == FHD_ERR_INVALID_ARG
        assert b"paths" in lib.fhd_last_error()
        assert lib.fhd_gather_paths(None, 0, *[None] * 5, 0, bad, None) == FHD_ERR_INVALID_ARG
        assert lib.fhd_forward_paths(*[None] * 10, 0, 0, bad, None) == FHD_ERR_INVALID_ARG
        assert lib.fhd_normal_paths(*[None] * 10, 0, 0, bad, None) == FHD_ERR_INVALID_ARG
        assert lib.fhd_cg_paths(*[None] * 10, 0, 0, 3, 0.0, ctypes.byref(done), None, bad,
                                None) == FHD_ERR_INVALID_ARG
    for good in (0, 1, 2):
        assert lib.fhd_compute_paths(*[None] * 10, 0, 0, good, None) == FHD_OK
        assert lib.fhd_gather_paths(None, 0, *[None] * 5, 0, good, None) == FHD_OK
        assert lib.fhd_forward_paths(*[None] * 10, 0, 0, good, None) == FHD_OK
        assert lib.fhd_normal_paths(*[None] * 10, 0, 0, good, None) == FHD_OK
        assert lib.fhd_cg_paths(*[None] * 10, 0, 0, 3, 0.0, ctypes.byref(done), None, good,
                                None) == FHD_OK


def test_kernel_timing_hook_arguments(lib):
    """fhd_time_kernel needs no device: it only copies the names and
    handles; bad arguments are refused and leave the hook disarmed."""
    lib.fhd_time_kernel.argtypes = [ctypes.c_char_p, ctypes.c_void_p, ctypes.c_int]
    lib.fhd_timed_launches.restype = ctypes.c_int
    two = (ctypes.c_void_p * 2)(1, 2)     # opaque handles, never used here
    assert lib.fhd_time_kernel(b"fhd_gather_kernel<16, true>", two, -1) == FHD_ERR_INVALID_ARG
    assert lib.fhd_time_kernel(b"fhd_gather_kernel<16, true>", None, 1) == FHD_ERR_INVALID_ARG
    holes = (ctypes.c_void_p * 2)(1, None)
    assert lib.fhd_time_kernel(b"fhd_gather_kernel<16, true>", holes, 1) == FHD_ERR_INVALID_ARG
    assert lib.fhd_time_kernel(b"fhd_gather_kernel<16, true>", two, 1) == FHD_OK
    assert lib.fhd_timed_launches() == 0
    assert lib.fhd_time_kernel(None, None, 0) == FHD_OK
    assert lib.fhd_timed_launches() == 0



def test_stale_library_is_rebuilt_when_a_source_is_newer(tmp_path):
    """ensure_built() rebuilds a library older than any of its sources or
    headers (here: a header's time set an hour ahead, then restored)."""
    build.ensure_built()
    assert not build.is_stale("libfhd.so")
    header = os.path.join(ROOT, "include", "fhd.h")
    st = os.stat(header)
    try:
        os.utime(header, (st.st_atime, os.path.getmtime(build.lib_path("libfhd.so")) + 3600))
        assert build.is_stale("libfhd.so")
    finally:
        os.utime(header, (st.st_atime, st.st_mtime))
    assert not build.is_stale("libfhd.so")
    assert header in build.sources_of("libfhd.so")


def test_noalloc_argument_checks(lib):
    """fhd_compute_noalloc refuses bad arguments, and a workspace beyond its
    scratch array, before touching any device memory: eight million samples
    need 160 MB of packed k-space alone, above FHD_NOALLOC_SCRATCH_BYTES
    (128 MiB). The pointers of that case are never dereferenced."""
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.fhd_compute_noalloc.argtypes = [vp] * 10 + [i32, i32, i32, vp]
    assert lib.fhd_compute_noalloc(*[None] * 10, -1, 5, 0, None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_compute_noalloc(*[None] * 10, 5, -1, 0, None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_compute_noalloc(*[None] * 10, 0, 0, 3, None) == FHD_ERR_INVALID_ARG
    assert lib.fhd_compute_noalloc(*[None] * 10, 0, 0, 0, None) == FHD_OK
    assert lib.fhd_compute_noalloc(*[None] * 10, 0, 5, 0, None) == FHD_ERR_INVALID_ARG
    fake = [0x10000000 * (i + 1) for i in range(10)]
    assert lib.fhd_compute_noalloc(*fake, 8_000_000, 4096, 0, None) == FHD_ERR_INVALID_ARG
    msg = lib.fhd_last_error()
    assert b"needs" in msg and str(128 * 1024 * 1024).encode() in msg


def test_release_workspaces_with_nothing_kept(lib):
    """With no call made on any stream there is nothing to free: FHD_OK,
    and no device is needed for it."""
    lib.fhd_release_workspaces.argtypes = []
    lib.fhd_release_workspaces.restype = ctypes.c_int
    assert lib.fhd_release_workspaces() == FHD_OK
