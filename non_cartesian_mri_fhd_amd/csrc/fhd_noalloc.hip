// fhd_noalloc.hip -- F^H D with no allocation: fhd_compute_noalloc, for
// callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// Its workspace -- the packed k-space, the unit classes, info words and
// line-pair records and the split partial sums -- lives in one file-scope
// device array, `scratch`, of kScratchBytes per GPU, held from the
// library's first use of a GPU until the process ends. The long-line and
// line-pair instances form their cos / sin factor operands in each
// workgroup instead of reading a per-call table (the same arithmetic),
// which keeps the workspace at 20 bytes per sample, 8 bytes per 4096
// voxels and, when the voxels are too few to fill the GPU in one pass, 8
// bytes per voxel and partial sum.
//
// In host code `scratch` names a host-side stand-in, not the array's device
// address: the address comes from hipGetSymbolAddress, once per device
// with that device current, and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>

#include "fhd_internal.h"

namespace fhd {

constexpr size_t kScratchBytes = FHD_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte blocks");

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
char *g_scratch_ptr[kMaxDevices] = {nullptr};

// The device address of `scratch` on the current device, looked up once
// per device; nullptr (with the error recorded) if the lookup fails.
char *device_scratch(int *status)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        *status = fail(FHD_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            *status = fail(FHD_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = static_cast<char *>(ptr);
    }
    return g_scratch_ptr[dev];
}

size_t up256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace
}  // namespace fhd

using namespace fhd;

extern "C" int fhd_compute_noalloc(const float *kx, const float *ky, const float *kz, const float *Dr,
                                   const float *Di, const float *x, const float *y, const float *z,
                                   float *rho_r, float *rho_i, int M, int N, int paths, void *stream)
{
    clear_error();
    if (M < 0) return fail(FHD_ERR_INVALID_ARG, "M < 0");
    if (N < 0) return fail(FHD_ERR_INVALID_ARG, "N < 0");
    if (!valid_paths(paths)) return fail_paths();
    if (N == 0) return FHD_OK;
    const int64_t mb = (int64_t)M * 4, nb = (int64_t)N * 4;
    const Span all[] = {{kx, mb, "kx"}, {ky, mb, "ky"}, {kz, mb, "kz"}, {Dr, mb, "Dr"},
                        {Di, mb, "Di"}, {x, nb, "x"},   {y, nb, "y"},   {z, nb, "z"},
                        {rho_r, nb, "rho_r"}, {rho_i, nb, "rho_i"}};
    int rc = check_host_side(all, 10);
    if (rc == FHD_OK) rc = check_no_overlap(all, 10, 8);
    if (rc != FHD_OK) return rc;
    const GatherPlan g = plan_gather(M, N, paths, false);
    const size_t packed_bytes = up256((size_t)packed_bytes_for(M));
    const size_t need = packed_bytes + g.work_bytes();
    if (need > kScratchBytes)
        return fail(FHD_ERR_INVALID_ARG, "fhd_compute_noalloc needs " + std::to_string(need) +
                                             " bytes of workspace for M = " + std::to_string(M) +
                                             ", N = " + std::to_string(N) + "; its scratch holds " +
                                             std::to_string(kScratchBytes));
    if ((rc = check_device_spans(all, 10)) != FHD_OK) return rc;
    char *base = device_scratch(&rc);
    if (!base) return rc;

    hipStream_t s = (hipStream_t)stream;
    float *packed = reinterpret_cast<float *>(base);
    if (M > 0 && (rc = launch_pack(kx, ky, kz, Dr, Di, M, packed, s)) != FHD_OK) return rc;
    return run_gather(g, base + packed_bytes, M > 0 ? packed : nullptr, M, x, y, z, rho_r, rho_i, N, s);
}
