// abi_checks.hip -- host-side argument checks and error reporting shared by
// every entry point of libfhd.so.
#include <cstdint>
#include <string>

#include "fhd_internal.h"

namespace fhd {

namespace {
thread_local std::string g_last_error;

bool overlaps(const Span &a, const Span &b)
{
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

int check_device_span(const Span &s, int device)
{
    if (s.bytes <= 0) return FHD_OK;
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, s.p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(FHD_ERR_INVALID_ARG, std::string(s.name) + " is not device-accessible memory (" +
                                             hipGetErrorString(e) + ")");
    }
    if (attr.type == hipMemoryTypeDevice) {
        if (attr.device != device)
            return fail(FHD_ERR_INVALID_ARG, std::string(s.name) + " lives on device " +
                                                 std::to_string(attr.device) + ", current is " +
                                                 std::to_string(device));
        // the span must end inside the allocation holding its first byte; if
        // the allocation cannot be found, refuse rather than launch blind
        hipDeviceptr_t base = nullptr;
        size_t size = 0;
        e = hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)s.p);
        if (e != hipSuccess || !base) {
            (void)hipGetLastError();
            return fail(FHD_ERR_INVALID_ARG, std::string(s.name) +
                                                 ": cannot find its allocation to check its size");
        }
        const uintptr_t b0 = (uintptr_t)base, p0 = (uintptr_t)s.p;
        if (p0 < b0 || p0 + (uintptr_t)s.bytes > b0 + size)
            return fail(FHD_ERR_INVALID_ARG, std::string(s.name) + " holds fewer than " +
                                                 std::to_string(s.bytes) + " bytes");
        return FHD_OK;
    }
    if (attr.type == hipMemoryTypeHost || attr.type == hipMemoryTypeManaged ||
        attr.type == hipMemoryTypeUnified)
        return FHD_OK;
    return fail(FHD_ERR_INVALID_ARG, std::string(s.name) + " is not device-accessible memory");
}
}  // namespace

int fail(int status, const std::string &msg)
{
    g_last_error = msg;
    return status;
}

void clear_error() { g_last_error.clear(); }

int check_host_side(const Span *spans, int count)
{
    for (int i = 0; i < count; ++i) {
        if (spans[i].bytes <= 0) continue;
        if (!spans[i].p) return fail(FHD_ERR_INVALID_ARG, std::string(spans[i].name) + " is NULL");
        if ((uintptr_t)spans[i].p % spans[i].align)
            return fail(FHD_ERR_INVALID_ARG, std::string(spans[i].name) + " is not " +
                                                 std::to_string(spans[i].align) + "-byte aligned");
    }
    return FHD_OK;
}

int check_no_overlap(const Span *spans, int count, int first_out)
{
    for (int i = first_out; i < count; ++i)
        for (int j = 0; j < count; ++j)
            if (j != i && overlaps(spans[i], spans[j]))
                return fail(FHD_ERR_INVALID_ARG, std::string(spans[i].name) + " overlaps " +
                                                     spans[j].name);
    return FHD_OK;
}

int check_device_spans(const Span *spans, int count)
{
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return fail(FHD_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    for (int i = 0; i < count; ++i) {
        const int rc = check_device_span(spans[i], device);
        if (rc != FHD_OK) return rc;
    }
    return FHD_OK;
}

int launch_status(const char *what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FHD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return FHD_OK;
}

}  // namespace fhd

extern "C" const char *fhd_status_string(int status)
{
    switch (status) {
    case FHD_OK: return "FHD_OK: success";
    case FHD_ERR_INVALID_ARG: return "FHD_ERR_INVALID_ARG: invalid pointer, size, alignment or overlap";
    case FHD_ERR_HIP: return "FHD_ERR_HIP: HIP runtime or launch error";
    case FHD_ERR_ALLOC: return "FHD_ERR_ALLOC: workspace allocation failed";
    default: return "unknown fhd status";
    }
}

extern "C" const char *fhd_last_error(void) { return fhd::g_last_error.c_str(); }
