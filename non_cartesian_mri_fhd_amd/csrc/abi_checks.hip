// abi_checks.hip -- host-side argument checks and error reporting shared by
// every entry point of libfhd.so.
#include <cstdint>
#include <string>
#include <vector>

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

namespace {
// The calling thread's armed kernel events (fhd_time_kernel).
struct KernelEvents {
    std::string name;
    std::vector<hipEvent_t> events;   // start, stop per launch
    int used = 0;
};
thread_local KernelEvents g_kernel_events;
}  // namespace

int timed_begin(const char *kernel, hipStream_t stream)
{
    KernelEvents &k = g_kernel_events;
    if (k.events.empty() || 2 * k.used >= (int)k.events.size() || k.name != kernel) return -1;
    const int slot = k.used++;
    (void)hipEventRecord(k.events[2 * slot], stream);
    return slot;
}

void timed_end(int slot, hipStream_t stream)
{
    if (slot >= 0) (void)hipEventRecord(g_kernel_events.events[2 * slot + 1], stream);
}

int fail_paths()
{
    return fail(FHD_ERR_INVALID_ARG, "paths must be FHD_GATHER_ALL, FHD_GATHER_VECTOR or FHD_GATHER_BF16X3");
}

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

int device_cus()
{
    static int cus_cached[64] = {0};
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= 64) {
        (void)hipGetLastError();
        return 0;
    }
    if (cus_cached[device] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
            cus <= 0) {
            (void)hipGetLastError();
            return 0;
        }
        cus_cached[device] = cus;
    }
    return cus_cached[device];
}

int split_count(int64_t blocks, int nchunks, int per_cu, int granule, double slack)
{
    const int cus = device_cus();
    if (cus <= 0) return 1;
    if (per_cu < 1) per_cu = 1;
    const int64_t resident = (int64_t)per_cu * cus;
    if (granule < 1) granule = 1;
    const int64_t stages = (nchunks + granule - 1) / granule;
    if (blocks <= 0 || stages <= 1) return 1;
    // Cutting the stream s ways makes every workgroup's work 1/s as long and
    // the launch ceil(s blocks / resident) rounds of them: time ~ rounds / s,
    // bounded below by blocks / resident. Take the fewest ways (at most one
    // per granule, and at most 16 or two rounds' worth) that come within
    // `slack` of the best.
    // s ways give every split ceil(stages / s) granules, so only
    // ceil(stages / that) of them have any: count those
    auto ways = [&](int64_t s) {
        const int64_t per = (stages + s - 1) / s;
        return (stages + per - 1) / per;
    };
    auto cost = [&](int64_t s) {
        const int64_t w = ways(s);
        return (double)((blocks * w + resident - 1) / resident) / (double)w;
    };
    int64_t most = 2 * resident / blocks;
    if (most < 16) most = 16;
    if (most > stages) most = stages;
    double lowest = cost(1);
    for (int64_t s = 2; s <= most; ++s) lowest = cost(s) < lowest ? cost(s) : lowest;
    for (int64_t s = 1; s <= most; ++s)
        if (cost(s) <= slack * lowest) return (int)ways(s);
    return 1;
}

namespace {
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float *__restrict__ part_r,
                                                            const float *__restrict__ part_i,
                                                            int splits, int64_t n,
                                                            float *__restrict__ out_r,
                                                            float *__restrict__ out_i,
                                                            const int *__restrict__ gate, int gate_want)
{
    if (gate != nullptr && lines_form_ran(gate) != (gate_want != 0)) return;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    // eight rows' loads in flight at a time, added in row order
    constexpr int kBatch = 8;
    float sr = 0.0f, si = 0.0f;
    int s = 0;
    for (; s + kBatch <= splits; s += kBatch) {
        float a[kBatch], b[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            a[k] = part_r[(int64_t)(s + k) * n + i];
            b[k] = part_i[(int64_t)(s + k) * n + i];
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            sr += a[k];
            si += b[k];
        }
    }
    for (; s < splits; ++s) {
        sr += part_r[(int64_t)s * n + i];
        si += part_i[(int64_t)s * n + i];
    }
    out_r[i] = sr;
    out_i[i] = si;
}

}  // namespace

int launch_reduce(const float *part_r, const float *part_i, int splits, int64_t n, float *out_r,
                  float *out_i, hipStream_t stream, const int *gate, bool gate_want)
{
    if (n == 0) return FHD_OK;
    reduce_splits_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(
        part_r, part_i, splits, n, out_r, out_i, gate, gate_want ? 1 : 0);
    return launch_status("reduce_splits_kernel launch");
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

extern "C" int fhd_time_kernel(const char *kernel, void *const *events, int count)
{
    fhd::clear_error();
    fhd::KernelEvents &k = fhd::g_kernel_events;
    k.events.clear();
    k.used = 0;
    k.name.clear();
    if (count < 0) return fhd::fail(FHD_ERR_INVALID_ARG, "count < 0");
    if (count == 0 || !kernel) return FHD_OK;
    if (!events) return fhd::fail(FHD_ERR_INVALID_ARG, "events is NULL");
    for (int i = 0; i < 2 * count; ++i)
        if (!events[i]) return fhd::fail(FHD_ERR_INVALID_ARG, "events holds a NULL event");
    k.name = kernel;
    for (int i = 0; i < 2 * count; ++i) k.events.push_back((hipEvent_t)events[i]);
    return FHD_OK;
}

extern "C" int fhd_timed_launches(void) { return fhd::g_kernel_events.used; }
