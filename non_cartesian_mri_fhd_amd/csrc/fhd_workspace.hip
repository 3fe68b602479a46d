// fhd_workspace.hip -- per-stream device workspaces kept between calls.
//
// A call of the allocating entry points needs device memory beyond its
// inputs and outputs (packed k-space, unit classes, the long-line factor
// table, split partial sums). Allocating and freeing it per call costs
// host time that, on small grids, is a large part of the call. So each
// (device, stream) pair keeps one buffer per use ("slot"), grown when a
// call needs more and otherwise reused: the calls on one stream run in
// stream order, so a call's kernels never overlap the previous call's.
//
// While a stream is being captured into a graph, a call instead takes
// stream-ordered allocations (hipMallocAsync / hipFreeAsync), which a graph
// records as its own allocation nodes, so that a graph never holds a
// cached buffer that a later call may free.
//
// Calls on one stream from several host threads are serialised: a call
// holds its stream's lock from its first workspace request to its end.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "fhd_internal.h"

namespace fhd {

struct WorkspaceEntry {
    std::recursive_mutex lock;
    char *ptr[kSlots] = {};
    size_t cap[kSlots] = {};
};

namespace {

// Never destroyed (entries included, which a call may still be waiting to
// lock): freeing device memory from a static destructor would run after
// the HIP runtime's own teardown.
std::mutex &map_lock()
{
    static std::mutex *m = new std::mutex;
    return *m;
}
std::map<std::pair<int, hipStream_t>, WorkspaceEntry *> &entries()
{
    static auto *m = new std::map<std::pair<int, hipStream_t>, WorkspaceEntry *>;
    return *m;
}

constexpr size_t kGrain = (size_t)2 << 20;   // buffers grow in 2 MiB steps

}  // namespace

StreamBuffer::StreamBuffer(hipStream_t stream, int slot) : stream_(stream), slot_(slot) {}

StreamBuffer::~StreamBuffer() { (void)finish(); }

int StreamBuffer::get(size_t bytes, char **out)
{
    *out = nullptr;
    if (bytes == 0) return FHD_OK;
    if (async_ || entry_) return fail(FHD_ERR_INVALID_ARG, "internal: one request per workspace buffer");
    hipStreamCaptureStatus status = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream_, &status);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(FHD_ERR_HIP, std::string("hipStreamIsCapturing: ") + hipGetErrorString(e));
    }
    if (status != hipStreamCaptureStatusNone) {
        e = hipMallocAsync(reinterpret_cast<void **>(&async_), bytes, stream_);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            async_ = nullptr;
            return fail(FHD_ERR_ALLOC, std::string("hipMallocAsync (workspace): ") + hipGetErrorString(e));
        }
        *out = async_;
        return FHD_OK;
    }
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(FHD_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    }
    WorkspaceEntry *entry;
    {
        std::lock_guard<std::mutex> g(map_lock());
        WorkspaceEntry *&slot = entries()[{dev, stream_}];
        if (!slot) slot = new WorkspaceEntry;
        entry = slot;
    }
    entry->lock.lock();
    entry_ = entry;
    if (entry->cap[slot_] < bytes) {
        if (entry->ptr[slot_]) {
            // the old buffer may still be in use by this stream's queued work
            e = hipStreamSynchronize(stream_);
            if (e == hipSuccess) e = hipFree(entry->ptr[slot_]);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                return fail(FHD_ERR_HIP, std::string("freeing a smaller workspace: ") + hipGetErrorString(e));
            }
            entry->ptr[slot_] = nullptr;
            entry->cap[slot_] = 0;
        }
        const size_t want = (bytes + kGrain - 1) / kGrain * kGrain;
        e = hipMalloc(reinterpret_cast<void **>(&entry->ptr[slot_]), want);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            entry->ptr[slot_] = nullptr;
            return fail(FHD_ERR_ALLOC, "hipMalloc (workspace, " + std::to_string(want) +
                                           " bytes): " + hipGetErrorString(e));
        }
        entry->cap[slot_] = want;
    }
    *out = entry->ptr[slot_];
    return FHD_OK;
}

int StreamBuffer::finish()
{
    int rc = FHD_OK;
    if (async_) {
        const hipError_t e = hipFreeAsync(async_, stream_);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            rc = fail(FHD_ERR_HIP, std::string("hipFreeAsync (workspace): ") + hipGetErrorString(e));
        }
        async_ = nullptr;
    }
    if (entry_) {
        entry_->lock.unlock();
        entry_ = nullptr;
    }
    return rc;
}

}  // namespace fhd

using namespace fhd;

extern "C" int fhd_release_workspaces(void)
{
    clear_error();
    // a call holds its entry's lock while it may still ask for the map's:
    // take the list first, then each entry's lock alone
    std::map<std::pair<int, hipStream_t>, WorkspaceEntry *> all;
    {
        std::lock_guard<std::mutex> g(map_lock());
        all = entries();
    }
    int rc = FHD_OK, current = 0;
    if (hipGetDevice(&current) != hipSuccess) {
        (void)hipGetLastError();
        current = -1;
    }
    for (auto &kv : all) {
        WorkspaceEntry *entry = kv.second;
        std::lock_guard<std::recursive_mutex> h(entry->lock);
        hipError_t e = hipSetDevice(kv.first.first);
        if (e == hipSuccess) e = hipDeviceSynchronize();
        for (int s = 0; s < kSlots && e == hipSuccess; ++s) {
            if (entry->ptr[s]) e = hipFree(entry->ptr[s]);
            if (e == hipSuccess) {
                entry->ptr[s] = nullptr;
                entry->cap[s] = 0;
            }
        }
        if (e != hipSuccess) {
            (void)hipGetLastError();
            if (rc == FHD_OK) rc = fail(FHD_ERR_HIP, std::string("fhd_release_workspaces: ") + hipGetErrorString(e));
        }
    }
    if (current >= 0) (void)hipSetDevice(current);
    return rc;
}
