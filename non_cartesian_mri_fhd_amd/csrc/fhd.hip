// fhd.hip -- F^H D (adjoint non-uniform DFT) for MI355X / gfx950.
//
// rho_n = sum_m D_m exp(+i 2 pi k_m . x_n)   (page "Case study -- iterative
// MRI reconstruction", section 17.3, F^H D equation)
//
// Two kernels, split by loop fission (section 17.3.2):
//
//  * fhd_pack_kernel -- per-sample pre-pass. Writes each sample as
//    (kx, ky, kz, psi, a) with a = |D| and psi = arg(D) / (2 pi) in
//    revolutions, so that D e^{i 2 pi p} = a e^{i 2 pi (p + psi)}. The
//    complex multiply-accumulate then needs two FMAs instead of four, and
//    psi folds into the phase dot product. Samples are stored in chunks of
//    kChunk, field-major inside a chunk ([kx x8][ky x8][kz x8][psi x8][a x8],
//    160 B = ten 16-byte vectors). The tail chunk is padded with a = 0
//    records, which add exactly 0.
//
//  * fhd_gather_kernel -- one lane per kVox consecutive voxels, no atomics
//    (sections 17.3.1, 17.3.3). Voxel coordinates and the 2*kVox
//    accumulators live in VGPRs. Every lane of the grid walks the same
//    sample stream (section 17.3.4's observation): a workgroup stages
//    kStageChunks chunks at a time in LDS (double buffered, the next stage
//    prefetched into registers while the current one is used) and every
//    lane reads each sample with a same-address ds_read_b128, which the LDS
//    broadcasts. The samples arrive in VGPRs: on gfx950 an FP32 FMA with an
//    SGPR operand issues at half the rate of an all-VGPR one, so a
//    scalar-load broadcast would halve the FMA rate.
//
//    Phases stay in revolutions and go straight into v_sin_f32 / v_cos_f32,
//    which take revolutions and reduce the argument exactly in hardware
//    (measured identical to an explicit v_fract_f32 reduction over the
//    whole fp32 range), so there is no 2 pi multiply and no fract (section
//    17.3.5, hardware trig).
//
//    When, in every lane of a wave, the kVox voxels share y and z bitwise
//    (any x-fastest voxel grid), ky*y + kz*z + psi is formed once per
//    sample and lane and each voxel adds kx*x with one FMA. The arithmetic
//    is the same FMA sequence as the general path, so results are bitwise
//    identical; waves that fail the test take the general path.
//
// Per voxel-sample term: phase 1 + 2/kVox FMA (3 FMA on the general path),
// v_cos_f32, v_sin_f32, 2 FMA accumulate.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>

#include "fhd.h"

namespace {

constexpr int kBlock = 256;        // gather workgroup: 4 wave64
constexpr int kVox = 8;            // consecutive voxels per lane
constexpr int kChunk = 8;          // samples per packed chunk
constexpr int kFields = 5;         // kx, ky, kz, psi, a
constexpr int kChunkVec4 = kChunk * kFields / 4;        // 10 float4 per chunk
constexpr int kStageChunks = 64;   // chunks per LDS stage (512 samples, 10 KB)
constexpr int kStageVec4 = kStageChunks * kChunkVec4;   // 640 float4
constexpr int kStageLoads = (kStageVec4 + kBlock - 1) / kBlock;   // 3 per lane
constexpr int kPackBlock = 256;

static_assert(kBlock % 64 == 0, "workgroup must be whole wave64s");
static_assert(kChunk * kFields % 4 == 0, "chunks must be whole float4s");
static_assert(kStageLoads == 3, "staging code below holds three float4 per lane");

thread_local std::string g_last_error;

int fail(int status, const std::string &msg)
{
    g_last_error = msg;
    return status;
}

int64_t packed_bytes_for(int64_t M)
{
    const int64_t chunks = (M + kChunk - 1) / kChunk;
    return chunks * kChunk * kFields * (int64_t)sizeof(float);
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPackBlock) void fhd_pack_kernel(
    const float *__restrict__ kx, const float *__restrict__ ky, const float *__restrict__ kz,
    const float *__restrict__ Dr, const float *__restrict__ Di,
    float *__restrict__ packed, int M, int64_t M_pad)
{
    const int64_t m = (int64_t)blockIdx.x * kPackBlock + threadIdx.x;
    if (m >= M_pad) return;
    float fx = 0.0f, fy = 0.0f, fz = 0.0f, psi = 0.0f, amp = 0.0f;
    if (m < M) {
        fx = kx[m];
        fy = ky[m];
        fz = kz[m];
        // polar form of D in double, rounded once to fp32
        const double re = Dr[m], im = Di[m];
        amp = (float)hypot(re, im);
        psi = (float)(atan2(im, re) * (0.5 / M_PI));   // [-0.5, 0.5] revolutions
    }
    float *c = packed + (m / kChunk) * (kFields * kChunk) + (m % kChunk);
    c[0 * kChunk] = fx;
    c[1 * kChunk] = fy;
    c[2 * kChunk] = fz;
    c[3 * kChunk] = psi;
    c[4 * kChunk] = amp;
}

// Unpack one chunk's float4s (read from LDS) into per-field arrays.
__device__ __forceinline__ void load_chunk(const float4 *ch, float (&f)[kFields][kChunk])
{
#pragma unroll
    for (int q = 0; q < kChunkVec4; ++q) {
        const float4 t = ch[q];
        const int field = (4 * q) / kChunk, at = (4 * q) % kChunk;
        f[field][at + 0] = t.x;
        f[field][at + 1] = t.y;
        f[field][at + 2] = t.z;
        f[field][at + 3] = t.w;
    }
}

// Accumulate one chunk of kChunk samples into a lane's V voxels.
// SHARED: all V voxels have the same y and z (checked by the caller).
template <int V, bool SHARED>
__device__ __forceinline__ void accumulate_chunk(const float4 *ch, const float (&px)[V],
                                                 const float (&py)[V], const float (&pz)[V],
                                                 float (&acc_r)[V], float (&acc_i)[V])
{
    float f[kFields][kChunk];
    load_chunk(ch, f);
    const float(&skx)[kChunk] = f[0];
    const float(&sky)[kChunk] = f[1];
    const float(&skz)[kChunk] = f[2];
    const float(&psi)[kChunk] = f[3];
    const float(&amp)[kChunk] = f[4];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
        float p[V], c[V], s[V];
        // phase in revolutions, including arg(D)
        if constexpr (SHARED) {
            const float q = __builtin_fmaf(sky[u], py[0], __builtin_fmaf(skz[u], pz[0], psi[u]));
#pragma unroll
            for (int v = 0; v < V; ++v) p[v] = __builtin_fmaf(skx[u], px[v], q);
        } else {
#pragma unroll
            for (int v = 0; v < V; ++v)
                p[v] = __builtin_fmaf(skx[u], px[v],
                                      __builtin_fmaf(sky[u], py[v], __builtin_fmaf(skz[u], pz[v], psi[u])));
        }
        // keep the transcendentals of a sample together: grouped, they
        // issue back to back instead of interleaving with the FMAs
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 0; v < V; ++v) c[v] = __builtin_amdgcn_cosf(p[v]);
#pragma unroll
        for (int v = 0; v < V; ++v) s[v] = __builtin_amdgcn_sinf(p[v]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            acc_r[v] = __builtin_fmaf(amp[u], c[v], acc_r[v]);
            acc_i[v] = __builtin_fmaf(amp[u], s[v], acc_i[v]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// At least 4 waves per SIMD (<= 128 VGPRs): a 128^3 grid at 8 voxels per
// lane is exactly 4 waves per SIMD, so all of them are resident at once.
template <int V>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void fhd_gather_kernel(
    const float *__restrict__ packed, int nchunks,
    const float *__restrict__ x, const float *__restrict__ y, const float *__restrict__ z,
    float *__restrict__ rho_r, float *__restrict__ rho_i, int N)
{
    __shared__ float4 stage[2][kStageVec4];
    const float4 *src = reinterpret_cast<const float4 *>(packed);

    // lane l of workgroup b owns voxels (b*kBlock + l)*V + v, v < V
    const int64_t n0 = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * V;
    float px[V], py[V], pz[V], acc_r[V], acc_i[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int64_t n = n0 + v;
        const bool live = n < N;
        px[v] = live ? x[n] : 0.0f;
        py[v] = live ? y[n] : 0.0f;
        pz[v] = live ? z[n] : 0.0f;
        acc_r[v] = 0.0f;
        acc_i[v] = 0.0f;
    }
    // voxels past N copy the lane's first voxel, so they never spoil the
    // shared-(y, z) test (their results are not stored)
#pragma unroll
    for (int v = 1; v < V; ++v)
        if (n0 + v >= N) {
            px[v] = px[0];
            py[v] = py[0];
            pz[v] = pz[0];
        }
    bool same_yz = true;
#pragma unroll
    for (int v = 1; v < V; ++v)
        same_yz = same_yz && __float_as_uint(py[v]) == __float_as_uint(py[0]) &&
                  __float_as_uint(pz[v]) == __float_as_uint(pz[0]);
    const bool shared = __all(same_yz);

    const int64_t total_vec4 = (int64_t)nchunks * kChunkVec4;
    const int nstages = (nchunks + kStageChunks - 1) / kStageChunks;
    for (int i = threadIdx.x; i < kStageVec4 && i < total_vec4; i += kBlock) stage[0][i] = src[i];
    __syncthreads();

    for (int st = 0; st < nstages; ++st) {
        // prefetch the next stage into registers (indices clamped in bounds,
        // the clamped copies are never written to LDS)
        const bool more = st + 1 < nstages;
        const int64_t next = (int64_t)(st + 1) * kStageVec4 + threadIdx.x;
        float4 r0, r1, r2;
        if (more) {
            r0 = src[min(next, total_vec4 - 1)];
            r1 = src[min(next + kBlock, total_vec4 - 1)];
            r2 = src[min(next + 2 * kBlock, total_vec4 - 1)];
        }
        const int chunks_here = min(kStageChunks, nchunks - st * kStageChunks);
        const float4 *buf = stage[st & 1];
        if (shared) {
            for (int c = 0; c < chunks_here; ++c)
                accumulate_chunk<V, true>(buf + c * kChunkVec4, px, py, pz, acc_r, acc_i);
        } else {
            for (int c = 0; c < chunks_here; ++c)
                accumulate_chunk<V, false>(buf + c * kChunkVec4, px, py, pz, acc_r, acc_i);
        }
        if (more) {
            // the other buffer was last read before the previous barrier
            float4 *dst = stage[(st + 1) & 1];
            const int i0 = threadIdx.x;
            if (next < total_vec4) dst[i0] = r0;
            if (i0 + kBlock < kStageVec4 && next + kBlock < total_vec4) dst[i0 + kBlock] = r1;
            if (i0 + 2 * kBlock < kStageVec4 && next + 2 * kBlock < total_vec4) dst[i0 + 2 * kBlock] = r2;
        }
        __syncthreads();
    }

#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int64_t n = n0 + v;
        if (n < N) {
            rho_r[n] = acc_r[v];
            rho_i[n] = acc_i[v];
        }
    }
}

// ---------------------------------------------------------------------------
// host-side checks
// ---------------------------------------------------------------------------
struct Span {
    const void *p;
    int64_t bytes;
    const char *name;
    unsigned align = 4;   // required alignment in bytes
};

bool overlaps(const Span &a, const Span &b)
{
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

// Null/alignment checks of spans with bytes > 0; no HIP call.
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

// Spans [first_out, count) are outputs: none may overlap any other span.
int check_no_overlap(const Span *spans, int count, int first_out)
{
    for (int i = first_out; i < count; ++i)
        for (int j = 0; j < count; ++j)
            if (j != i && overlaps(spans[i], spans[j]))
                return fail(FHD_ERR_INVALID_ARG, std::string(spans[i].name) + " overlaps " +
                                                     spans[j].name);
    return FHD_OK;
}

// The span must be memory the current device can access, and (for device
// allocations) lie inside one allocation.
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

// Launches without argument checks; callers have checked.
int launch_pack(const float *kx, const float *ky, const float *kz, const float *Dr, const float *Di,
                int M, float *packed, hipStream_t stream)
{
    if (M == 0) return FHD_OK;
    const int64_t M_pad = (int64_t)((M + kChunk - 1) / kChunk) * kChunk;
    const int64_t blocks = (M_pad + kPackBlock - 1) / kPackBlock;
    fhd_pack_kernel<<<dim3((unsigned)blocks), dim3(kPackBlock), 0, stream>>>(kx, ky, kz, Dr, Di,
                                                                             packed, M, M_pad);
    return launch_status("fhd_pack_kernel launch");
}

int launch_gather(const float *packed, int M, const float *x, const float *y, const float *z,
                  float *rho_r, float *rho_i, int N, hipStream_t stream)
{
    if (N == 0) return FHD_OK;
    const int nchunks = (int)(((int64_t)M + kChunk - 1) / kChunk);
    const int64_t per_block = (int64_t)kBlock * kVox;
    const int64_t blocks = ((int64_t)N + per_block - 1) / per_block;
    fhd_gather_kernel<kVox><<<dim3((unsigned)blocks), dim3(kBlock), 0, stream>>>(
        packed, nchunks, x, y, z, rho_r, rho_i, N);
    return launch_status("fhd_gather_kernel launch");
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" int64_t fhd_packed_bytes(int M)
{
    if (M < 0) return -1;
    return packed_bytes_for(M);
}

extern "C" void fhd_gather_config(int *voxels_per_lane, int *samples_per_chunk, int *block_threads)
{
    if (voxels_per_lane) *voxels_per_lane = kVox;
    if (samples_per_chunk) *samples_per_chunk = kChunk;
    if (block_threads) *block_threads = kBlock;
}

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

extern "C" const char *fhd_last_error(void) { return g_last_error.c_str(); }

extern "C" int fhd_pack(const float *kx, const float *ky, const float *kz, const float *Dr,
                        const float *Di, int M, void *packed, int64_t packed_bytes, void *stream)
{
    g_last_error.clear();
    if (M < 0) return fail(FHD_ERR_INVALID_ARG, "M < 0");
    if (M == 0) return FHD_OK;
    const int64_t need = packed_bytes_for(M), mb = (int64_t)M * 4;
    if (packed_bytes < need)
        return fail(FHD_ERR_INVALID_ARG, "packed_bytes " + std::to_string(packed_bytes) + " < " +
                                             std::to_string(need));
    const Span all[] = {{kx, mb, "kx"}, {ky, mb, "ky"}, {kz, mb, "kz"}, {Dr, mb, "Dr"},
                        {Di, mb, "Di"}, {packed, need, "packed", 16}};
    int rc = check_host_side(all, 6);
    if (rc == FHD_OK) rc = check_no_overlap(all, 6, 5);
    if (rc == FHD_OK) rc = check_device_spans(all, 6);
    if (rc != FHD_OK) return rc;
    return launch_pack(kx, ky, kz, Dr, Di, M, (float *)packed, (hipStream_t)stream);
}

extern "C" int fhd_gather(const void *packed, int M, const float *x, const float *y, const float *z,
                          float *rho_r, float *rho_i, int N, void *stream)
{
    g_last_error.clear();
    if (M < 0) return fail(FHD_ERR_INVALID_ARG, "M < 0");
    if (N < 0) return fail(FHD_ERR_INVALID_ARG, "N < 0");
    if (N == 0) return FHD_OK;
    const int64_t nb = (int64_t)N * 4;
    const Span all[] = {{packed, M > 0 ? packed_bytes_for(M) : 0, "packed", 16},
                        {x, nb, "x"}, {y, nb, "y"}, {z, nb, "z"},
                        {rho_r, nb, "rho_r"}, {rho_i, nb, "rho_i"}};
    int rc = check_host_side(all, 6);
    if (rc == FHD_OK) rc = check_no_overlap(all, 6, 4);
    if (rc == FHD_OK) rc = check_device_spans(all, 6);
    if (rc != FHD_OK) return rc;
    return launch_gather((const float *)packed, M, x, y, z, rho_r, rho_i, N, (hipStream_t)stream);
}

extern "C" int fhd_compute(const float *kx, const float *ky, const float *kz, const float *Dr,
                           const float *Di, const float *x, const float *y, const float *z,
                           float *rho_r, float *rho_i, int M, int N, void *stream)
{
    g_last_error.clear();
    if (M < 0) return fail(FHD_ERR_INVALID_ARG, "M < 0");
    if (N < 0) return fail(FHD_ERR_INVALID_ARG, "N < 0");
    if (N == 0) return FHD_OK;
    const int64_t mb = (int64_t)M * 4, nb = (int64_t)N * 4;
    const Span all[] = {{kx, mb, "kx"}, {ky, mb, "ky"}, {kz, mb, "kz"}, {Dr, mb, "Dr"},
                        {Di, mb, "Di"}, {x, nb, "x"},   {y, nb, "y"},   {z, nb, "z"},
                        {rho_r, nb, "rho_r"}, {rho_i, nb, "rho_i"}};
    int rc = check_host_side(all, 10);
    if (rc == FHD_OK) rc = check_no_overlap(all, 10, 8);
    if (rc == FHD_OK) rc = check_device_spans(all, 10);
    if (rc != FHD_OK) return rc;

    hipStream_t s = (hipStream_t)stream;
    float *packed = nullptr;
    if (M > 0) {
        const hipError_t e = hipMallocAsync((void **)&packed, (size_t)packed_bytes_for(M), s);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(FHD_ERR_ALLOC, std::string("hipMallocAsync: ") + hipGetErrorString(e));
        }
        rc = launch_pack(kx, ky, kz, Dr, Di, M, packed, s);
    }
    if (rc == FHD_OK) rc = launch_gather(packed, M, x, y, z, rho_r, rho_i, N, s);
    if (packed) {
        const hipError_t e = hipFreeAsync(packed, s);
        if (e != hipSuccess && rc == FHD_OK)
            rc = fail(FHD_ERR_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(e));
    }
    return rc;
}
