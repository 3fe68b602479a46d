// fhd.hip -- F^H D (adjoint non-uniform DFT) for MI355X / gfx950.
//
// rho_n = sum_m D_m exp(+i 2 pi k_m . x_n)   (page "Case study -- iterative
// MRI reconstruction", section 17.3, F^H D equation)
//
// Two kernels, split by loop fission (section 17.3.2):
//
//  * fhd_pack_kernel -- per-sample pre-pass. Writes each sample as the
//    record (kx, ky, kz, psi, a) with a = |D| and psi = arg(D) / (2 pi) in
//    revolutions, so that D e^{i 2 pi p} = a e^{i 2 pi (p + psi)}: the
//    complex multiply-accumulate needs two FMAs instead of four and psi
//    folds into the phase dot product (record format: fhd_internal.h).
//
//  * fhd_gather_kernel -- one lane per kVox consecutive voxels, no atomics
//    (sections 17.3.1, 17.3.3). Voxel coordinates and the 2*kVox
//    accumulators live in VGPRs. Every lane of the grid walks the same
//    sample stream (section 17.3.4's observation), delivered by
//    stream_chunks() as an LDS broadcast into VGPRs.
//
//    Phases stay in revolutions and go straight into v_sin_f32 / v_cos_f32,
//    which take revolutions and reduce the argument exactly in hardware
//    (measured identical to an explicit v_fract_f32 reduction over the
//    whole fp32 range), so there is no 2 pi multiply and no fract (section
//    17.3.5, hardware trig).
//
//    When, in every lane of a workgroup, the kVox voxels share y and z
//    bitwise (any x-fastest voxel grid), ky*y + kz*z + psi is formed once
//    per sample and lane and each voxel adds kx*x with one FMA. The
//    arithmetic is the same FMA sequence as the general path, so results
//    are bitwise identical; workgroups that fail the test take the general
//    path.
//
//    When, in addition, each lane's voxels are equally spaced along x
//    (x_v = x_0 + v dx to fp32 rounding, checked exactly), the phase is a
//    ramp p_v = p_0 + v d with d = kx dx, and the phasors follow from two
//    seeds: a e^{i 2 pi p_0} by v_cos/v_sin, its rotation by e^{i 2 pi d}
//    (also v_cos/v_sin), then the three-term recurrence
//    w_{v+1} = 2 cos(2 pi d) w_v - w_{v-1}, which holds for any sinusoid of
//    step d and is linear, so the amplitude rides along. Four
//    transcendentals per sample and lane instead of 2 kVox. Rounding in the
//    recurrence grows at most like v^2 ulp (v < kVox); the seeds carry the
//    same phase rounding as the direct evaluation.
//
// Per voxel-sample term: direct paths, phase 1 + 2/kVox FMA (3 FMA on the
// general path), v_cos_f32, v_sin_f32, 2 FMA accumulate; ramp path, 4/kVox
// transcendentals and about 5 VALU operations.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <string>

#include "fhd_internal.h"

namespace fhd {
namespace {

constexpr int kVox = 16;        // consecutive voxels per lane
constexpr int kDirectGroup = 8; // voxels per transcendental group on the direct paths
static_assert(kVox % kDirectGroup == 0, "direct groups tile a lane's voxels");
constexpr int kRampGroup = 4;   // samples per transcendental group on the ramp path
static_assert(kChunk % kRampGroup == 0, "ramp groups tile a chunk");

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
    store_record(packed, m, fx, fy, fz, psi, amp);
}

// Accumulate one chunk of kChunk samples into a lane's V voxels.
// SHARED: all V voxels have the same y and z (checked by the caller).
template <int V, bool SHARED>
__device__ __forceinline__ void accumulate_chunk(const float4 *ch, const float (&px)[V],
                                                 const float (&py)[V], const float (&pz)[V],
                                                 float (&acc_r)[V], float (&acc_i)[V])
{
    // a sample's five fields are read from LDS when needed (same address in
    // every lane: a broadcast), which keeps registers for the V voxels
    const float *f = reinterpret_cast<const float *>(ch);
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
        const float skx = f[0 * kChunk + u], amp = f[4 * kChunk + u];
        float q = 0.0f;
        if constexpr (SHARED) q = __builtin_fmaf(f[1 * kChunk + u], py[0], __builtin_fmaf(f[2 * kChunk + u], pz[0], f[3 * kChunk + u]));
        // voxels in groups of kDirectGroup
#pragma unroll
        for (int g0 = 0; g0 < V; g0 += kDirectGroup) {
            float p[kDirectGroup], c[kDirectGroup], s[kDirectGroup];
            // phase in revolutions, including arg(D)
#pragma unroll
            for (int v = 0; v < kDirectGroup; ++v) {
                if constexpr (SHARED)
                    p[v] = __builtin_fmaf(skx, px[g0 + v], q);
                else
                    p[v] = __builtin_fmaf(skx, px[g0 + v],
                                          __builtin_fmaf(f[1 * kChunk + u], py[g0 + v],
                                                         __builtin_fmaf(f[2 * kChunk + u], pz[g0 + v], f[3 * kChunk + u])));
            }
            // The transcendentals of a group issue together at raised wave
            // priority. A transcendental holds its SIMD's issue port for two
            // quad-cycles and never pairs; plain all-VGPR FMAs from two waves
            // can issue in one quad-cycle. Letting the transcendental groups
            // go first makes the waves' FMA runs coincide, so more FMAs pair
            // (measured 14 % faster at 128^3 x 100k, identical results).
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int v = 0; v < kDirectGroup; ++v) c[v] = __builtin_amdgcn_cosf(p[v]);
#pragma unroll
            for (int v = 0; v < kDirectGroup; ++v) s[v] = __builtin_amdgcn_sinf(p[v]);
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int v = 0; v < kDirectGroup; ++v) {
                acc_r[g0 + v] = __builtin_fmaf(amp, c[v], acc_r[g0 + v]);
                acc_i[g0 + v] = __builtin_fmaf(amp, s[v], acc_i[g0 + v]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Ramp path: a lane's V voxels share y and z and sit at x0 + v dx.
template <int V>
__device__ __forceinline__ void accumulate_chunk_ramp(const float4 *ch, float x0, float dx, float y,
                                                      float z, float (&acc_r)[V], float (&acc_i)[V])
{
    float f[kFields][kChunk];
    load_chunk(ch, f);
    const float(&skx)[kChunk] = f[0];
    const float(&sky)[kChunk] = f[1];
    const float(&skz)[kChunk] = f[2];
    const float(&psi)[kChunk] = f[3];
    const float(&amp)[kChunk] = f[4];
    // the transcendentals of kRampGroup samples issue as one group at raised
    // wave priority (longer groups let more of the other waves' VALU work
    // pair up; 4 measured best)
#pragma unroll
    for (int u0 = 0; u0 < kChunk; u0 += kRampGroup) {
        float p0[kRampGroup], d[kRampGroup], c0[kRampGroup], s0[kRampGroup], cd[kRampGroup],
            sd[kRampGroup];
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            const int u = u0 + t;
            p0[t] = __builtin_fmaf(skx[u], x0, __builtin_fmaf(sky[u], y, __builtin_fmaf(skz[u], z, psi[u])));
            d[t] = skx[u] * dx;
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            c0[t] = __builtin_amdgcn_cosf(p0[t]);
            s0[t] = __builtin_amdgcn_sinf(p0[t]);
            cd[t] = __builtin_amdgcn_cosf(d[t]);
            sd[t] = __builtin_amdgcn_sinf(d[t]);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            const int u = u0 + t;
            // w_0 = a e^{i 2 pi p0}; w_1 = w_0 e^{i 2 pi d}
            float wr0 = amp[u] * c0[t], wi0 = amp[u] * s0[t];
            float wr1 = __builtin_fmaf(wr0, cd[t], -wi0 * sd[t]);
            float wi1 = __builtin_fmaf(wi0, cd[t], wr0 * sd[t]);
            const float two_cd = cd[t] + cd[t];
            acc_r[0] += wr0;
            acc_i[0] += wi0;
            acc_r[1] += wr1;
            acc_i[1] += wi1;
#pragma unroll
            for (int v = 2; v < V; ++v) {
                const float wr2 = __builtin_fmaf(two_cd, wr1, -wr0);
                const float wi2 = __builtin_fmaf(two_cd, wi1, -wi0);
                acc_r[v] += wr2;
                acc_i[v] += wi2;
                wr0 = wr1;
                wi0 = wi1;
                wr1 = wr2;
                wi1 = wi2;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// At least 4 waves per SIMD (<= 128 VGPRs): a 128^3 grid at 8 voxels per
// lane is exactly 4 waves per SIMD, so all of them are resident at once.
// Split s = blockIdx.y of `splits` takes its share of the sample stream and
// writes rho (splits == 1) or its partial sums at out + s*N.
template <int V>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void fhd_gather_kernel(
    const float *__restrict__ packed, int nchunks, int splits,
    const float *__restrict__ x, const float *__restrict__ y, const float *__restrict__ z,
    float *__restrict__ out_r, float *__restrict__ out_i, int N)
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
    // equal spacing along x: every x_v is x0 + v dx rounded once (lanes with
    // voxels past N never qualify)
    const float dx = px[1] - px[0];
    bool ramp = same_yz && n0 + V <= N && __builtin_isfinite(dx);
#pragma unroll
    for (int v = 1; v < V; ++v)
        ramp = ramp && __builtin_fmaf((float)v, dx, px[0]) == px[v];
    // one decision per workgroup, so every branch's stage barriers are
    // reached by every wave of the workgroup
    const bool all_ramp = __syncthreads_and(ramp);
    const bool shared = __syncthreads_and(same_yz);

    int c0, c1;
    split_range(nchunks, splits, blockIdx.y, &c0, &c1);
    if (all_ramp)
        stream_chunks(src, c0, c1, stage, [&](const float4 *ch) {
            accumulate_chunk_ramp<V>(ch, px[0], dx, py[0], pz[0], acc_r, acc_i);
        });
    else if (shared)
        stream_chunks(src, c0, c1, stage, [&](const float4 *ch) {
            accumulate_chunk<V, true>(ch, px, py, pz, acc_r, acc_i);
        });
    else
        stream_chunks(src, c0, c1, stage, [&](const float4 *ch) {
            accumulate_chunk<V, false>(ch, px, py, pz, acc_r, acc_i);
        });

    float *dst_r = out_r + (int64_t)blockIdx.y * N, *dst_i = out_i + (int64_t)blockIdx.y * N;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int64_t n = n0 + v;
        if (n < N) {
            dst_r[n] = acc_r[v];
            dst_i[n] = acc_i[v];
        }
    }
}

}  // namespace

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
    const int splits = split_count(blocks, nchunks);
    if (splits == 1) {
        fhd_gather_kernel<kVox><<<dim3((unsigned)blocks), dim3(kBlock), 0, stream>>>(
            packed, nchunks, 1, x, y, z, rho_r, rho_i, N);
        return launch_status("fhd_gather_kernel launch");
    }
    float *part = nullptr;
    const hipError_t e = hipMallocAsync((void **)&part, (size_t)splits * 2 * N * sizeof(float), stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(FHD_ERR_ALLOC, std::string("hipMallocAsync (split partials): ") +
                                       hipGetErrorString(e));
    }
    float *part_r = part, *part_i = part + (int64_t)splits * N;
    fhd_gather_kernel<kVox><<<dim3((unsigned)blocks, (unsigned)splits), dim3(kBlock), 0, stream>>>(
        packed, nchunks, splits, x, y, z, part_r, part_i, N);
    int rc = launch_status("fhd_gather_kernel launch");
    if (rc == FHD_OK) rc = launch_reduce(part_r, part_i, splits, N, rho_r, rho_i, stream);
    const hipError_t f = hipFreeAsync(part, stream);
    if (f != hipSuccess && rc == FHD_OK)
        rc = fail(FHD_ERR_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(f));
    return rc;
}

int adjoint_gather_vox_per_lane() { return kVox; }

}  // namespace fhd

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
using namespace fhd;

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

extern "C" int fhd_pack(const float *kx, const float *ky, const float *kz, const float *Dr,
                        const float *Di, int M, void *packed, int64_t packed_bytes, void *stream)
{
    clear_error();
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
    clear_error();
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
    clear_error();
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
