// microbench.hip -- issue-rate micro-benchmarks that fix the denominator of
// the F^H D gather kernel's ALU roofline on gfx950.
//
// The gather kernel spends each voxel-sample term on plain fp32 VALU work
// (FMA, fract) and two transcendentals (v_sin_f32, v_cos_f32). Its ceiling
// depends on three hardware facts that no page states for this chip:
//   * the plain fp32 FMA issue rate (expected: one wave64 instruction per 4
//     cycles per SIMD, 64 FMA / CU / cycle without packed math);
//   * the transcendental issue rate;
//   * whether transcendentals block plain VALU issue on their SIMD or run
//     beside it.
// mix_kernel<A, B> runs, per lane and iteration, S independent streams that
// each issue A plain FMAs and B transcendentals (B = 1: sin; B = 2: sin and
// cos). Timing several (A, B) pairs answers all three questions: with
// blocking issue, time ~ A*t_fma + B*t_trans; with side-by-side issue, time
// ~ max(A*t_fma, B*t_trans).
//
// The kernels also read the shader clock counter (clock64) and the constant
// wall clock (wall_clock64) at the start and end of each workgroup, so the
// host can report the clock the SIMDs actually ran at.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

namespace {

constexpr int kBlock = 256;
constexpr int kStreams = 8;

template <int A, int B>
__global__ __launch_bounds__(kBlock) void mix_kernel(float *__restrict__ out,
                                                     long long *__restrict__ clocks, int iters,
                                                     float seed)
{
    const long long t0 = clock64(), w0 = wall_clock64();
    float xs[kStreams];
    constexpr int NACC = A > 1 ? A - 1 : 1;
    float acc[kStreams][NACC];
#pragma unroll
    for (int s = 0; s < kStreams; ++s) {
        xs[s] = seed + 0.01f * (float)(threadIdx.x + s);
#pragma unroll
        for (int j = 0; j < NACC; ++j) acc[s][j] = 0.0f;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < kStreams; ++s) {
            if constexpr (A == 0) {
                // transcendental-only chain: B per stream and iteration
                float t = __builtin_amdgcn_sinf(xs[s]);
                if constexpr (B == 2) t = __builtin_amdgcn_cosf(t);
                xs[s] = t;
            } else {
                // one FMA moves the stream, B transcendentals read it and
                // A - 1 FMAs accumulate them (or the stream, if B = 0)
                xs[s] = __builtin_fmaf(xs[s], 0.9990234375f, 0.0009765625f);
                float t0v = xs[s], t1v = xs[s];
                if constexpr (B >= 1) t0v = __builtin_amdgcn_sinf(xs[s]);
                if constexpr (B >= 2) t1v = __builtin_amdgcn_cosf(xs[s]);
                if constexpr (A > 1) {
#pragma unroll
                    for (int j = 0; j < A - 1; ++j)
                        acc[s][j] = __builtin_fmaf((j & 1) ? t1v : t0v, 0.5f, acc[s][j]);
                }
            }
        }
    }
    float sum = 0.0f;
#pragma unroll
    for (int s = 0; s < kStreams; ++s) {
        sum += xs[s];
#pragma unroll
        for (int j = 0; j < NACC; ++j) sum += acc[s][j];
    }
    out[(size_t)blockIdx.x * kBlock + threadIdx.x] = sum;
    if (threadIdx.x == 0) {
        clocks[4 * blockIdx.x + 0] = t0;
        clocks[4 * blockIdx.x + 1] = clock64();
        clocks[4 * blockIdx.x + 2] = w0;
        clocks[4 * blockIdx.x + 3] = wall_clock64();
    }
}

using MixFn = void (*)(float *, long long *, int, float);

struct MixEntry {
    int a, b;
    MixFn fn;
};

const MixEntry kMixes[] = {
    {8, 0, mix_kernel<8, 0>},   {0, 1, mix_kernel<0, 1>},   {0, 2, mix_kernel<0, 2>},
    {3, 2, mix_kernel<3, 2>},   {4, 2, mix_kernel<4, 2>},   {5, 2, mix_kernel<5, 2>},
    {6, 2, mix_kernel<6, 2>},   {8, 2, mix_kernel<8, 2>},   {12, 2, mix_kernel<12, 2>},
    {16, 2, mix_kernel<16, 2>}, {6, 1, mix_kernel<6, 1>},
};

}  // namespace

// Number of (A, B) pairs and the pair at index i.
extern "C" int fhdmb_mix_count(void) { return (int)(sizeof(kMixes) / sizeof(kMixes[0])); }

extern "C" int fhdmb_mix_pair(int i, int *a, int *b)
{
    if (i < 0 || i >= fhdmb_mix_count()) return -1;
    *a = kMixes[i].a;
    *b = kMixes[i].b;
    return 0;
}

// Runs mix_kernel<a, b> on `blocks` workgroups of 256 lanes for `iters`
// iterations of 8 streams: one untimed launch, then one launch timed with
// HIP events on a private stream. Writes the elapsed milliseconds, the mean
// shader clock in MHz over the workgroups, and a checksum of the outputs.
// Returns 0, -1 for an unknown pair or bad size, -2 on a HIP error.
extern "C" int fhdmb_mix(int a, int b, int blocks, int iters, double *ms, double *sclk_mhz,
                         double *checksum)
{
    MixFn fn = nullptr;
    for (const MixEntry &e : kMixes)
        if (e.a == a && e.b == b) fn = e.fn;
    if (!fn || blocks <= 0 || iters <= 0) return -1;

    float *out = nullptr;
    long long *clocks = nullptr;
    hipStream_t stream = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int rc = 0;
    int wall_khz = 0;
    const size_t nout = (size_t)blocks * kBlock;
    if (hipMalloc(&out, nout * sizeof(float)) != hipSuccess ||
        hipMalloc(&clocks, (size_t)blocks * 4 * sizeof(long long)) != hipSuccess ||
        hipStreamCreate(&stream) != hipSuccess || hipEventCreate(&e0) != hipSuccess ||
        hipEventCreate(&e1) != hipSuccess ||
        hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, 0) != hipSuccess) {
        rc = -2;
    }
    if (rc == 0) {
        fn<<<blocks, kBlock, 0, stream>>>(out, clocks, iters, 0.25f);
        hipEventRecord(e0, stream);
        fn<<<blocks, kBlock, 0, stream>>>(out, clocks, iters, 0.25f);
        hipEventRecord(e1, stream);
        if (hipStreamSynchronize(stream) != hipSuccess || hipGetLastError() != hipSuccess) rc = -2;
    }
    if (rc == 0) {
        float f = 0.0f;
        hipEventElapsedTime(&f, e0, e1);
        *ms = f;
        std::vector<long long> c((size_t)blocks * 4);
        std::vector<float> o(nout);
        hipMemcpy(c.data(), clocks, c.size() * sizeof(long long), hipMemcpyDeviceToHost);
        hipMemcpy(o.data(), out, o.size() * sizeof(float), hipMemcpyDeviceToHost);
        double cyc = 0.0, wall = 0.0, sum = 0.0;
        for (int i = 0; i < blocks; ++i) {
            cyc += (double)(c[4 * i + 1] - c[4 * i + 0]);
            wall += (double)(c[4 * i + 3] - c[4 * i + 2]);
        }
        for (float v : o) sum += v;
        *sclk_mhz = wall > 0 ? cyc / wall * (wall_khz / 1000.0) : 0.0;
        *checksum = sum;
    }
    if (e0) hipEventDestroy(e0);
    if (e1) hipEventDestroy(e1);
    if (stream) hipStreamDestroy(stream);
    if (out) hipFree(out);
    if (clocks) hipFree(clocks);
    return rc;
}
