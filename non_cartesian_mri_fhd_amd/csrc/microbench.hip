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
// form_kernel<F> times one exact VALU instruction form, written as inline
// assembly so the compiler can neither reorder, fuse nor re-encode it: eight
// independent accumulator chains per lane, so every instruction has seven
// independent neighbours. The forms separate what decides the FP32 issue
// rate on gfx950: operand source (VGPR, inline constant, literal, SGPR),
// encoding (VOP2, VOP3), v_fract_f32, the transcendental unit, and the
// gather kernel's own mix of 2 transcendentals and 5 FMAs. One more form
// reads the LDS (ds_read_b128, conflict-free, eight reads in flight per
// wave) to give the LDS read bandwidth per CU that the matrix-core kernels'
// operand reads share; four more time v_mfma_f32_16x16x32_f16 alone and
// each followed by independent work (4 FMAs; a v_sin_f32 and an FMA; one
// ds_read_b128), at one and at two waves per SIMD, to show what a wave's
// other instructions cost its matrix products.
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
typedef unsigned mb_u32x4 __attribute__((ext_vector_type(4)));
typedef float mb_f32x4 __attribute__((ext_vector_type(4)));

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


// ---------------------------------------------------------------------------
// instruction forms (inline assembly; VALU only)
// ---------------------------------------------------------------------------
#define FHDMB_R8(X) X(0) X(1) X(2) X(3) X(4) X(5) X(6) X(7)

template <int F>
__global__ __launch_bounds__(kBlock) void form_kernel(float *__restrict__ out,
                                                      long long *__restrict__ clocks, int iters,
                                                      float sv)
{
    float a0 = threadIdx.x, a1 = a0 + 1, a2 = a0 + 2, a3 = a0 + 3, a4 = a0 + 4, a5 = a0 + 5,
          a6 = a0 + 6, a7 = a0 + 7;
    float t0 = 0, t1 = 0, t2 = 0, t3 = 0, t4 = 0, t5 = 0, t6 = 0, t7 = 0;
    const float x = threadIdx.x * 0.001f, y = x + 0.5f;
    // matrix-core forms: eight independent 16x16x32 fp16 accumulators
    mb_f32x4 m0 = {0, 0, 0, 0}, m1 = m0, m2 = m0, m3 = m0, m4 = m0, m5 = m0, m6 = m0, m7 = m0;
    const mb_u32x4 ma = {threadIdx.x, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u}, mb = {0x3c003c00u, 1u, 2u, 3u};
    const long long c0 = clock64(), w0 = wall_clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (F == 0) {   // v_fmac_f32_e32, VGPR operands
#define FHDMB_I(i) asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a##i) : "v"(y), "v"(x));
                FHDMB_R8(FHDMB_I)
#undef FHDMB_I
            } else if constexpr (F == 1) {   // v_fmac_f32_e32, SGPR src0
#define FHDMB_I(i) asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a##i) : "s"(sv), "v"(x));
                FHDMB_R8(FHDMB_I)
#undef FHDMB_I
            } else if constexpr (F == 2) {   // v_fmac_f32_e32, inline constant
#define FHDMB_I(i) asm volatile("v_fmac_f32_e32 %0, 0.5, %1" : "+v"(a##i) : "v"(x));
                FHDMB_R8(FHDMB_I)
#undef FHDMB_I
            } else if constexpr (F == 3) {   // v_fma_f32 (VOP3), VGPR operands
#define FHDMB_I(i) asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(a##i) : "v"(y), "v"(x));
                FHDMB_R8(FHDMB_I)
#undef FHDMB_I
            } else if constexpr (F == 4) {   // v_fma_f32 (VOP3), SGPR operand
#define FHDMB_I(i) asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(a##i) : "s"(sv), "v"(x));
                FHDMB_R8(FHDMB_I)
#undef FHDMB_I
            } else if constexpr (F == 5) {   // v_fmamk_f32, literal constant
#define FHDMB_I(i) asm volatile("v_fmamk_f32 %0, %1, 0x3f000000, %0" : "+v"(a##i) : "v"(x));
                FHDMB_R8(FHDMB_I)
#undef FHDMB_I
            } else if constexpr (F == 6) {   // v_fract_f32
#define FHDMB_I(i) asm volatile("v_fract_f32_e32 %0, %0" : "+v"(a##i));
                FHDMB_R8(FHDMB_I)
#undef FHDMB_I
            } else if constexpr (F == 7) {   // v_sin_f32 into distinct live registers
#define FHDMB_I(i) asm volatile("v_sin_f32_e32 %0, %1" : "+v"(t##i) : "v"(a##i));
                FHDMB_R8(FHDMB_I)
#undef FHDMB_I
            } else if constexpr (F == 8) {   // gather mix, grouped: sin, cos, 5 VGPR FMAs
                asm volatile("v_sin_f32_e32 %0, %1" : "+v"(t0) : "v"(x));
                asm volatile("v_cos_f32_e32 %0, %1" : "+v"(t1) : "v"(x));
                asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a0) : "v"(y), "v"(x));
                asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a1) : "v"(y), "v"(x));
                asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a2) : "v"(y), "v"(x));
                asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a3) : "v"(y), "v"(x));
                asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a4) : "v"(y), "v"(x));
            } else if constexpr (F == 10) {   // v_fmac_f32 with a DPP row broadcast of src0
#define FHDMB_I(i) asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:5 row_mask:0xf bank_mask:0xf" : "+v"(a##i) : "v"(y), "v"(x));
                FHDMB_R8(FHDMB_I)
#undef FHDMB_I
            } else if constexpr (F == 11) {   // v_mov_b32 with a DPP row broadcast
#define FHDMB_I(i) asm volatile("v_mov_b32_dpp %0, %1 row_newbcast:5 row_mask:0xf bank_mask:0xf" : "=v"(t##i) : "v"(a##i));
                FHDMB_R8(FHDMB_I)
#undef FHDMB_I
            } else if constexpr (F == 12) {   // ds_read_b128, 1 KB per wave and read, no bank conflicts
                // 16 KB per workgroup: its 256 lanes' 16 B at 4 offsets
                __shared__ uint4 lds[4 * kBlock];
                if (it == 0 && r == 0) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) lds[k * kBlock + threadIdx.x] = make_uint4(threadIdx.x, k, 1, 2);
                    __syncthreads();
                }
                // the LDS offset of this lane's 16 B (the low half of its flat address)
                const unsigned addr = (unsigned)reinterpret_cast<uintptr_t>(&lds[threadIdx.x]);
                mb_u32x4 q0, q1, q2, q3, q4, q5, q6, q7;
                asm volatile("ds_read_b128 %0, %1 offset:0" : "=v"(q0) : "v"(addr) : "memory");
                asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(q1) : "v"(addr) : "memory");
                asm volatile("ds_read_b128 %0, %1 offset:8192" : "=v"(q2) : "v"(addr) : "memory");
                asm volatile("ds_read_b128 %0, %1 offset:12288" : "=v"(q3) : "v"(addr) : "memory");
                asm volatile("ds_read_b128 %0, %1 offset:0" : "=v"(q4) : "v"(addr) : "memory");
                asm volatile("ds_read_b128 %0, %1 offset:4096" : "=v"(q5) : "v"(addr) : "memory");
                asm volatile("ds_read_b128 %0, %1 offset:8192" : "=v"(q6) : "v"(addr) : "memory");
                asm volatile("ds_read_b128 %0, %1 offset:12288" : "=v"(q7) : "v"(addr) : "memory");
                // the waits tie the loaded registers, so nothing reads them before
                asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(q0), "+v"(q1), "+v"(q2), "+v"(q3)::"memory");
                asm volatile("" : "+v"(q4), "+v"(q5), "+v"(q6), "+v"(q7));
                t0 = __uint_as_float(__float_as_uint(t0) ^ q0.x);
                t1 = __uint_as_float(__float_as_uint(t1) ^ q1.y);
                t2 = __uint_as_float(__float_as_uint(t2) ^ q2.z);
                t3 = __uint_as_float(__float_as_uint(t3) ^ q3.w);
                t4 = __uint_as_float(__float_as_uint(t4) ^ q4.x);
                t5 = __uint_as_float(__float_as_uint(t5) ^ q5.y);
                t6 = __uint_as_float(__float_as_uint(t6) ^ q6.z);
                t7 = __uint_as_float(__float_as_uint(t7) ^ q7.w);
            } else if constexpr (F == 13) {   // v_mfma_f32_16x16x32_f16 alone
#define FHDMB_I(i) asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(m##i) : "v"(ma), "v"(mb));
                FHDMB_R8(FHDMB_I)
#undef FHDMB_I
            } else if constexpr (F == 14) {   // each MFMA followed by 4 independent VGPR FMAs
#define FHDMB_I(i)                                                                            \
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(m##i) : "v"(ma), "v"(mb));   \
    asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a0) : "v"(y), "v"(x));                     \
    asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a1) : "v"(y), "v"(x));                     \
    asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a2) : "v"(y), "v"(x));                     \
    asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a3) : "v"(y), "v"(x));
                FHDMB_R8(FHDMB_I)
#undef FHDMB_I
            } else if constexpr (F == 15) {   // each MFMA followed by a v_sin_f32 and an FMA
#define FHDMB_I(i)                                                                            \
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(m##i) : "v"(ma), "v"(mb));   \
    asm volatile("v_sin_f32_e32 %0, %1" : "+v"(t##i) : "v"(a##i));                             \
    asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a##i) : "v"(y), "v"(x));
                FHDMB_R8(FHDMB_I)
#undef FHDMB_I
            } else if constexpr (F == 16) {   // each MFMA followed by one ds_read_b128
                __shared__ uint4 lds2[4 * kBlock];
                if (it == 0 && r == 0) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) lds2[k * kBlock + threadIdx.x] = make_uint4(threadIdx.x, k, 1, 2);
                    __syncthreads();
                }
                // the LDS offset of this lane's 16 B (the low half of its flat address)
                const unsigned addr = (unsigned)reinterpret_cast<uintptr_t>(&lds2[threadIdx.x]);
                mb_u32x4 q0, q1, q2, q3, q4, q5, q6, q7;
#define FHDMB_I(i, off)                                                                       \
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(m##i) : "v"(ma), "v"(mb));   \
    asm volatile("ds_read_b128 %0, %1 offset:" #off : "=v"(q##i) : "v"(addr) : "memory");
                FHDMB_I(0, 0) FHDMB_I(1, 4096) FHDMB_I(2, 8192) FHDMB_I(3, 12288)
                FHDMB_I(4, 0) FHDMB_I(5, 4096) FHDMB_I(6, 8192) FHDMB_I(7, 12288)
#undef FHDMB_I
                // the wait ties the loaded registers, so nothing reads them before;
                // one of them is used (one vector instruction per 8 MFMAs)
                asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(q0), "+v"(q1), "+v"(q2), "+v"(q3)::"memory");
                asm volatile("" : "+v"(q4), "+v"(q5), "+v"(q6), "+v"(q7));
                t0 = __uint_as_float(__float_as_uint(t0) ^ q0.x);
            } else if constexpr (F == 9) {   // gather mix with SGPR operands
                asm volatile("v_sin_f32_e32 %0, %1" : "+v"(t0) : "v"(x));
                asm volatile("v_cos_f32_e32 %0, %1" : "+v"(t1) : "v"(x));
                asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a0) : "s"(sv), "v"(x));
                asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a1) : "s"(sv), "v"(x));
                asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a2) : "s"(sv), "v"(x));
                asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a3) : "s"(sv), "v"(x));
                asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a4) : "s"(sv), "v"(x));
            }
        }
    }
    const long long c1 = clock64(), w1 = wall_clock64();
    const mb_f32x4 m = m0 + m1 + m2 + m3 + m4 + m5 + m6 + m7;
    out[(size_t)blockIdx.x * kBlock + threadIdx.x] =
        a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7 + t0 + t1 + t2 + t3 + t4 + t5 + t6 + t7 + m[0] + m[1] + m[2] + m[3];
    if (threadIdx.x == 0) {
        clocks[4 * blockIdx.x + 0] = c0;
        clocks[4 * blockIdx.x + 1] = c1;
        clocks[4 * blockIdx.x + 2] = w0;
        clocks[4 * blockIdx.x + 3] = w1;
    }
}
#undef FHDMB_R8

struct FormEntry {
    const char *name;
    int instrs_per_group;   // instructions per unrolled group (4 groups per iteration)
    MixFn fn;
};

const FormEntry kForms[] = {
    {"fmac_vop2_vgpr", 8, form_kernel<0>}, {"fmac_vop2_sgpr", 8, form_kernel<1>},
    {"fmac_vop2_inline_const", 8, form_kernel<2>}, {"fma_vop3_vgpr", 8, form_kernel<3>},
    {"fma_vop3_sgpr", 8, form_kernel<4>}, {"fmamk_literal", 8, form_kernel<5>},
    {"fract", 8, form_kernel<6>}, {"sin", 8, form_kernel<7>},
    {"mix_2trans_5fma_vgpr", 7, form_kernel<8>}, {"mix_2trans_5fma_sgpr", 7, form_kernel<9>},
    {"fmac_vop2_dpp_row_bcast", 8, form_kernel<10>}, {"mov_dpp_row_bcast", 8, form_kernel<11>},
    {"lds_read_b128", 8, form_kernel<12>},
    {"mfma_f16_16x16x32", 8, form_kernel<13>}, {"mfma_f16_plus_4fma", 8, form_kernel<14>},
    {"mfma_f16_plus_sin_fma", 8, form_kernel<15>}, {"mfma_f16_plus_lds_read_b128", 8, form_kernel<16>},
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

namespace {

// One untimed launch, then one launch timed with HIP events on a private
// stream. Writes the elapsed milliseconds, the mean shader clock (MHz) over
// the workgroups and a checksum of the outputs. 0 on success, -2 on a HIP
// error.
int time_kernel(MixFn fn, int blocks, int iters, float arg, double *ms, double *sclk_mhz,
                double *checksum)
{
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
        fn<<<blocks, kBlock, 0, stream>>>(out, clocks, iters, arg);
        (void)hipEventRecord(e0, stream);
        fn<<<blocks, kBlock, 0, stream>>>(out, clocks, iters, arg);
        (void)hipEventRecord(e1, stream);
        if (hipStreamSynchronize(stream) != hipSuccess || hipGetLastError() != hipSuccess) rc = -2;
    }
    if (rc == 0) {
        float f = 0.0f;
        (void)hipEventElapsedTime(&f, e0, e1);
        *ms = f;
        std::vector<long long> c((size_t)blocks * 4);
        std::vector<float> o(nout);
        if (hipMemcpy(c.data(), clocks, c.size() * sizeof(long long), hipMemcpyDeviceToHost) !=
                hipSuccess ||
            hipMemcpy(o.data(), out, o.size() * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess)
            rc = -2;
        double cyc = 0.0, wall = 0.0, sum = 0.0;
        for (int i = 0; i < blocks; ++i) {
            cyc += (double)(c[4 * i + 1] - c[4 * i + 0]);
            wall += (double)(c[4 * i + 3] - c[4 * i + 2]);
        }
        for (float v : o) sum += v;
        *sclk_mhz = wall > 0 ? cyc / wall * (wall_khz / 1000.0) : 0.0;
        *checksum = sum;
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (stream) (void)hipStreamDestroy(stream);
    if (out) (void)hipFree(out);
    if (clocks) (void)hipFree(clocks);
    return rc;
}

}  // namespace

// Runs mix_kernel<a, b> on `blocks` workgroups of 256 lanes for `iters`
// iterations of 8 streams (see time_kernel). Returns 0, -1 for an unknown
// pair or bad size, -2 on a HIP error.
extern "C" int fhdmb_mix(int a, int b, int blocks, int iters, double *ms, double *sclk_mhz,
                         double *checksum)
{
    MixFn fn = nullptr;
    for (const MixEntry &e : kMixes)
        if (e.a == a && e.b == b) fn = e.fn;
    if (!fn || blocks <= 0 || iters <= 0) return -1;
    return time_kernel(fn, blocks, iters, 0.25f, ms, sclk_mhz, checksum);
}

// Number of instruction forms, and the name and instructions per group of
// form i (each iteration runs 4 groups per lane).
extern "C" int fhdmb_form_count(void) { return (int)(sizeof(kForms) / sizeof(kForms[0])); }

extern "C" const char *fhdmb_form_name(int i)
{
    return (i >= 0 && i < fhdmb_form_count()) ? kForms[i].name : nullptr;
}

extern "C" int fhdmb_form_instrs(int i)
{
    return (i >= 0 && i < fhdmb_form_count()) ? kForms[i].instrs_per_group : -1;
}

// Times form i (see time_kernel). Returns 0, -1 for a bad index or size,
// -2 on a HIP error.
extern "C" int fhdmb_form(int i, int blocks, int iters, double *ms, double *sclk_mhz,
                          double *checksum)
{
    if (i < 0 || i >= fhdmb_form_count() || blocks <= 0 || iters <= 0) return -1;
    return time_kernel(kForms[i].fn, blocks, iters, 1.0001f, ms, sclk_mhz, checksum);
}
