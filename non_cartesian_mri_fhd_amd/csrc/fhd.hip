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
//    ramp with step d = kx dx. The voxels pair up symmetrically about the
//    lane's centre, where one phasor u = a e^{i 2 pi p_c} is evaluated; a
//    pair at +-(j + 1/2) dx from it gets u (C_j +- i S_j) with real
//    C_j = cos(2 pi (j + 1/2) d), S_j = sin(2 pi (j + 1/2) d), which follow
//    from cos and sin of half a step by the three-term recurrence of any
//    sinusoid. The lane accumulates u C_j and i u S_j per pair and unfolds
//    them into the two voxels at the end: four FMAs per voxel pair. When
//    all lanes of the workgroup share the step (any grid), C_j and S_j are
//    the same for every lane, so one lane per sample forms them into an LDS
//    record and the others read it back: per sample and lane, 3 FMAs of
//    phase, 2 transcendentals and 32 FMAs for 16 terms. Otherwise each lane
//    forms them itself (4 transcendentals and 55 VALU operations). Rounding
//    in the recurrence grows at most like j^2 ulp (j < kVox / 2); the centre
//    phase carries one more rounding than a direct evaluation.
//
// Per voxel-sample term: direct paths, phase 1 + 2/kVox FMA (3 FMA on the
// general path), v_cos_f32, v_sin_f32, 2 FMA accumulate; ramp path, 2/kVox
// transcendentals and 35/kVox VALU operations (shared step).
//
//  * fhd_classify_kernel -- tests every unit of 4096 voxels once per call and
//    records which instance takes it. Units whose voxels form lines along x
//    at one step (every x-fastest grid with rows of a multiple of 64) go to
//    the matrix-core instances, fhd_gather_long_lines_kernel (lines of 128,
//    two units per workgroup) and fhd_gather_lines_kernel (lines of 64):
//    the voxels pair up about each line's centre and the sum becomes real
//    matrix products (lines x samples)(samples x pairs) in split bf16 (see
//    "Lines on the matrix cores" below); the rest go to fhd_gather_kernel.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <string>
#include <type_traits>

#include "fhd_internal.h"

namespace fhd {
namespace {

constexpr int kVox = 16;        // consecutive voxels per lane
constexpr int kVecGranuleChunks = 8;   // the vector instances' split granule (64 samples)
constexpr int kDirectGroup = 8; // voxels per transcendental group on the direct paths
static_assert(kVox % kDirectGroup == 0, "direct groups tile a lane's voxels");
constexpr int kRampGroup = 4;   // samples per transcendental group on the ramp path
static_assert(kChunk % kRampGroup == 0, "ramp groups tile a chunk");
static_assert(kVox % 2 == 0, "the ramp path pairs a lane's voxels");

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

// 2 cos(2 pi d) of the ramp path's recurrence from s = sin(2 pi d / 2),
// as 2 - 4 s^2, which stays accurate for small steps d.
__device__ __forceinline__ float ramp_k2(float s) { return __builtin_fmaf(-4.0f * s, s, 2.0f); }

// Ramp path: a lane's V voxels share y and z and sit at x0 + v dx. They
// pair up around the lane's centre x_c = x0 + (V-1)/2 dx: voxel V/2 + j and
// voxel V/2 - 1 - j sit at x_c +- (j + 1/2) dx. With h = d/2 = kx dx / 2,
// p_c = p_0 + (V-1) h and u = a e^{i 2 pi p_c}, their phasors are
// u (C_j +- i S_j), C_j = cos(2 pi (2j+1) h), S_j = sin(2 pi (2j+1) h), both
// real. So the lane accumulates, per pair,
//   sum_j = sum over samples of u C_j      (acc[j])
//   dif_j = sum over samples of i u S_j    (acc[V/2 + j])
// at four FMAs per pair, and ramp_unfold() turns them into the two voxels'
// sums (sum_j + dif_j and sum_j - dif_j). C_j and S_j follow from
// (cos 2 pi h, sin 2 pi h) by the three-term recurrence
// c_{j+1} = 2 cos(2 pi d) c_j - c_{j-1} (started at c_{-1} = C_0,
// s_{-1} = -S_0). Per sample and lane: 4 transcendentals and 55 other VALU
// instructions for V = 16 terms. (Workgroups whose lanes all share one step
// take ramp_one_step() instead, which forms the sample-only part once per
// workgroup.)
template <int V>
__device__ __forceinline__ void accumulate_chunk_ramp(const float4 *ch, float x0, float hdx, float y,
                                                      float z, float (&acc_r)[V], float (&acc_i)[V])
{
    constexpr int P = V / 2;   // voxel pairs per lane
    float f[kFields][kChunk];
    load_chunk(ch, f);
    const float(&skx)[kChunk] = f[0];
    const float(&sky)[kChunk] = f[1];
    const float(&skz)[kChunk] = f[2];
    const float(&psi)[kChunk] = f[3];
    const float(&amp)[kChunk] = f[4];
    // the transcendentals of kRampGroup samples issue as one group at raised
    // wave priority (longer groups let more of the other waves' VALU work
    // pair up)
#pragma unroll
    for (int u0 = 0; u0 < kChunk; u0 += kRampGroup) {
        float pc[kRampGroup], h[kRampGroup], cc[kRampGroup], sc[kRampGroup], ch1[kRampGroup],
            sh1[kRampGroup];
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            const int u = u0 + t;
            const float p0 = __builtin_fmaf(skx[u], x0, __builtin_fmaf(sky[u], y, __builtin_fmaf(skz[u], z, psi[u])));
            h[t] = skx[u] * hdx;
            pc[t] = __builtin_fmaf((float)(V - 1), h[t], p0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            cc[t] = __builtin_amdgcn_cosf(pc[t]);
            sc[t] = __builtin_amdgcn_sinf(pc[t]);
            ch1[t] = __builtin_amdgcn_cosf(h[t]);
            sh1[t] = __builtin_amdgcn_sinf(h[t]);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            const int u = u0 + t;
            const float ur = amp[u] * cc[t], ui = amp[u] * sc[t];
            const float k2 = ramp_k2(sh1[t]);
            float cp = ch1[t], sp = -sh1[t];   // index -1
            float c = ch1[t], s = sh1[t];      // index 0
#pragma unroll
            for (int j = 0; j < P; ++j) {
                if (j > 0) {
                    const float cn = __builtin_fmaf(k2, c, -cp), sn = __builtin_fmaf(k2, s, -sp);
                    cp = c;
                    sp = s;
                    c = cn;
                    s = sn;
                }
                acc_r[j] = __builtin_fmaf(ur, c, acc_r[j]);
                acc_i[j] = __builtin_fmaf(ui, c, acc_i[j]);
                acc_r[P + j] = __builtin_fmaf(-ui, s, acc_r[P + j]);
                acc_i[P + j] = __builtin_fmaf(ur, s, acc_i[P + j]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Ramp path for a workgroup whose lanes all step by the same dx. Then C_j,
// S_j and the centre offset (V-1) h are sample-only: one lane per sample
// forms them (with the amplitude folded in) into an LDS record
//   [a C_0 .. a C_{P-1}][a S_0 .. a S_{P-1}][kx ky kz psi + (V-1) h]
// (kRampRecord float4), and every lane reads the records back as LDS
// broadcasts. Per sample and lane: 3 FMAs for the centre phase p_c, cos and
// sin of it (u / a), and the 4 P accumulating FMAs -- 35 VALU and 2
// transcendentals for V = 16 terms.
constexpr int kRampRecord = kVox / 4 + 1;      // float4 per sample record
constexpr int kSideSamples = 128;               // records per LDS round
static_assert(kVox % 8 == 0, "a record holds whole float4s of C and S");
static_assert((kStageChunks * kChunk) % kSideSamples == 0, "rounds tile a stage");
static_assert(kSideSamples % kRampGroup == 0 && kSideSamples <= kBlock, "one record per lane");

// Lane i < n writes the record of the stage's sample r0 + i.
template <int V>
__device__ __forceinline__ void ramp_records(const float4 *buf, int r0, int n, float hdx,
                                             float4 *side)
{
    constexpr int P = V / 2;
    const int i = threadIdx.x;
    if (i >= n) return;
    const int s = r0 + i;
    const float *b = reinterpret_cast<const float *>(buf) + (s / kChunk) * (kFields * kChunk) + s % kChunk;
    const float kx = b[0], ky = b[kChunk], kz = b[2 * kChunk], psi = b[3 * kChunk], amp = b[4 * kChunk];
    const float h = kx * hdx;
    const float c1 = __builtin_amdgcn_cosf(h), s1 = __builtin_amdgcn_sinf(h), k2 = ramp_k2(s1);
    float C[P], S[P];
    float cp = c1, sp = -s1, c = c1, sn = s1;
#pragma unroll
    for (int j = 0; j < P; ++j) {
        if (j > 0) {
            const float cn = __builtin_fmaf(k2, c, -cp), snn = __builtin_fmaf(k2, sn, -sp);
            cp = c;
            sp = sn;
            c = cn;
            sn = snn;
        }
        C[j] = amp * c;
        S[j] = amp * sn;
    }
    float4 *rec = side + i * kRampRecord;
#pragma unroll
    for (int q = 0; q < P / 4; ++q) {
        rec[q] = make_float4(C[4 * q], C[4 * q + 1], C[4 * q + 2], C[4 * q + 3]);
        rec[P / 4 + q] = make_float4(S[4 * q], S[4 * q + 1], S[4 * q + 2], S[4 * q + 3]);
    }
    rec[P / 2] = make_float4(kx, ky, kz, __builtin_fmaf((float)(V - 1), h, psi));
}

// Accumulates records [0, n) of `side` (n a multiple of kRampGroup) into
// the pair sums (acc[j] = sum_j, acc[V/2 + j] = dif_j). The LDS reads run
// ahead of their use: a group's phase inputs during the previous group's
// last sample's FMAs, a sample's C and S during the previous sample's FMAs
// (the first sample's during the transcendentals).
template <int V>
__device__ __forceinline__ void ramp_accumulate_records(const float4 *side, int n, float x0, float y,
                                                        float z, float (&acc_r)[V], float (&acc_i)[V])
{
    constexpr int P = V / 2;
    constexpr int Q = P / 2;   // float4 of C and S per record
    static_assert(Q == kRampGroup, "a sample's C and S and a group's phase inputs are equally many reads");
    float4 q[kRampGroup];
#pragma unroll
    for (int t = 0; t < kRampGroup; ++t) q[t] = side[t * kRampRecord + Q];
    for (int i = 0; i < n; i += kRampGroup) {
        const float4 *rec = side + i * kRampRecord;
        float cc[kRampGroup], sc[kRampGroup];
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t)
            cc[t] = __builtin_fmaf(q[t].x, x0, __builtin_fmaf(q[t].y, y, __builtin_fmaf(q[t].z, z, q[t].w)));
        float4 cs[Q];
#pragma unroll
        for (int e = 0; e < Q; ++e) cs[e] = rec[e];
        // the next group's phase inputs (this group's again after the last)
        const float4 *nxt = i + kRampGroup < n ? rec + kRampGroup * kRampRecord : rec;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            sc[t] = __builtin_amdgcn_sinf(cc[t]);
            cc[t] = __builtin_amdgcn_cosf(cc[t]);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            // the next sample's C and S, or during the group's last sample
            // (in the registers C and S would take) the next group's phase
            // inputs
            float4 cn[Q];
            if (t + 1 < kRampGroup) {
#pragma unroll
                for (int e = 0; e < Q; ++e) cn[e] = rec[(t + 1) * kRampRecord + e];
            } else {
#pragma unroll
                for (int u = 0; u < kRampGroup; ++u) q[u] = nxt[u * kRampRecord + Q];
            }
            float C[P], S[P];
#pragma unroll
            for (int e = 0; e < Q / 2; ++e) {
                C[4 * e] = cs[e].x;
                C[4 * e + 1] = cs[e].y;
                C[4 * e + 2] = cs[e].z;
                C[4 * e + 3] = cs[e].w;
                S[4 * e] = cs[Q / 2 + e].x;
                S[4 * e + 1] = cs[Q / 2 + e].y;
                S[4 * e + 2] = cs[Q / 2 + e].z;
                S[4 * e + 3] = cs[Q / 2 + e].w;
            }
#pragma unroll
            for (int j = 0; j < P; ++j) {
                acc_r[j] = __builtin_fmaf(cc[t], C[j], acc_r[j]);
                acc_i[j] = __builtin_fmaf(sc[t], C[j], acc_i[j]);
                acc_r[P + j] = __builtin_fmaf(-sc[t], S[j], acc_r[P + j]);
                acc_i[P + j] = __builtin_fmaf(cc[t], S[j], acc_i[P + j]);
            }
            if (t + 1 < kRampGroup) {
#pragma unroll
                for (int e = 0; e < Q; ++e) cs[e] = cn[e];
            }
            // the reads go out after this sample's first FMAs (whose
            // operands are then in), so waiting for them never waits for
            // the reads just issued
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, Q, 0);   // Q == kRampGroup reads either way
            __builtin_amdgcn_sched_group_barrier(0x002, 4 * P - 2, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Streams chunks [c_begin, c_end) like stream_chunks(), and turns each stage
// into sample records kSideSamples at a time: records written, LDS barrier,
// accumulated by every lane, LDS barrier. The next stage's copy is issued
// after the first round's records are written, so no barrier waits for it
// before the stage's end.
template <int V>
__device__ __forceinline__ void ramp_one_step(const float4 *__restrict__ src, int c_begin, int c_end,
                                              float4 (*stage)[kStageVec4], float4 *side, float x0,
                                              float hdx, float y, float z, float (&acc_r)[V],
                                              float (&acc_i)[V])
{
    const int nchunks = c_end > c_begin ? c_end - c_begin : 0;
    src += (int64_t)c_begin * kChunkVec4;
    const int64_t total_vec4 = (int64_t)nchunks * kChunkVec4;
    const int nstages = (nchunks + kStageChunks - 1) / kStageChunks;
    if (nstages > 0) issue_stage_load(src, total_vec4, 0, stage[0]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int st = 0; st < nstages; ++st) {
        const int samples = min(kStageChunks, nchunks - st * kStageChunks) * kChunk;
        const float4 *buf = stage[st & 1];
        for (int r0 = 0; r0 < samples; r0 += kSideSamples) {
            const int n = min(kSideSamples, samples - r0);
            ramp_records<V>(buf, r0, n, hdx, side);
            lds_barrier();
            if (r0 == 0 && st + 1 < nstages) issue_stage_load(src, total_vec4, st + 1, stage[(st + 1) & 1]);
            ramp_accumulate_records<V>(side, n, x0, y, z, acc_r, acc_i);
            lds_barrier();
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
}

// Pair sums of the ramp path (acc[j] = sum_j, acc[V/2 + j] = dif_j) to the
// voxels' sums: voxel V/2 + j gets sum_j + dif_j, voxel V/2 - 1 - j gets
// sum_j - dif_j.
template <int V>
__device__ __forceinline__ void ramp_unfold(float (&acc_r)[V], float (&acc_i)[V])
{
    constexpr int P = V / 2;
    float out_r[V], out_i[V];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        out_r[P + j] = acc_r[j] + acc_r[P + j];
        out_i[P + j] = acc_i[j] + acc_i[P + j];
        out_r[P - 1 - j] = acc_r[j] - acc_r[P + j];
        out_i[P - 1 - j] = acc_i[j] - acc_i[P + j];
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
        acc_r[v] = out_r[v];
        acc_i[v] = out_i[v];
    }
}

// ---------------------------------------------------------------------------
// Units and their classes
// ---------------------------------------------------------------------------
// Every gather instance takes voxels in units of kUnitVox consecutive
// voxels (a workgroup takes one unit, or an aligned pair of units). The
// classify kernel tests each unit once and records which instance takes
// it; a "line" is a run of voxels along x at a common step (same y and z
// bitwise, x_v = x_0 + v dx rounded once), and the classes are
//   kClassLongPair -- both units of an aligned pair are whole and their
//                     aligned runs of kLongLineVox voxels are lines of one
//                     step for the pair (any x-fastest grid whose rows are a
//                     multiple of 128 voxels): the long-line matrix-core
//                     instance, two units per workgroup;
//   kClassLines    -- otherwise, the unit is whole and its aligned runs of
//                     kLineVox voxels are lines of one step for the unit
//                     (rows a multiple of 64): the matrix-core instance;
//   kClassOneStep  -- otherwise, every lane's kVox voxels are such a ramp
//                     and all lanes share the step: the ramp path with
//                     sample records;
//   kClassGeneral  -- everything else (per-lane ramps, shared (y, z), direct).
static_assert(kUnitVox == kBlock * kVox, "a unit is one workgroup of the vector instances");
static_assert(kLineVox % kVox == 0 && 64 % (kLineVox / kVox) == 0, "a line is whole lanes of one wave");
static_assert(kLongLineVox % kVox == 0 && 64 % (kLongLineVox / kVox) == 0, "a line is whole lanes of one wave");

// Lane l of workgroup b owns voxels (b kBlock + l) V + v, v < V. Voxels past
// N copy the lane's first voxel, so they never spoil the shared-(y, z) test
// (their results are not stored). With VEC4, a lane with all V voxels in
// range reads them as float4s when the coordinate arrays are 16-byte
// aligned (the classification; the gather instances keep scalar loads,
// which leave their register allocation as it is).
template <int V, bool VEC4 = false>
__device__ __forceinline__ void load_lane_voxels(const float *__restrict__ x, const float *__restrict__ y,
                                                 const float *__restrict__ z, int N, int64_t n0,
                                                 float (&px)[V], float (&py)[V], float (&pz)[V])
{
    if constexpr (VEC4 && V % 4 == 0) {
        const bool aligned = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y) |
                               reinterpret_cast<uintptr_t>(z)) & 15) == 0;
        if (aligned && n0 + V <= N) {
            const float4 *x4 = reinterpret_cast<const float4 *>(x + n0);
            const float4 *y4 = reinterpret_cast<const float4 *>(y + n0);
            const float4 *z4 = reinterpret_cast<const float4 *>(z + n0);
#pragma unroll
            for (int q = 0; q < V / 4; ++q) {
                const float4 a = x4[q], b = y4[q], c = z4[q];
                px[4 * q] = a.x, px[4 * q + 1] = a.y, px[4 * q + 2] = a.z, px[4 * q + 3] = a.w;
                py[4 * q] = b.x, py[4 * q + 1] = b.y, py[4 * q + 2] = b.z, py[4 * q + 3] = b.w;
                pz[4 * q] = c.x, pz[4 * q + 1] = c.y, pz[4 * q + 2] = c.z, pz[4 * q + 3] = c.w;
            }
            return;
        }
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int64_t n = n0 + v;
        const bool live = n < N;
        px[v] = live ? x[n] : 0.0f;
        py[v] = live ? y[n] : 0.0f;
        pz[v] = live ? z[n] : 0.0f;
    }
#pragma unroll
    for (int v = 1; v < V; ++v)
        if (n0 + v >= N) {
            px[v] = px[0];
            py[v] = py[0];
            pz[v] = pz[0];
        }
}

// Whether the lane's voxels share y and z bitwise (*same_yz) and, in
// addition, sit at x_0 + v dx rounded once with dx = x_1 - x_0 (returned;
// lanes with voxels past N never qualify); *dx gets that step.
template <int V>
__device__ __forceinline__ bool lane_ramp(const float (&px)[V], const float (&py)[V],
                                          const float (&pz)[V], int64_t n0, int N, bool *same_yz,
                                          float *dx)
{
    bool same = true;
#pragma unroll
    for (int v = 1; v < V; ++v)
        same = same && __float_as_uint(py[v]) == __float_as_uint(py[0]) &&
               __float_as_uint(pz[v]) == __float_as_uint(pz[0]);
    const float d = px[1] - px[0];
    bool ramp = same && n0 + V <= N && __builtin_isfinite(d);
#pragma unroll
    for (int v = 1; v < V; ++v) ramp = ramp && __builtin_fmaf((float)v, d, px[0]) == px[v];
    *same_yz = same;
    *dx = d;
    return ramp;
}

// Whether the lane's voxels lie on the line of LINE voxels that its group
// of LINE / V lanes forms: y and z equal to the line's first voxel's
// bitwise and x_v = x_0 + v dx rounded once, dx = x_1 - x_0 of the line;
// *dx gets the line's step.
template <int LINE, int V>
__device__ __forceinline__ bool lane_on_line(const float (&px)[V], const float (&py)[V],
                                             const float (&pz)[V], float *dx)
{
    constexpr int kLanes = LINE / V;
    const int lane = threadIdx.x & 63;
    const int lead = lane & ~(kLanes - 1);
    const float x0 = __shfl(px[0], lead), x1 = __shfl(px[1], lead);
    const float y0 = __shfl(py[0], lead), z0 = __shfl(pz[0], lead);
    const float d = x1 - x0;
    const int first = V * (lane & (kLanes - 1));
    bool ok = __builtin_isfinite(d);
#pragma unroll
    for (int v = 0; v < V; ++v)
        ok = ok && __builtin_fmaf((float)(first + v), d, x0) == px[v] &&
             __float_as_uint(py[v]) == __float_as_uint(y0) && __float_as_uint(pz[v]) == __float_as_uint(z0);
    *dx = d;
    return ok;
}

// One workgroup per aligned pair of units (units 2b and 2b + 1 < units),
// one half of the workgroup (kBlock lanes, the lane-to-voxel map of the
// gather instances) per unit, both tested at once: cls[u] = the class of
// unit u (never a matrix-core class unless allow_lines); the first pair's
// workgroup also records whether that pair is of class kClassLongPair
// (info[0]) and its lines' step (info[1], bits), and clears info[2] and
// info[3] (flags the forward operator's line and line-pair pre-passes set). Two barriers: one to publish
// each unit's first-lane steps, one to combine the waves' votes.
//
// With `patches` set, the workgroup also records in patches[2 b] and
// patches[2 b + 1] whether the pair's lines, taken two by two (lines 2i
// and 2i + 1), are all one line and that line moved by one common offset d
// (bitwise the same difference of their first voxels' x, y and z), with
// the lines' step dx and d (bits): {flag, dx, e.x, e.y} and {d.x, d.y,
// d.z, e.z}; flag 1 for the 64 lines of 128 voxels of a long pair, 2 for
// the 128 lines of 64 voxels of two units of class kClassLines with one
// step, 3 for those when, beyond that, the lines 4i + 2 are the lines 4i
// moved by one common offset e (so lines 4i .. 4i + 3 sit at 0, d, e and
// e + d from line 4i).
//
// When the grid holds kAmpSlots more workgroups than pairs, workgroup
// pairs + s instead writes slot s (info[4 + s]) with the largest amplitude
// (bits) of the chunks c = s kClassifyBlock + t, s kClassifyBlock + t +
// kAmpSlots kClassifyBlock, ... of `packed` (nchunks chunks): the
// matrix-core products in fp16 scale the amplitudes by it (amp_shift).
constexpr int kClassifyBlock = 2 * kBlock;
__global__ __launch_bounds__(kClassifyBlock) void fhd_classify_kernel(const float *__restrict__ x,
                                                                      const float *__restrict__ y,
                                                                      const float *__restrict__ z, int N,
                                                                      int64_t units, int allow_lines,
                                                                      int *__restrict__ cls,
                                                                      int *__restrict__ info,
                                                                      const float4 *__restrict__ packed,
                                                                      int nchunks, int4 *__restrict__ patches)
{
    constexpr int kWavesPerUnit = kBlock / 64;
    const int64_t pairs = (units + 1) / 2;
    if ((int64_t)blockIdx.x >= pairs) {   // an amplitude slot (uniform over the workgroup)
        __shared__ unsigned wave_max[kClassifyBlock / 64];
        const int slot = (int)((int64_t)blockIdx.x - pairs);
        unsigned m = 0u;
        for (int64_t c = (int64_t)slot * kClassifyBlock + threadIdx.x; c < nchunks;
             c += (int64_t)kAmpSlots * kClassifyBlock) {
            // the amplitude field: the chunk's float4s 8 and 9
            const float4 a = packed[c * kChunkVec4 + 8], b = packed[c * kChunkVec4 + 9];
            const unsigned v[8] = {__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z),
                                   __float_as_uint(a.w), __float_as_uint(b.x), __float_as_uint(b.y),
                                   __float_as_uint(b.z), __float_as_uint(b.w)};
#pragma unroll
            for (int i = 0; i < 8; ++i) m = v[i] > m ? v[i] : m;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const unsigned t = (unsigned)__shfl_xor((int)m, o);
            m = t > m ? t : m;
        }
        if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x / 64] = m;
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 1; w < kClassifyBlock / 64; ++w) m = wave_max[w] > m ? wave_max[w] : m;
            info[4 + slot] = (int)m;
        }
        return;
    }
    __shared__ float wg_step[2][3];                // each unit's first lane's ramp and line steps
    __shared__ float wg_shift[3][3];               // the pair's first lines' offsets (128, 64, 64 by 2)
    __shared__ int votes[2 * kWavesPerUnit][6];    // per wave: one step, 64-lines, 128-lines, shifts
    const int half = threadIdx.x / kBlock, t = threadIdx.x % kBlock;
    const int64_t u = 2 * (int64_t)blockIdx.x + half;
    const bool present = u < units;   // the grid's last pair may hold one unit
    const int64_t unit = u * kUnitVox;
    const int64_t n0 = unit + (int64_t)t * kVox;
    bool ramp = false, on64 = false, on128 = false;
    float dx = 0.0f, d64 = 0.0f, d128 = 0.0f;
    // this lane's line pair (lines 2i and 2i + 1 of kLongLineVox voxels:
    // the lanes from a_lead and from a_lead + 8 of the wave): the offset of
    // the second's first voxel from the first's
    constexpr int kLineLanes = kLongLineVox / kVox, kLine64Lanes = kLineVox / kVox;
    static_assert(kLineLanes == 8 && 64 % (2 * kLineLanes) == 0, "a wave holds whole line pairs");
    static_assert(kLine64Lanes == 4, "a 64-voxel line pair is 8 lanes");
    float sx = 0.0f, sy = 0.0f, sz = 0.0f, sx64 = 0.0f, sy64 = 0.0f, sz64 = 0.0f;
    float ex64 = 0.0f, ey64 = 0.0f, ez64 = 0.0f;
    if (present) {   // uniform over each wave
        float px[kVox], py[kVox], pz[kVox];
        load_lane_voxels<kVox, true>(x, y, z, N, n0, px, py, pz);
        bool same_yz;
        ramp = lane_ramp<kVox>(px, py, pz, n0, N, &same_yz, &dx);
        const bool whole = unit + kUnitVox <= N;
        on64 = whole && lane_on_line<kLineVox, kVox>(px, py, pz, &d64);
        on128 = whole && lane_on_line<kLongLineVox, kVox>(px, py, pz, &d128);
        const int a_lead = (threadIdx.x & 63) & ~(2 * kLineLanes - 1);
        sx = __shfl(px[0], a_lead + kLineLanes) - __shfl(px[0], a_lead);
        sy = __shfl(py[0], a_lead + kLineLanes) - __shfl(py[0], a_lead);
        sz = __shfl(pz[0], a_lead + kLineLanes) - __shfl(pz[0], a_lead);
        const int a64 = (threadIdx.x & 63) & ~(2 * kLine64Lanes - 1);
        sx64 = __shfl(px[0], a64 + kLine64Lanes) - __shfl(px[0], a64);
        sy64 = __shfl(py[0], a64 + kLine64Lanes) - __shfl(py[0], a64);
        sz64 = __shfl(pz[0], a64 + kLine64Lanes) - __shfl(pz[0], a64);
        // this lane's group of four 64-voxel lines (16 lanes): line 4i + 2's
        // offset from line 4i
        const int a4 = (threadIdx.x & 63) & ~(4 * kLine64Lanes - 1);
        ex64 = __shfl(px[0], a4 + 2 * kLine64Lanes) - __shfl(px[0], a4);
        ey64 = __shfl(py[0], a4 + 2 * kLine64Lanes) - __shfl(py[0], a4);
        ez64 = __shfl(pz[0], a4 + 2 * kLine64Lanes) - __shfl(pz[0], a4);
        if (t == 0) {
            wg_step[half][0] = dx;
            wg_step[half][1] = d64;
            wg_step[half][2] = d128;
            if (half == 0) {
                wg_shift[0][0] = sx;
                wg_shift[0][1] = sy;
                wg_shift[0][2] = sz;
                wg_shift[1][0] = sx64;
                wg_shift[1][1] = sy64;
                wg_shift[1][2] = sz64;
                wg_shift[2][0] = ex64;
                wg_shift[2][1] = ey64;
                wg_shift[2][2] = ez64;
            }
        }
    }
    __syncthreads();
    const bool one = ramp && __float_as_uint(dx) == __float_as_uint(wg_step[half][0]);
    const bool l64 = on64 && __float_as_uint(d64) == __float_as_uint(wg_step[half][1]);
    const bool l128 = on128 && __float_as_uint(d128) == __float_as_uint(wg_step[half][2]);
    const bool shifted = l128 && __builtin_isfinite(sx) && __builtin_isfinite(sy) && __builtin_isfinite(sz) &&
                         __float_as_uint(sx) == __float_as_uint(wg_shift[0][0]) &&
                         __float_as_uint(sy) == __float_as_uint(wg_shift[0][1]) &&
                         __float_as_uint(sz) == __float_as_uint(wg_shift[0][2]);
    const bool shifted64 = l64 && __builtin_isfinite(sx64) && __builtin_isfinite(sy64) &&
                           __builtin_isfinite(sz64) && __float_as_uint(sx64) == __float_as_uint(wg_shift[1][0]) &&
                           __float_as_uint(sy64) == __float_as_uint(wg_shift[1][1]) &&
                           __float_as_uint(sz64) == __float_as_uint(wg_shift[1][2]);
    const bool grouped64 = shifted64 && __builtin_isfinite(ex64) && __builtin_isfinite(ey64) &&
                           __builtin_isfinite(ez64) && __float_as_uint(ex64) == __float_as_uint(wg_shift[2][0]) &&
                           __float_as_uint(ey64) == __float_as_uint(wg_shift[2][1]) &&
                           __float_as_uint(ez64) == __float_as_uint(wg_shift[2][2]);
    const int wave = threadIdx.x / 64;
    const bool all_one = __all(one), all64 = __all(l64), all128 = __all(l128), all_shift = __all(shifted);
    const bool all_shift64 = __all(shifted64), all_group64 = __all(grouped64);
    if ((threadIdx.x & 63) == 0) {
        votes[wave][0] = all_one;
        votes[wave][1] = all64;
        votes[wave][2] = all128;
        votes[wave][3] = all_shift;
        votes[wave][4] = all_shift64;
        votes[wave][5] = all_group64;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int c[2], lng[2], shf = 1, shf64 = 1, grp64 = 1;
        for (int k = 0; k < 2; ++k) {
            int v[6] = {1, 1, 1, 1, 1, 1};
            for (int w = 0; w < kWavesPerUnit; ++w)
                for (int q = 0; q < 6; ++q) v[q] &= votes[k * kWavesPerUnit + w][q];
            c[k] = allow_lines && v[1] ? kClassLines : v[0] ? kClassOneStep : kClassGeneral;
            lng[k] = v[2];
            shf &= v[3];
            shf64 &= v[4];
            grp64 &= v[5];
        }
        const bool has_second = 2 * (int64_t)blockIdx.x + 1 < units;
        const bool pair = allow_lines && has_second && lng[0] && lng[1] &&
                          __float_as_uint(wg_step[0][2]) == __float_as_uint(wg_step[1][2]);
        cls[2 * (int64_t)blockIdx.x] = pair ? kClassLongPair : c[0];
        if (has_second) cls[2 * (int64_t)blockIdx.x + 1] = pair ? kClassLongPair : c[1];
        if (blockIdx.x == 0) {
            info[0] = pair ? 1 : 0;
            info[1] = (int)__float_as_uint(wg_step[0][2]);
            info[2] = 0;
            info[3] = 0;
        }
        if (patches) {
            // 1: 128-voxel line pairs (a long pair); 2: 64-voxel line pairs
            // (both units of class kClassLines with one step for the pair);
            // 3: those in groups of four lines with one second offset
            const bool pair64 = !pair && has_second && c[0] == kClassLines && c[1] == kClassLines &&
                                __float_as_uint(wg_step[0][1]) == __float_as_uint(wg_step[1][1]) && shf64;
            const int flag = pair && shf ? 1 : pair64 && grp64 ? 3 : pair64 ? 2 : 0;
            const int sel = flag >= 2 ? 1 : 0;
            patches[2 * (int64_t)blockIdx.x] =
                make_int4(flag, (int)__float_as_uint(wg_step[0][flag >= 2 ? 1 : 2]),
                          (int)__float_as_uint(wg_shift[2][0]), (int)__float_as_uint(wg_shift[2][1]));
            patches[2 * (int64_t)blockIdx.x + 1] =
                make_int4((int)__float_as_uint(wg_shift[sel][0]), (int)__float_as_uint(wg_shift[sel][1]),
                          (int)__float_as_uint(wg_shift[sel][2]), (int)__float_as_uint(wg_shift[2][2]));
        }
    }
}

// Two VALU instances share the grid: ONE_STEP = true takes the units of
// class kClassOneStep (the ramp path with sample records, at 5 waves per
// SIMD, <= 96 VGPRs) and ONE_STEP = false those of class kClassGeneral (at
// 4 waves per SIMD, <= 128 VGPRs); each returns at once for the others.
// Split s = blockIdx.y of `splits` takes its share of the sample stream, in
// whole granules of kVecGranuleChunks chunks (so that a grid of few units
// can still fill the chip), and writes rho (splits == 1) or its partial
// sums at out + s*N.
template <int V, bool ONE_STEP>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(ONE_STEP ? 5 : 4))) void fhd_gather_kernel(
    const float *__restrict__ packed, int nchunks, int splits, const int *__restrict__ cls,
    const float *__restrict__ x, const float *__restrict__ y, const float *__restrict__ z,
    float *__restrict__ out_r, float *__restrict__ out_i, int N)
{
    static_assert(V * kBlock == kUnitVox, "a workgroup is one unit");
    if (cls[blockIdx.x] != (ONE_STEP ? kClassOneStep : kClassGeneral)) return;
    __shared__ float4 stage[2][kStageVec4];
    __shared__ float4 side[kSideSamples * kRampRecord];   // ramp path with one step per workgroup
    const float4 *src = reinterpret_cast<const float4 *>(packed);

    const int64_t n0 = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * V;
    float px[V], py[V], pz[V], acc_r[V], acc_i[V];
    load_lane_voxels<V>(x, y, z, N, n0, px, py, pz);
#pragma unroll
    for (int v = 0; v < V; ++v) {
        acc_r[v] = 0.0f;
        acc_i[v] = 0.0f;
    }
    bool same_yz;
    float dx;
    const bool ramp = lane_ramp<V>(px, py, pz, n0, N, &same_yz, &dx);

    int c0, c1;
    split_range<kVecGranuleChunks>(nchunks, splits, blockIdx.y, &c0, &c1);
    if constexpr (ONE_STEP) {
        // every lane is a ramp of the unit's common step
        ramp_one_step<V>(src, c0, c1, stage, side, px[0], 0.5f * dx, py[0], pz[0], acc_r, acc_i);
        ramp_unfold<V>(acc_r, acc_i);
    } else {
        // one decision per workgroup, so every branch's stage barriers are
        // reached by every wave of the workgroup
        const bool all_ramp = __syncthreads_and(ramp);
        const bool shared = __syncthreads_and(same_yz);
        if (all_ramp) {
            const float hdx = 0.5f * dx;
            stream_chunks(src, c0, c1, stage, [&](const float4 *ch) {
                accumulate_chunk_ramp<V>(ch, px[0], hdx, py[0], pz[0], acc_r, acc_i);
            });
            ramp_unfold<V>(acc_r, acc_i);
        } else if (shared)
            stream_chunks(src, c0, c1, stage, [&](const float4 *ch) {
                accumulate_chunk<V, true>(ch, px, py, pz, acc_r, acc_i);
            });
        else
            stream_chunks(src, c0, c1, stage, [&](const float4 *ch) {
                accumulate_chunk<V, false>(ch, px, py, pz, acc_r, acc_i);
            });
    }

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

// ---------------------------------------------------------------------------
// Which line-pair workgroups take a group of units
// ---------------------------------------------------------------------------
// Whether quad q (units 4q .. 4q + 3) is taken by the line-pair instance:
// both of its unit pairs are long pairs with the line-pair structure, the
// same step and the same offset (records from the classification, two
// int4 per unit pair).
__device__ __forceinline__ bool patch_quad(const int *__restrict__ cls, const int4 *__restrict__ patches,
                                           int64_t units, int64_t q)
{
    if (patches == nullptr || 4 * q + 3 >= units) return false;
    if (cls[4 * q] != kClassLongPair || cls[4 * q + 2] != kClassLongPair) return false;
    const int4 a0 = patches[4 * q], a1 = patches[4 * q + 1], b0 = patches[4 * q + 2], b1 = patches[4 * q + 3];
    return a0.x == 1 && b0.x == 1 && a0.y == b0.y && a1.x == b1.x && a1.y == b1.y && a1.z == b1.z;
}

// How the line-pair instance runs in a call: not at all, with a B table
// formed for quad 0's step and offsets (it then takes the quads of quad
// 0's kind that share them; the long-line and 64-voxel line-pair
// instances take the other unit pairs), or forming each step's B operands
// itself (it takes every quad of either kind).
enum : int { kPatchNone = 0, kPatchTable = 1, kPatchFormed = 2 };

// Whether quad q (units 4q .. 4q + 3) is one of four-line groups of
// 64-voxel lines: all four units of class kClassLines, both unit pairs'
// records flag 3, with the same step and offsets.
__device__ __forceinline__ bool group64_quad(const int *__restrict__ cls, const int4 *__restrict__ patches,
                                             int64_t units, int64_t q)
{
    if (patches == nullptr || 4 * q + 3 >= units) return false;
    if (cls[4 * q] != kClassLines || cls[4 * q + 1] != kClassLines || cls[4 * q + 2] != kClassLines ||
        cls[4 * q + 3] != kClassLines)
        return false;
    const int4 a0 = patches[4 * q], a1 = patches[4 * q + 1], b0 = patches[4 * q + 2], b1 = patches[4 * q + 3];
    return a0.x == 3 && b0.x == 3 && a0.y == b0.y && a0.z == b0.z && a0.w == b0.w && a1.x == b1.x &&
           a1.y == b1.y && a1.z == b1.z && a1.w == b1.w;
}

// Whether quad q is taken by the line-pair instance as four-line groups
// of 64-voxel lines in `mode` (in the table mode: quad 0 so too, with the
// same step and offsets).
__device__ __forceinline__ bool group64_taken(const int *__restrict__ cls, const int4 *__restrict__ patches,
                                              int64_t units, int64_t q, int mode)
{
    if (mode == kPatchNone || !group64_quad(cls, patches, units, q)) return false;
    if (mode == kPatchFormed || q == 0) return true;
    if (!group64_quad(cls, patches, units, 0)) return false;
    const int4 r0 = patches[0], r1 = patches[1], a0 = patches[4 * q], a1 = patches[4 * q + 1];
    return r0.y == a0.y && r0.z == a0.z && r0.w == a0.w && r1.x == a1.x && r1.y == a1.y && r1.z == a1.z &&
           r1.w == a1.w;
}

// Whether unit pair p (units 2p, 2p + 1) is one the 64-voxel line-pair
// instance may take: both units of class kClassLines, the pair's record
// says its 64-voxel lines pair up (flag 2 or 3), and its quad is not
// taken as four-line groups in the line-pair instance's mode.
__device__ __forceinline__ bool pair64_open(const int *__restrict__ cls, const int4 *__restrict__ patches,
                                            int64_t units, int64_t p, int quad_mode)
{
    if (patches == nullptr || 2 * p + 1 >= units) return false;
    if (cls[2 * p] != kClassLines || cls[2 * p + 1] != kClassLines) return false;
    if (patches[2 * p].x != 2 && patches[2 * p].x != 3) return false;
    return !group64_taken(cls, patches, units, p / 2, quad_mode);
}

// Whether unit pair p is taken by the 64-voxel line-pair instance in
// `mode` (in the table mode also pair 0 so, with the same step and
// offset), the line-pair instance running in `quad_mode`.
__device__ __forceinline__ bool pair64_taken(const int *__restrict__ cls, const int4 *__restrict__ patches,
                                             int64_t units, int64_t p, int mode, int quad_mode)
{
    if (mode == kPatchNone || !pair64_open(cls, patches, units, p, quad_mode)) return false;
    if (mode == kPatchFormed || p == 0) return true;
    if (!pair64_open(cls, patches, units, 0, quad_mode)) return false;
    const int4 r0 = patches[0], r1 = patches[1], a0 = patches[2 * p], a1 = patches[2 * p + 1];
    return r0.y == a0.y && r1.x == a1.x && r1.y == a1.y && r1.z == a1.z;
}

// Whether quad q is taken by the line-pair instance in `mode` as 128-voxel
// line pairs.
__device__ __forceinline__ bool patch_taken(const int *__restrict__ cls, const int4 *__restrict__ patches,
                                            int64_t units, int64_t q, int mode)
{
    if (mode == kPatchNone || !patch_quad(cls, patches, units, q)) return false;
    if (mode == kPatchFormed) return true;
    if (q == 0) return true;
    if (!patch_quad(cls, patches, units, 0)) return false;
    const int4 r0 = patches[0], r1 = patches[1], a0 = patches[4 * q], a1 = patches[4 * q + 1];
    return r0.y == a0.y && r1.x == a1.x && r1.y == a1.y && r1.z == a1.z;
}

// ---------------------------------------------------------------------------
// Lines on the matrix cores
// ---------------------------------------------------------------------------
// In a unit of class kClassLines the voxels of a line pair up about its
// centre x_c = x_0 + (kLineVox - 1) dx / 2, and pair j, at x_c +- (j + 1/2)
// dx, gets
//
//   sum_m U[l, m] (B_C[m, j] +- i B_S[m, j])
//   U[l, m]   = exp(i 2 pi (k_m . x_c(l) + psi_m))     (line l's centre)
//   B_C[m, j] = a_m cos(2 pi (2j + 1) kx_m dx / 2)      (real, the same for
//   B_S[m, j] = a_m sin(2 pi (2j + 1) kx_m dx / 2)       every line)
//
// i.e. four real matrix products (lines x samples) by (samples x pairs):
// P_rc = U_r B_C, P_ic = U_i B_C, P_is = U_i B_S, P_rs = U_r B_S, and voxel
// kLineVox/2 + j gets (P_rc - P_is, P_ic + P_rs), voxel kLineVox/2 - 1 - j
// (P_rc + P_is, P_ic - P_rs). They run on the bf16 matrix cores with every
// fp32 operand split into a bf16 high part and a bf16 remainder, three
// products per real product (the remainders' product, below 2^-17 of it,
// dropped), accumulated in fp32: 12 v_mfma_f32_32x32x16_bf16 per 32 lines
// x 32 pairs x 16 samples, 6 bf16 multiply-adds per term in place of two
// transcendentals per 16 terms and 2 FMAs per term on the vector ALUs.
//
// Operand layout of v_mfma_f32_32x32x16_bf16 (measured): lane l supplies
// A[l % 32][8 (l / 32) + i] and B[8 (l / 32) + i][l % 32], i < 8, and
// accumulator register r of lane l holds C[8 (r / 4) + 4 (l / 32) + r % 4]
// [l % 32]. A wave takes 32 lines (rows) and all 32 pairs (columns); per 16
// samples (a chunk pair, chunk l / 32 for lane l) a lane forms U of its
// line for its 8 samples (3 FMA, 2 transcendentals each) and, shared by the
// workgroup through LDS, 8 elements of B_C (wave 0) or B_S (wave 1) for its
// pair (1 multiply, 1 transcendental, 1 multiply each), split, published
// with one LDS barrier (double buffered).
constexpr int kLinesBlock = 128;                    // 2 waves
constexpr int kLinePairs = kLineVox / 2;
// stages of 32 chunks (5 KB, double buffered): with B's 8 KB the LDS holds
// as many workgroups as the registers allow (3 waves per SIMD)
constexpr int kLinesStageChunks = 32;
constexpr int kLinesStageVec4 = kLinesStageChunks * kChunkVec4;
static_assert(kLinePairs == 32, "the pairs fill one 32-column tile");
static_assert(kUnitVox == 32 * kLineVox * (kLinesBlock / 64), "a wave takes 32 lines of the unit");
static_assert(kLinesBlock / 64 == 2, "wave 0 forms B_C, wave 1 B_S");

template <bool F16>
__global__ __launch_bounds__(kLinesBlock) __attribute__((amdgpu_waves_per_eu(3))) void fhd_gather_lines_kernel(
    const float *__restrict__ packed, int nchunks, int splits, const int *__restrict__ cls,
    const int4 *__restrict__ patches, int64_t units, int pair_mode, int quad_mode, const int *__restrict__ info,
    const float *__restrict__ x, const float *__restrict__ y, const float *__restrict__ z,
    float *__restrict__ out_r, float *__restrict__ out_i, int N)
{
    // units the line-pair or 64-voxel line-pair instance takes are theirs
    if (cls[blockIdx.x] != kClassLines || group64_taken(cls, patches, units, blockIdx.x / 4, quad_mode) ||
        pair64_taken(cls, patches, units, blockIdx.x / 2, pair_mode, quad_mode))
        return;
    __shared__ float4 stage[2][kLinesStageVec4];
    // [buffer][B_C hi, B_C lo, B_S hi, B_S lo][k half][pair]: one lane's
    // 8-sample operand each; a half-wave reads 32 consecutive entries
    __shared__ u32x4 bshare[2][4][2][kLinePairs];
    const float4 *src = reinterpret_cast<const float4 *>(packed);
    const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // fp16 products: amplitudes scaled by 2^sh into fp16's range, the sums
    // scaled back at the end (powers of two: exact)
    const int sh = F16 ? read_amp_shift(info) : 0;

    // line 32 wave + col of the unit (the whole unit lies below N)
    const int64_t unit = (int64_t)blockIdx.x * kUnitVox;
    const int64_t first = unit + (int64_t)(32 * wave + col) * kLineVox;
    const float x0 = x[first], dx = x[first + 1] - x0, ly = y[first], lz = z[first];
    const float xc = __builtin_fmaf(0.5f * (float)(kLineVox - 1), dx, x0);
    // pair `col`'s angle per unit kx: (2 col + 1) dx / 2 (dx is the unit's)
    const float tj = (float)(2 * col + 1) * (0.5f * dx);

    float16v prc, pic, pis, prs;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        prc[r] = 0.0f;
        pic[r] = 0.0f;
        pis[r] = 0.0f;
        prs[r] = 0.0f;
    }

    int c0, c1, kb = 0;
    split_range<kLinesStageChunks>(nchunks, splits, blockIdx.y, &c0, &c1);
    const int nch = c1 > c0 ? c1 - c0 : 0;
    src += (int64_t)c0 * kChunkVec4;
    const int64_t total_vec4 = (int64_t)nch * kChunkVec4;
    const int nstages = (nch + kLinesStageChunks - 1) / kLinesStageChunks;
    if (nstages > 0) issue_stage_load<kLinesBlock, kLinesStageVec4>(src, total_vec4, 0, stage[0]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // one group of 16 samples: chunks ch and ch + 1 of the stage (the
    // second replaced by zeros, i.e. amplitude 0 in B, when ONE)
    auto group = [&](const float4 *ch, auto one) {
        float f[kFields][kChunk];
        if constexpr (decltype(one)::value) {
            if (half == 0) {
                load_chunk(ch, f);
            } else {
#pragma unroll
                for (int q = 0; q < kFields; ++q)
#pragma unroll
                    for (int u = 0; u < kChunk; ++u) f[q][u] = 0.0f;
            }
        } else {
            load_chunk(ch + half * kChunkVec4, f);
        }
        __builtin_amdgcn_s_setprio(1);
        float b[kChunk], amp[kChunk];
#pragma unroll
        for (int i = 0; i < kChunk; ++i) amp[i] = scale_amp<F16>(f[4][i], sh);
        if (wave == 0) {
#pragma unroll
            for (int i = 0; i < kChunk; ++i) b[i] = amp[i] * __builtin_amdgcn_cosf(f[0][i] * tj);
        } else {
#pragma unroll
            for (int i = 0; i < kChunk; ++i) b[i] = amp[i] * __builtin_amdgcn_sinf(f[0][i] * tj);
        }
        unsigned bh[4], bl[4];
        split_parts<F16, kChunk>(b, bh, bl);
        bshare[kb][2 * wave + 0][half][col] = (u32x4){bh[0], bh[1], bh[2], bh[3]};
        bshare[kb][2 * wave + 1][half][col] = (u32x4){bl[0], bl[1], bl[2], bl[3]};
        float ur[kChunk], ui[kChunk];
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            const float p = __builtin_fmaf(f[0][i], xc, __builtin_fmaf(f[1][i], ly, __builtin_fmaf(f[2][i], lz, f[3][i])));
            ur[i] = __builtin_amdgcn_cosf(p);
            ui[i] = __builtin_amdgcn_sinf(p);
        }
        unsigned wa[4][4];
        split_parts<F16, kChunk>(ur, wa[0], wa[1]);
        split_parts<F16, kChunk>(ui, wa[2], wa[3]);
        const u32x4 arh = {wa[0][0], wa[0][1], wa[0][2], wa[0][3]}, arl = {wa[1][0], wa[1][1], wa[1][2], wa[1][3]};
        const u32x4 aih = {wa[2][0], wa[2][1], wa[2][2], wa[2][3]}, ail = {wa[3][0], wa[3][1], wa[3][2], wa[3][3]};
        __builtin_amdgcn_s_setprio(0);
        lds_barrier();   // this group's B is in LDS
        const u32x4 bch = bshare[kb][0][half][col], bcl = bshare[kb][1][half][col];
        const u32x4 bsh = bshare[kb][2][half][col], bsl = bshare[kb][3][half][col];
        prc = mfma32<F16>(arh, bch, prc);
        pic = mfma32<F16>(aih, bch, pic);
        pis = mfma32<F16>(aih, bsh, pis);
        prs = mfma32<F16>(arh, bsh, prs);
        prc = mfma32<F16>(arh, bcl, prc);
        pic = mfma32<F16>(aih, bcl, pic);
        pis = mfma32<F16>(aih, bsl, pis);
        prs = mfma32<F16>(arh, bsl, prs);
        prc = mfma32<F16>(arl, bch, prc);
        pic = mfma32<F16>(ail, bch, pic);
        pis = mfma32<F16>(ail, bsh, pis);
        prs = mfma32<F16>(arl, bsh, prs);
        kb ^= 1;
    };
    for (int st = 0; st < nstages; ++st) {
        const int chunks_here = min(kLinesStageChunks, nch - st * kLinesStageChunks);
        const float4 *buf = stage[st & 1];
        for (int c = 0; c + 1 < chunks_here; c += 2) {
            group(buf + c * kChunkVec4, std::false_type{});
            // the next stage's copy goes out once the stage's first group
            // has passed its barrier, so no later barrier waits long for it
            if (c == 0 && st + 1 < nstages)
                issue_stage_load<kLinesBlock, kLinesStageVec4>(src, total_vec4, st + 1, stage[(st + 1) & 1]);
        }
        // an odd chunk at the stream's end (the last stage only)
        if (chunks_here & 1) group(buf + (chunks_here - 1) * kChunkVec4, std::true_type{});
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // unfold the pair sums into the line's voxels: row 8 (r / 4) + 4 half +
    // r % 4 of the wave's 32 lines, pair col
    float *dst_r = out_r + (int64_t)blockIdx.y * N, *dst_i = out_i + (int64_t)blockIdx.y * N;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t line = unit + (int64_t)(32 * wave + 8 * (r / 4) + 4 * half + (r % 4)) * kLineVox;
        dst_r[line + kLinePairs + col] = unscale<F16>(prc[r] - pis[r], sh);
        dst_i[line + kLinePairs + col] = unscale<F16>(pic[r] + prs[r], sh);
        dst_r[line + kLinePairs - 1 - col] = unscale<F16>(prc[r] + pis[r], sh);
        dst_i[line + kLinePairs - 1 - col] = unscale<F16>(pic[r] - prs[r], sh);
    }
}

// ---------------------------------------------------------------------------
// Long lines on the matrix cores
// ---------------------------------------------------------------------------
// An aligned pair of units of class kClassLongPair is 64 lines of
// kLongLineVox voxels with one step: the same four real products as the
// matrix-core instance above, with 64 pairs per line about the centre
// x_0 + (kLongLineVox - 1) dx / 2 and the B factors of a sample shared by all
// 64 lines of the workgroup. Per sample, the workgroup forms 64 U elements
// and 128 B values for 8192 voxels (the single-unit form: 64 and 64 for
// 4096), so the vector work per term is 36 % lower and matches the matrix
// cores' 6 bf16 multiply-adds per term.
//
// Four waves of 16 lines each, on v_mfma_f32_16x16x32_bf16 (operand layout
// measured: lane l supplies A[l % 16][8 (l / 16) + i] and B[8 (l / 16) +
// i][l % 16], i < 8; accumulator register r of lane l holds C[4 (l / 16) +
// r][l % 16]): per 32 samples (four chunks, chunk l / 16 for lane l) a lane
// forms U of its line for its 8 samples and 16 B values -- wave w the
// B_C (w < 2) or B_S (w >= 2, as a cosine a quarter turn later) elements of
// pair tiles 2 (w % 2) and 2 (w % 2) + 1 for its pair l % 16 -- published
// through LDS (double buffered, one barrier per 32 samples); each wave then
// takes 4 pair tiles of 16: 48 products of 16 x 16 x 32.
constexpr int kLongPairs = kLongLineVox / 2;       // 64
constexpr int kLongTiles = kLongPairs / 16;        // 16-pair tiles
constexpr int kPairVox = 2 * kUnitVox;             // voxels per workgroup
constexpr int kLongBlock = 256;                    // 4 waves of 16 lines
constexpr int kLongGroup = 4;                      // chunks per product step (32 samples)
static_assert(kPairVox == kLongLineVox * 16 * (kLongBlock / 64), "a wave takes 16 lines of the pair");
static_assert(kLongTiles == 4 && kLongBlock / 64 == 4, "each wave forms 2 tiles of B_C or B_S");
static_assert(kLinesStageChunks % kLongGroup == 0, "product steps tile a stage");

// B operands of one product step (32 samples), laid out as the operands are
// read: [B_C hi, B_C lo, B_S hi, B_S lo][tile][k quarter][pair in tile],
// 8 bf16 (one lane's operand) each; a wave reads 64 consecutive entries
// (no bank conflicts). 16 KB.
constexpr int kLongStepVec4 = 4 * kLongTiles * 4 * 16;
typedef u32x4 LongStepB[4][kLongTiles][4][16];
// A product step's LDS buffer: its B operands and its four sample chunks.
constexpr int kLongStepChunkVec4 = kLongGroup * kChunkVec4;   // 40 float4
struct LongStep {
    LongStepB b;
    float4 chunks[kLongStepChunkVec4];
};

// Lane (wave w, lane l) of a step's B: B_C (w < 2) or B_S (w >= 2, as a
// cosine a quarter turn later) of pair tiles 2 (w % 2) and 2 (w % 2) + 1,
// pair l % 16 of each, samples 8 (l / 16) .. + 7 (f: their chunk; dx: the
// step of the lines; sh: the amplitudes' scaling in the fp16 form), split
// and stored at their place in `dst`.
template <bool F16>
__device__ __forceinline__ void long_step_b(const float (&f)[kFields][kChunk], float dx, int wave,
                                            int quarter_k, int col, int sh, LongStepB &dst)
{
    const int part = wave >> 1, t0 = 2 * (wave & 1);
    const float turn = part == 0 ? 0.0f : -0.25f;
    const float tj0 = (float)(2 * (16 * t0 + col) + 1) * (0.5f * dx);
    const float tj1 = (float)(2 * (16 * (t0 + 1) + col) + 1) * (0.5f * dx);
    float b0[kChunk], b1[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        const float amp = scale_amp<F16>(f[4][i], sh);
        b0[i] = amp * __builtin_amdgcn_cosf(__builtin_fmaf(f[0][i], tj0, turn));
        b1[i] = amp * __builtin_amdgcn_cosf(__builtin_fmaf(f[0][i], tj1, turn));
    }
    unsigned h0[4], l0[4], h1[4], l1[4];
    split_parts<F16, kChunk>(b0, h0, l0);
    split_parts<F16, kChunk>(b1, h1, l1);
    dst[2 * part + 0][t0][quarter_k][col] = (u32x4){h0[0], h0[1], h0[2], h0[3]};
    dst[2 * part + 1][t0][quarter_k][col] = (u32x4){l0[0], l0[1], l0[2], l0[3]};
    dst[2 * part + 0][t0 + 1][quarter_k][col] = (u32x4){h1[0], h1[1], h1[2], h1[3]};
    dst[2 * part + 1][t0 + 1][quarter_k][col] = (u32x4){l1[0], l1[1], l1[2], l1[3]};
}

constexpr int kQuadVox = 2 * kPairVox;              // voxels of a quad
constexpr int kPatchBlock = 256;                    // 4 waves of 16 rows

// The line-pair instance for groups of SIDES lines of LINE voxels
// symmetric about a centre c (128, 2: a line and the line moved by d, the
// quads of long pairs; 64, 4: lines at 0, d, e, e + d, four-line groups of
// 64-voxel lines; 64, 2: unit pairs of 64-voxel lines). A group is one row
// of the products; its voxels pair up by point reflection about c, one
// column per pair: side s (sigma_1, sigma_2) = (s & 1 ? -1 : 1, s & 2 ?
// -1 : 1) and j < LINE / 2 hold the voxel at c + sigma_1 d / 2 + sigma_2 e
// / 2 + o_j (line SIDES - 1 - s of the group, voxel LINE / 2 + j) and its
// reflection (line s, voxel LINE / 2 - 1 - j), o_j = (j + 1/2) dx e_x. A
// workgroup takes 64 rows with SIDES LINE / 2 columns in kTiles tiles of
// 16. B operands of one step: [B_C hi, B_C lo, B_S hi, B_S lo][tile][k
// quarter][column in tile], one lane's 8 fp16 or bf16 each: 32 KB for 8
// tiles, 16 KB for 4.
template <int TILES>
struct PatchStep {
    u32x4 b[4][TILES][4][16];
    float4 chunks[kLongStepChunkVec4];
};
template <int LINE, int SIDES>
struct PatchShape {
    static constexpr int kHalf = LINE / 2;                  // columns per side
    static constexpr int kTiles = SIDES * kHalf / 16;
    static constexpr int kSideTiles = kHalf / 16;
    static constexpr int kGroupVox = 64 * SIDES * LINE;
    static constexpr int kStepVec4 = 4 * kTiles * 4 * 16;
    typedef u32x4 StepB[4][kTiles][4][16];
    typedef PatchStep<kTiles> Step;
};
typedef PatchShape<kLongLineVox, 2> PairShape128;
typedef PatchShape<kLineVox, 4> GroupShape64;
typedef PatchShape<kLineVox, 2> PairShape64;
static_assert(PairShape128::kGroupVox == kQuadVox, "a 128-voxel line-pair workgroup is a quad");
static_assert(GroupShape64::kGroupVox == kQuadVox, "a 64-voxel four-line-group workgroup is a quad");
static_assert(PairShape64::kGroupVox == kPairVox, "a 64-voxel line-pair workgroup is a unit pair");
static_assert(PairShape128::kTiles == GroupShape64::kTiles, "both quad kinds share one step layout");
constexpr int kPatchStepVec4 = PairShape128::kStepVec4;
static_assert(PairShape64::kStepVec4 == kLongStepVec4, "the 64-voxel line-pair B shares the long-line table");

// The offsets of a group (from its records): d and, for four sides, e.
struct GroupOffsets {
    float dx, d[3], e[3];
};
__device__ __forceinline__ GroupOffsets group_offsets(const int4 *__restrict__ rec)
{
    const int4 a = rec[0], b = rec[1];
    GroupOffsets o;
    o.dx = __int_as_float(a.y);
    o.d[0] = __int_as_float(b.x);
    o.d[1] = __int_as_float(b.y);
    o.d[2] = __int_as_float(b.z);
    o.e[0] = __int_as_float(a.z);
    o.e[1] = __int_as_float(a.w);
    o.e[2] = __int_as_float(b.w);
    return o;
}

// Lane (wave w, lane l) of a step's B: B_C (w < 2) or B_S (w >= 2, as a
// cosine a quarter turn later) of the tiles of sides (w & 1) SIDES / 2 ..
// + SIDES / 2 - 1, column l % 16 of each, samples 8 (l / 16) .. + 7 (f:
// their chunk; sh: the amplitudes' scaling in the fp16 form), split and
// stored at their place in `dst`.
template <bool F16, int LINE, int SIDES>
__device__ __forceinline__ void patch_step_b(const float (&f)[kFields][kChunk], const GroupOffsets &o, int wave,
                                             int quarter_k, int col, int sh,
                                             typename PatchShape<LINE, SIDES>::StepB &dst)
{
    using Shape = PatchShape<LINE, SIDES>;
    constexpr int kSidesPerWave = SIDES / 2;
    const int part = wave >> 1;
    const float turn = part == 0 ? 0.0f : -0.25f;
    float hd[kChunk], he[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        hd[i] = 0.5f * __builtin_fmaf(f[0][i], o.d[0], __builtin_fmaf(f[1][i], o.d[1], f[2][i] * o.d[2]));
        he[i] = SIDES == 4 ? 0.5f * __builtin_fmaf(f[0][i], o.e[0], __builtin_fmaf(f[1][i], o.e[1], f[2][i] * o.e[2]))
                           : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < kSidesPerWave; ++q) {
        const int side = (wave & 1) * kSidesPerWave + q;
        const float s1 = (side & 1) ? -1.0f : 1.0f, s2 = (side & 2) ? -1.0f : 1.0f;
#pragma unroll
        for (int tt = 0; tt < Shape::kSideTiles; ++tt) {
            const int j = 16 * tt + col, t = side * Shape::kSideTiles + tt;
            const float tj = (float)(2 * j + 1) * (0.5f * o.dx);
            float b[kChunk];
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                const float off = SIDES == 4 ? __builtin_fmaf(s2, he[i], s1 * hd[i]) : s1 * hd[i];
                const float amp = scale_amp<F16>(f[4][i], sh);
                b[i] = amp * __builtin_amdgcn_cosf(__builtin_fmaf(f[0][i], tj, off + turn));
            }
            unsigned h[4], l[4];
            split_parts<F16, kChunk>(b, h, l);
            dst[2 * part + 0][t][quarter_k][col] = (u32x4){h[0], h[1], h[2], h[3]};
            dst[2 * part + 1][t][quarter_k][col] = (u32x4){l[0], l[1], l[2], l[3]};
        }
    }
}

// Step g of the B table for a group's step and offsets (the records at
// rec[0], rec[1]): chunks past the stream's end as zeros.
template <bool F16, int LINE, int SIDES>
__device__ __forceinline__ void patch_table_step(const float *__restrict__ packed, int nchunks,
                                                 const int4 *__restrict__ rec, const int *__restrict__ info,
                                                 float4 *__restrict__ table)
{
    using Shape = PatchShape<LINE, SIDES>;
    const GroupOffsets o = group_offsets(rec);
    const int sh = F16 ? read_amp_shift(info) : 0;
    const int lane = threadIdx.x & 63, quarter_k = lane >> 4, col = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t chunk = (int64_t)blockIdx.x * kLongGroup + quarter_k;
    float f[kFields][kChunk];
    if (chunk < nchunks) {
        load_chunk(reinterpret_cast<const float4 *>(packed) + chunk * kChunkVec4, f);
    } else {
#pragma unroll
        for (int q = 0; q < kFields; ++q)
#pragma unroll
            for (int u = 0; u < kChunk; ++u) f[q][u] = 0.0f;
    }
    patch_step_b<F16, LINE, SIDES>(
        f, o, wave, quarter_k, col, sh,
        *reinterpret_cast<typename Shape::StepB *>(table + (int64_t)blockIdx.x * Shape::kStepVec4));
}

// The B operands of every product step of the sample stream, formed once per
// call for the step of the first pair of units when that pair is of class
// kClassLongPair (info[0] = 1, info[1] = its step's bits, as the classify
// kernel records them) and not taken by the line-pair instance (which then
// most likely takes every long pair): step g at table + g kLongStepVec4,
// chunks past the stream's end as zeros. The long-line workgroups whose
// lines have that step copy them into LDS instead of forming them (same
// arithmetic, same bits). When pair 0 is instead taken by the 64-voxel
// line-pair instance (in table mode), the same buffer gets that instance's
// B operands for pair 0's step and offset (the same size per step).
template <bool F16>
__global__ __launch_bounds__(kLongBlock) void fhd_long_table_kernel(const float *__restrict__ packed, int nchunks,
                                                                    const int *__restrict__ cls,
                                                                    const int4 *__restrict__ patches, int64_t units,
                                                                    int patch_mode, int pair64_mode,
                                                                    const int *__restrict__ info,
                                                                    float4 *__restrict__ table)
{
    if (pair64_mode == kPatchTable && pair64_taken(cls, patches, units, 0, kPatchTable, patch_mode)) {
        patch_table_step<F16, kLineVox, 2>(packed, nchunks, patches, info, table);
        return;
    }
    if (info[0] == 0 || patch_taken(cls, patches, units, 0, patch_mode)) return;
    const float dx = __int_as_float(info[1]);
    const int sh = F16 ? read_amp_shift(info) : 0;
    const int lane = threadIdx.x & 63, quarter_k = lane >> 4, col = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t chunk = (int64_t)blockIdx.x * kLongGroup + quarter_k;
    float f[kFields][kChunk];
    if (chunk < nchunks) {
        const float4 *c = reinterpret_cast<const float4 *>(packed) + chunk * kChunkVec4;
#pragma unroll
        for (int q = 0; q < kChunkVec4; ++q) {
            const float4 t = c[q];
            const int field = (4 * q) / kChunk, at = (4 * q) % kChunk;
            f[field][at + 0] = t.x;
            f[field][at + 1] = t.y;
            f[field][at + 2] = t.z;
            f[field][at + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < kFields; ++q)
#pragma unroll
            for (int u = 0; u < kChunk; ++u) f[q][u] = 0.0f;
    }
    long_step_b<F16>(f, dx, wave, quarter_k, col, sh,
                     *reinterpret_cast<LongStepB *>(table + (int64_t)blockIdx.x * kLongStepVec4));
}

template <bool F16>
__global__ __launch_bounds__(kLongBlock) __attribute__((amdgpu_waves_per_eu(3))) void fhd_gather_long_lines_kernel(
    const float *__restrict__ packed, int nchunks, int splits, int pairs, const int *__restrict__ cls,
    const int4 *__restrict__ patches, int64_t units, int patch_mode, const int *__restrict__ info,
    const float4 *__restrict__ table, const float *__restrict__ x, const float *__restrict__ y,
    const float *__restrict__ z, float *__restrict__ out_r, float *__restrict__ out_i, int N)
{
    // workgroup -> (pair, split), split-major over the XCDs (see xcd_unit)
    const int64_t unit = xcd_unit(blockIdx.x, (int64_t)pairs * splits);
    const int64_t pair = unit % pairs;
    const int split = (int)(unit / pairs);
    if (cls[2 * pair] != kClassLongPair || patch_taken(cls, patches, units, pair / 2, patch_mode)) return;
    // Two step buffers, each a step's B operands and its four sample
    // chunks, used alternately: while the workgroup works on one step, the
    // next step's data is copied straight into the other buffer (buffer_load
    // ... lds). They are two variables, not one array, so the copy in flight
    // into one is known not to alias reads of the other, and no read waits
    // for a copy it does not need.
    __shared__ LongStep buf0, buf1;
    const float4 *src = reinterpret_cast<const float4 *>(packed);
    const int lane = threadIdx.x & 63, quarter_k = lane >> 4, col = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sh = F16 ? read_amp_shift(info) : 0;

    // line 16 wave + col of the pair (both units lie below N)
    const int64_t base = pair * kPairVox;
    const int64_t first = base + (int64_t)(16 * wave + col) * kLongLineVox;
    const float x0 = x[first], dx = x[first + 1] - x0, ly = y[first], lz = z[first];
    const float xc = __builtin_fmaf(0.5f * (float)(kLongLineVox - 1), dx, x0);
    // every line of the pair has the step dx (bitwise), so this is uniform;
    // the table exists when the first pair is a long pair outside the
    // line-pair instance's quads
    const bool use_table = table != nullptr && info[0] != 0 && !patch_taken(cls, patches, units, 0, patch_mode) &&
                           __float_as_uint(dx) == (unsigned)info[1];

    float4v prc[kLongTiles], pic[kLongTiles], pis[kLongTiles], prs[kLongTiles];
#pragma unroll
    for (int t = 0; t < kLongTiles; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            prc[t][r] = 0.0f;
            pic[t][r] = 0.0f;
            pis[t][r] = 0.0f;
            prs[t][r] = 0.0f;
        }

    // this split's chunks [c0, c1): steps g0 .. g0 + nsteps - 1 of the
    // sample stream (splits are whole stages of 32 chunks, so whole steps;
    // only the stream's last step may hold fewer than four chunks)
    int c0, c1;
    split_range<kLinesStageChunks>(nchunks, splits, split, &c0, &c1);
    const int nch = c1 > c0 ? c1 - c0 : 0;
    src += (int64_t)c0 * kChunkVec4;
    const int64_t total_vec4 = (int64_t)nch * kChunkVec4;
    const int nsteps = (nch + kLongGroup - 1) / kLongGroup;
    const int64_t table_vec4 = (((int64_t)nchunks + kLongGroup - 1) / kLongGroup) * kLongStepVec4;
    const int g0 = c0 / kLongGroup;

    // Copies step i of the split (its chunks and, from the table, its B
    // operands) into `dst`. Chunks past the split's end read as zeros
    // (amplitude 0: they add nothing), as do the table's past the stream's.
    auto copy_step = [&](int i, LongStep &dst, auto from_table) {
        issue_stage_load<kLongBlock, kLongStepChunkVec4>(src, total_vec4, i, dst.chunks);
        if constexpr (decltype(from_table)::value)
            issue_stage_load<kLongBlock, kLongStepVec4>(table, table_vec4, g0 + i,
                                                         reinterpret_cast<float4 *>(&dst.b));
    };

    // Step i of the split, in `cur`, whose copy was issued during the
    // previous step. The copies are shared work (lanes of every wave copy
    // parts of the buffer, and wave 0 alone the chunks), and a wave's own
    // wait covers only its own copies, so the step opens with every wave
    // waiting for its copies and a barrier: after it `cur` is whole in LDS,
    // and every wave has finished reading `next` (the previous step's
    // buffer), into which the copy of step i + 1 then goes. Without the
    // table, the workgroup forms the step's B operands into `cur` itself,
    // behind a second barrier.
    auto step = [&](int i, LongStep &cur, LongStep &next, auto from_table) {
        constexpr bool kTable = decltype(from_table)::value;
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();
        if (i + 1 < nsteps) copy_step(i + 1, next, from_table);
        float f[kFields][kChunk];
        load_chunk(cur.chunks + quarter_k * kChunkVec4, f);
        if constexpr (!kTable) {
            long_step_b<F16>(f, dx, wave, quarter_k, col, sh, cur.b);
            lds_barrier();
        }
        float ur[kChunk], ui[kChunk];
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
            const float p = __builtin_fmaf(f[0][k], xc, __builtin_fmaf(f[1][k], ly, __builtin_fmaf(f[2][k], lz, f[3][k])));
            ur[k] = __builtin_amdgcn_cosf(p);
            ui[k] = __builtin_amdgcn_sinf(p);
        }
        unsigned wa[4][4];
        split_parts<F16, kChunk>(ur, wa[0], wa[1]);
        split_parts<F16, kChunk>(ui, wa[2], wa[3]);
        const u32x4 arh = {wa[0][0], wa[0][1], wa[0][2], wa[0][3]}, arl = {wa[1][0], wa[1][1], wa[1][2], wa[1][3]};
        const u32x4 aih = {wa[2][0], wa[2][1], wa[2][2], wa[2][3]}, ail = {wa[3][0], wa[3][1], wa[3][2], wa[3][3]};
        // the products run at raised wave priority: a wave with MFMAs to
        // issue goes before the other waves' operand work, which keeps the
        // matrix core fed (measured 3 % faster than raising the operand
        // work instead, identical results)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < kLongTiles; ++t) {
            const u32x4 bch = cur.b[0][t][quarter_k][col], bcl = cur.b[1][t][quarter_k][col];
            const u32x4 bsh = cur.b[2][t][quarter_k][col], bsl = cur.b[3][t][quarter_k][col];
            prc[t] = mfma16<F16>(arh, bch, prc[t]);
            pic[t] = mfma16<F16>(aih, bch, pic[t]);
            pis[t] = mfma16<F16>(aih, bsh, pis[t]);
            prs[t] = mfma16<F16>(arh, bsh, prs[t]);
            prc[t] = mfma16<F16>(arh, bcl, prc[t]);
            pic[t] = mfma16<F16>(aih, bcl, pic[t]);
            pis[t] = mfma16<F16>(aih, bsl, pis[t]);
            prs[t] = mfma16<F16>(arh, bsl, prs[t]);
            prc[t] = mfma16<F16>(arl, bch, prc[t]);
            pic[t] = mfma16<F16>(ail, bch, pic[t]);
            pis[t] = mfma16<F16>(ail, bsh, pis[t]);
            prs[t] = mfma16<F16>(arl, bsh, prs[t]);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // steps in pairs, so each buffer is named statically
    auto walk = [&](auto from_table) {
        if (nsteps > 0) copy_step(0, buf0, from_table);
        int i = 0;
        for (; i + 1 < nsteps; i += 2) {
            step(i, buf0, buf1, from_table);
            step(i + 1, buf1, buf0, from_table);
        }
        if (i < nsteps) step(i, buf0, buf1, from_table);
    };
    if (use_table)
        walk(std::true_type{});
    else
        walk(std::false_type{});

    // unfold: row 4 (l / 16) + r of the wave's 16 lines, pair 16 t + l % 16
    float *dst_r = out_r + (int64_t)split * N, *dst_i = out_i + (int64_t)split * N;
#pragma unroll
    for (int t = 0; t < kLongTiles; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t line = base + (int64_t)(16 * wave + 4 * quarter_k + r) * kLongLineVox;
            const int j = 16 * t + col;
            dst_r[line + kLongPairs + j] = unscale<F16>(prc[t][r] - pis[t][r], sh);
            dst_i[line + kLongPairs + j] = unscale<F16>(pic[t][r] + prs[t][r], sh);
            dst_r[line + kLongPairs - 1 - j] = unscale<F16>(prc[t][r] + pis[t][r], sh);
            dst_i[line + kLongPairs - 1 - j] = unscale<F16>(pic[t][r] - prs[t][r], sh);
        }
}

// ---------------------------------------------------------------------------
// Line pairs on the matrix cores
// ---------------------------------------------------------------------------
// A quad -- two aligned long pairs of units, 16384 voxels, 128 lines of
// kLongLineVox -- whose lines, two by two, are one line and the same line
// moved by an offset d (lines 2i and 2i + 1; every pair of the quad with the
// same step dx and the same d, as the classification's records say: the
// rows of an x-fastest grid, with d one row along y, or, for rows of 256
// voxels, the second half of the row along x). The 256 voxels of a line
// pair sit symmetrically about
//
//   c = x_c(line 2i) + d / 2
//
// as 128 symmetric pairs: for j < 64,
//   pair j      (tiles 0-3)  c +- o, o = (j + 1/2) dx e_x + d / 2
//               (+: line 2i + 1's voxel 64 + j; -: line 2i's voxel 63 - j)
//   pair 64 + j (tiles 4-7)  c +- o, o = (j + 1/2) dx e_x - d / 2
//               (+: line 2i's voxel 64 + j; -: line 2i + 1's voxel 63 - j)
// so the sum is the long-line form's four real products with one U element
// per line pair instead of per line and 128 pair columns,
//
//   B_C[m, p] = a_m cos(2 pi k_m . o_p),  B_S[m, p] = a_m sin(2 pi k_m . o_p),
//   k_m . o_p = kx_m (2j + 1) dx / 2 +- k_m . d / 2,
//
// twice the matrix-core work per U element: the vector work per term (the
// U elements' phases, transcendentals and splits) is half the long-line
// form's, while the matrix cores run the same 12 FLOP per term.
//
// Four waves of 16 line pairs (waves 0 and 1 the quad's first unit pair,
// waves 2 and 3 its second), each with all 8 tiles of 16 pair columns: 96
// products of 16 x 16 x 32 per 32 samples. The B operands of a step are
// 32 KB (formed once per call into a table, or by the workgroup itself),
// double buffered with the step's four sample chunks: 66.8 KB of LDS, two
// workgroups (8 waves) per CU.
// The B operands of every step of the sample stream for quad 0's kind,
// step and offsets, formed once per call when quad 0 is taken by the
// line-pair instance (as 128-voxel line pairs or as four-line groups of
// 64-voxel lines): step g at table + g kPatchStepVec4. Quads of that kind
// with that step and those offsets copy them into LDS instead of forming
// them (same arithmetic, same bits).
template <bool F16>
__global__ __launch_bounds__(kPatchBlock) void fhd_patch_table_kernel(const float *__restrict__ packed, int nchunks,
                                                                      const int *__restrict__ cls,
                                                                      const int4 *__restrict__ patches,
                                                                      int64_t units, const int *__restrict__ info,
                                                                      float4 *__restrict__ table)
{
    if (patch_quad(cls, patches, units, 0))
        patch_table_step<F16, kLongLineVox, 2>(packed, nchunks, patches, info, table);
    else if (group64_quad(cls, patches, units, 0))
        patch_table_step<F16, kLineVox, 4>(packed, nchunks, patches, info, table);
}

// One workgroup of the line-pair instance for groups of SIDES lines of LINE
// voxels: group `group` (a quad for PairShape128 and GroupShape64, a unit
// pair for PairShape64), sample split `split` of `splits`. TABLE: the B
// operands come from `table`; else the workgroup forms them (the same
// arithmetic).
template <bool F16, bool TABLE, int LINE, int SIDES>
__device__ __forceinline__ void patch_group(const float *__restrict__ packed, int nchunks, int splits, int64_t group,
                                            int split, const int4 *__restrict__ rec, const int *__restrict__ info,
                                            const float4 *__restrict__ table, const float *__restrict__ x,
                                            const float *__restrict__ y, const float *__restrict__ z,
                                            float *__restrict__ out_r, float *__restrict__ out_i, int N,
                                            typename PatchShape<LINE, SIDES>::Step &buf0,
                                            typename PatchShape<LINE, SIDES>::Step &buf1)
{
    using Shape = PatchShape<LINE, SIDES>;
    using Step = typename Shape::Step;
    constexpr int kTiles = Shape::kTiles, kHalf = Shape::kHalf;
    const float4 *src = reinterpret_cast<const float4 *>(packed);
    const int lane = threadIdx.x & 63, quarter_k = lane >> 4, col = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sh = F16 ? read_amp_shift(info) : 0;
    const GroupOffsets o = group_offsets(rec);

    // row 16 wave + col of the group: its lines SIDES row .. + SIDES - 1,
    // centre x_c(line 0) + d / 2 (+ e / 2)
    const int64_t base = group * Shape::kGroupVox;
    const int64_t first = base + (int64_t)(SIDES * (16 * wave + col)) * LINE;
    const float x0 = x[first], ly = y[first], lz = z[first];
    float cx = __builtin_fmaf(0.5f * (float)(LINE - 1), o.dx, x0) + 0.5f * o.d[0];
    float cy = ly + 0.5f * o.d[1], cz = lz + 0.5f * o.d[2];
    if constexpr (SIDES == 4) {
        cx += 0.5f * o.e[0];
        cy += 0.5f * o.e[1];
        cz += 0.5f * o.e[2];
    }

    float4v prc[kTiles], pic[kTiles], pis[kTiles], prs[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            prc[t][r] = 0.0f;
            pic[t][r] = 0.0f;
            pis[t][r] = 0.0f;
            prs[t][r] = 0.0f;
        }

    int c0, c1;
    split_range<kLinesStageChunks>(nchunks, splits, split, &c0, &c1);
    const int nch = c1 > c0 ? c1 - c0 : 0;
    src += (int64_t)c0 * kChunkVec4;
    const int64_t total_vec4 = (int64_t)nch * kChunkVec4;
    const int nsteps = (nch + kLongGroup - 1) / kLongGroup;
    const int64_t table_vec4 = (((int64_t)nchunks + kLongGroup - 1) / kLongGroup) * Shape::kStepVec4;
    const int g0 = c0 / kLongGroup;

    auto copy_step = [&](int i, Step &dst) __attribute__((always_inline)) {
        issue_stage_load<kPatchBlock, kLongStepChunkVec4>(src, total_vec4, i, dst.chunks);
        if constexpr (TABLE)
            issue_stage_load<kPatchBlock, Shape::kStepVec4>(table, table_vec4, g0 + i,
                                                             reinterpret_cast<float4 *>(&dst.b));
    };

    // step i in `cur` (see the long-line instance's step for the order of
    // waits, barriers and copies)
    auto step = [&](int i, Step &cur, Step &next) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();
        if (i + 1 < nsteps) copy_step(i + 1, next);
        float f[kFields][kChunk];
        load_chunk(cur.chunks + quarter_k * kChunkVec4, f);
        if constexpr (!TABLE) {
            patch_step_b<F16, LINE, SIDES>(f, o, wave, quarter_k, col, sh, cur.b);
            lds_barrier();
        }
        float ur[kChunk], ui[kChunk];
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
            const float p = __builtin_fmaf(f[0][k], cx, __builtin_fmaf(f[1][k], cy, __builtin_fmaf(f[2][k], cz, f[3][k])));
            ur[k] = __builtin_amdgcn_cosf(p);
            ui[k] = __builtin_amdgcn_sinf(p);
        }
        unsigned wa[4][4];
        split_parts<F16, kChunk>(ur, wa[0], wa[1]);
        split_parts<F16, kChunk>(ui, wa[2], wa[3]);
        const u32x4 arh = {wa[0][0], wa[0][1], wa[0][2], wa[0][3]}, arl = {wa[1][0], wa[1][1], wa[1][2], wa[1][3]};
        const u32x4 aih = {wa[2][0], wa[2][1], wa[2][2], wa[2][3]}, ail = {wa[3][0], wa[3][1], wa[3][2], wa[3][3]};
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
            const u32x4 bch = cur.b[0][t][quarter_k][col], bcl = cur.b[1][t][quarter_k][col];
            const u32x4 bsh = cur.b[2][t][quarter_k][col], bsl = cur.b[3][t][quarter_k][col];
            prc[t] = mfma16<F16>(arh, bch, prc[t]);
            pic[t] = mfma16<F16>(aih, bch, pic[t]);
            pis[t] = mfma16<F16>(aih, bsh, pis[t]);
            prs[t] = mfma16<F16>(arh, bsh, prs[t]);
            prc[t] = mfma16<F16>(arh, bcl, prc[t]);
            pic[t] = mfma16<F16>(aih, bcl, pic[t]);
            pis[t] = mfma16<F16>(aih, bsl, pis[t]);
            prs[t] = mfma16<F16>(arh, bsl, prs[t]);
            prc[t] = mfma16<F16>(arl, bch, prc[t]);
            pic[t] = mfma16<F16>(ail, bch, pic[t]);
            pis[t] = mfma16<F16>(ail, bsh, pis[t]);
            prs[t] = mfma16<F16>(arl, bsh, prs[t]);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    if (nsteps > 0) copy_step(0, buf0);
    int i = 0;
    for (; i + 1 < nsteps; i += 2) {
        step(i, buf0, buf1);
        step(i + 1, buf1, buf0);
    }
    if (i < nsteps) step(i, buf0, buf1);

    // unfold: row 4 (l / 16) + r of the wave's 16 rows, column 16 t + l % 16
    // (side t / kSideTiles, j = 16 (t % kSideTiles) + l % 16): the voxel of
    // the side's line SIDES - 1 - side at kHalf + j and its reflection on
    // line `side` at kHalf - 1 - j
    float *dst_r = out_r + (int64_t)split * N, *dst_i = out_i + (int64_t)split * N;
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row0 = base + (int64_t)(SIDES * (16 * wave + 4 * quarter_k + r)) * LINE;
            const int side = t / Shape::kSideTiles;
            const int j = 16 * (t % Shape::kSideTiles) + col;
            const int64_t plus = row0 + (int64_t)(SIDES - 1 - side) * LINE + kHalf + j;
            const int64_t minus = row0 + (int64_t)side * LINE + kHalf - 1 - j;
            dst_r[plus] = unscale<F16>(prc[t][r] - pis[t][r], sh);
            dst_i[plus] = unscale<F16>(pic[t][r] + prs[t][r], sh);
            dst_r[minus] = unscale<F16>(prc[t][r] + pis[t][r], sh);
            dst_i[minus] = unscale<F16>(pic[t][r] - prs[t][r], sh);
        }
}

// The line-pair instance on quads: quads of long pairs whose lines pair up
// (128-voxel line pairs, splits_long sample splits, into out_long) and
// quads of 64-voxel lines in four-line groups (splits_lines splits, into
// out_lines; the reduce sums class kClassLines units over that many rows).
// TABLE: the B operands come from the table (mode kPatchTable, the quads of
// quad 0's kind that share its step and offsets); else the workgroup
// forms them (mode kPatchFormed, every quad; two separate instances, so
// the table form's register allocation does not carry the forming code's).
// The grid is quads x max(splits_long, splits_lines); a workgroup past its
// kind's split count returns.
template <bool F16, bool TABLE>
__global__ __launch_bounds__(kPatchBlock) __attribute__((amdgpu_waves_per_eu(2))) void fhd_gather_patch_kernel(
    const float *__restrict__ packed, int nchunks, int splits_long, int splits_lines, int64_t quads, int64_t units,
    const int *__restrict__ cls, const int4 *__restrict__ patches, const int *__restrict__ info,
    const float4 *__restrict__ table, const float *__restrict__ x, const float *__restrict__ y,
    const float *__restrict__ z, float *__restrict__ out_long_r, float *__restrict__ out_long_i,
    float *__restrict__ out_lines_r, float *__restrict__ out_lines_i, int N)
{
    // workgroup -> (quad, split), split-major over the XCDs (see xcd_unit)
    const int splits = splits_long > splits_lines ? splits_long : splits_lines;
    const int64_t unit = xcd_unit(blockIdx.x, quads * splits);
    const int64_t quad = unit % quads;
    const int split = (int)(unit / quads);
    constexpr int kMode = TABLE ? kPatchTable : kPatchFormed;
    // two step buffers used alternately, as in the long-line instance
    __shared__ PairShape128::Step buf0, buf1;
    if (patch_taken(cls, patches, units, quad, kMode)) {
        if (split >= splits_long) return;
        patch_group<F16, TABLE, kLongLineVox, 2>(packed, nchunks, splits_long, quad, split, patches + 4 * quad, info,
                                                 table, x, y, z, out_long_r, out_long_i, N, buf0, buf1);
    } else if (group64_taken(cls, patches, units, quad, kMode)) {
        if (split >= splits_lines) return;
        patch_group<F16, TABLE, kLineVox, 4>(packed, nchunks, splits_lines, quad, split, patches + 4 * quad, info,
                                             table, x, y, z, out_lines_r, out_lines_i, N, buf0, buf1);
    }
}

// The 64-voxel line-pair instance: unit pairs whose 64-voxel lines pair up
// (record flag 2 or 3, outside the quads taken as four-line groups in
// quad_mode), with the B table (16 KB per step, in the long-line table's
// buffer) for pair 0's step and offset, or formed.
template <bool F16, bool TABLE>
__global__ __launch_bounds__(kPatchBlock) __attribute__((amdgpu_waves_per_eu(3))) void fhd_gather_patch64_kernel(
    const float *__restrict__ packed, int nchunks, int splits, int64_t pairs, int64_t units, int quad_mode,
    const int *__restrict__ cls, const int4 *__restrict__ patches, const int *__restrict__ info,
    const float4 *__restrict__ table, const float *__restrict__ x, const float *__restrict__ y,
    const float *__restrict__ z, float *__restrict__ out_r, float *__restrict__ out_i, int N)
{
    const int64_t unit = xcd_unit(blockIdx.x, pairs * splits);
    const int64_t pair = unit % pairs;
    const int split = (int)(unit / pairs);
    if (!pair64_taken(cls, patches, units, pair, TABLE ? kPatchTable : kPatchFormed, quad_mode)) return;
    __shared__ PairShape64::Step buf0, buf1;
    patch_group<F16, TABLE, kLineVox, 2>(packed, nchunks, splits, pair, split, patches + 2 * pair, info, table, x,
                                         y, z, out_r, out_i, N, buf0, buf1);
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

// Workgroups of a gather instance that fit on one CU at once (register
// and LDS budget), asked of the runtime once per device and instance.
template <int KERNEL>
int blocks_per_cu(const void *kernel, int block)
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 4;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block, 0) != hipSuccess || n < 1) n = 4;
        cached[dev] = n;
    }
    return cached[dev];
}

int launch_classify(const float *x, const float *y, const float *z, int N, bool allow_lines, int *cls,
                    int *info, hipStream_t stream, bool amp_slots, const float *packed, int M, int4 *patches)
{
    const int64_t blocks = ((int64_t)N + kUnitVox - 1) / kUnitVox;
    const int64_t pairs = (blocks + 1) / 2;
    const int nchunks = amp_slots && M > 0 ? (int)(((int64_t)M + kChunk - 1) / kChunk) : 0;
    const int64_t grid = pairs + (amp_slots ? kAmpSlots : 0);
    fhd_classify_kernel<<<dim3((unsigned)grid), dim3(kClassifyBlock), 0, stream>>>(
        x, y, z, N, blocks, allow_lines ? 1 : 0, cls, info, reinterpret_cast<const float4 *>(packed), nchunks,
        patches);
    return launch_status("fhd_classify_kernel launch");
}

// The matrix-core instances of one split type (F16: fp16 parts, the
// default; else bf16 parts). Each writes rho itself when its split count
// is 1, else its partial sums. The line-pair and long-line instances share
// one split count (both take units of class kClassLongPair).
template <bool F16>
int launch_line_instances(const GatherPlan &g, const int *cls, const int4 *patches, const int *info,
                          float4 *long_table, float4 *patch_table, const float *x, const float *y, const float *z,
                          float *rho_r, float *rho_i, float *part_r, float *part_i, int N, const float *packed,
                          hipStream_t stream)
{
    int rc = FHD_OK;
    // a class needs whole units: with fewer than four (two, one) whole
    // units no unit can take the line-pair (long-line, line) instance,
    // which is not launched
    const bool quads = g.quads > 0, long_pairs = (int64_t)N >= 2 * (int64_t)kUnitVox, whole_unit = N >= kUnitVox;
    const bool direct_long = g.s_long == 1, direct_lines = g.s_lines == 1;
    if (quads && patch_table) {
        fhd_patch_table_kernel<F16><<<dim3((unsigned)g.steps), dim3(kPatchBlock), 0, stream>>>(
            packed, g.nchunks, cls, patches, g.blocks, info, patch_table);
        rc = launch_status("fhd_patch_table_kernel launch");
    }
    const int mode = !quads ? kPatchNone : patch_table ? kPatchTable : kPatchFormed;
    if (rc == FHD_OK && quads) {
        // quads of long pairs take the long pairs' split count, four-line
        // groups of 64-voxel lines the lines' one
        const int s_quad = g.s_long > g.s_lines ? g.s_long : g.s_lines;
        const dim3 grid((unsigned)(g.quads * s_quad));
        float *long_r = direct_long ? rho_r : part_r, *long_i = direct_long ? rho_i : part_i;
        float *lines_r = direct_lines ? rho_r : part_r, *lines_i = direct_lines ? rho_i : part_i;
        if (mode == kPatchTable) {
            TimedLaunch timed(F16 ? "fhd_gather_patch_kernel<true, true>" : "fhd_gather_patch_kernel<false, true>",
                              stream);
            fhd_gather_patch_kernel<F16, true><<<grid, dim3(kPatchBlock), 0, stream>>>(
                packed, g.nchunks, g.s_long, g.s_lines, g.quads, g.blocks, cls, patches, info, patch_table, x, y, z,
                long_r, long_i, lines_r, lines_i, N);
        } else {
            TimedLaunch timed(F16 ? "fhd_gather_patch_kernel<true, false>" : "fhd_gather_patch_kernel<false, false>",
                              stream);
            fhd_gather_patch_kernel<F16, false><<<grid, dim3(kPatchBlock), 0, stream>>>(
                packed, g.nchunks, g.s_long, g.s_lines, g.quads, g.blocks, cls, patches, info, nullptr, x, y, z,
                long_r, long_i, lines_r, lines_i, N);
        }
        rc = launch_status("fhd_gather_patch_kernel launch");
    }
    // the 64-voxel line-pair instance shares the long-line table's buffer
    const int mode64 = !long_pairs ? kPatchNone : long_table ? kPatchTable : kPatchFormed;
    if (rc == FHD_OK && long_pairs && long_table) {
        fhd_long_table_kernel<F16><<<dim3((unsigned)g.steps), dim3(kLongBlock), 0, stream>>>(
            packed, g.nchunks, cls, patches, g.blocks, mode, mode64, info, long_table);
        rc = launch_status("fhd_long_table_kernel launch");
    }
    if (rc == FHD_OK && long_pairs) {
        TimedLaunch timed(F16 ? "fhd_gather_long_lines_kernel<true>" : "fhd_gather_long_lines_kernel<false>", stream);
        fhd_gather_long_lines_kernel<F16><<<dim3((unsigned)(g.pairs * g.s_long)), dim3(kLongBlock), 0, stream>>>(
            packed, g.nchunks, g.s_long, (int)g.pairs, cls, patches, g.blocks, mode, info, long_table, x, y, z,
            direct_long ? rho_r : part_r, direct_long ? rho_i : part_i, N);
        rc = launch_status("fhd_gather_long_lines_kernel launch");
    }
    // the four-line groups, the 64-voxel line-pair and the line instances
    // share one split count (all take units of class kClassLines)
    if (rc == FHD_OK && long_pairs) {
        const dim3 grid((unsigned)(g.pairs * g.s_lines));
        float *out_r = direct_lines ? rho_r : part_r, *out_i = direct_lines ? rho_i : part_i;
        if (mode64 == kPatchTable) {
            TimedLaunch timed(F16 ? "fhd_gather_patch64_kernel<true, true>" : "fhd_gather_patch64_kernel<false, true>",
                              stream);
            fhd_gather_patch64_kernel<F16, true><<<grid, dim3(kPatchBlock), 0, stream>>>(
                packed, g.nchunks, g.s_lines, g.pairs, g.blocks, mode, cls, patches, info, long_table, x, y, z,
                out_r, out_i, N);
        } else {
            TimedLaunch timed(F16 ? "fhd_gather_patch64_kernel<true, false>"
                                  : "fhd_gather_patch64_kernel<false, false>",
                              stream);
            fhd_gather_patch64_kernel<F16, false><<<grid, dim3(kPatchBlock), 0, stream>>>(
                packed, g.nchunks, g.s_lines, g.pairs, g.blocks, mode, cls, patches, info, nullptr, x, y, z, out_r,
                out_i, N);
        }
        rc = launch_status("fhd_gather_patch64_kernel launch");
    }
    if (rc == FHD_OK && whole_unit) {
        TimedLaunch timed(F16 ? "fhd_gather_lines_kernel<true>" : "fhd_gather_lines_kernel<false>", stream);
        fhd_gather_lines_kernel<F16><<<dim3((unsigned)g.blocks, (unsigned)g.s_lines), dim3(kLinesBlock), 0,
                                        stream>>>(packed, g.nchunks, g.s_lines, cls, patches, g.blocks, mode64, mode,
                                                  info, x, y, z, direct_lines ? rho_r : part_r,
                                                  direct_lines ? rho_i : part_i, N);
        rc = launch_status("fhd_gather_lines_kernel launch");
    }
    return rc;
}

// rho_n = the sum over s < S of part[s N + n] in increasing s, where S is
// the split count of the instance that took voxel n's unit; nothing where
// S = 1 (that instance wrote rho itself).
__global__ __launch_bounds__(256) void fhd_reduce_units_kernel(const float *__restrict__ part_r,
                                                               const float *__restrict__ part_i,
                                                               const int *__restrict__ cls, int s_vec,
                                                               int s_lines, int s_long, int N,
                                                               float *__restrict__ out_r,
                                                               float *__restrict__ out_i)
{
    static_assert(kUnitVox % 256 == 0, "a workgroup lies in one unit");
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= N) return;
    const int c = cls[i / kUnitVox];
    const int splits = c == kClassLongPair ? s_long : c == kClassLines ? s_lines : s_vec;
    if (splits <= 1) return;
    // eight rows' loads in flight at a time, added in row order
    constexpr int kBatch = 8;
    float sr = 0.0f, si = 0.0f;
    int s = 0;
    for (; s + kBatch <= splits; s += kBatch) {
        float a[kBatch], b[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            a[k] = part_r[(int64_t)(s + k) * N + i];
            b[k] = part_i[(int64_t)(s + k) * N + i];
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            sr += a[k];
            si += b[k];
        }
    }
    for (; s < splits; ++s) {
        sr += part_r[(int64_t)s * N + i];
        si += part_i[(int64_t)s * N + i];
    }
    out_r[i] = sr;
    out_i[i] = si;
}

// Partial sums beyond the first instance's own rows: at most this many
// bytes. The first instance in the plan -- the long-line one where it can
// run, else the 64-voxel line one, else the vector ones -- takes the split
// count that balances it; the instances behind it (which take what the
// first one leaves: rows of other lengths, voxels off a grid) at most as
// many rows as the first one's or this budget allows.
constexpr size_t kPartBudget = (size_t)48 << 20;

GatherPlan plan_gather(int M, int N, int paths, bool with_table)
{
    GatherPlan g;
    g.paths = paths;
    g.nchunks = (int)(((int64_t)M + kChunk - 1) / kChunk);
    g.blocks = ((int64_t)N + kUnitVox - 1) / kUnitVox;
    g.pairs = (g.blocks + 1) / 2;
    const bool matrix_cores = paths != FHD_GATHER_VECTOR;
    const bool long_pairs = matrix_cores && (int64_t)N >= 2 * (int64_t)kUnitVox;
    const bool whole_unit = matrix_cores && N >= kUnitVox;
    g.quads = matrix_cores ? (int64_t)N / kQuadVox : 0;   // whole quads only
    // the long pairs' split count: sized for the line-pair instance where
    // quads can exist (on grids it takes every long pair), else for the
    // long-line one
    if (g.quads > 0)
        g.s_long = split_count(g.quads, g.nchunks,
                               blocks_per_cu<4>(reinterpret_cast<const void *>(fhd_gather_patch_kernel<true, true>),
                                                kPatchBlock),
                               kLinesStageChunks);
    else if (long_pairs)
        g.s_long = split_count(g.pairs, g.nchunks,
                               blocks_per_cu<1>(reinterpret_cast<const void *>(fhd_gather_long_lines_kernel<true>),
                                                kLongBlock),
                               kLinesStageChunks);
    // the lines' split count: sized for the 64-voxel line-pair instance
    // where unit pairs exist (on grids with rows of 64 it takes them all),
    // else for the line one
    if (long_pairs)
        g.s_lines = split_count(g.pairs, g.nchunks,
                                blocks_per_cu<5>(reinterpret_cast<const void *>(fhd_gather_patch64_kernel<true, true>),
                                                 kPatchBlock),
                                kLinesStageChunks);
    else if (whole_unit)
        g.s_lines = split_count(g.blocks, g.nchunks,
                                blocks_per_cu<3>(reinterpret_cast<const void *>(fhd_gather_lines_kernel<true>),
                                                 kLinesBlock),
                                kLinesStageChunks);
    // the vector instances split as the one-step ramp instance needs: at
    // its full occupancy when the units alone fill the CUs (the splits then
    // even out the last round), else to two workgroups per CU (measured:
    // more, each with fewer samples, take longer on grids of a few units)
    const int vec_occupancy =
        blocks_per_cu<2>(reinterpret_cast<const void *>(fhd_gather_kernel<kVox, true>), kBlock);
    const int vec_per_cu = g.blocks >= device_cus() || vec_occupancy < 2 ? vec_occupancy : 2;
    g.s_vec = split_count(g.blocks, g.nchunks, vec_per_cu, kVecGranuleChunks);
    if (matrix_cores) {
        const int first = long_pairs ? g.s_long : whole_unit ? g.s_lines : g.s_vec;
        const int64_t budget_rows = N > 0 ? (int64_t)(kPartBudget / (2 * sizeof(float) * (size_t)N)) : 1;
        const int cap = (int)(budget_rows > first ? (budget_rows < (1 << 20) ? budget_rows : (1 << 20)) : first);
        if (long_pairs && g.s_lines > cap) g.s_lines = cap;
        if (g.s_vec > cap) g.s_vec = cap;
    }
    g.splits = g.s_vec;
    if (g.s_long > g.splits) g.splits = g.s_long;
    if (g.s_lines > g.splits) g.splits = g.s_lines;
    // the workspace: the unit classes and the info words, the unit pairs'
    // line-pair records (two int4 each), the B tables of the long-line
    // (16 KB per 32 samples) and line-pair (32 KB) instances, then (splits
    // > 1) the partial sums
    g.patch_offset = ((size_t)g.blocks * sizeof(int) + kInfoWords * sizeof(int) + 15) / 16 * 16;
    g.cls_bytes = (g.patch_offset + (matrix_cores ? (size_t)g.pairs * 2 * sizeof(int4) : 0) + 255) / 256 * 256;
    g.steps = M > 0 && long_pairs && with_table ? ((int64_t)g.nchunks + kLongGroup - 1) / kLongGroup : 0;
    g.table_bytes = (size_t)g.steps * kLongStepVec4 * sizeof(float4);
    g.patch_table_bytes = g.quads > 0 ? (size_t)g.steps * kPatchStepVec4 * sizeof(float4) : 0;
    g.part_bytes = g.splits > 1 ? (size_t)g.splits * 2 * N * sizeof(float) : 0;
    return g;
}

int run_gather(const GatherPlan &g, char *work, const float *packed, int M, const float *x, const float *y,
               const float *z, float *rho_r, float *rho_i, int N, hipStream_t stream)
{
    const bool matrix_cores = g.paths != FHD_GATHER_VECTOR;
    int *cls = reinterpret_cast<int *>(work);
    int *info = cls + g.blocks;
    int4 *patches = matrix_cores ? reinterpret_cast<int4 *>(work + g.patch_offset) : nullptr;
    float4 *long_table = g.table_bytes > 0 ? reinterpret_cast<float4 *>(work + g.cls_bytes) : nullptr;
    float4 *patch_table =
        g.patch_table_bytes > 0 ? reinterpret_cast<float4 *>(work + g.cls_bytes + g.table_bytes) : nullptr;
    float *part_r = nullptr, *part_i = nullptr;
    if (g.splits > 1) {
        part_r = reinterpret_cast<float *>(work + g.cls_bytes + g.table_bytes + g.patch_table_bytes);
        part_i = part_r + (int64_t)g.splits * N;
    }
    // the fp16 products need the largest amplitude: the classification's
    // extra workgroups reduce it
    const bool f16 = g.paths == FHD_GATHER_ALL;
    int rc = launch_classify(x, y, z, N, matrix_cores, cls, info, stream, f16, packed, M, patches);
    // which launched instance splits (the others write rho themselves)
    bool any_split = false;
    if (rc == FHD_OK && matrix_cores) {
        rc = f16 ? launch_line_instances<true>(g, cls, patches, info, long_table, patch_table, x, y, z, rho_r,
                                               rho_i, part_r, part_i, N, packed, stream)
                 : launch_line_instances<false>(g, cls, patches, info, long_table, patch_table, x, y, z, rho_r,
                                                rho_i, part_r, part_i, N, packed, stream);
        any_split = ((int64_t)N >= 2 * (int64_t)kUnitVox && g.s_long > 1) || (N >= kUnitVox && g.s_lines > 1);
    }
    const dim3 grid((unsigned)g.blocks, (unsigned)g.s_vec);
    float *vec_r = g.s_vec > 1 ? part_r : rho_r, *vec_i = g.s_vec > 1 ? part_i : rho_i;
    any_split = any_split || g.s_vec > 1;
    // the one-step ramp class also needs a whole unit
    if (rc == FHD_OK && N >= kUnitVox) {
        TimedLaunch timed("fhd_gather_kernel<16, true>", stream);
        fhd_gather_kernel<kVox, true><<<grid, dim3(kBlock), 0, stream>>>(packed, g.nchunks, g.s_vec, cls, x, y, z,
                                                                          vec_r, vec_i, N);
        rc = launch_status("fhd_gather_kernel<one step> launch");
    }
    if (rc == FHD_OK) {
        TimedLaunch timed("fhd_gather_kernel<16, false>", stream);
        fhd_gather_kernel<kVox, false><<<grid, dim3(kBlock), 0, stream>>>(packed, g.nchunks, g.s_vec, cls, x, y,
                                                                           z, vec_r, vec_i, N);
        rc = launch_status("fhd_gather_kernel launch");
    }
    if (rc == FHD_OK && any_split) {
        fhd_reduce_units_kernel<<<dim3((unsigned)(((int64_t)N + 255) / 256)), dim3(256), 0, stream>>>(
            part_r, part_i, cls, g.s_vec, g.s_lines, g.s_long, N, rho_r, rho_i);
        rc = launch_status("fhd_reduce_units_kernel launch");
    }
    return rc;
}

int launch_gather(const float *packed, int M, const float *x, const float *y, const float *z,
                  float *rho_r, float *rho_i, int N, hipStream_t stream, int paths)
{
    if (N == 0) return FHD_OK;
    const GatherPlan g = plan_gather(M, N, paths, true);
    StreamBuffer buf(stream, kSlotGather);
    char *work = nullptr;
    int rc = buf.get(g.work_bytes(), &work);
    if (rc == FHD_OK) rc = run_gather(g, work, packed, M, x, y, z, rho_r, rho_i, N, stream);
    const int f = buf.finish();
    return rc != FHD_OK ? rc : f;
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

extern "C" int fhd_gather_paths(const void *packed, int M, const float *x, const float *y,
                                const float *z, float *rho_r, float *rho_i, int N, int paths,
                                void *stream)
{
    clear_error();
    if (M < 0) return fail(FHD_ERR_INVALID_ARG, "M < 0");
    if (N < 0) return fail(FHD_ERR_INVALID_ARG, "N < 0");
    if (!valid_paths(paths)) return fail_paths();
    if (N == 0) return FHD_OK;
    const int64_t nb = (int64_t)N * 4;
    const Span all[] = {{packed, M > 0 ? packed_bytes_for(M) : 0, "packed", 16},
                        {x, nb, "x"}, {y, nb, "y"}, {z, nb, "z"},
                        {rho_r, nb, "rho_r"}, {rho_i, nb, "rho_i"}};
    int rc = check_host_side(all, 6);
    if (rc == FHD_OK) rc = check_no_overlap(all, 6, 4);
    if (rc == FHD_OK) rc = check_device_spans(all, 6);
    if (rc != FHD_OK) return rc;
    return launch_gather((const float *)packed, M, x, y, z, rho_r, rho_i, N, (hipStream_t)stream, paths);
}

extern "C" int fhd_gather(const void *packed, int M, const float *x, const float *y, const float *z,
                          float *rho_r, float *rho_i, int N, void *stream)
{
    return fhd_gather_paths(packed, M, x, y, z, rho_r, rho_i, N, FHD_GATHER_ALL, stream);
}

extern "C" int fhd_compute_paths(const float *kx, const float *ky, const float *kz, const float *Dr,
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
    if (rc == FHD_OK) rc = check_device_spans(all, 10);
    if (rc != FHD_OK) return rc;

    hipStream_t s = (hipStream_t)stream;
    StreamBuffer buf(s, kSlotPacked);
    char *mem = nullptr;
    rc = buf.get(M > 0 ? (size_t)packed_bytes_for(M) : 0, &mem);
    float *packed = reinterpret_cast<float *>(mem);
    if (rc == FHD_OK && M > 0) rc = launch_pack(kx, ky, kz, Dr, Di, M, packed, s);
    if (rc == FHD_OK) rc = launch_gather(packed, M, x, y, z, rho_r, rho_i, N, s, paths);
    const int f = buf.finish();
    return rc != FHD_OK ? rc : f;
}

extern "C" int fhd_compute(const float *kx, const float *ky, const float *kz, const float *Dr,
                           const float *Di, const float *x, const float *y, const float *z,
                           float *rho_r, float *rho_i, int M, int N, void *stream)
{
    return fhd_compute_paths(kx, ky, kz, Dr, Di, x, y, z, rho_r, rho_i, M, N, FHD_GATHER_ALL, stream);
}
