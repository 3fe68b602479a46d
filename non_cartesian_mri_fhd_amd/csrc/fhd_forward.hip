// fhd_forward.hip -- the forward operator F (image to k-space) for gfx950.
//
// D_m = sum_n rho_n exp(-i 2 pi k_m . x_n)   (page "Case study -- iterative
// MRI reconstruction", section 17.2: F maps the image to k-space and F^H,
// section 17.3, is its adjoint; section 17.3.2 names F^H F, whose first
// half this is)
//
// The same two-kernel split as F^H D with the roles of voxels and samples
// swapped:
//
//  * fhd_forward_pack_kernel -- per-voxel pre-pass. Writes each voxel as the
//    record (x, y, z, s, a) with a = |rho| and s = -arg(rho) / (2 pi), so
//    that rho e^{-i 2 pi k.x} = a e^{-i 2 pi (k.x + s)}. Voxels on a line
//    in x at equal steps (checked exactly; every x-fastest grid) are
//    written instead as
//      - a 16-voxel ramp, when both chunks of an aligned chunk pair are one
//        ramp: the first chunk holds, for the voxel pairs 8 + j and 7 - j
//        about the centre, A_j = c_{8+j} + c_{7-j} and B_j = c_{8+j} - c_{7-j}
//        (c = conj(rho)) and (x0, dx/2, y, z), marked by -2 in the last
//        slot of the amplitude field; the second chunk holds zeros and -3;
//      - else an 8-voxel ramp chunk: Re rho_u, -Im rho_u, then
//        (x0, dx, y, z), marked by -1 (amplitudes are never negative).
//
//  * fhd_forward_gather_kernel -- one lane per kSamp consecutive samples,
//    no atomics; every lane walks the same voxel stream through LDS, a
//    chunk pair at a time, and accumulates conj(D). Per term of a general
//    chunk: p = kx x + ky y + kz z + s (3 FMA; 2 + 1/kSamp when all of a
//    lane's samples share kz, as within a plane of a stack of spirals --
//    bitwise identical), v_cos_f32, v_sin_f32, 2 FMA. A 16-voxel ramp is
//    e^{i 2 pi k.x_c} sum_j (A_j C_j + i B_j S_j) with the real factors
//    C_j, S_j = cos, sin(2 pi (j + 1/2) kx dx) from a three-term recurrence,
//    which the lane keeps for its samples while the step repeats (on a
//    grid they are formed once): 2 transcendentals and 40 other VALU
//    instructions per sample for 16 terms. Two samples per lane leave the
//    registers for those factors. An 8-voxel ramp chunk is a polynomial in z = e^{i 2 pi kx dx},
//    e^{i 2 pi k.x_0} sum_u conj(rho_u) z^u, by Horner's rule (4 FMA per
//    voxel) after 4 transcendentals per sample. The accumulated imaginary
//    part is negated once at the end (exact).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <string>
#include <type_traits>

#include "fhd_internal.h"

namespace fhd {
namespace {

constexpr int kSamp = 2;        // consecutive samples per lane (2, 1, 4, 8 measured: 2 best)
constexpr int kRampGroup = 2;   // samples per transcendental group on ramp chunks
static_assert(kSamp % kRampGroup == 0, "ramp groups tile a lane's samples");

__global__ __launch_bounds__(kPackBlock) void fhd_forward_pack_kernel(
    const float *__restrict__ x, const float *__restrict__ y, const float *__restrict__ z,
    const float *__restrict__ rho_r, const float *__restrict__ rho_i,
    float *__restrict__ packed, int N, int64_t N_pad, const int *__restrict__ gate)
{
    if (gate != nullptr && lines_form_ran(gate)) return;   // a matrix-core form took F
    // every lane stays to the end: the ramp test exchanges values between
    // the 8 lanes of a chunk (a chunk never straddles N_pad or a wave)
    const int64_t n = (int64_t)blockIdx.x * kPackBlock + threadIdx.x;
    const bool live = n < N;
    float fx = 0.0f, fy = 0.0f, fz = 0.0f, re = 0.0f, im = 0.0f;
    if (live) {
        fx = x[n];
        fy = y[n];
        fz = z[n];
        re = rho_r[n];
        im = rho_i[n];
    }
    const int lane = threadIdx.x & 63;
    // 16-voxel ramps: chunk pairs (2c, 2c + 1), 16 lanes of one wave
    const int base16 = lane & ~(2 * kChunk - 1), w = lane & (2 * kChunk - 1);
    const float x0 = __shfl(fx, base16), x1 = __shfl(fx, base16 + 1);
    const float y0 = __shfl(fy, base16), z0 = __shfl(fz, base16);
    const float dx = x1 - x0;
    const bool same = live && __float_as_uint(fy) == __float_as_uint(y0) &&
                      __float_as_uint(fz) == __float_as_uint(z0) && __builtin_isfinite(dx);
    const bool mine16 = same && __builtin_fmaf((float)w, dx, x0) == fx;
    const bool ramp16 = ((__ballot(mine16) >> base16) & 0xffffull) == 0xffffull;
    // 8-voxel ramps: single chunks
    const int base = lane & ~(kChunk - 1), u = lane & (kChunk - 1);
    const float x0c = __shfl(fx, base), x1c = __shfl(fx, base + 1);
    const float y0c = __shfl(fy, base), z0c = __shfl(fz, base);
    const float dxc = x1c - x0c;
    const bool mine = live && __float_as_uint(fy) == __float_as_uint(y0c) &&
                      __float_as_uint(fz) == __float_as_uint(z0c) && __builtin_isfinite(dxc) &&
                      __builtin_fmaf((float)u, dxc, x0c) == fx;
    const bool ramp = ((__ballot(mine) >> base) & 0xffull) == 0xffull;
    // pair sums of conj(rho) about the 16-voxel centre: slot j < 8 of the
    // pair's first chunk gets A_j = c_{8+j} + c_{7-j}, B_j = c_{8+j} - c_{7-j}
    const float hr = __shfl(re, base16 + kChunk + (w & (kChunk - 1)));
    const float hi = -__shfl(im, base16 + kChunk + (w & (kChunk - 1)));
    const float lr = __shfl(re, base16 + kChunk - 1 - (w & (kChunk - 1)));
    const float li = -__shfl(im, base16 + kChunk - 1 - (w & (kChunk - 1)));
    if (n >= N_pad) return;
    if (ramp16) {
        if (w < kChunk) {
            const float geo = w == 0 ? x0 : w == 1 ? 0.5f * dx : w == 2 ? y0 : w == 3 ? z0 : 0.0f;
            store_record(packed, n, hr + lr, hi + li, hr - lr, hi - li, w == kChunk - 1 ? -2.0f : geo);
        } else {
            // the pair's second chunk carries nothing: zero amplitudes and a
            // marker, so that it adds 0 however it is read
            store_record(packed, n, 0.0f, 0.0f, 0.0f, 0.0f, w == 2 * kChunk - 1 ? -3.0f : 0.0f);
        }
    } else if (ramp) {
        const float geo = u == 0 ? x0c : u == 1 ? dxc : u == 2 ? y0c : u == 3 ? z0c : 0.0f;
        store_record(packed, n, re, -im, geo, 0.0f, u == kChunk - 1 ? -1.0f : 0.0f);
    } else {
        float s = 0.0f, amp = 0.0f;
        if (live) {
            amp = (float)hypot((double)re, (double)im);
            s = (float)(-atan2((double)im, (double)re) * (0.5 / M_PI));   // [-0.5, 0.5] revolutions
        }
        store_record(packed, n, fx, fy, fz, s, amp);
    }
}

// A ramp chunk: acc_j += e^{i 2 pi k_j.x_0} sum_u c_u z_j^u with
// c_u = conj(rho_u), z_j = e^{i 2 pi kx_j dx} (Horner, highest u first).
template <int S>
__device__ __forceinline__ void accumulate_ramp_chunk(const float (&f)[kFields][kChunk],
                                                      const float (&kx)[S], const float (&ky)[S],
                                                      const float (&kz)[S], float (&acc_r)[S],
                                                      float (&acc_i)[S])
{
    const float x0 = f[2][0], dx = f[2][1], y = f[2][2], z = f[2][3];
    // the transcendentals of kRampGroup samples issue as one group at raised
    // wave priority (2 measured best)
#pragma unroll
    for (int j0 = 0; j0 < S; j0 += kRampGroup) {
        float p[kRampGroup], d[kRampGroup], er[kRampGroup], ei[kRampGroup], zr[kRampGroup],
            zi[kRampGroup];
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            const int j = j0 + t;
            p[t] = __builtin_fmaf(kx[j], x0, __builtin_fmaf(ky[j], y, kz[j] * z));
            d[t] = kx[j] * dx;
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            er[t] = __builtin_amdgcn_cosf(p[t]);
            ei[t] = __builtin_amdgcn_sinf(p[t]);
            zr[t] = __builtin_amdgcn_cosf(d[t]);
            zi[t] = __builtin_amdgcn_sinf(d[t]);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            const int j = j0 + t;
            float hr = f[0][kChunk - 1], hi = f[1][kChunk - 1];
#pragma unroll
            for (int u = kChunk - 2; u >= 0; --u) {
                const float tr = __builtin_fmaf(hr, zr[t], __builtin_fmaf(-hi, zi[t], f[0][u]));
                const float ti = __builtin_fmaf(hr, zi[t], __builtin_fmaf(hi, zr[t], f[1][u]));
                hr = tr;
                hi = ti;
            }
            acc_r[j] = __builtin_fmaf(er[t], hr, __builtin_fmaf(-ei[t], hi, acc_r[j]));
            acc_i[j] = __builtin_fmaf(er[t], hi, __builtin_fmaf(ei[t], hr, acc_i[j]));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// A 16-voxel ramp (a chunk pair): with c_u = conj(rho_u), centre
// x_c = x_0 + 7.5 dx, h = kx dx / 2 and theta_j = 2 pi (2j + 1) h,
//   sum_u c_u e^{i 2 pi k.x_u} = e^{i 2 pi k.x_c} sum_j (A_j C_j + i B_j S_j)
// with A_j = c_{8+j} + c_{7-j}, B_j = c_{8+j} - c_{7-j} (written by the
// pre-pass), C_j = cos theta_j and S_j = sin theta_j by the three-term
// recurrence from cos and sin of 2 pi h. C_j, S_j and h depend on the
// sample and the step alone, so the lane keeps them for its samples
// (RampFactors) and forms them again only when a ramp's step differs from
// the last one (on a grid: once). Per sample and ramp then: 2
// transcendentals and 40 other VALU instructions for 16 terms.
template <int S>
struct RampFactors {
    float hdx;                       // the step they were formed for (NaN: none yet)
    float h[S], c[S][kChunk], s[S][kChunk];
};

template <int S>
__device__ __forceinline__ void ramp_factors(float hdx, const float (&kx)[S], RampFactors<S> &rf)
{
    rf.hdx = hdx;
#pragma unroll
    for (int j = 0; j < S; ++j) {
        const float h = kx[j] * hdx;
        const float c1 = __builtin_amdgcn_cosf(h), s1 = __builtin_amdgcn_sinf(h);
        const float k2 = __builtin_fmaf(-4.0f * s1, s1, 2.0f);   // 2 cos(4 pi h)
        float cp = c1, sp = -s1, c = c1, sn = s1;
        rf.h[j] = h;
#pragma unroll
        for (int q = 0; q < kChunk; ++q) {
            if (q > 0) {
                const float cn = __builtin_fmaf(k2, c, -cp), snn = __builtin_fmaf(k2, sn, -sp);
                cp = c;
                sp = sn;
                c = cn;
                sn = snn;
            }
            rf.c[j][q] = c;
            rf.s[j][q] = sn;
        }
    }
}

template <int S>
__device__ __forceinline__ void accumulate_ramp_pair(const float4 *ch, const float (&kx)[S],
                                                     const float (&ky)[S], const float (&kz)[S],
                                                     RampFactors<S> &rf, float (&acc_r)[S],
                                                     float (&acc_i)[S])
{
    constexpr int P = kChunk;   // voxel pairs
    float f[kFields][kChunk];
    load_chunk(ch, f);
    const float(&ar)[P] = f[0];
    const float(&ai)[P] = f[1];
    const float(&br)[P] = f[2];
    const float(&bi)[P] = f[3];
    const float x0 = f[4][0], hdx = f[4][1], y = f[4][2], z = f[4][3];
    // every lane reads the same pair: a scalar branch
    if (__builtin_bit_cast(unsigned, hdx) != __builtin_bit_cast(unsigned, rf.hdx))
        ramp_factors<S>(hdx, kx, rf);
#pragma unroll
    for (int j0 = 0; j0 < S; j0 += kRampGroup) {
        float pc[kRampGroup], er[kRampGroup], ei[kRampGroup];
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            const int j = j0 + t;
            pc[t] = __builtin_fmaf(2.0f * kChunk - 1.0f, rf.h[j],
                                   __builtin_fmaf(kx[j], x0, __builtin_fmaf(ky[j], y, kz[j] * z)));
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            er[t] = __builtin_amdgcn_cosf(pc[t]);
            ei[t] = __builtin_amdgcn_sinf(pc[t]);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kRampGroup; ++t) {
            const int j = j0 + t;
            float pr = 0.0f, pi = 0.0f;
#pragma unroll
            for (int q = 0; q < P; ++q) {
                // P += A_q C_q + i B_q S_q
                pr = __builtin_fmaf(ar[q], rf.c[j][q], __builtin_fmaf(-bi[q], rf.s[j][q], pr));
                pi = __builtin_fmaf(ai[q], rf.c[j][q], __builtin_fmaf(br[q], rf.s[j][q], pi));
            }
            acc_r[j] = __builtin_fmaf(er[t], pr, __builtin_fmaf(-ei[t], pi, acc_r[j]));
            acc_i[j] = __builtin_fmaf(er[t], pi, __builtin_fmaf(ei[t], pr, acc_i[j]));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Accumulate one chunk of kChunk voxels into a lane's S samples.
// SHARED: all S samples have the same kz (checked by the caller).
template <int S, bool SHARED>
__device__ __forceinline__ void accumulate_voxels(const float4 *ch, const float (&kx)[S],
                                                  const float (&ky)[S], const float (&kz)[S],
                                                  float (&acc_r)[S], float (&acc_i)[S])
{
    float f[kFields][kChunk];
    load_chunk(ch, f);
    // every lane reads the same chunk: a scalar branch
    const float mark = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                      __builtin_bit_cast(int, f[4][kChunk - 1])));
    if (mark < 0.0f) {
        accumulate_ramp_chunk<S>(f, kx, ky, kz, acc_r, acc_i);
        return;
    }
    const float(&vx)[kChunk] = f[0];
    const float(&vy)[kChunk] = f[1];
    const float(&vz)[kChunk] = f[2];
    const float(&vs)[kChunk] = f[3];
    const float(&amp)[kChunk] = f[4];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
        float p[S], c[S], sn[S];
        if constexpr (SHARED) {
            const float q = __builtin_fmaf(kz[0], vz[u], vs[u]);
#pragma unroll
            for (int j = 0; j < S; ++j) p[j] = __builtin_fmaf(kx[j], vx[u], __builtin_fmaf(ky[j], vy[u], q));
        } else {
#pragma unroll
            for (int j = 0; j < S; ++j)
                p[j] = __builtin_fmaf(kx[j], vx[u],
                                      __builtin_fmaf(ky[j], vy[u], __builtin_fmaf(kz[j], vz[u], vs[u])));
        }
        // transcendentals as one group at raised wave priority, so the
        // waves' FMA runs coincide and pair (as in the F^H D gather)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int j = 0; j < S; ++j) c[j] = __builtin_amdgcn_cosf(p[j]);
#pragma unroll
        for (int j = 0; j < S; ++j) sn[j] = __builtin_amdgcn_sinf(p[j]);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < S; ++j) {
            acc_r[j] = __builtin_fmaf(amp[u], c[j], acc_r[j]);
            acc_i[j] = __builtin_fmaf(amp[u], sn[j], acc_i[j]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Split s = blockIdx.y of `splits` takes its share of the voxel stream and
// writes D (splits == 1) or its partial sums at out + s*M.
template <int S>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void fhd_forward_gather_kernel(
    const float *__restrict__ packed, int nchunks, int splits,
    const float *__restrict__ kx, const float *__restrict__ ky, const float *__restrict__ kz,
    float *__restrict__ out_r, float *__restrict__ out_i, int M, const int *__restrict__ gate)
{
    if (gate != nullptr && lines_form_ran(gate)) return;   // a matrix-core form took F
    __shared__ float4 stage[2][kStageVec4];
    const float4 *src = reinterpret_cast<const float4 *>(packed);

    // lane l of workgroup b owns samples (b*kBlock + l)*S + j, j < S
    const int64_t m0 = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * S;
    float sx[S], sy[S], sz[S], acc_r[S], acc_i[S];
#pragma unroll
    for (int j = 0; j < S; ++j) {
        const int64_t m = m0 + j;
        const bool live = m < M;
        sx[j] = live ? kx[m] : 0.0f;
        sy[j] = live ? ky[m] : 0.0f;
        sz[j] = live ? kz[m] : 0.0f;
        acc_r[j] = 0.0f;
        acc_i[j] = 0.0f;
    }
#pragma unroll
    for (int j = 1; j < S; ++j)
        if (m0 + j >= M) {
            sx[j] = sx[0];
            sy[j] = sy[0];
            sz[j] = sz[0];
        }
    bool same_kz = true;
#pragma unroll
    for (int j = 1; j < S; ++j) same_kz = same_kz && __float_as_uint(sz[j]) == __float_as_uint(sz[0]);
    const bool shared = __syncthreads_and(same_kz);

    RampFactors<S> rf;
    rf.hdx = __builtin_nanf("");
    int c0, c1;
    split_range(nchunks, splits, blockIdx.y, &c0, &c1);
    // chunk pairs (2c, 2c + 1): stages and splits start at even chunks, so a
    // 16-voxel ramp's two chunks always arrive together
    auto pair = [&](const float4 *ch, int count, auto shared_kz) {
        // every lane reads the same chunk: a scalar branch
        const float mark = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(
                                                          int, reinterpret_cast<const float *>(ch)[kFields * kChunk - 1])));
        if (count == 2 && mark == -2.0f) {
            accumulate_ramp_pair<S>(ch, sx, sy, sz, rf, acc_r, acc_i);
            return;
        }
        for (int c = 0; c < count; ++c)
            accumulate_voxels<S, decltype(shared_kz)::value>(ch + c * kChunkVec4, sx, sy, sz, acc_r, acc_i);
    };
    if (shared)
        stream_chunk_groups<2>(src, c0, c1, stage, [&](const float4 *ch, int count) {
            pair(ch, count, std::true_type());
        });
    else
        stream_chunk_groups<2>(src, c0, c1, stage, [&](const float4 *ch, int count) {
            pair(ch, count, std::false_type());
        });

    float *dst_r = out_r + (int64_t)blockIdx.y * M, *dst_i = out_i + (int64_t)blockIdx.y * M;
#pragma unroll
    for (int j = 0; j < S; ++j) {
        const int64_t m = m0 + j;
        if (m < M) {
            dst_r[m] = acc_r[j];
            dst_i[m] = -acc_i[j];
        }
    }
}

// ---------------------------------------------------------------------------
// F on lines of voxels, on the matrix cores
// ---------------------------------------------------------------------------
// When the voxels are lines of kLongLineVox along x with one step dx (every
// aligned pair of units of class kClassLongPair, one step throughout), the
// voxels of a line pair up about its centre x_c = x_0 + (kLongLineVox - 1)
// dx / 2, and with rho+_j, rho-_j the voxels at x_c +- (j + 1/2) dx,
//
//   D_m = sum_l conj(V[l, m]) T[l, m],   V = exp(i 2 pi k_m . x_c(l))
//   T[l, m] = sum_j (P_j C_j(m) - i Q_j S_j(m)),
//   P_j = rho+_j + rho-_j, Q_j = rho+_j - rho-_j,
//   C_j, S_j = cos, sin(2 pi (2j + 1) kx_m dx / 2),
//
// i.e. T_re = sum_K A_re[l, K] B[K, m], T_im = sum_K A_im[l, K] B[K, m]
// over K = (j, cos part) then (j, sin part), with A_re = [P_r | Q_i],
// A_im = [P_i | -Q_r], B = [C | S]: two real products with K = 2 x 64, in
// split bf16 (three bf16 products per fp32 product, fp32 accumulation), 6
// bf16 multiply-adds per term; then per line and sample one phasor (2
// transcendentals for 128 terms) and a complex multiply-add.
//
// fhd_forward_lines_pack_kernel forms A once per call, in operand order,
// in tiles of 16 lines; fhd_forward_lines_kernel gives each wave 32
// samples (two 16-sample columns of v_mfma_f32_16x16x32_bf16, layout:
// lane l supplies A[l % 16][8 (l / 16) + i] and B[8 (l / 16) + i][l % 16],
// accumulator register r holds C[4 (l / 16) + r][l % 16]), keeps their B
// operands in registers, and walks the tiles of its split through LDS.
constexpr int kFwdBlock = 256;                          // 4 waves
constexpr int kFwdTileLines = 16;
constexpr int kFwdPairs = kLongLineVox / 2;             // 64
constexpr int kFwdKSteps = 2 * kFwdPairs / 32;          // 4 products of K = 32
constexpr int kFwdOpsVec4 = kFwdKSteps * 4 * 64;        // [k step][re hi, re lo, im hi, im lo][lane]
constexpr int kFwdTileVec4 = kFwdOpsVec4 + kFwdTileLines;   // then (x_c, y, z, 0) per line
constexpr int kFwdTileVox = kFwdTileLines * kLongLineVox;
constexpr int kFwdColumns = 2;                          // 16-sample columns per wave
constexpr int kFwdBlockSamples = (kFwdBlock / 64) * 16 * kFwdColumns;
constexpr int kFwdStageRegs = (kFwdTileVec4 + kFwdBlock - 1) / kFwdBlock;
static_assert(kFwdBlock / 64 == kFwdKSteps, "one pre-pass wave per k step");
static_assert((2 * kUnitVox) % kFwdTileVox == 0, "tiles tile a pair of units");

// One workgroup per tile of 16 lines: wave s forms k step s of the A
// operands (lane l: line l % 16, K = 32 s + 8 (l / 16) + i), the first 16
// lanes of wave 0 the lines' centres; a line that breaks the rule (its unit
// pair not of class kClassLongPair, or a step other than the first pair's)
// sets info[2], and the vector form then takes F. F16: the operands are
// split into fp16 parts, each line's scaled by a power of two 2^sh (with
// the line's largest |value| times 2^sh in [2^14, 2^15): amp_shift), and
// sh is stored in the line's centre record for the gather to undo.
template <bool F16>
__global__ __launch_bounds__(kFwdBlock) void fhd_forward_lines_pack_kernel(
    const float *__restrict__ x, const float *__restrict__ y, const float *__restrict__ z,
    const float *__restrict__ rho_r, const float *__restrict__ rho_i, const int *__restrict__ cls,
    int *__restrict__ info, u32x4 *__restrict__ tiles)
{
    if (pairs_form_ran(info)) return;   // the line-pair form took F
    const int s = threadIdx.x >> 6, lane = threadIdx.x & 63, row = lane & 15, quarter_k = lane >> 4;
    const int64_t base = ((int64_t)blockIdx.x * kFwdTileLines + row) * kLongLineVox;
    const bool sine = s >= kFwdKSteps / 2;   // K >= 64: the S part
    float re[kChunk], im[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        const int j = (32 * s + 8 * quarter_k + i) % kFwdPairs;
        const int64_t up = base + kFwdPairs + j, dn = base + kFwdPairs - 1 - j;
        const float ur = rho_r[up], ui = rho_i[up], dr = rho_r[dn], di = rho_i[dn];
        re[i] = sine ? ui - di : ur + dr;      // Q_i | P_r
        im[i] = sine ? dr - ur : ui + di;      // -Q_r | P_i
    }
    int sh = 0;
    if constexpr (F16) {
        // the line's largest magnitude: over the lane's values, the wave's
        // four lanes of the row, then the four waves (LDS)
        __shared__ unsigned row_max[kFwdKSteps][kFwdTileLines];
        unsigned m = 0u;
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            const unsigned a = __float_as_uint(re[i]) & 0x7fffffffu, b = __float_as_uint(im[i]) & 0x7fffffffu;
            m = a > m ? a : m;
            m = b > m ? b : m;
        }
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {
            const unsigned t = (unsigned)__shfl_xor((int)m, o);
            m = t > m ? t : m;
        }
        if (quarter_k == 0) row_max[s][row] = m;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kFwdKSteps; ++w) m = row_max[w][row] > m ? row_max[w][row] : m;
        sh = amp_shift(m);
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            re[i] = __builtin_ldexpf(re[i], sh);
            im[i] = __builtin_ldexpf(im[i], sh);
        }
    }
    unsigned rh[4], rl[4], ih[4], il[4];
    split_parts<F16, kChunk>(re, rh, rl);
    split_parts<F16, kChunk>(im, ih, il);
    u32x4 *t = tiles + (int64_t)blockIdx.x * kFwdTileVec4 + s * 4 * 64 + lane;
    t[0 * 64] = (u32x4){rh[0], rh[1], rh[2], rh[3]};
    t[1 * 64] = (u32x4){rl[0], rl[1], rl[2], rl[3]};
    t[2 * 64] = (u32x4){ih[0], ih[1], ih[2], ih[3]};
    t[3 * 64] = (u32x4){il[0], il[1], il[2], il[3]};
    if (s == 0 && quarter_k == 0) {
        const float x0 = x[base], dx = x[base + 1] - x0;
        const float xc = __builtin_fmaf(0.5f * (float)(kLongLineVox - 1), dx, x0);
        tiles[(int64_t)blockIdx.x * kFwdTileVec4 + kFwdOpsVec4 + row] =
            (u32x4){__float_as_uint(xc), __float_as_uint(y[base]), __float_as_uint(z[base]), (unsigned)sh};
        const bool ok = info[0] != 0 && cls[base / kUnitVox] == kClassLongPair &&
                        __float_as_uint(dx) == (unsigned)info[1];
        if (!ok) atomicOr(&info[2], 1);
    }
}

// Workgroup b, split s: samples b kFwdBlockSamples .. + 127 (wave w the 32
// from 32 w; lane l the sample l % 16 of each of its two columns, rows 4
// (l / 16) .. + 3 of each tile), tiles of split s of the line stream; writes
// D (splits == 1) or its partial sums at out + s M.
template <bool F16>
__global__ __launch_bounds__(kFwdBlock) __attribute__((amdgpu_waves_per_eu(3))) void fhd_forward_lines_kernel(
    const u32x4 *__restrict__ tiles, int ntiles, int splits, const int *__restrict__ info,
    const float *__restrict__ kx, const float *__restrict__ ky, const float *__restrict__ kz,
    float *__restrict__ out_r, float *__restrict__ out_i, int M)
{
    // the line-pair form took F, or the vector form takes it
    if (pairs_form_ran(info) || !lines_form_ran(info)) return;
    __shared__ u32x4 stage[2][kFwdTileVec4];
    const int lane = threadIdx.x & 63, quarter_k = lane >> 4, col = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float hdx = 0.5f * __int_as_float(info[1]);

    int64_t m[kFwdColumns];
    float skx[kFwdColumns], sky[kFwdColumns], skz[kFwdColumns];
#pragma unroll
    for (int t = 0; t < kFwdColumns; ++t) {
        m[t] = (int64_t)blockIdx.x * kFwdBlockSamples + wave * 16 * kFwdColumns + t * 16 + col;
        const bool live = m[t] < M;   // samples past M compute with k = 0 and are not stored
        skx[t] = live ? kx[m[t]] : 0.0f;
        sky[t] = live ? ky[m[t]] : 0.0f;
        skz[t] = live ? kz[m[t]] : 0.0f;
    }
    // B operands (cos and sin, |B| <= 1: no scaling), held for the whole
    // walk: K = 32 s + 8 (l / 16) + i, pair j = K % 64, cos (K < 64) or sin
    u32x4 bh[kFwdColumns][kFwdKSteps], bl[kFwdColumns][kFwdKSteps];
#pragma unroll
    for (int t = 0; t < kFwdColumns; ++t)
#pragma unroll
        for (int s = 0; s < kFwdKSteps; ++s) {
            float v[kChunk];
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                const int j = (32 * s + 8 * quarter_k + i) % kFwdPairs;
                const float a = skx[t] * ((float)(2 * j + 1) * hdx);
                v[i] = s < kFwdKSteps / 2 ? __builtin_amdgcn_cosf(a) : __builtin_amdgcn_sinf(a);
            }
            unsigned h[4], l[4];
            split_parts<F16, kChunk>(v, h, l);
            bh[t][s] = (u32x4){h[0], h[1], h[2], h[3]};
            bl[t][s] = (u32x4){l[0], l[1], l[2], l[3]};
        }

    float dr[kFwdColumns], di[kFwdColumns];
#pragma unroll
    for (int t = 0; t < kFwdColumns; ++t) {
        dr[t] = 0.0f;
        di[t] = 0.0f;
    }
    const int per = (ntiles + splits - 1) / splits;
    const int t0 = min(ntiles, (int)blockIdx.y * per), t1 = min(ntiles, t0 + per);

    // tiles reach LDS through registers: loaded at the start of the
    // previous tile, stored at its end
    u32x4 sreg[kFwdStageRegs];
    auto load_tile = [&](int tau) {
#pragma unroll
        for (int k = 0; k < kFwdStageRegs; ++k) {
            const int i = k * kFwdBlock + threadIdx.x;
            if (i < kFwdTileVec4) sreg[k] = tiles[(int64_t)tau * kFwdTileVec4 + i];
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int k = 0; k < kFwdStageRegs; ++k) {
            const int i = k * kFwdBlock + threadIdx.x;
            if (i < kFwdTileVec4) stage[buf][i] = sreg[k];
        }
    };
    if (t0 < t1) {
        load_tile(t0);
        store_tile(0);
    }
    lds_barrier();
    int b = 0;
    for (int tau = t0; tau < t1; ++tau) {
        const bool more = tau + 1 < t1;   // uniform
        if (more) load_tile(tau + 1);
        float4v tre[kFwdColumns], tim[kFwdColumns];
#pragma unroll
        for (int t = 0; t < kFwdColumns; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                tre[t][r] = 0.0f;
                tim[t][r] = 0.0f;
            }
        // the products at raised wave priority, the phasor work after them
        // at normal priority: a wave with MFMAs to issue goes first (measured
        // 1-3 % faster than the other way round, identical results)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < kFwdKSteps; ++s) {
            const u32x4 *op = &stage[b][s * 4 * 64 + lane];
            const u32x4 arh = op[0 * 64], arl = op[1 * 64], aih = op[2 * 64], ail = op[3 * 64];
#pragma unroll
            for (int t = 0; t < kFwdColumns; ++t) {
                tre[t] = mfma16<F16>(arh, bh[t][s], tre[t]);
                tim[t] = mfma16<F16>(aih, bh[t][s], tim[t]);
                tre[t] = mfma16<F16>(arh, bl[t][s], tre[t]);
                tim[t] = mfma16<F16>(aih, bl[t][s], tim[t]);
                tre[t] = mfma16<F16>(arl, bh[t][s], tre[t]);
                tim[t] = mfma16<F16>(ail, bh[t][s], tim[t]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // D += conj(V) T for rows 4 (l / 16) + r, with V of the row's centre
        // (scaled by the row's 2^-sh in the fp16 form)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const u32x4 c = stage[b][kFwdOpsVec4 + 4 * quarter_k + r];
            const float xc = __uint_as_float(c.x), ly = __uint_as_float(c.y), lz = __uint_as_float(c.z);
#pragma unroll
            for (int t = 0; t < kFwdColumns; ++t) {
                const float p = __builtin_fmaf(skx[t], xc, __builtin_fmaf(sky[t], ly, skz[t] * lz));
                const float vc = unscale<F16>(__builtin_amdgcn_cosf(p), (int)c.w);
                const float vs = unscale<F16>(__builtin_amdgcn_sinf(p), (int)c.w);
                dr[t] = __builtin_fmaf(vc, tre[t][r], __builtin_fmaf(vs, tim[t][r], dr[t]));
                di[t] = __builtin_fmaf(vc, tim[t][r], __builtin_fmaf(-vs, tre[t][r], di[t]));
            }
        }
        // the other buffer was last read before the previous barrier
        if (more) store_tile(b ^ 1);
        lds_barrier();
        b ^= 1;
    }

    // each column's four row groups (lanes col + 16 q) add up
#pragma unroll
    for (int t = 0; t < kFwdColumns; ++t) {
        dr[t] += __shfl_xor(dr[t], 16);
        di[t] += __shfl_xor(di[t], 16);
        dr[t] += __shfl_xor(dr[t], 32);
        di[t] += __shfl_xor(di[t], 32);
    }
    if (quarter_k == 0) {
        float *dst_r = out_r + (int64_t)blockIdx.y * M, *dst_i = out_i + (int64_t)blockIdx.y * M;
#pragma unroll
        for (int t = 0; t < kFwdColumns; ++t)
            if (m[t] < M) {
                dst_r[m[t]] = dr[t];
                dst_i[m[t]] = di[t];
            }
    }
}

// ---------------------------------------------------------------------------
// F on line pairs, on the matrix cores
// ---------------------------------------------------------------------------
// When, beyond the line form's rule, the lines 2i + 1 of every unit are
// the lines 2i moved by one offset d, the same throughout (the line-pair
// records of the classification: flag 1 in every unit pair, with pair 0's
// step and offset), each line pair sums about its centre c = x_c(2i) +
// d / 2. Its voxels lie at c + sigma (d / 2 + o_j) and c - sigma (d / 2 +
// o_j) with o_j = (j + 1/2) dx e_x, j < 64, and sigma = +1 (side 0: line
// 2i + 1 from its centre up, line 2i from its centre down) or -1 (side 1:
// the other halves). With rho+ and rho- the two voxels of (side, j),
//
//   D_m = sum_pairs conj(V) sum_{side, j} (P C - i Q S),
//   V = exp(i 2 pi k_m . c),  P, Q = rho+ +- rho-,
//   C, S = cos, sin(2 pi k_m . (sigma d / 2 + o_j)),
//
// the line form's products with K = 2 x 128 per line pair instead of
// 2 x 64 per line: the same matrix-core work per term, and half the phasor
// work (one V per line pair and sample).
//
// Units of 64-voxel lines (class kClassLines) whose lines come four by
// four at 0, d, e and e + d from line 4i (record flag 3 in every unit
// pair, pair 0's step and offsets throughout; rows y .. y + 3 of a grid
// with rows of 64) take the same form with four sides of 32 columns: the
// group's voxels at c + sigma_1 d / 2 + sigma_2 e / 2 + o_j (line 3 - s of
// the group) and their reflections (line s), side s = (sigma_1, sigma_2)
// = (s & 1 ? -1 : 1, s & 2 ? -1 : 1), j < 32, c = x_c(4i) + d / 2 + e / 2;
// again K = 2 x 128 per group and sample.
//
// fhd_forward_pairs_pack_kernel forms A in tiles of 16 groups (one unit;
// K = 32 s + 8 (l / 16) + i: cos part for K < 128, then sin; within a
// part, side (K % 128) / (LINE / 2), j = K % (LINE / 2)) and checks the
// rule; fhd_forward_pairs_kernel walks the tiles with each wave's B (all
// sides) in registers. In the fp16 form a tile's operands share one
// power-of-two scale (the tile's largest |value| times 2^sh in [2^14,
// 2^15)), undone once per tile.
constexpr int kFwpTilePairs = 16;
constexpr int kFwpKSteps = 2 * 2 * kFwdPairs / 32;      // 8 products of K = 32
constexpr int kFwpOpsVec4 = kFwpKSteps * 4 * 64;
constexpr int kFwpTileVec4 = kFwpOpsVec4 + kFwpTilePairs;   // then (c_x, c_y, c_z, sh) per pair
static_assert(2 * kFwpTilePairs * kLongLineVox == kUnitVox, "a tile of line pairs is one unit");
static_assert(4 * kFwpTilePairs * kLineVox == kUnitVox, "a tile of four-line groups is one unit");

// The group kind of a call, from pair 0's record: 128-voxel line pairs
// (flag 1) or four-line groups of 64-voxel lines (flag 3); else none.
enum : int { kFwpNone = 0, kFwpPairs128 = 1, kFwpGroups64 = 3 };
__device__ __forceinline__ int fwp_kind(const int4 *__restrict__ patches)
{
    const int f = patches[0].x;
    return f == kFwpPairs128 || f == kFwpGroups64 ? f : kFwpNone;
}

// Whether unit `unit` has the group structure of the call's kind, with
// pair 0's step and offsets.
__device__ __forceinline__ bool fwp_unit_ok(const int *__restrict__ cls, const int4 *__restrict__ patches,
                                            const int *__restrict__ info, int64_t unit, int kind)
{
    const int4 r0 = patches[2 * (unit / 2)], r1 = patches[2 * (unit / 2) + 1], q0 = patches[0], q1 = patches[1];
    const bool same = r0.x == q0.x && r0.y == q0.y && r1.x == q1.x && r1.y == q1.y && r1.z == q1.z;
    if (kind == kFwpPairs128) return info[0] != 0 && cls[unit] == kClassLongPair && same && r0.y == info[1];
    if (kind == kFwpGroups64)
        return cls[unit] == kClassLines && same && r0.z == q0.z && r0.w == q0.w && r1.w == q1.w;
    return false;
}

// Unit `unit`'s voxels of row `row` (a group of SIDES lines of LINE) and
// column K of the operand, as the pre-pass pairs them.
template <int LINE, int SIDES>
__device__ __forceinline__ void fwp_voxels(int64_t unit, int row, int K, int64_t *up, int64_t *dn)
{
    constexpr int kHalf = LINE / 2;
    const int kk = K % (2 * kFwdPairs), side = kk / kHalf, j = kk % kHalf;
    const int64_t row0 = unit * kUnitVox + (int64_t)(SIDES * row) * LINE;
    *up = row0 + (int64_t)(SIDES - 1 - side) * LINE + kHalf + j;
    *dn = row0 + (int64_t)side * LINE + kHalf - 1 - j;
}
static_assert(kFwpKSteps == 2 * (kFwdBlock / 64), "two k steps per pre-pass wave");

// One workgroup per unit (tile): wave w forms k steps 2 w and 2 w + 1
// (lane l: row l % 16, a line pair or a four-line group), the first 16
// lanes of wave 0 the rows' centres; the first lane checks the unit
// against pair 0's record and, when it differs (or pair 0 has no group
// kind), sets info[3] (the line-pair form then stands aside).
template <bool F16>
__global__ __launch_bounds__(kFwdBlock) void fhd_forward_pairs_pack_kernel(
    const float *__restrict__ x, const float *__restrict__ y, const float *__restrict__ z,
    const float *__restrict__ rho_r, const float *__restrict__ rho_i, const int *__restrict__ cls,
    const int4 *__restrict__ patches, int *__restrict__ info, u32x4 *__restrict__ tiles)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, row = lane & 15, quarter_k = lane >> 4;
    const int64_t unit = blockIdx.x;
    const int kind = fwp_kind(patches);   // uniform
    if (threadIdx.x == 0 && !fwp_unit_ok(cls, patches, info, unit, kind)) atomicOr(&info[3], 1);
    if (kind == kFwpNone) return;
    const bool pairs = kind == kFwpPairs128;
    const int line = pairs ? kLongLineVox : kLineVox, sides = pairs ? 2 : 4;
    float re[2][kChunk], im[2][kChunk];
    auto gather_rows = [&](auto line_c, auto sides_c) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int s = 2 * w + h;
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                const int K = 32 * s + 8 * quarter_k + i;
                const bool sine = K >= 2 * kFwdPairs;
                int64_t up, dn;
                fwp_voxels<decltype(line_c)::value, decltype(sides_c)::value>(unit, row, K, &up, &dn);
                const float ur = rho_r[up], ui = rho_i[up], dr = rho_r[dn], di = rho_i[dn];
                re[h][i] = sine ? ui - di : ur + dr;   // Q_i | P_r
                im[h][i] = sine ? dr - ur : ui + di;   // -Q_r | P_i
            }
        }
    };
    if (pairs)   // uniform
        gather_rows(std::integral_constant<int, kLongLineVox>(), std::integral_constant<int, 2>());
    else
        gather_rows(std::integral_constant<int, kLineVox>(), std::integral_constant<int, 4>());
    int sh = 0;
    if constexpr (F16) {
        // the tile's largest magnitude: the lane's values, the wave, the
        // four waves (LDS)
        __shared__ unsigned wave_max[kFwdBlock / 64];
        unsigned m = 0u;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                const unsigned a = __float_as_uint(re[h][i]) & 0x7fffffffu;
                const unsigned b = __float_as_uint(im[h][i]) & 0x7fffffffu;
                m = a > m ? a : m;
                m = b > m ? b : m;
            }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const unsigned t = (unsigned)__shfl_xor((int)m, o);
            m = t > m ? t : m;
        }
        if (lane == 0) wave_max[w] = m;
        __syncthreads();
#pragma unroll
        for (int v = 0; v < kFwdBlock / 64; ++v) m = wave_max[v] > m ? wave_max[v] : m;
        sh = amp_shift(m);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                re[h][i] = __builtin_ldexpf(re[h][i], sh);
                im[h][i] = __builtin_ldexpf(im[h][i], sh);
            }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        unsigned rh[4], rl[4], ih[4], il[4];
        split_parts<F16, kChunk>(re[h], rh, rl);
        split_parts<F16, kChunk>(im[h], ih, il);
        u32x4 *t = tiles + unit * kFwpTileVec4 + (2 * w + h) * 4 * 64 + lane;
        t[0 * 64] = (u32x4){rh[0], rh[1], rh[2], rh[3]};
        t[1 * 64] = (u32x4){rl[0], rl[1], rl[2], rl[3]};
        t[2 * 64] = (u32x4){ih[0], ih[1], ih[2], ih[3]};
        t[3 * 64] = (u32x4){il[0], il[1], il[2], il[3]};
    }
    if (w == 0 && quarter_k == 0) {
        // the row's centre: x_c of its first line plus d / 2 (plus e / 2)
        const int4 r0 = patches[2 * (unit / 2)], r1 = patches[2 * (unit / 2) + 1];
        const float dx = __int_as_float(r0.y);
        const int64_t first = unit * kUnitVox + (int64_t)(sides * row) * line;
        float cx = __builtin_fmaf(0.5f * (float)(line - 1), dx, x[first]) + 0.5f * __int_as_float(r1.x);
        float cy = y[first] + 0.5f * __int_as_float(r1.y), cz = z[first] + 0.5f * __int_as_float(r1.z);
        if (!pairs) {
            cx += 0.5f * __int_as_float(r0.z);
            cy += 0.5f * __int_as_float(r0.w);
            cz += 0.5f * __int_as_float(r1.w);
        }
        tiles[unit * kFwpTileVec4 + kFwpOpsVec4 + row] =
            (u32x4){__float_as_uint(cx), __float_as_uint(cy), __float_as_uint(cz), (unsigned)sh};
    }
}

// Workgroup b, split s: samples b kFwdBlockSamples .. + 127 as in the line
// form (wave w the 32 from 32 w, two 16-sample columns), the tiles of
// split s of the line-pair stream, staged into LDS by buffer loads (two
// buffers); writes D (splits == 1) or its partial sums at out + s M.
template <bool F16>
__global__ __launch_bounds__(kFwdBlock) __attribute__((amdgpu_waves_per_eu(2))) void fhd_forward_pairs_kernel(
    const u32x4 *__restrict__ tiles, int ntiles, int splits, const int *__restrict__ info,
    const int4 *__restrict__ patches, const float *__restrict__ kx, const float *__restrict__ ky,
    const float *__restrict__ kz, float *__restrict__ out_r, float *__restrict__ out_i, int M)
{
    if (!pairs_form_ran(info)) return;
    __shared__ u32x4 stage[2][kFwpTileVec4];
    const int lane = threadIdx.x & 63, quarter_k = lane >> 4, col = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int4 r0 = patches[0], r1 = patches[1];
    const float hdx = 0.5f * __int_as_float(r0.y);
    const float ddx = __int_as_float(r1.x), ddy = __int_as_float(r1.y), ddz = __int_as_float(r1.z);

    int64_t m[kFwdColumns];
    float skx[kFwdColumns], sky[kFwdColumns], skz[kFwdColumns];
#pragma unroll
    for (int t = 0; t < kFwdColumns; ++t) {
        m[t] = (int64_t)blockIdx.x * kFwdBlockSamples + wave * 16 * kFwdColumns + t * 16 + col;
        const bool live = m[t] < M;   // samples past M compute with k = 0 and are not stored
        skx[t] = live ? kx[m[t]] : 0.0f;
        sky[t] = live ? ky[m[t]] : 0.0f;
        skz[t] = live ? kz[m[t]] : 0.0f;
    }
    // B operands, held for the whole walk: K = 32 s + 8 (l / 16) + i, cos
    // (K < 128) or sin of 2 pi (kx (j + 1/2) dx + sigma_1 k . d / 2 +
    // sigma_2 k . e / 2) for side (K % 128) / (LINE / 2), j = K % (LINE / 2)
    const float hex = __int_as_float(r0.z), hey = __int_as_float(r0.w), hez = __int_as_float(r1.w);
    u32x4 bh[kFwdColumns][kFwpKSteps], bl[kFwdColumns][kFwpKSteps];
    auto form_b = [&](auto half_c) __attribute__((always_inline)) {
        constexpr int kHalf = decltype(half_c)::value;
        constexpr bool kPairs = kHalf == kFwdPairs;
#pragma unroll
        for (int t = 0; t < kFwdColumns; ++t) {
            const float hd = 0.5f * __builtin_fmaf(skx[t], ddx, __builtin_fmaf(sky[t], ddy, skz[t] * ddz));
            const float he =
                kPairs ? 0.0f : 0.5f * __builtin_fmaf(skx[t], hex, __builtin_fmaf(sky[t], hey, skz[t] * hez));
#pragma unroll
            for (int s = 0; s < kFwpKSteps; ++s) {
                float v[kChunk];
#pragma unroll
                for (int i = 0; i < kChunk; ++i) {
                    const int K = 32 * s + 8 * quarter_k + i, kk = K % (2 * kFwdPairs);
                    const int side = kk / kHalf, j = kk % kHalf;
                    const float s1 = (side & 1) ? -1.0f : 1.0f, s2 = (side & 2) ? -1.0f : 1.0f;
                    const float off = kPairs ? s1 * hd : __builtin_fmaf(s2, he, s1 * hd);
                    const float a = __builtin_fmaf(skx[t], (float)(2 * j + 1) * hdx, off);
                    v[i] = K < 2 * kFwdPairs ? __builtin_amdgcn_cosf(a) : __builtin_amdgcn_sinf(a);
                }
                unsigned h[4], l[4];
                split_parts<F16, kChunk>(v, h, l);
                bh[t][s] = (u32x4){h[0], h[1], h[2], h[3]};
                bl[t][s] = (u32x4){l[0], l[1], l[2], l[3]};
            }
        }
    };
    if (r0.x == kFwpPairs128)   // uniform
        form_b(std::integral_constant<int, kFwdPairs>());
    else
        form_b(std::integral_constant<int, kLineVox / 2>());

    float dr[kFwdColumns], di[kFwdColumns];
#pragma unroll
    for (int t = 0; t < kFwdColumns; ++t) {
        dr[t] = 0.0f;
        di[t] = 0.0f;
    }
    const int per = (ntiles + splits - 1) / splits;
    const int t0 = min(ntiles, (int)blockIdx.y * per), t1 = min(ntiles, t0 + per);
    const float4 *src = reinterpret_cast<const float4 *>(tiles);
    const int64_t total_vec4 = (int64_t)ntiles * kFwpTileVec4;
    if (t0 < t1) issue_stage_load<kFwdBlock, kFwpTileVec4>(src, total_vec4, t0, reinterpret_cast<float4 *>(stage[0]));

    // V = exp(i 2 pi k . c) of a tile's rows 4 (l / 16) + r and the lane's
    // columns, and the tile's scale 2^-sh
    struct Phasors {
        float c[4][kFwdColumns], s[4][kFwdColumns];
        float scale;
    };
    auto phasors = [&](const u32x4 *st, Phasors &v) __attribute__((always_inline)) {
        int sh = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const u32x4 c = st[kFwpOpsVec4 + 4 * quarter_k + r];
            const float cx = __uint_as_float(c.x), cy = __uint_as_float(c.y), cz = __uint_as_float(c.z);
            sh = (int)c.w;
#pragma unroll
            for (int t = 0; t < kFwdColumns; ++t) {
                const float p = __builtin_fmaf(skx[t], cx, __builtin_fmaf(sky[t], cy, skz[t] * cz));
                v.c[r][t] = __builtin_amdgcn_cosf(p);
                v.s[r][t] = __builtin_amdgcn_sinf(p);
            }
        }
        v.scale = unscale<F16>(1.0f, sh);
    };
    // D += 2^-sh conj(V) T over the lane's four rows
    float4v tre[kFwdColumns], tim[kFwdColumns];
    auto accumulate = [&](const Phasors &v) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < kFwdColumns; ++t) {
            float tdr = 0.0f, tdi = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                tdr = __builtin_fmaf(v.c[r][t], tre[t][r], __builtin_fmaf(v.s[r][t], tim[t][r], tdr));
                tdi = __builtin_fmaf(v.c[r][t], tim[t][r], __builtin_fmaf(-v.s[r][t], tre[t][r], tdi));
            }
            dr[t] = __builtin_fmaf(tdr, v.scale, dr[t]);
            di[t] = __builtin_fmaf(tdi, v.scale, di[t]);
        }
    };

    // Tile tau (in stage[b]): its phasors go to `cur` first, while the
    // previous tile's products (tre / tim) drain; those are then folded
    // into D with the previous tile's phasors `prev`, and tile tau's
    // products start. So the phasor work never waits on the matrix cores.
    auto tile = [&](int tau, int b, Phasors &cur, const Phasors &prev) __attribute__((always_inline)) {
        // tile tau is in stage[b] once every wave's copies have landed; the
        // other buffer was last read before this barrier
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();
        if (tau + 1 < t1)
            issue_stage_load<kFwdBlock, kFwpTileVec4>(src, total_vec4, tau + 1,
                                                      reinterpret_cast<float4 *>(stage[b ^ 1]));
        phasors(stage[b], cur);
        // formed here, not sunk towards their use a tile later
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int t = 0; t < kFwdColumns; ++t) asm volatile("" : "+v"(cur.c[r][t]), "+v"(cur.s[r][t]));
        __builtin_amdgcn_sched_barrier(0);   // keep the phasors ahead of the fold
        accumulate(prev);
#pragma unroll
        for (int t = 0; t < kFwdColumns; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                tre[t][r] = 0.0f;
                tim[t][r] = 0.0f;
            }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < kFwpKSteps; ++s) {
            const u32x4 *op = &stage[b][s * 4 * 64 + lane];
            const u32x4 arh = op[0 * 64], arl = op[1 * 64], aih = op[2 * 64], ail = op[3 * 64];
#pragma unroll
            for (int t = 0; t < kFwdColumns; ++t) {
                tre[t] = mfma16<F16>(arh, bh[t][s], tre[t]);
                tim[t] = mfma16<F16>(aih, bh[t][s], tim[t]);
                tre[t] = mfma16<F16>(arh, bl[t][s], tre[t]);
                tim[t] = mfma16<F16>(aih, bl[t][s], tim[t]);
                tre[t] = mfma16<F16>(arl, bh[t][s], tre[t]);
                tim[t] = mfma16<F16>(ail, bh[t][s], tim[t]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // the fold before the first tile adds zeros
    Phasors va, vb;
#pragma unroll
    for (int t = 0; t < kFwdColumns; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            tre[t][r] = 0.0f;
            tim[t][r] = 0.0f;
            vb.c[r][t] = 0.0f;
            vb.s[r][t] = 0.0f;
        }
    vb.scale = 0.0f;
    int tau = t0;
    for (; tau + 1 < t1; tau += 2) {
        tile(tau, 0, va, vb);
        tile(tau + 1, 1, vb, va);
    }
    if (tau < t1) {
        tile(tau, 0, va, vb);
        accumulate(va);
    } else if (t0 < t1) {
        accumulate(vb);
    }

    // each column's four row groups (lanes col + 16 q) add up
#pragma unroll
    for (int t = 0; t < kFwdColumns; ++t) {
        dr[t] += __shfl_xor(dr[t], 16);
        di[t] += __shfl_xor(di[t], 16);
        dr[t] += __shfl_xor(dr[t], 32);
        di[t] += __shfl_xor(di[t], 32);
    }
    if (quarter_k == 0) {
        float *dst_r = out_r + (int64_t)blockIdx.y * M, *dst_i = out_i + (int64_t)blockIdx.y * M;
#pragma unroll
        for (int t = 0; t < kFwdColumns; ++t)
            if (m[t] < M) {
                dst_r[m[t]] = dr[t];
                dst_i[m[t]] = di[t];
            }
    }
}

}  // namespace

int launch_forward_pack(const float *x, const float *y, const float *z, const float *rho_r,
                        const float *rho_i, int N, float *packed, hipStream_t stream, const int *gate)
{
    if (N == 0) return FHD_OK;
    const int64_t N_pad = (int64_t)((N + kChunk - 1) / kChunk) * kChunk;
    const int64_t blocks = (N_pad + kPackBlock - 1) / kPackBlock;
    fhd_forward_pack_kernel<<<dim3((unsigned)blocks), dim3(kPackBlock), 0, stream>>>(
        x, y, z, rho_r, rho_i, packed, N, N_pad, gate);
    return launch_status("fhd_forward_pack_kernel launch");
}

int launch_forward_gather(const float *packed, int N, const float *kx, const float *ky,
                          const float *kz, float *Dr, float *Di, int M, hipStream_t stream, const int *gate)
{
    if (M == 0) return FHD_OK;
    const int nchunks = (int)(((int64_t)N + kChunk - 1) / kChunk);
    const int64_t per_block = (int64_t)kBlock * kSamp;
    const int64_t blocks = ((int64_t)M + per_block - 1) / per_block;
    const int splits = split_count(blocks, nchunks);
    if (splits == 1) {
        {
            TimedLaunch timed("fhd_forward_gather_kernel<2>", stream);
            fhd_forward_gather_kernel<kSamp><<<dim3((unsigned)blocks), dim3(kBlock), 0, stream>>>(
                packed, nchunks, 1, kx, ky, kz, Dr, Di, M, gate);
        }
        return launch_status("fhd_forward_gather_kernel launch");
    }
    StreamBuffer buf(stream, kSlotForwardPart);
    char *mem = nullptr;
    int rc = buf.get((size_t)splits * 2 * M * sizeof(float), &mem);
    if (rc != FHD_OK) return rc;
    float *part_r = reinterpret_cast<float *>(mem), *part_i = part_r + (int64_t)splits * M;
    {
        TimedLaunch timed("fhd_forward_gather_kernel<2>", stream);
        fhd_forward_gather_kernel<kSamp>
            <<<dim3((unsigned)blocks, (unsigned)splits), dim3(kBlock), 0, stream>>>(
                packed, nchunks, splits, kx, ky, kz, part_r, part_i, M, gate);
    }
    rc = launch_status("fhd_forward_gather_kernel launch");
    if (rc == FHD_OK) rc = launch_reduce(part_r, part_i, splits, M, Dr, Di, stream, gate, false);
    const int f = buf.finish();
    return rc != FHD_OK ? rc : f;
}


// The line-pair form's pre-pass and gather of one split type (F16: fp16
// parts).
template <bool F16>
int launch_forward_pairs(const float *x, const float *y, const float *z, const float *rho_r,
                         const float *rho_i, const int *cls, const int4 *patches, int *info, u32x4 *tiles,
                         int64_t units, int64_t blocks, int splits, const float *kx, const float *ky,
                         const float *kz, float *part_r, float *part_i, int M, hipStream_t stream)
{
    fhd_forward_pairs_pack_kernel<F16><<<dim3((unsigned)units), dim3(kFwdBlock), 0, stream>>>(
        x, y, z, rho_r, rho_i, cls, patches, info, tiles);
    int rc = launch_status("fhd_forward_pairs_pack_kernel launch");
    if (rc == FHD_OK) {
        TimedLaunch timed(F16 ? "fhd_forward_pairs_kernel<true>" : "fhd_forward_pairs_kernel<false>", stream);
        fhd_forward_pairs_kernel<F16><<<dim3((unsigned)blocks, (unsigned)splits), dim3(kFwdBlock), 0, stream>>>(
            tiles, (int)units, splits, info, patches, kx, ky, kz, part_r, part_i, M);
        rc = launch_status("fhd_forward_pairs_kernel launch");
    }
    return rc;
}

// The line form's pre-pass and gather of one split type (F16: fp16 parts).
template <bool F16>
int launch_forward_lines(const float *x, const float *y, const float *z, const float *rho_r,
                         const float *rho_i, const int *cls, int *info, u32x4 *tiles, int64_t ntiles,
                         int64_t blocks, int splits, const float *kx, const float *ky, const float *kz,
                         float *part_r, float *part_i, int M, hipStream_t stream)
{
    fhd_forward_lines_pack_kernel<F16><<<dim3((unsigned)ntiles), dim3(kFwdBlock), 0, stream>>>(
        x, y, z, rho_r, rho_i, cls, info, tiles);
    int rc = launch_status("fhd_forward_lines_pack_kernel launch");
    if (rc == FHD_OK) {
        TimedLaunch timed(F16 ? "fhd_forward_lines_kernel<true>" : "fhd_forward_lines_kernel<false>", stream);
        fhd_forward_lines_kernel<F16><<<dim3((unsigned)blocks, (unsigned)splits), dim3(kFwdBlock), 0, stream>>>(
            tiles, (int)ntiles, splits, info, kx, ky, kz, part_r, part_i, M);
        rc = launch_status("fhd_forward_lines_kernel launch");
    }
    return rc;
}

int launch_forward(const float *x, const float *y, const float *z, const float *rho_r,
                   const float *rho_i, int N, const float *kx, const float *ky, const float *kz,
                   float *Dr, float *Di, int M, float *vox, hipStream_t stream, int paths)
{
    if (M == 0) return FHD_OK;
    if (N == 0 || N % (2 * kUnitVox) != 0 || paths == FHD_GATHER_VECTOR) {
        // not whole pairs of units (or the vector form asked for)
        int rc = launch_forward_pack(x, y, z, rho_r, rho_i, N, vox, stream);
        return rc == FHD_OK ? launch_forward_gather(vox, N, kx, ky, kz, Dr, Di, M, stream) : rc;
    }
    const int64_t units = N / kUnitVox, ntiles = N / kFwdTileVox;
    const int64_t blocks = ((int64_t)M + kFwdBlockSamples - 1) / kFwdBlockSamples;
    // workgroups per CU of the line-pair gather (the split count's, shared
    // with the line form, which stands in when the line-pair rule fails)
    static int per_cu_cache[64] = {0};
    int dev = 0, per_cu = 2;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
        if (per_cu_cache[dev] == 0) {
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &n, reinterpret_cast<const void *>(fhd_forward_pairs_kernel<true>), kFwdBlock, 0) != hipSuccess ||
                n < 1)
                n = 2;
            per_cu_cache[dev] = n;
        }
        per_cu = per_cu_cache[dev];
    }
    // cut the tile stream so the sample blocks fill whole rounds (each part
    // at least one line-pair tile, two line tiles), within 0.5 % of the
    // cheapest count: a part's own cost (its workgroups form their B
    // operands, one row of partial sums of D) is small against a walk of
    // tens of tiles (at 128^3 x 100k: 13 parts rather than 7; 11 or 15
    // parts ran 0.8 % faster than 7, interleaved on one machine)
    const int splits = split_count(blocks, (int)(units * kStageChunks), per_cu, kStageChunks, 1.005);
    // one workspace: unit classes and the flag words | line-pair records |
    // tiles (either form's) | partials
    const size_t cls_bytes = ((size_t)units * sizeof(int) + kInfoWords * sizeof(int) + 255) / 256 * 256;
    const size_t rec_bytes = ((size_t)units * sizeof(int4) + 255) / 256 * 256;
    const size_t line_tile_bytes = (size_t)ntiles * kFwdTileVec4 * sizeof(u32x4);
    const size_t pair_tile_bytes = (size_t)units * kFwpTileVec4 * sizeof(u32x4);
    const size_t tile_bytes = line_tile_bytes > pair_tile_bytes ? line_tile_bytes : pair_tile_bytes;
    const size_t part_bytes = splits > 1 ? (size_t)splits * 2 * M * sizeof(float) : 0;
    StreamBuffer buf(stream, kSlotForward);
    char *work = nullptr;
    int rc = buf.get(cls_bytes + rec_bytes + tile_bytes + part_bytes, &work);
    if (rc != FHD_OK) return rc;
    int *cls = reinterpret_cast<int *>(work), *info = cls + units;
    int4 *patches = reinterpret_cast<int4 *>(work + cls_bytes);
    u32x4 *tiles = reinterpret_cast<u32x4 *>(work + cls_bytes + rec_bytes);
    float *part_r = Dr, *part_i = Di;
    if (splits > 1) {
        part_r = reinterpret_cast<float *>(work + cls_bytes + rec_bytes + tile_bytes);
        part_i = part_r + (int64_t)splits * M;
    }
    rc = launch_classify(x, y, z, N, true, cls, info, stream, false, nullptr, 0, patches);
    // the line-pair form, else the line form (each stands aside when the
    // other runs or its rule fails), with one split count
    const bool f16 = paths != FHD_GATHER_BF16X3;
    if (rc == FHD_OK)
        rc = f16 ? launch_forward_pairs<true>(x, y, z, rho_r, rho_i, cls, patches, info, tiles, units, blocks,
                                              splits, kx, ky, kz, part_r, part_i, M, stream)
                 : launch_forward_pairs<false>(x, y, z, rho_r, rho_i, cls, patches, info, tiles, units, blocks,
                                               splits, kx, ky, kz, part_r, part_i, M, stream);
    if (rc == FHD_OK)
        rc = f16 ? launch_forward_lines<true>(x, y, z, rho_r, rho_i, cls, info, tiles, ntiles, blocks, splits, kx,
                                              ky, kz, part_r, part_i, M, stream)
                 : launch_forward_lines<false>(x, y, z, rho_r, rho_i, cls, info, tiles, ntiles, blocks, splits, kx,
                                               ky, kz, part_r, part_i, M, stream);
    if (rc == FHD_OK && splits > 1) rc = launch_reduce(part_r, part_i, splits, M, Dr, Di, stream, info, true);
    // the vector form, which stands aside when either matrix-core form ran
    if (rc == FHD_OK) rc = launch_forward_pack(x, y, z, rho_r, rho_i, N, vox, stream, info);
    if (rc == FHD_OK) rc = launch_forward_gather(vox, N, kx, ky, kz, Dr, Di, M, stream, info);
    const int f = buf.finish();
    return rc != FHD_OK ? rc : f;
}

}  // namespace fhd

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
using namespace fhd;

extern "C" int fhd_forward_pack(const float *x, const float *y, const float *z, const float *rho_r,
                                const float *rho_i, int N, void *packed, int64_t packed_bytes,
                                void *stream)
{
    clear_error();
    if (N < 0) return fail(FHD_ERR_INVALID_ARG, "N < 0");
    if (N == 0) return FHD_OK;
    const int64_t need = packed_bytes_for(N), nb = (int64_t)N * 4;
    if (packed_bytes < need)
        return fail(FHD_ERR_INVALID_ARG, "packed_bytes " + std::to_string(packed_bytes) + " < " +
                                             std::to_string(need));
    const Span all[] = {{x, nb, "x"}, {y, nb, "y"}, {z, nb, "z"}, {rho_r, nb, "rho_r"},
                        {rho_i, nb, "rho_i"}, {packed, need, "packed", 16}};
    int rc = check_host_side(all, 6);
    if (rc == FHD_OK) rc = check_no_overlap(all, 6, 5);
    if (rc == FHD_OK) rc = check_device_spans(all, 6);
    if (rc != FHD_OK) return rc;
    return launch_forward_pack(x, y, z, rho_r, rho_i, N, (float *)packed, (hipStream_t)stream);
}

extern "C" int fhd_forward_gather(const void *packed, int N, const float *kx, const float *ky,
                                  const float *kz, float *Dr, float *Di, int M, void *stream)
{
    clear_error();
    if (N < 0) return fail(FHD_ERR_INVALID_ARG, "N < 0");
    if (M < 0) return fail(FHD_ERR_INVALID_ARG, "M < 0");
    if (M == 0) return FHD_OK;
    const int64_t mb = (int64_t)M * 4;
    const Span all[] = {{packed, N > 0 ? packed_bytes_for(N) : 0, "packed", 16},
                        {kx, mb, "kx"}, {ky, mb, "ky"}, {kz, mb, "kz"},
                        {Dr, mb, "Dr"}, {Di, mb, "Di"}};
    int rc = check_host_side(all, 6);
    if (rc == FHD_OK) rc = check_no_overlap(all, 6, 4);
    if (rc == FHD_OK) rc = check_device_spans(all, 6);
    if (rc != FHD_OK) return rc;
    return launch_forward_gather((const float *)packed, N, kx, ky, kz, Dr, Di, M,
                                 (hipStream_t)stream);
}

extern "C" int fhd_forward_paths(const float *kx, const float *ky, const float *kz, const float *x,
                                 const float *y, const float *z, const float *rho_r, const float *rho_i,
                                 float *Dr, float *Di, int M, int N, int paths, void *stream)
{
    clear_error();
    if (M < 0) return fail(FHD_ERR_INVALID_ARG, "M < 0");
    if (N < 0) return fail(FHD_ERR_INVALID_ARG, "N < 0");
    if (!valid_paths(paths)) return fail_paths();
    if (M == 0) return FHD_OK;
    const int64_t mb = (int64_t)M * 4, nb = (int64_t)N * 4;
    const Span all[] = {{kx, mb, "kx"}, {ky, mb, "ky"}, {kz, mb, "kz"},
                        {x, nb, "x"},   {y, nb, "y"},   {z, nb, "z"},
                        {rho_r, nb, "rho_r"}, {rho_i, nb, "rho_i"},
                        {Dr, mb, "Dr"}, {Di, mb, "Di"}};
    int rc = check_host_side(all, 10);
    if (rc == FHD_OK) rc = check_no_overlap(all, 10, 8);
    if (rc == FHD_OK) rc = check_device_spans(all, 10);
    if (rc != FHD_OK) return rc;

    hipStream_t s = (hipStream_t)stream;
    StreamBuffer buf(s, kSlotForwardPacked);
    char *mem = nullptr;
    rc = buf.get(N > 0 ? (size_t)packed_bytes_for(N) : 0, &mem);
    if (rc == FHD_OK)
        rc = launch_forward(x, y, z, rho_r, rho_i, N, kx, ky, kz, Dr, Di, M, reinterpret_cast<float *>(mem), s,
                            paths);
    const int f = buf.finish();
    return rc != FHD_OK ? rc : f;
}

extern "C" int fhd_forward(const float *kx, const float *ky, const float *kz, const float *x,
                           const float *y, const float *z, const float *rho_r, const float *rho_i,
                           float *Dr, float *Di, int M, int N, void *stream)
{
    return fhd_forward_paths(kx, ky, kz, x, y, z, rho_r, rho_i, Dr, Di, M, N, FHD_GATHER_ALL, stream);
}

// q = F^H F p: F into a k-space temporary, then F^H (loop fission of the
// normal operator into its two halves, page "Case study -- iterative MRI
// reconstruction", section 17.3.2).
extern "C" int fhd_normal_paths(const float *kx, const float *ky, const float *kz, const float *x,
                                const float *y, const float *z, const float *p_r, const float *p_i,
                                float *q_r, float *q_i, int M, int N, int paths, void *stream)
{
    clear_error();
    if (M < 0) return fail(FHD_ERR_INVALID_ARG, "M < 0");
    if (N < 0) return fail(FHD_ERR_INVALID_ARG, "N < 0");
    if (!valid_paths(paths)) return fail_paths();
    if (N == 0) return FHD_OK;
    const int64_t mb = (int64_t)M * 4, nb = (int64_t)N * 4;
    const Span all[] = {{kx, mb, "kx"}, {ky, mb, "ky"}, {kz, mb, "kz"},
                        {x, nb, "x"},   {y, nb, "y"},   {z, nb, "z"},
                        {p_r, nb, "p_r"}, {p_i, nb, "p_i"},
                        {q_r, nb, "q_r"}, {q_i, nb, "q_i"}};
    int rc = check_host_side(all, 10);
    if (rc == FHD_OK) rc = check_no_overlap(all, 10, 8);
    if (rc == FHD_OK) rc = check_device_spans(all, 10);
    if (rc != FHD_OK) return rc;

    hipStream_t s = (hipStream_t)stream;
    if (M == 0) return launch_gather(nullptr, 0, x, y, z, q_r, q_i, N, s, paths);   // empty sum
    // one workspace: packed voxels | packed samples | D (real, imaginary)
    const int64_t vox_bytes = packed_bytes_for(N), smp_bytes = packed_bytes_for(M);
    const int64_t d_bytes = 2 * mb;
    StreamBuffer buf(s, kSlotNormal);
    char *ws = nullptr;
    rc = buf.get((size_t)(vox_bytes + smp_bytes + d_bytes), &ws);
    if (rc != FHD_OK) return rc;
    float *vox = (float *)ws, *smp = (float *)(ws + vox_bytes);
    float *d_r = (float *)(ws + vox_bytes + smp_bytes), *d_i = d_r + M;
    rc = launch_forward(x, y, z, p_r, p_i, N, kx, ky, kz, d_r, d_i, M, vox, s, paths);
    if (rc == FHD_OK) rc = launch_pack(kx, ky, kz, d_r, d_i, M, smp, s);
    if (rc == FHD_OK) rc = launch_gather(smp, M, x, y, z, q_r, q_i, N, s, paths);
    const int f = buf.finish();
    return rc != FHD_OK ? rc : f;
}

extern "C" int fhd_normal(const float *kx, const float *ky, const float *kz, const float *x,
                          const float *y, const float *z, const float *p_r, const float *p_i,
                          float *q_r, float *q_i, int M, int N, void *stream)
{
    return fhd_normal_paths(kx, ky, kz, x, y, z, p_r, p_i, q_r, q_i, M, N, FHD_GATHER_ALL, stream);
}
