// fhd_grid.hip -- F^H D on a Cartesian voxel grid as a complex GEMM on the
// gfx950 matrix cores.
//
// rho_n = sum_m D_m exp(+i 2 pi k_m . x_n)   (page "Case study -- iterative
// MRI reconstruction", section 17.3, F^H D equation) with the voxels on a
// grid, x = x0 + ix dx, y = y0 + iy dy, z = z0 + iz dz, n = ix + nx (iy +
// ny iz). The exponential factors, exp(i 2 pi k.x) = exp(i 2 pi kx x) *
// exp(i 2 pi (ky y + kz z)), so with D_m = a_m exp(i 2 pi psi_m):
//
//     rho[(iy, iz), ix] = sum_m A[(iy, iz), m] B[m, ix]
//     A[(iy, iz), m] = a_m exp(i 2 pi (ky_m y + kz_m z + psi_m))
//     B[m, ix]       = exp(i 2 pi kx_m x)
//
// a complex (nyz x M) by (M x nx) product. Each term then costs one complex
// multiply-add on the matrix cores (4 real v_mfma_f32_32x32x2_f32 per 2
// samples and 32 x 32 outputs) instead of two transcendentals and ~3 FMAs
// on the vector ALUs; the operands are generated on the fly from the packed
// samples (fhd_pack's format), amortised over a 32 x 64 output tile per
// wave: per lane and 2 samples, one A element (2 FMA, 2 transcendentals,
// 3 multiplies) and two B elements (1 multiply, 2 transcendentals each)
// feed 8 MFMAs. The voxel coordinates are the grid's, rounded once to fp32
// from their double values. Rows and columns past the grid's edge are
// computed like the others and never stored: in C = A B a row of A only
// reaches its own row of C and a column of B its own column.
//
// v_mfma_f32_32x32x2_f32 operand layout (measured): lane l supplies
// A[l % 32][l / 32] and B[l / 32][l % 32]; accumulator register r of lane l
// holds C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]. Both operands of a lane
// therefore belong to the same sample, m0 + l / 32.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <string>

#include "fhd_internal.h"

namespace fhd {
namespace {

constexpr int kTileYZ = 32;           // A rows per wave
constexpr int kTilesX = 2;            // 32-column B tiles per wave
constexpr int kWaves = kBlock / 64;   // 4 waves per workgroup, stacked along yz

struct GridAxis {
    float x0, dx, y0, dy, z0, dz;
};

__device__ __forceinline__ float grid_coord(float c0, float d, int64_t i)
{
    return (float)((double)c0 + (double)i * (double)d);
}

// Workgroup b covers ix tile bx = b % tiles_x (64 columns) and yz rows
// (b / tiles_x) * 128 .. + 127, one 32-row slab per wave; split s =
// blockIdx.y takes its share of the sample stream.
__global__ __launch_bounds__(kBlock) void fhd_grid_kernel(
    const float *__restrict__ packed, int nchunks, int splits, int nx, int ny, int64_t nyz,
    int tiles_x, GridAxis g, float *__restrict__ out_r, float *__restrict__ out_i)
{
    __shared__ float4 stage[2][kStageVec4];
    const float4 *src = reinterpret_cast<const float4 *>(packed);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;

    const int bx = blockIdx.x % tiles_x;
    const int64_t yz0 = (int64_t)(blockIdx.x / tiles_x) * (kTileYZ * kWaves) + (int64_t)wave * kTileYZ;

    // this lane's A row (yz) and B columns (ix)
    const int64_t yz = yz0 + col;
    const float ry = grid_coord(g.y0, g.dy, yz % ny);
    const float rz = grid_coord(g.z0, g.dz, yz / ny);
    float cx[kTilesX];
#pragma unroll
    for (int t = 0; t < kTilesX; ++t) cx[t] = grid_coord(g.x0, g.dx, bx * (32 * kTilesX) + 32 * t + col);

    float16v acc_r[kTilesX], acc_i[kTilesX];
#pragma unroll
    for (int t = 0; t < kTilesX; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc_r[t][r] = 0.0f;
            acc_i[t][r] = 0.0f;
        }

    int c0, c1;
    split_range(nchunks, splits, blockIdx.y, &c0, &c1);
    stream_chunks(src, c0, c1, stage, [&](const float4 *ch) {
        const float *f = reinterpret_cast<const float *>(ch);
        // 8 samples = 4 k-steps of 2; this lane's sample of step j is
        // 2 j + half
#pragma unroll
        for (int j = 0; j < kChunk / 2; ++j) {
            const int u = 2 * j + half;
            const float skx = f[0 * kChunk + u], sky = f[1 * kChunk + u];
            const float skz = f[2 * kChunk + u], psi = f[3 * kChunk + u];
            const float amp = f[4 * kChunk + u];
            // A element: a e^{i 2 pi (ky y + kz z + psi)}
            const float q = __builtin_fmaf(sky, ry, __builtin_fmaf(skz, rz, psi));
            const float a_r = amp * __builtin_amdgcn_cosf(q);
            const float a_i = amp * __builtin_amdgcn_sinf(q);
            const float na_i = -a_i;
            // B elements: e^{i 2 pi kx x}
            float b_r[kTilesX], b_i[kTilesX];
#pragma unroll
            for (int t = 0; t < kTilesX; ++t) {
                const float p = skx * cx[t];
                b_r[t] = __builtin_amdgcn_cosf(p);
                b_i[t] = __builtin_amdgcn_sinf(p);
            }
            // (a_r + i a_i)(b_r + i b_i), the four accumulators in turn. The
            // operand generation around this runs at raised wave priority,
            // the matrix-core issue at normal priority (measured 2 % faster
            // than one priority throughout).
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int t = 0; t < kTilesX; ++t) {
                acc_r[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a_r, b_r[t], acc_r[t], 0, 0, 0);
                acc_i[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a_r, b_i[t], acc_i[t], 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < kTilesX; ++t) {
                acc_r[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(na_i, b_i[t], acc_r[t], 0, 0, 0);
                acc_i[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a_i, b_r[t], acc_i[t], 0, 0, 0);
            }
            __builtin_amdgcn_s_setprio(1);
            __builtin_amdgcn_sched_barrier(0);
        }
    });
    __builtin_amdgcn_s_setprio(0);

    const int64_t N = nyz * nx;
    float *dst_r = out_r + (int64_t)blockIdx.y * N, *dst_i = out_i + (int64_t)blockIdx.y * N;
#pragma unroll
    for (int t = 0; t < kTilesX; ++t) {
        const int ix = bx * (32 * kTilesX) + 32 * t + col;
        if (ix >= nx) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = yz0 + 8 * (r / 4) + 4 * half + (r % 4);
            if (row < nyz) {
                dst_r[row * nx + ix] = acc_r[t][r];
                dst_i[row * nx + ix] = acc_i[t][r];
            }
        }
    }
}

// The same product with bf16 matrix-core instructions in three passes:
// a b = a_hi b_hi + a_hi b_lo + a_lo b_hi (a_lo b_lo, below 2^-17 |a b|,
// dropped), accumulated in fp32 by v_mfma_f32_32x32x16_bf16. One such
// instruction takes 16 samples (two chunks); lane l supplies
// A[l % 32][8 (l / 32) + i] and B[8 (l / 32) + i][l % 32], i < 8 (layout
// measured), so half-wave h takes chunk h of the pair, and the accumulator
// layout is the fp32 instruction's. A wave covers 32 (y, z) rows and TILES
// 32-column tiles; the four waves of a workgroup are stacked along (y, z)
// and share their 32 TILES columns, so B is made once per workgroup: each
// lane computes 2 TILES of the 16 x 32 TILES elements, splits them and
// writes them to LDS in operand order (double buffered, one barrier per 16
// samples); each wave then reads its operands with ds_read_b128.
template <int TILES>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(TILES == 4 ? 2 : 3))) void fhd_grid_bf16x3_kernel(
    const float *__restrict__ packed, int nchunks, int splits, int nx, int ny, int64_t nyz,
    int tiles_x, GridAxis g, float *__restrict__ out_r, float *__restrict__ out_i)
{
    constexpr int kCols = 32 * TILES;          // columns per workgroup
    constexpr int kPer = 16 * kCols / kBlock;  // B elements per lane and 16 samples
    static_assert(kPer == 4 || kPer == 8, "a lane's B elements lie in one chunk");
    __shared__ float4 stage[2][kStageVec4];
    // [buffer][part: b_r hi, b_r lo, b_i hi, b_i lo][tile][k half][column],
    // 8 bf16 each: one lane's operand; a half-wave reads 32 consecutive
    // entries (no bank conflicts)
    __shared__ u32x4 bshare[2][4][TILES][2][32];
    const float4 *src = reinterpret_cast<const float4 *>(packed);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;

    const int bx = blockIdx.x % tiles_x;
    const int64_t yz0 = (int64_t)(blockIdx.x / tiles_x) * (kTileYZ * kWaves) + (int64_t)wave * kTileYZ;
    const int64_t yz = yz0 + col;
    const float ry = grid_coord(g.y0, g.dy, yz % ny);
    const float rz = grid_coord(g.z0, g.dz, yz / ny);

    // B producer role: column pc of the workgroup's kCols, samples
    // kPer pg .. kPer pg + kPer - 1 of each group of 16
    const int pc = threadIdx.x % kCols, pg = threadIdx.x / kCols;
    const float pxc = grid_coord(g.x0, g.dx, (int64_t)bx * kCols + pc);
    const int p_tile = pc / 32, p_col = pc % 32, p_half = (kPer * pg) / kChunk;
    const int p_vec = ((kPer * pg) % kChunk) / 4;   // first float4 of f0 in the chunk

    float16v acc_r[TILES], acc_i[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc_r[t][r] = 0.0f;
            acc_i[t][r] = 0.0f;
        }

    int c0, c1, kb = 0;
    split_range(nchunks, splits, blockIdx.y, &c0, &c1);
    stream_chunk_groups<2>(src, c0, c1, stage, [&](const float4 *ch, int count) {
        __builtin_amdgcn_s_setprio(1);
        // B elements e^{i 2 pi kx x} of this lane's kPer samples and column;
        // a missing second chunk (odd stream end) gives kx = 0 (its samples
        // have zero amplitude in A)
        {
            float kxs[kPer];
#pragma unroll
            for (int v = 0; v < kPer / 4; ++v) {
                float4 k4 = {0.0f, 0.0f, 0.0f, 0.0f};
                if (p_half < count) k4 = ch[p_half * kChunkVec4 + p_vec + v];
                kxs[4 * v + 0] = k4.x;
                kxs[4 * v + 1] = k4.y;
                kxs[4 * v + 2] = k4.z;
                kxs[4 * v + 3] = k4.w;
            }
            float br[kPer], bi[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const float p = kxs[i] * pxc;
                br[i] = __builtin_amdgcn_cosf(p);
                bi[i] = __builtin_amdgcn_sinf(p);
            }
            unsigned w[4][kPer / 2];
            split_bf16<kPer>(br, w[0], w[1]);
            split_bf16<kPer>(bi, w[2], w[3]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                unsigned *dst = reinterpret_cast<unsigned *>(&bshare[kb][q][p_tile][p_half][p_col]) +
                                ((kPer * pg) % kChunk) / 2;
#pragma unroll
                for (int i = 0; i < kPer / 2; ++i) dst[i] = w[q][i];
            }
        }
        // A elements of this lane's row, chunk `half` of the pair:
        // a e^{i 2 pi (ky y + kz z + psi)}
        float f[kFields][kChunk];
        if (half < count) {
            load_chunk(ch + half * kChunkVec4, f);
        } else {
#pragma unroll
            for (int q = 0; q < kFields; ++q)
#pragma unroll
                for (int u = 0; u < kChunk; ++u) f[q][u] = 0.0f;
        }
        float ar[kChunk], ai[kChunk];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const float q = __builtin_fmaf(f[1][u], ry, __builtin_fmaf(f[2][u], rz, f[3][u]));
            ar[u] = f[4][u] * __builtin_amdgcn_cosf(q);
            ai[u] = f[4][u] * __builtin_amdgcn_sinf(q);
        }
        unsigned wa[4][4];
        split_bf16<kChunk>(ar, wa[0], wa[1]);
        split_bf16<kChunk>(ai, wa[2], wa[3]);
        const bf16x8 arh = as_bf16x8(wa[0]), arl = as_bf16x8(wa[1]);
        const bf16x8 aih = as_bf16x8(wa[2]), ail = as_bf16x8(wa[3]);
        const u32x4 sign = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        const bf16x8 naih = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, aih) ^ sign);
        const bf16x8 nail = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, ail) ^ sign);
        __syncthreads();   // this group's B is in LDS
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int t = 0; t < TILES; ++t) {
            const bf16x8 brh = __builtin_bit_cast(bf16x8, bshare[kb][0][t][half][col]);
            const bf16x8 brl = __builtin_bit_cast(bf16x8, bshare[kb][1][t][half][col]);
            const bf16x8 bih = __builtin_bit_cast(bf16x8, bshare[kb][2][t][half][col]);
            const bf16x8 bil = __builtin_bit_cast(bf16x8, bshare[kb][3][t][half][col]);
            // real part: a_r b_r - a_i b_i; imaginary part: a_r b_i + a_i b_r
            acc_r[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(arh, brh, acc_r[t], 0, 0, 0);
            acc_i[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(arh, bih, acc_i[t], 0, 0, 0);
            acc_r[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(arh, brl, acc_r[t], 0, 0, 0);
            acc_i[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(arh, bil, acc_i[t], 0, 0, 0);
            acc_r[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(arl, brh, acc_r[t], 0, 0, 0);
            acc_i[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(arl, bih, acc_i[t], 0, 0, 0);
            acc_r[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(naih, bih, acc_r[t], 0, 0, 0);
            acc_i[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aih, brh, acc_i[t], 0, 0, 0);
            acc_r[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(naih, bil, acc_r[t], 0, 0, 0);
            acc_i[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aih, brl, acc_i[t], 0, 0, 0);
            acc_r[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(nail, bih, acc_r[t], 0, 0, 0);
            acc_i[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ail, brh, acc_i[t], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        kb ^= 1;
    });
    __builtin_amdgcn_s_setprio(0);

    const int64_t N = nyz * nx;
    float *dst_r = out_r + (int64_t)blockIdx.y * N, *dst_i = out_i + (int64_t)blockIdx.y * N;
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        const int64_t ix = (int64_t)bx * kCols + 32 * t + col;
        if (ix >= nx) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = yz0 + 8 * (r / 4) + 4 * half + (r % 4);
            if (row < nyz) {
                dst_r[row * nx + ix] = acc_r[t][r];
                dst_i[row * nx + ix] = acc_i[t][r];
            }
        }
    }
}

// Workgroups of a grid kernel that fit on one CU at once (its register
// and LDS budget), asked of the runtime once per device and kernel.
template <int KERNEL>
int grid_blocks_per_cu(const void *kernel)
{
    static int cached[64] = {0};
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= 64) {
        (void)hipGetLastError();
        return 2;
    }
    if (cached[device] == 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kBlock, 0) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 2;
        }
        cached[device] = n;
    }
    return cached[device];
}

// ---------------------------------------------------------------------------
// Forward F on a grid: D_m = sum_n rho_n e^{-i 2 pi k_m.x_n}, the other side
// of the page's F^H D (section 17.2 defines F as the image-to-k-space map).
// On the grid the exponential factors as before, but now the separable
// side is the sum:
//
//     C[(iy, iz), m] = sum_ix rho[(iy, iz), ix] e^{-i 2 pi kx_m x_ix}
//     D_m = sum_(iy, iz) e^{-i 2 pi (ky_m y + kz_m z)} C[(iy, iz), m]
//
// a complex (nyz x nx) by (nx x M) product followed by a phase and a sum
// over its rows. Workgroup = 128 rows (4 waves of 32) x 64 of the nx
// columns (4 groups of 16, the bf16 instruction's k); a wave keeps its
// split rho operands in registers for the whole launch and walks the
// samples 32 at a time. The e^{-i 2 pi kx x} operand (cos, and sin with
// the sign folded into the accumulators) is made once per workgroup, 8
// elements per lane, and shared through LDS. Per 32 samples a wave then
// runs 48 MFMAs into three accumulators (Re: rho_r cos + rho_i sin; rho_r
// sin; rho_i cos), applies the row phases, sums its 16 rows per lane, the
// two half-waves and the four waves, and writes one partial D per sample.
// The partials of all workgroups (rows x column groups) are added in a
// fixed order afterwards.
constexpr int kFwdK = 64;                 // x columns per workgroup
constexpr int kFwdSteps = kFwdK / 16;     // bf16 MFMA k-groups per workgroup

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void fhd_forward_grid_bf16x3_kernel(
    const float *__restrict__ rho_r, const float *__restrict__ rho_i, int nx, int ny, int64_t nyz,
    const float *__restrict__ kx, const float *__restrict__ ky, const float *__restrict__ kz, int M,
    int m_per_split, int kranges, GridAxis g, float *__restrict__ part_r, float *__restrict__ part_i)
{
    // [part: cos hi, cos lo, sin hi, sin lo][k-group][k half][sample]
    __shared__ u32x4 bE[4][kFwdSteps][2][32];
    __shared__ float red[kWaves][32][2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int64_t slab = blockIdx.x / kranges;
    const int kr = blockIdx.x % kranges;
    const int64_t row0 = slab * (kTileYZ * kWaves) + (int64_t)wave * kTileYZ;

    // A operands: rho of row row0 + col, columns kr*64 + 16 s + 8 half + i,
    // zero past the grid's edge
    bf16x8 arh[kFwdSteps], arl[kFwdSteps], aih[kFwdSteps], ail[kFwdSteps];
    {
        const int64_t yz = row0 + col;
#pragma unroll
        for (int s = 0; s < kFwdSteps; ++s) {
            float vr[kChunk], vi[kChunk];
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                const int ix = kr * kFwdK + 16 * s + 8 * half + i;
                const bool ok = yz < nyz && ix < nx;
                vr[i] = ok ? rho_r[yz * nx + ix] : 0.0f;
                vi[i] = ok ? rho_i[yz * nx + ix] : 0.0f;
            }
            unsigned w[4][4];
            split_bf16<kChunk>(vr, w[0], w[1]);
            split_bf16<kChunk>(vi, w[2], w[3]);
            arh[s] = as_bf16x8(w[0]);
            arl[s] = as_bf16x8(w[1]);
            aih[s] = as_bf16x8(w[2]);
            ail[s] = as_bf16x8(w[3]);
        }
    }
    // producer role: sample pm of each group of 32, columns kr*64 + 8 pg + i
    const int pm = threadIdx.x & 31, pg = threadIdx.x >> 5;
    const int p_s = pg / 2, p_h = pg % 2;
    float pxv[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) pxv[i] = grid_coord(g.x0, g.dx, (int64_t)kr * kFwdK + 8 * pg + i);
    // epilogue rows of this lane (accumulator layout): their y and z
    float ey[16], ez[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t yz = row0 + 8 * (r / 4) + 4 * half + (r % 4);
        ey[r] = grid_coord(g.y0, g.dy, yz % ny);
        ez[r] = grid_coord(g.z0, g.dz, yz / ny);
    }

    const int m_begin = blockIdx.y * m_per_split;
    const int m_end = min(M, m_begin + m_per_split);
    for (int mb = m_begin; mb < m_end; mb += 32) {
        __builtin_amdgcn_s_setprio(1);
        {
            // e^{-i 2 pi kx x} = cos - i sin for this lane's sample and 8
            // columns (samples past M: kx = 0, never stored)
            const int m = mb + pm;
            const float pk = m < M ? kx[m] : 0.0f;
            float c[kChunk], sn[kChunk];
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                const float p = pk * pxv[i];
                c[i] = __builtin_amdgcn_cosf(p);
                sn[i] = __builtin_amdgcn_sinf(p);
            }
            unsigned w[4][4];
            split_bf16<kChunk>(c, w[0], w[1]);
            split_bf16<kChunk>(sn, w[2], w[3]);
#pragma unroll
            for (int q = 0; q < 4; ++q) bE[q][p_s][p_h][pm] = (u32x4){w[q][0], w[q][1], w[q][2], w[q][3]};
        }
        __syncthreads();   // B of these 32 samples is in LDS
        __builtin_amdgcn_s_setprio(0);
        float16v acc_r, acc_p, acc_q;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc_r[r] = 0.0f;
            acc_p[r] = 0.0f;
            acc_q[r] = 0.0f;
        }
#pragma unroll
        for (int s = 0; s < kFwdSteps; ++s) {
            const bf16x8 ch = __builtin_bit_cast(bf16x8, bE[0][s][half][col]);
            const bf16x8 cl = __builtin_bit_cast(bf16x8, bE[1][s][half][col]);
            const bf16x8 sh = __builtin_bit_cast(bf16x8, bE[2][s][half][col]);
            const bf16x8 sl = __builtin_bit_cast(bf16x8, bE[3][s][half][col]);
            // Re C = rho_r cos + rho_i sin; Im C = rho_i cos - rho_r sin
            acc_r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(arh[s], ch, acc_r, 0, 0, 0);
            acc_p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(arh[s], sh, acc_p, 0, 0, 0);
            acc_q = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aih[s], ch, acc_q, 0, 0, 0);
            acc_r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(arh[s], cl, acc_r, 0, 0, 0);
            acc_p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(arh[s], sl, acc_p, 0, 0, 0);
            acc_q = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aih[s], cl, acc_q, 0, 0, 0);
            acc_r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(arl[s], ch, acc_r, 0, 0, 0);
            acc_p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(arl[s], sh, acc_p, 0, 0, 0);
            acc_q = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ail[s], ch, acc_q, 0, 0, 0);
            acc_r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aih[s], sh, acc_r, 0, 0, 0);
            acc_r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aih[s], sl, acc_r, 0, 0, 0);
            acc_r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ail[s], sh, acc_r, 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(1);
        // D_m += e^{-i 2 pi (ky y + kz z)} C over this lane's 16 rows
        const int m = mb + col;
        const float eky = m < M ? ky[m] : 0.0f, ekz = m < M ? kz[m] : 0.0f;
        float dr = 0.0f, di = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float ph = __builtin_fmaf(eky, ey[r], ekz * ez[r]);
            const float cp = __builtin_amdgcn_cosf(ph), sp = __builtin_amdgcn_sinf(ph);
            const float cr = acc_r[r], ci = acc_q[r] - acc_p[r];
            dr = __builtin_fmaf(cp, cr, __builtin_fmaf(sp, ci, dr));
            di = __builtin_fmaf(cp, ci, __builtin_fmaf(-sp, cr, di));
        }
        dr += __shfl_xor(dr, 32);
        di += __shfl_xor(di, 32);
        if (half == 0) {
            red[wave][col][0] = dr;
            red[wave][col][1] = di;
        }
        __syncthreads();   // all waves' sums are in LDS; B may be rewritten
        if (threadIdx.x < 32 && mb + (int)threadIdx.x < m_end) {
            float sr = 0.0f, si = 0.0f;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) {
                sr += red[v][threadIdx.x][0];
                si += red[v][threadIdx.x][1];
            }
            part_r[(int64_t)blockIdx.x * M + mb + threadIdx.x] = sr;
            part_i[(int64_t)blockIdx.x * M + mb + threadIdx.x] = si;
        }
    }
    __builtin_amdgcn_s_setprio(0);
}

}  // namespace

int launch_grid_gather(const float *packed, int M, int nx, int ny, int nz, const float *axis,
                       int precision, float *rho_r, float *rho_i, hipStream_t stream)
{
    const int64_t nyz = (int64_t)ny * nz, N = nyz * nx;
    if (N == 0) return FHD_OK;
    // fp32: 2 tiles per wave; bf16x3: 4 tiles (2 when the grid is at most 64
    // columns wide, where 4 would leave half of them idle)
    const int kernel_id = precision == FHD_GRID_BF16X3 ? (nx > 64 ? 2 : 1) : 0;
    const int tiles = kernel_id == 2 ? 4 : 2;
    const int nchunks = (int)(((int64_t)M + kChunk - 1) / kChunk);
    const int tiles_x = (int)((nx + 32 * tiles - 1) / (32 * tiles));
    const int64_t slabs = (nyz + kTileYZ * kWaves - 1) / (kTileYZ * kWaves);
    const int64_t blocks = slabs * tiles_x;
    const GridAxis g{axis[0], axis[1], axis[2], axis[3], axis[4], axis[5]};
    int per_cu = 2;
    const char *name = "fhd_grid_kernel launch";
    if (kernel_id == 0) {
        per_cu = grid_blocks_per_cu<0>((const void *)fhd_grid_kernel);
    } else if (kernel_id == 1) {
        per_cu = grid_blocks_per_cu<1>((const void *)fhd_grid_bf16x3_kernel<2>);
        name = "fhd_grid_bf16x3_kernel<2> launch";
    } else {
        per_cu = grid_blocks_per_cu<2>((const void *)fhd_grid_bf16x3_kernel<4>);
        name = "fhd_grid_bf16x3_kernel<4> launch";
    }
    const int splits = split_count(blocks, nchunks, per_cu);
    auto launch = [&](int nsplit, float *out_r, float *out_i) {
        const dim3 grid((unsigned)blocks, (unsigned)nsplit);
        if (kernel_id == 0) {
            TimedLaunch timed("fhd_grid_kernel", stream);
            fhd_grid_kernel<<<grid, dim3(kBlock), 0, stream>>>(packed, nchunks, nsplit, nx, ny, nyz,
                                                              tiles_x, g, out_r, out_i);
        } else if (kernel_id == 1) {
            TimedLaunch timed("fhd_grid_bf16x3_kernel<2>", stream);
            fhd_grid_bf16x3_kernel<2><<<grid, dim3(kBlock), 0, stream>>>(
                packed, nchunks, nsplit, nx, ny, nyz, tiles_x, g, out_r, out_i);
        } else {
            TimedLaunch timed("fhd_grid_bf16x3_kernel<4>", stream);
            fhd_grid_bf16x3_kernel<4><<<grid, dim3(kBlock), 0, stream>>>(
                packed, nchunks, nsplit, nx, ny, nyz, tiles_x, g, out_r, out_i);
        }
        return launch_status(name);
    };
    if (splits == 1) return launch(1, rho_r, rho_i);
    float *part = nullptr;
    const hipError_t e = hipMallocAsync((void **)&part, (size_t)splits * 2 * N * sizeof(float), stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(FHD_ERR_ALLOC, std::string("hipMallocAsync (split partials): ") +
                                       hipGetErrorString(e));
    }
    float *part_r = part, *part_i = part + (int64_t)splits * N;
    int rc = launch(splits, part_r, part_i);
    if (rc == FHD_OK) rc = launch_reduce(part_r, part_i, splits, N, rho_r, rho_i, stream);
    const hipError_t f = hipFreeAsync(part, stream);
    if (f != hipSuccess && rc == FHD_OK)
        rc = fail(FHD_ERR_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(f));
    return rc;
}

int launch_forward_grid(const float *rho_r, const float *rho_i, int nx, int ny, int nz,
                        const float *axis, int precision, const float *kx, const float *ky,
                        const float *kz, int M, float *Dr, float *Di, hipStream_t stream)
{
    if (M == 0) return FHD_OK;
    if (precision != FHD_GRID_BF16X3) return fail(FHD_ERR_INVALID_ARG, "precision");
    const int64_t nyz = (int64_t)ny * nz;
    const int kranges = (nx + kFwdK - 1) / kFwdK;
    const int64_t slabs = (nyz + kTileYZ * kWaves - 1) / (kTileYZ * kWaves);
    const int64_t blocks = slabs * kranges;
    const GridAxis g{axis[0], axis[1], axis[2], axis[3], axis[4], axis[5]};
    // cut the samples into parts of whole 32s so that the launch fills the
    // chip (2 workgroups per CU at this kernel's register budget)
    const int per_cu = grid_blocks_per_cu<3>((const void *)fhd_forward_grid_bf16x3_kernel);
    int device = 0, cus = 0;
    if (hipGetDevice(&device) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    const int64_t groups = ((int64_t)M + 31) / 32;
    int64_t msplits = ((int64_t)per_cu * cus + blocks - 1) / blocks;
    msplits = std::max<int64_t>(1, std::min<int64_t>(msplits, groups));
    const int m_per_split = (int)(((groups + msplits - 1) / msplits) * 32);
    msplits = ((int64_t)M + m_per_split - 1) / m_per_split;
    float *part = nullptr;
    const hipError_t e = hipMallocAsync((void **)&part, (size_t)blocks * 2 * M * sizeof(float), stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(FHD_ERR_ALLOC, std::string("hipMallocAsync (row partials): ") + hipGetErrorString(e));
    }
    float *part_r = part, *part_i = part + blocks * M;
    {
        TimedLaunch timed("fhd_forward_grid_bf16x3_kernel", stream);
        fhd_forward_grid_bf16x3_kernel<<<dim3((unsigned)blocks, (unsigned)msplits), dim3(kBlock), 0, stream>>>(
            rho_r, rho_i, nx, ny, nyz, kx, ky, kz, M, m_per_split, kranges, g, part_r, part_i);
    }
    int rc = launch_status("fhd_forward_grid_bf16x3_kernel launch");
    if (rc == FHD_OK) rc = launch_reduce(part_r, part_i, (int)blocks, M, Dr, Di, stream);
    const hipError_t f = hipFreeAsync(part, stream);
    if (f != hipSuccess && rc == FHD_OK)
        rc = fail(FHD_ERR_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(f));
    return rc;
}

}  // namespace fhd

using namespace fhd;

namespace {
int check_grid_args(int M, int nx, int ny, int nz, const float *axis, int precision, int64_t *N)
{
    if (M < 0) return fail(FHD_ERR_INVALID_ARG, "M < 0");
    if (precision != FHD_GRID_FP32 && precision != FHD_GRID_BF16X3)
        return fail(FHD_ERR_INVALID_ARG, "precision must be FHD_GRID_FP32 or FHD_GRID_BF16X3");
    if (nx < 0 || ny < 0 || nz < 0) return fail(FHD_ERR_INVALID_ARG, "negative grid size");
    const int64_t n = (int64_t)nx * ny * nz;
    if (n > INT32_MAX) return fail(FHD_ERR_INVALID_ARG, "nx*ny*nz exceeds 2^31 - 1");
    if (!axis) return fail(FHD_ERR_INVALID_ARG, "axis is NULL");
    for (int i = 0; i < 6; ++i)
        if (!std::isfinite(axis[i])) return fail(FHD_ERR_INVALID_ARG, "axis holds a non-finite value");
    *N = n;
    return FHD_OK;
}
}  // namespace

extern "C" int fhd_grid_gather(const void *packed, int M, int nx, int ny, int nz, const float *axis,
                               int precision, float *rho_r, float *rho_i, void *stream)
{
    clear_error();
    int64_t N = 0;
    int rc = check_grid_args(M, nx, ny, nz, axis, precision, &N);
    if (rc != FHD_OK || N == 0) return rc;
    const int64_t nb = N * 4;
    const Span all[] = {{packed, M > 0 ? packed_bytes_for(M) : 0, "packed", 16},
                        {rho_r, nb, "rho_r"}, {rho_i, nb, "rho_i"}};
    rc = check_host_side(all, 3);
    if (rc == FHD_OK) rc = check_no_overlap(all, 3, 1);
    if (rc == FHD_OK) rc = check_device_spans(all, 3);
    if (rc != FHD_OK) return rc;
    return launch_grid_gather((const float *)packed, M, nx, ny, nz, axis, precision, rho_r, rho_i,
                              (hipStream_t)stream);
}

extern "C" int fhd_compute_grid(const float *kx, const float *ky, const float *kz, const float *Dr,
                                const float *Di, int M, int nx, int ny, int nz, const float *axis,
                                int precision, float *rho_r, float *rho_i, void *stream)
{
    clear_error();
    int64_t N = 0;
    int rc = check_grid_args(M, nx, ny, nz, axis, precision, &N);
    if (rc != FHD_OK || N == 0) return rc;
    const int64_t mb = (int64_t)M * 4, nb = N * 4;
    const Span all[] = {{kx, mb, "kx"}, {ky, mb, "ky"}, {kz, mb, "kz"}, {Dr, mb, "Dr"},
                        {Di, mb, "Di"}, {rho_r, nb, "rho_r"}, {rho_i, nb, "rho_i"}};
    rc = check_host_side(all, 7);
    if (rc == FHD_OK) rc = check_no_overlap(all, 7, 5);
    if (rc == FHD_OK) rc = check_device_spans(all, 7);
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
    if (rc == FHD_OK) rc = launch_grid_gather(packed, M, nx, ny, nz, axis, precision, rho_r, rho_i, s);
    if (packed) {
        const hipError_t e = hipFreeAsync(packed, s);
        if (e != hipSuccess && rc == FHD_OK)
            rc = fail(FHD_ERR_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(e));
    }
    return rc;
}

extern "C" int fhd_forward_grid(const float *kx, const float *ky, const float *kz, int M, int nx, int ny,
                                int nz, const float *axis, int precision, const float *rho_r,
                                const float *rho_i, float *Dr, float *Di, void *stream)
{
    clear_error();
    int64_t N = 0;
    int rc = check_grid_args(M, nx, ny, nz, axis, precision, &N);
    if (rc != FHD_OK || M == 0) return rc;
    if (precision != FHD_GRID_BF16X3)
        return fail(FHD_ERR_INVALID_ARG, "fhd_forward_grid supports FHD_GRID_BF16X3 only");
    const int64_t mb = (int64_t)M * 4, nb = N * 4;
    const Span all[] = {{kx, mb, "kx"},       {ky, mb, "ky"},       {kz, mb, "kz"},
                        {rho_r, nb, "rho_r"}, {rho_i, nb, "rho_i"}, {Dr, mb, "Dr"},
                        {Di, mb, "Di"}};
    rc = check_host_side(all, 7);
    if (rc == FHD_OK) rc = check_no_overlap(all, 7, 5);
    if (rc == FHD_OK) rc = check_device_spans(all, 7);
    if (rc != FHD_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (N == 0) return launch_reduce(nullptr, nullptr, 0, M, Dr, Di, s);   // empty image: D = 0
    return launch_forward_grid(rho_r, rho_i, nx, ny, nz, axis, precision, kx, ky, kz, M, Dr, Di, s);
}
