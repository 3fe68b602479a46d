// F^H D in the scatter form: one lane per k-space sample, which adds its
// term D_m e^{+i 2 pi k_m . x_n} into every voxel's rho_n with atomic adds.
// This is the first of the two mappings that "scatter vs gather" (section
// 17.3.1 of the F^H D chapter) compares, kept as measured evidence for the
// choice of the gather form (fhd_gather), which needs no atomics at all.
//
// gfx950 reading of the mapping: the voxel index is uniform across a wave,
// so x_n, y_n, z_n come through scalar loads. The 64 lanes' additions to
// the one address rho_n are combined by the compiler (a lane-by-lane loop
// over the active lanes on the scalar unit) into one hardware fp32 atomic
// per wave (unsafeAtomicAdd: global_atomic_add_f32, no compare-and-swap
// loop). The atomics of the M / 64 waves that add into the same N voxels
// then serialise at the L2; their order varies from run to run, so results
// agree with the gather's to rounding only, not bitwise.
//
// To fill the chip when M / 256 workgroups are few, the voxels are cut
// into slices (grid dimension y); every workgroup still takes 256 samples
// and adds them into every voxel of its slice.

#include "fhd_internal.h"

namespace fhd {
namespace {

constexpr int kScatterBlock = 256;      // samples per workgroup
constexpr int kScatterMinBlocks = 2048; // workgroups to aim for
constexpr int kScatterMinSlice = 64;    // fewest voxels per slice

__global__ __launch_bounds__(kScatterBlock) void fhd_zero_kernel(float *__restrict__ a, float *__restrict__ b,
                                                                 int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * kScatterBlock + threadIdx.x;
    if (i < n) {
        a[i] = 0.0f;
        b[i] = 0.0f;
    }
}

__global__ __launch_bounds__(kScatterBlock) void fhd_scatter_kernel(
    const float *__restrict__ kx, const float *__restrict__ ky, const float *__restrict__ kz,
    const float *__restrict__ Dr, const float *__restrict__ Di, int M,
    const float *__restrict__ x, const float *__restrict__ y, const float *__restrict__ z, int N, int slices,
    float *__restrict__ rho_r, float *__restrict__ rho_i)
{
    const int64_t m = (int64_t)blockIdx.x * kScatterBlock + threadIdx.x;
    const bool live = m < M;
    const float skx = live ? kx[m] : 0.0f, sky = live ? ky[m] : 0.0f, skz = live ? kz[m] : 0.0f;
    const float dr = live ? Dr[m] : 0.0f, di = live ? Di[m] : 0.0f;
    // this workgroup's slice of voxels [n0, n1)
    const int n0 = (int)((int64_t)N * blockIdx.y / slices);
    const int n1 = (int)((int64_t)N * (blockIdx.y + 1) / slices);
    for (int n = n0; n < n1; ++n) {
        // phase in revolutions; the hardware sine and cosine take
        // revolutions, after reduction to [0, 1)
        const float p = __builtin_amdgcn_fractf(__builtin_fmaf(skx, x[n], __builtin_fmaf(sky, y[n], skz * z[n])));
        const float c = __builtin_amdgcn_cosf(p), s = __builtin_amdgcn_sinf(p);
        if (live) {
            unsafeAtomicAdd(&rho_r[n], __builtin_fmaf(dr, c, -di * s));
            unsafeAtomicAdd(&rho_i[n], __builtin_fmaf(dr, s, di * c));
        }
    }
}

}  // namespace
}  // namespace fhd

using namespace fhd;

extern "C" int fhd_scatter(const float *kx, const float *ky, const float *kz, const float *Dr,
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
    const int64_t zero_blocks = ((int64_t)N + kScatterBlock - 1) / kScatterBlock;
    fhd_zero_kernel<<<dim3((unsigned)zero_blocks), dim3(kScatterBlock), 0, s>>>(rho_r, rho_i, N);
    rc = launch_status("fhd_zero_kernel launch");
    if (rc != FHD_OK || M == 0) return rc;

    const int64_t sample_blocks = ((int64_t)M + kScatterBlock - 1) / kScatterBlock;
    int64_t slices = (kScatterMinBlocks + sample_blocks - 1) / sample_blocks;
    const int64_t max_slices = ((int64_t)N + kScatterMinSlice - 1) / kScatterMinSlice;
    if (slices > max_slices) slices = max_slices;
    if (slices < 1) slices = 1;
    fhd_scatter_kernel<<<dim3((unsigned)sample_blocks, (unsigned)slices), dim3(kScatterBlock), 0, s>>>(
        kx, ky, kz, Dr, Di, M, x, y, z, N, (int)slices, rho_r, rho_i);
    return launch_status("fhd_scatter_kernel launch");
}
