// fhd_cg.hip -- conjugate-gradient reconstruction on the normal equations.
//
// Page "Case study -- iterative MRI reconstruction", section 17.2 states the
// reconstruction as argmin_rho ||F rho - D||^2 + lambda R(rho) and solves it
// with conjugate gradients, whose loop (the CG skeleton after section 17.3.6)
// needs b = F^H D once and F^H F p every iteration. The regulariser R is not
// specified on the pages, so this solves lambda = 0:
//
//     F^H F rho = F^H D,  rho_0 = 0,  r_0 = p_0 = b,  rs_0 = <r_0, r_0>
//     repeat: Ap = F^H F p;  alpha = rs / <p, Ap>
//             rho += alpha p;  r -= alpha Ap;  rs' = <r, r>
//             stop if rs' < tol;  p = r + (rs' / rs) p;  rs = rs'
//
// Vectors are complex fp32 (separate real and imaginary arrays); inner
// products are Re sum conj(u) v accumulated in fp64 by a two-stage
// reduction with a fixed order (per-block partials, then one block), so
// every run is bitwise repeatable. As on the pages, the scalars come back
// to the host each iteration (two 8-byte reads), which decides the early
// stop; F^H F dominates the iteration by orders of magnitude.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <string>
#include <vector>

#include "fhd_internal.h"

namespace fhd {
namespace {

constexpr int kVecBlock = 256;
constexpr int kDotBlocks = 1024;   // partial sums per inner product

// partial[b] = sum over the block's grid-stride share of (ur*vr + ui*vi)
__global__ __launch_bounds__(kVecBlock) void dot_partial_kernel(
    const float *__restrict__ ur, const float *__restrict__ ui, const float *__restrict__ vr,
    const float *__restrict__ vi, int64_t n, double *__restrict__ partial)
{
    __shared__ double red[kVecBlock];
    double acc = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * kVecBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kVecBlock)
        acc += (double)ur[i] * vr[i] + (double)ui[i] * vi[i];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = kVecBlock / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

// out[0] = sum of partial[0 .. count) in a fixed order
__global__ __launch_bounds__(kVecBlock) void dot_final_kernel(const double *__restrict__ partial,
                                                              int count, double *__restrict__ out)
{
    __shared__ double red[kVecBlock];
    double acc = 0.0;
    for (int i = threadIdx.x; i < count; i += kVecBlock) acc += partial[i];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = kVecBlock / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = red[0];
}

// rho += alpha p;  r -= alpha Ap
__global__ __launch_bounds__(kVecBlock) void cg_step_kernel(
    float *__restrict__ rho_r, float *__restrict__ rho_i, float *__restrict__ r_r,
    float *__restrict__ r_i, const float *__restrict__ p_r, const float *__restrict__ p_i,
    const float *__restrict__ ap_r, const float *__restrict__ ap_i, float alpha, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * kVecBlock + threadIdx.x;
    if (i >= n) return;
    rho_r[i] = __builtin_fmaf(alpha, p_r[i], rho_r[i]);
    rho_i[i] = __builtin_fmaf(alpha, p_i[i], rho_i[i]);
    r_r[i] = __builtin_fmaf(-alpha, ap_r[i], r_r[i]);
    r_i[i] = __builtin_fmaf(-alpha, ap_i[i], r_i[i]);
}

// p = r + beta p
__global__ __launch_bounds__(kVecBlock) void cg_direction_kernel(
    float *__restrict__ p_r, float *__restrict__ p_i, const float *__restrict__ r_r,
    const float *__restrict__ r_i, float beta, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * kVecBlock + threadIdx.x;
    if (i >= n) return;
    p_r[i] = __builtin_fmaf(beta, p_r[i], r_r[i]);
    p_i[i] = __builtin_fmaf(beta, p_i[i], r_i[i]);
}

// rho = 0;  p = r
__global__ __launch_bounds__(kVecBlock) void cg_start_kernel(
    float *__restrict__ rho_r, float *__restrict__ rho_i, float *__restrict__ p_r,
    float *__restrict__ p_i, const float *__restrict__ r_r, const float *__restrict__ r_i,
    int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * kVecBlock + threadIdx.x;
    if (i >= n) return;
    rho_r[i] = 0.0f;
    rho_i[i] = 0.0f;
    p_r[i] = r_r[i];
    p_i[i] = r_i[i];
}

unsigned vec_blocks(int64_t n) { return (unsigned)((n + kVecBlock - 1) / kVecBlock); }

struct CgWork {
    float *r_r, *r_i, *p_r, *p_i, *ap_r, *ap_i;   // N each
    float *vox, *smp, *d_r, *d_i;                 // normal-operator temporaries
    double *partial, *scalar;
};

// <u, v> into host `out` (synchronises the stream)
int dot(const float *ur, const float *ui, const float *vr, const float *vi, int64_t n,
        const CgWork &w, hipStream_t s, double *out)
{
    const int blocks = (int)std::min<int64_t>(kDotBlocks, std::max<int64_t>(1, vec_blocks(n)));
    dot_partial_kernel<<<blocks, kVecBlock, 0, s>>>(ur, ui, vr, vi, n, w.partial);
    dot_final_kernel<<<1, kVecBlock, 0, s>>>(w.partial, blocks, w.scalar);
    int rc = launch_status("dot kernels launch");
    if (rc != FHD_OK) return rc;
    hipError_t e = hipMemcpyAsync(out, w.scalar, sizeof(double), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(FHD_ERR_HIP, std::string("dot readback: ") + hipGetErrorString(e));
    return FHD_OK;
}

// Ap = F^H F p
int normal(const float *kx, const float *ky, const float *kz, const float *x, const float *y,
           const float *z, int M, int N, const CgWork &w, hipStream_t s)
{
    int rc = launch_forward_pack(x, y, z, w.p_r, w.p_i, N, w.vox, s);
    if (rc == FHD_OK) rc = launch_forward_gather(w.vox, N, kx, ky, kz, w.d_r, w.d_i, M, s);
    if (rc == FHD_OK) rc = launch_pack(kx, ky, kz, w.d_r, w.d_i, M, w.smp, s);
    if (rc == FHD_OK) rc = launch_gather(w.smp, M, x, y, z, w.ap_r, w.ap_i, N, s);
    return rc;
}

int run_cg(const float *kx, const float *ky, const float *kz, const float *Dr, const float *Di,
           const float *x, const float *y, const float *z, float *rho_r, float *rho_i, int M, int N,
           int max_iter, float tol, int *iters_done, float *residuals, const CgWork &w,
           hipStream_t s)
{
    const int64_t n = N;
    // b = F^H D into r; rho = 0; p = r
    int rc = launch_pack(kx, ky, kz, Dr, Di, M, w.smp, s);
    if (rc == FHD_OK) rc = launch_gather(w.smp, M, x, y, z, w.r_r, w.r_i, N, s);
    if (rc != FHD_OK) return rc;
    cg_start_kernel<<<vec_blocks(n), kVecBlock, 0, s>>>(rho_r, rho_i, w.p_r, w.p_i, w.r_r, w.r_i, n);
    if ((rc = launch_status("cg_start_kernel launch")) != FHD_OK) return rc;
    double rs = 0.0;
    if ((rc = dot(w.r_r, w.r_i, w.r_r, w.r_i, n, w, s, &rs)) != FHD_OK) return rc;
    if (residuals) residuals[0] = (float)rs;
    int it = 0;
    while (it < max_iter && !(rs < (double)tol) && rs > 0.0) {
        if ((rc = normal(kx, ky, kz, x, y, z, M, N, w, s)) != FHD_OK) return rc;
        double pap = 0.0;
        if ((rc = dot(w.p_r, w.p_i, w.ap_r, w.ap_i, n, w, s, &pap)) != FHD_OK) return rc;
        if (!(pap > 0.0)) break;   // p is in the null space of F: nothing left to do
        const float alpha = (float)(rs / pap);
        cg_step_kernel<<<vec_blocks(n), kVecBlock, 0, s>>>(rho_r, rho_i, w.r_r, w.r_i, w.p_r, w.p_i,
                                                           w.ap_r, w.ap_i, alpha, n);
        if ((rc = launch_status("cg_step_kernel launch")) != FHD_OK) return rc;
        double rs_new = 0.0;
        if ((rc = dot(w.r_r, w.r_i, w.r_r, w.r_i, n, w, s, &rs_new)) != FHD_OK) return rc;
        ++it;
        if (residuals) residuals[it] = (float)rs_new;
        if (rs_new < (double)tol) {
            rs = rs_new;
            break;
        }
        const float beta = (float)(rs_new / rs);
        cg_direction_kernel<<<vec_blocks(n), kVecBlock, 0, s>>>(w.p_r, w.p_i, w.r_r, w.r_i, beta, n);
        if ((rc = launch_status("cg_direction_kernel launch")) != FHD_OK) return rc;
        rs = rs_new;
    }
    *iters_done = it;
    return FHD_OK;
}

}  // namespace
}  // namespace fhd

using namespace fhd;

extern "C" int64_t fhd_cg_workspace_bytes(int M, int N)
{
    if (M < 0 || N < 0) return -1;
    const int64_t nb = (int64_t)N * 4, mb = (int64_t)M * 4;
    auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
    return 6 * up(nb) + up(packed_bytes_for(N)) + up(packed_bytes_for(M)) + 2 * up(mb) +
           up(kDotBlocks * 8) + up(8);
}

extern "C" int fhd_cg(const float *kx, const float *ky, const float *kz, const float *Dr,
                      const float *Di, const float *x, const float *y, const float *z,
                      float *rho_r, float *rho_i, int M, int N, int max_iter, float tol,
                      int *iters_done, float *residuals, void *stream)
{
    clear_error();
    if (M < 0) return fail(FHD_ERR_INVALID_ARG, "M < 0");
    if (N < 0) return fail(FHD_ERR_INVALID_ARG, "N < 0");
    if (max_iter < 0) return fail(FHD_ERR_INVALID_ARG, "max_iter < 0");
    if (!iters_done) return fail(FHD_ERR_INVALID_ARG, "iters_done is NULL");
    if (!(tol >= 0.0f)) return fail(FHD_ERR_INVALID_ARG, "tol must be >= 0");
    *iters_done = 0;
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
    char *ws = nullptr;
    const int64_t bytes = fhd_cg_workspace_bytes(M, N);
    hipError_t e = hipMallocAsync((void **)&ws, (size_t)bytes, s);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(FHD_ERR_ALLOC, std::string("hipMallocAsync: ") + hipGetErrorString(e));
    }
    auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
    char *c = ws;
    auto take = [&](int64_t b) {
        char *p = c;
        c += up(b);
        return p;
    };
    CgWork w;
    w.r_r = (float *)take(nb);
    w.r_i = (float *)take(nb);
    w.p_r = (float *)take(nb);
    w.p_i = (float *)take(nb);
    w.ap_r = (float *)take(nb);
    w.ap_i = (float *)take(nb);
    w.vox = (float *)take(packed_bytes_for(N));
    w.smp = (float *)take(packed_bytes_for(M));
    w.d_r = (float *)take(mb);
    w.d_i = (float *)take(mb);
    w.partial = (double *)take(kDotBlocks * 8);
    w.scalar = (double *)take(8);
    rc = run_cg(kx, ky, kz, Dr, Di, x, y, z, rho_r, rho_i, M, N, max_iter, tol, iters_done,
                residuals, w, s);
    e = hipFreeAsync(ws, s);
    if (e != hipSuccess && rc == FHD_OK)
        rc = fail(FHD_ERR_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(e));
    return rc;
}
