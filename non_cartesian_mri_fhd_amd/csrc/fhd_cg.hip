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
// every run is bitwise repeatable. The scalars (rs, <p, Ap>, alpha, beta,
// the iteration count and the residual history) live in device memory and
// are produced and consumed by kernels, so an iteration is a fixed launch
// sequence with no host round trip. Once the stopping rule fires, a device
// flag turns the remaining updates into no-ops; the host looks at that flag
// only between batches of kBatch iterations (skipping batches that would do
// nothing) and reads the count and history back once at the end.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
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
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

// Device-resident CG scalars. `active` is 1 while iterating; the kernels of
// an iteration do nothing once it is 0.
struct CgState {
    double rs;        // ||r||^2 of the current residual
    double pap;       // <p, Ap>
    float alpha, beta;
    int active;
    int iters;        // iterations completed
};

// Stage 2 of the inner products: sum the partials in a fixed order, then
// thread 0 applies one step of the CG scalar logic.
enum class DotUse { kStart, kAlpha, kResidual };

template <DotUse USE>
__global__ __launch_bounds__(kVecBlock) void dot_final_kernel(const double *__restrict__ partial,
                                                              int count, CgState *st,
                                                              double *__restrict__ history,
                                                              int max_iter, float tol)
{
    __shared__ double red[kVecBlock];
    if (USE != DotUse::kStart && !st->active) return;
    double acc = 0.0;
    for (int i = threadIdx.x; i < count; i += kVecBlock) acc += partial[i];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = kVecBlock / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x != 0) return;
    const double v = red[0];
    if (USE == DotUse::kStart) {
        // rs_0 = ||F^H D||^2; iterate unless it is already small enough or zero
        st->rs = v;
        st->iters = 0;
        history[0] = v;
        st->active = (max_iter > 0 && !(v < (double)tol) && v > 0.0) ? 1 : 0;
    } else if (USE == DotUse::kAlpha) {
        st->pap = v;
        if (v > 0.0) {
            st->alpha = (float)(st->rs / v);
        } else {
            st->active = 0;   // p lies in the null space of F: nothing left to do
        }
    } else {
        const int k = st->iters + 1;
        st->iters = k;
        history[k] = v;
        if (v < (double)tol || !(v > 0.0) || k >= max_iter) {
            st->active = 0;
        } else {
            st->beta = (float)(v / st->rs);
            st->rs = v;
        }
    }
}

// rho += alpha p;  r -= alpha Ap
__global__ __launch_bounds__(kVecBlock) void cg_step_kernel(
    float *__restrict__ rho_r, float *__restrict__ rho_i, float *__restrict__ r_r,
    float *__restrict__ r_i, const float *__restrict__ p_r, const float *__restrict__ p_i,
    const float *__restrict__ ap_r, const float *__restrict__ ap_i, const CgState *st, int64_t n)
{
    if (!st->active) return;
    const float alpha = st->alpha;
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
    const float *__restrict__ r_i, const CgState *st, int64_t n)
{
    if (!st->active) return;
    const float beta = st->beta;
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

constexpr int kBatch = 8;   // iterations enqueued between looks at the stop flag

struct CgWork {
    float *r_r, *r_i, *p_r, *p_i, *ap_r, *ap_i;   // N each
    float *vox, *smp, *d_r, *d_i;                 // normal-operator temporaries
    double *partial;                              // kDotBlocks
    CgState *state;
    double *history;                              // max_iter + 1
};

// <u, v>, consumed on the device by dot_final_kernel<USE>
template <DotUse USE>
int dot(const float *ur, const float *ui, const float *vr, const float *vi, int64_t n,
        const CgWork &w, int max_iter, float tol, hipStream_t s)
{
    const int blocks = (int)std::min<int64_t>(kDotBlocks, std::max<int64_t>(1, vec_blocks(n)));
    dot_partial_kernel<<<blocks, kVecBlock, 0, s>>>(ur, ui, vr, vi, n, w.partial);
    dot_final_kernel<USE><<<1, kVecBlock, 0, s>>>(w.partial, blocks, w.state, w.history, max_iter,
                                                  tol);
    return launch_status("dot kernels launch");
}

// Ap = F^H F p
int normal(const float *kx, const float *ky, const float *kz, const float *x, const float *y,
           const float *z, int M, int N, const CgWork &w, hipStream_t s, int paths)
{
    int rc = launch_forward(x, y, z, w.p_r, w.p_i, N, kx, ky, kz, w.d_r, w.d_i, M, w.vox, s, paths);
    if (rc == FHD_OK) rc = launch_pack(kx, ky, kz, w.d_r, w.d_i, M, w.smp, s);
    if (rc == FHD_OK) rc = launch_gather(w.smp, M, x, y, z, w.ap_r, w.ap_i, N, s, paths);
    return rc;
}

int read_back(void *dst, const void *src, size_t bytes, hipStream_t s)
{
    hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(FHD_ERR_HIP, std::string("CG readback: ") + hipGetErrorString(e));
    return FHD_OK;
}

// The CG loop over operator callbacks: rhs() writes b = F^H D into w.r,
// normal() writes F^H F p (p in w.p) into w.ap; both enqueue on `s`.
template <class Rhs, class Normal>
int run_cg(Rhs &&rhs, Normal &&normal_op, float *rho_r, float *rho_i, int N, int max_iter, float tol,
           int *iters_done, float *residuals, const CgWork &w, hipStream_t s)
{
    const int64_t n = N;
    // b = F^H D into r; rho = 0; p = r; rs = <r, r>
    int rc = rhs();
    if (rc != FHD_OK) return rc;
    cg_start_kernel<<<vec_blocks(n), kVecBlock, 0, s>>>(rho_r, rho_i, w.p_r, w.p_i, w.r_r, w.r_i, n);
    if ((rc = launch_status("cg_start_kernel launch")) != FHD_OK) return rc;
    if ((rc = dot<DotUse::kStart>(w.r_r, w.r_i, w.r_r, w.r_i, n, w, max_iter, tol, s)) != FHD_OK)
        return rc;
    for (int launched = 0; launched < max_iter;) {
        int active = 0;
        if ((rc = read_back(&active, &w.state->active, sizeof(int), s)) != FHD_OK) return rc;
        if (!active) break;
        const int batch = std::min(kBatch, max_iter - launched);
        for (int b = 0; b < batch; ++b) {
            if ((rc = normal_op()) != FHD_OK) return rc;
            rc = dot<DotUse::kAlpha>(w.p_r, w.p_i, w.ap_r, w.ap_i, n, w, max_iter, tol, s);
            if (rc != FHD_OK) return rc;
            cg_step_kernel<<<vec_blocks(n), kVecBlock, 0, s>>>(rho_r, rho_i, w.r_r, w.r_i, w.p_r,
                                                               w.p_i, w.ap_r, w.ap_i, w.state, n);
            if ((rc = launch_status("cg_step_kernel launch")) != FHD_OK) return rc;
            rc = dot<DotUse::kResidual>(w.r_r, w.r_i, w.r_r, w.r_i, n, w, max_iter, tol, s);
            if (rc != FHD_OK) return rc;
            cg_direction_kernel<<<vec_blocks(n), kVecBlock, 0, s>>>(w.p_r, w.p_i, w.r_r, w.r_i,
                                                                    w.state, n);
            if ((rc = launch_status("cg_direction_kernel launch")) != FHD_OK) return rc;
        }
        launched += batch;
    }
    CgState st;
    if ((rc = read_back(&st, w.state, sizeof st, s)) != FHD_OK) return rc;
    *iters_done = st.iters;
    if (residuals) {
        std::vector<double> h((size_t)st.iters + 1);
        if ((rc = read_back(h.data(), w.history, h.size() * sizeof(double), s)) != FHD_OK) return rc;
        for (size_t k = 0; k < h.size(); ++k) residuals[k] = (float)h[k];
    }
    return FHD_OK;
}

// Carves the workspace of fhd_cg_workspace_bytes(M, N, max_iter) bytes
// (stream-ordered) into the CG vectors and scratch.
int64_t work_bytes(int M, int N, int max_iter)
{
    const int64_t nb = (int64_t)N * 4, mb = (int64_t)M * 4;
    auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
    return 6 * up(nb) + up(packed_bytes_for(N)) + up(packed_bytes_for(M)) + 2 * up(mb) +
           up(kDotBlocks * 8) + up(sizeof(CgState)) + up(((int64_t)max_iter + 1) * 8);
}

int alloc_work(int M, int N, int max_iter, hipStream_t s, char **ws, CgWork *w)
{
    const int64_t mb = (int64_t)M * 4, nb = (int64_t)N * 4;
    auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
    const int64_t bytes = work_bytes(M, N, max_iter);
    const hipError_t e = hipMallocAsync((void **)ws, (size_t)bytes, s);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(FHD_ERR_ALLOC, std::string("hipMallocAsync: ") + hipGetErrorString(e));
    }
    char *c = *ws;
    auto take = [&](int64_t b) {
        char *p = c;
        c += up(b);
        return p;
    };
    w->r_r = (float *)take(nb);
    w->r_i = (float *)take(nb);
    w->p_r = (float *)take(nb);
    w->p_i = (float *)take(nb);
    w->ap_r = (float *)take(nb);
    w->ap_i = (float *)take(nb);
    w->vox = (float *)take(packed_bytes_for(N));
    w->smp = (float *)take(packed_bytes_for(M));
    w->d_r = (float *)take(mb);
    w->d_i = (float *)take(mb);
    w->partial = (double *)take(kDotBlocks * 8);
    w->state = (CgState *)take(sizeof(CgState));
    w->history = (double *)take(((int64_t)max_iter + 1) * 8);
    return FHD_OK;
}

}  // namespace
}  // namespace fhd

using namespace fhd;

extern "C" int64_t fhd_cg_workspace_bytes(int M, int N, int max_iter)
{
    if (M < 0 || N < 0 || max_iter < 0) return -1;
    return work_bytes(M, N, max_iter);
}

extern "C" int fhd_cg_paths(const float *kx, const float *ky, const float *kz, const float *Dr,
                            const float *Di, const float *x, const float *y, const float *z,
                            float *rho_r, float *rho_i, int M, int N, int max_iter, float tol,
                            int *iters_done, float *residuals, int paths, void *stream)
{
    clear_error();
    if (M < 0) return fail(FHD_ERR_INVALID_ARG, "M < 0");
    if (N < 0) return fail(FHD_ERR_INVALID_ARG, "N < 0");
    if (max_iter < 0) return fail(FHD_ERR_INVALID_ARG, "max_iter < 0");
    if (!valid_paths(paths)) return fail_paths();
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
    CgWork w;
    if ((rc = alloc_work(M, N, max_iter, s, &ws, &w)) != FHD_OK) return rc;
    rc = run_cg(
        [&] {
            int r = launch_pack(kx, ky, kz, Dr, Di, M, w.smp, s);
            return r == FHD_OK ? launch_gather(w.smp, M, x, y, z, w.r_r, w.r_i, N, s, paths) : r;
        },
        [&] { return normal(kx, ky, kz, x, y, z, M, N, w, s, paths); }, rho_r, rho_i, N, max_iter, tol,
        iters_done, residuals, w, s);
    const hipError_t e = hipFreeAsync(ws, s);
    if (e != hipSuccess && rc == FHD_OK)
        rc = fail(FHD_ERR_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(e));
    return rc;
}

extern "C" int fhd_cg(const float *kx, const float *ky, const float *kz, const float *Dr,
                      const float *Di, const float *x, const float *y, const float *z,
                      float *rho_r, float *rho_i, int M, int N, int max_iter, float tol,
                      int *iters_done, float *residuals, void *stream)
{
    return fhd_cg_paths(kx, ky, kz, Dr, Di, x, y, z, rho_r, rho_i, M, N, max_iter, tol, iters_done,
                        residuals, FHD_GATHER_ALL, stream);
}

// ---------------------------------------------------------------------------
// The same on a Cartesian voxel grid with the matrix-core operators
// (F by fhd_forward_grid's kernel, F^H by fhd_grid_gather's).
// ---------------------------------------------------------------------------
namespace {
int check_grid_cg_args(int M, int nx, int ny, int nz, const float *axis, int precision, int64_t *N)
{
    if (M < 0) return fail(FHD_ERR_INVALID_ARG, "M < 0");
    if (nx < 0 || ny < 0 || nz < 0) return fail(FHD_ERR_INVALID_ARG, "negative grid size");
    const int64_t n = (int64_t)nx * ny * nz;
    if (n > INT32_MAX) return fail(FHD_ERR_INVALID_ARG, "nx*ny*nz exceeds 2^31 - 1");
    if (!axis) return fail(FHD_ERR_INVALID_ARG, "axis is NULL");
    for (int i = 0; i < 6; ++i)
        if (!std::isfinite(axis[i])) return fail(FHD_ERR_INVALID_ARG, "axis holds a non-finite value");
    if (precision != FHD_GRID_BF16X3)
        return fail(FHD_ERR_INVALID_ARG, "the grid operators F^H F and CG support FHD_GRID_BF16X3 only");
    *N = n;
    return FHD_OK;
}
}  // namespace

extern "C" int fhd_normal_grid(const float *kx, const float *ky, const float *kz, int M, int nx, int ny,
                               int nz, const float *axis, int precision, const float *p_r,
                               const float *p_i, float *q_r, float *q_i, void *stream)
{
    clear_error();
    int64_t N = 0;
    int rc = check_grid_cg_args(M, nx, ny, nz, axis, precision, &N);
    if (rc != FHD_OK || N == 0) return rc;
    const int64_t mb = (int64_t)M * 4, nb = N * 4;
    const Span all[] = {{kx, mb, "kx"}, {ky, mb, "ky"},   {kz, mb, "kz"},  {p_r, nb, "p_r"},
                        {p_i, nb, "p_i"}, {q_r, nb, "q_r"}, {q_i, nb, "q_i"}};
    rc = check_host_side(all, 7);
    if (rc == FHD_OK) rc = check_no_overlap(all, 7, 5);
    if (rc == FHD_OK) rc = check_device_spans(all, 7);
    if (rc != FHD_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (M == 0) return launch_reduce(nullptr, nullptr, 0, N, q_r, q_i, s);   // no samples: 0
    // workspace: D (2 M floats) and the packed samples
    const int64_t up_d = (2 * mb + 255) / 256 * 256;
    char *ws = nullptr;
    hipError_t e = hipMallocAsync((void **)&ws, (size_t)(up_d + packed_bytes_for(M)), s);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(FHD_ERR_ALLOC, std::string("hipMallocAsync: ") + hipGetErrorString(e));
    }
    float *d_r = (float *)ws, *d_i = d_r + M, *smp = (float *)(ws + up_d);
    rc = launch_forward_grid(p_r, p_i, nx, ny, nz, axis, precision, kx, ky, kz, M, d_r, d_i, s);
    if (rc == FHD_OK) rc = launch_pack(kx, ky, kz, d_r, d_i, M, smp, s);
    if (rc == FHD_OK) rc = launch_grid_gather(smp, M, nx, ny, nz, axis, precision, q_r, q_i, s);
    e = hipFreeAsync(ws, s);
    if (e != hipSuccess && rc == FHD_OK)
        rc = fail(FHD_ERR_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(e));
    return rc;
}

extern "C" int fhd_cg_grid(const float *kx, const float *ky, const float *kz, const float *Dr,
                           const float *Di, int M, int nx, int ny, int nz, const float *axis,
                           int precision, float *rho_r, float *rho_i, int max_iter, float tol,
                           int *iters_done, float *residuals, void *stream)
{
    clear_error();
    int64_t N64 = 0;
    int rc = check_grid_cg_args(M, nx, ny, nz, axis, precision, &N64);
    if (rc != FHD_OK) return rc;
    if (max_iter < 0) return fail(FHD_ERR_INVALID_ARG, "max_iter < 0");
    if (!iters_done) return fail(FHD_ERR_INVALID_ARG, "iters_done is NULL");
    if (!(tol >= 0.0f)) return fail(FHD_ERR_INVALID_ARG, "tol must be >= 0");
    *iters_done = 0;
    if (N64 == 0) return FHD_OK;
    const int N = (int)N64;
    const int64_t mb = (int64_t)M * 4, nb = N64 * 4;
    const Span all[] = {{kx, mb, "kx"}, {ky, mb, "ky"}, {kz, mb, "kz"}, {Dr, mb, "Dr"},
                        {Di, mb, "Di"}, {rho_r, nb, "rho_r"}, {rho_i, nb, "rho_i"}};
    rc = check_host_side(all, 7);
    if (rc == FHD_OK) rc = check_no_overlap(all, 7, 5);
    if (rc == FHD_OK) rc = check_device_spans(all, 7);
    if (rc != FHD_OK) return rc;

    hipStream_t s = (hipStream_t)stream;
    char *ws = nullptr;
    CgWork w;
    if ((rc = alloc_work(M, N, max_iter, s, &ws, &w)) != FHD_OK) return rc;
    rc = run_cg(
        [&] {
            if (M == 0) return launch_reduce(nullptr, nullptr, 0, N, w.r_r, w.r_i, s);
            int r = launch_pack(kx, ky, kz, Dr, Di, M, w.smp, s);
            return r == FHD_OK ? launch_grid_gather(w.smp, M, nx, ny, nz, axis, precision, w.r_r, w.r_i, s)
                               : r;
        },
        [&] {
            if (M == 0) return launch_reduce(nullptr, nullptr, 0, N, w.ap_r, w.ap_i, s);
            int r = launch_forward_grid(w.p_r, w.p_i, nx, ny, nz, axis, precision, kx, ky, kz, M, w.d_r,
                                        w.d_i, s);
            if (r == FHD_OK) r = launch_pack(kx, ky, kz, w.d_r, w.d_i, M, w.smp, s);
            return r == FHD_OK ? launch_grid_gather(w.smp, M, nx, ny, nz, axis, precision, w.ap_r, w.ap_i, s)
                               : r;
        },
        rho_r, rho_i, N, max_iter, tol, iters_done, residuals, w, s);
    const hipError_t e = hipFreeAsync(ws, s);
    if (e != hipSuccess && rc == FHD_OK)
        rc = fail(FHD_ERR_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(e));
    return rc;
}
