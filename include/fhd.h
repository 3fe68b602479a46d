/*
 * fhd.h -- C ABI of the MI355X (gfx950) F^H D library, libfhd.so.
 *
 * F^H D is the adjoint non-uniform discrete Fourier transform at the heart
 * of iterative non-Cartesian MRI reconstruction (page "Case study --
 * iterative MRI reconstruction", section 17.3, the F^H D equation):
 *
 *     rho_n = sum_{m < M} D_m * exp(+i * 2*pi * (kx_m*x_n + ky_m*y_n + kz_m*z_n))
 *
 * for every voxel n < N. k is in cycles per field of view and (x, y, z) in
 * field-of-view units. D_m = Dr[m] + i*Di[m] and rho_n = rho_r[n] +
 * i*rho_i[n]. There is no weighting and no normalisation. The argument
 * names and order follow the gather kernel on that page (section 17.3.1),
 * with a HIP stream added.
 *
 * Conventions shared by every entry point:
 *   - All arrays are fp32 (or the packed buffer, see fhd_pack), contiguous,
 *     4-byte aligned, in device memory of the current HIP device (or in
 *     pinned host memory the device can access). They are owned by the
 *     caller; the library never frees or retains them.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the default
 *     stream) and the call returns without synchronising. Calls on one
 *     stream run in order.
 *   - Outputs are overwritten, never accumulated into.
 *   - Temporaries (packed k-space, unit classes, factor tables, split
 *     partial sums) live in device buffers the library keeps per (device,
 *     stream) between calls, grown when a call needs more, until
 *     fhd_release_workspaces(). While `stream` is being captured into a
 *     graph, a call takes stream-ordered allocations (hipMallocAsync) and
 *     frees them (hipFreeAsync) instead. Calls on one stream from several
 *     host threads are serialised by the library.
 *   - Return value: FHD_OK (0) or a negative FHD_ERR_* status. Argument
 *     checks that need no device (null pointers, negative sizes, overlaps,
 *     alignment) run before any HIP call; then pointers are checked to be
 *     device-accessible, on the current device and large enough for the
 *     stated sizes. fhd_last_error() gives a message for the calling
 *     thread's last failure.
 */
#ifndef FHD_H
#define FHD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FHD_OK 0
#define FHD_ERR_INVALID_ARG (-1) /* bad pointer, size, alignment or overlap */
#define FHD_ERR_HIP (-2)         /* a HIP runtime or launch error */
#define FHD_ERR_ALLOC (-3)       /* the library could not get its workspace */

/*
 * Paths (the `paths` argument of the *_paths entry points). Voxels are
 * taken in units of 4096 consecutive ones. A unit whose aligned runs of 64
 * (or, for a pair of units, 128) voxels are lines along x with one common
 * step -- same y and z bitwise, x_v = x_0 + v dx rounded once to fp32; the
 * rows of any x-fastest grid whose rows are a multiple of 64 voxels -- can
 * be summed on the matrix cores: the voxels pair up about each line's
 * centre and F^H D (or F) becomes real matrix products of per-line centre
 * phasors and per-sample cos / sin factors (the same sum, evaluated in a
 * different order). Where, in four units (lines of 128) or two units
 * (lines of 64), the lines also come two by two as one line and that line
 * moved by one offset (the rows of a grid), F^H D pairs the voxels of each
 * two lines about their common centre instead, with half the per-line
 * work; where, in four units of lines of 64, they come four by four at
 * offsets 0, d, e and e + d from the first (rows y .. y + 3), about the
 * four lines' common centre, with a quarter. Every other unit is summed on
 * the vector ALUs in fp32.
 *
 *   FHD_GATHER_ALL    (the default of fhd_compute, fhd_gather, fhd_forward,
 *                     fhd_normal, fhd_cg) lines on the matrix cores with
 *                     fp32-class products: each fp32 operand is split into
 *                     an fp16 part and an fp16 remainder (22 significant
 *                     bits together; amplitudes scaled by a power of two
 *                     into fp16's range first, and the sums scaled back),
 *                     three fp16 products per fp32 product with fp32
 *                     accumulation: per product within 2^-21 relative of
 *                     the exact product at worst and about 2^-24 on
 *                     average, the order of fp32's own rounding (2^-24)
 *                     and below the hardware sine's error (about 2^-21).
 *   FHD_GATHER_VECTOR every unit on the vector ALUs in fp32.
 *   FHD_GATHER_BF16X3 lines on the matrix cores as above but with bf16 parts
 *                     (16 significant bits together): per product within
 *                     about 3 x 2^-17 relative, roughly 1e-5 relative on a
 *                     sum. Faster on some shapes; an explicit opt-in.
 */
#define FHD_GATHER_ALL 0
#define FHD_GATHER_VECTOR 1
#define FHD_GATHER_BF16X3 2

/* Arithmetic of the grid form's matrix products (fhd_compute_grid). */
#define FHD_GRID_FP32 0   /* fp32 matrix-core products, fp32 accumulation */
#define FHD_GRID_BF16X3 1 /* each fp32 operand split into two bf16 parts,
                             three bf16 products per fp32 product (the
                             lo x lo part, under 2^-17 relative, dropped),
                             fp32 accumulation */

/*
 * rho = F^H D over N voxels and M samples (section 17.3, F^H D equation).
 * Runs the loop-fission pre-pass (fhd_pack, section 17.3.2) into a
 * workspace of fhd_packed_bytes(M) bytes that the library keeps for
 * `stream`, then the gather (fhd_gather, one lane
 * per voxel with no atomics, section 17.3.1) with the default paths,
 * FHD_GATHER_ALL: units of lines along x on the matrix cores with
 * fp32-class split-fp16 products, the rest on the vector ALUs in fp32 (see
 * the paths above).
 *   kx, ky, kz, Dr, Di : M fp32 values each (read only)
 *   x, y, z            : N fp32 values each (read only)
 *   rho_r, rho_i       : N fp32 values each (written); they must not
 *                        overlap each other or any input
 *   M >= 0, N >= 0     : M = 0 writes zeros (an empty sum); N = 0 does
 *                        nothing. Pointers may be NULL only when the
 *                        matching size is 0.
 * Non-finite inputs give non-finite outputs where they enter the sum.
 * Errors: FHD_ERR_INVALID_ARG, FHD_ERR_ALLOC, FHD_ERR_HIP.
 */
int fhd_compute(const float *kx, const float *ky, const float *kz,
                const float *Dr, const float *Di,
                const float *x, const float *y, const float *z,
                float *rho_r, float *rho_i, int M, int N, void *stream);

/*
 * fhd_compute with a choice of paths (FHD_GATHER_ALL, FHD_GATHER_VECTOR or
 * FHD_GATHER_BF16X3; anything else is FHD_ERR_INVALID_ARG). Same arguments,
 * workspace and errors otherwise.
 */
int fhd_compute_paths(const float *kx, const float *ky, const float *kz,
                      const float *Dr, const float *Di,
                      const float *x, const float *y, const float *z,
                      float *rho_r, float *rho_i, int M, int N, int paths,
                      void *stream);

/*
 * rho = F^H D in the scatter form that section 17.3.1 compares with the
 * gather form: one lane per sample m adds D_m e^{+i 2 pi k_m . x_n} into
 * every rho_n with fp32 atomic adds (the compiler merges a wave's 64 adds to
 * one address into one). Kept as the measured evidence for fhd_compute's
 * gather form; slow by design at large N x M (every term ends in an atomic
 * path). The summation order varies from run to run, so results match
 * fhd_compute's to rounding only. No workspace.
 *   arguments : as for fhd_compute (same layout, ownership, overlap rules)
 * M = 0 writes zeros; N = 0 does nothing.
 * Errors: FHD_ERR_INVALID_ARG, FHD_ERR_HIP.
 */
int fhd_scatter(const float *kx, const float *ky, const float *kz,
                const float *Dr, const float *Di,
                const float *x, const float *y, const float *z,
                float *rho_r, float *rho_i, int M, int N, void *stream);

/*
 * Size in bytes of the packed k-space that fhd_pack writes for M samples,
 * or -1 if M < 0. M is padded up to a whole chunk of samples.
 */
int64_t fhd_packed_bytes(int M);

/*
 * Loop-fission pre-pass (section 17.3.2: move per-sample work out of the
 * voxel loop; section 17.3.4: keep a sample's values together). Packs the
 * SoA k-space into `packed`, chunk-interleaved records of (kx, ky, kz,
 * arg(D) in revolutions, |D|), zero-padded to a whole chunk. The padding
 * records have |D| = 0 and add exactly nothing.
 *   kx..Di       : M fp32 values each (read only)
 *   packed       : device buffer of at least packed_bytes bytes (written),
 *                  16-byte aligned, packed_bytes >= fhd_packed_bytes(M); it
 *                  must not overlap any input
 * M = 0 does nothing. Errors: FHD_ERR_INVALID_ARG, FHD_ERR_HIP.
 */
int fhd_pack(const float *kx, const float *ky, const float *kz,
             const float *Dr, const float *Di, int M,
             void *packed, int64_t packed_bytes, void *stream);

/*
 * Gather kernel over packed k-space (section 17.3.1, gather form; 17.3.3,
 * accumulators in registers; 17.3.4, every lane reads the same sample at
 * once; 17.3.5, hardware sin/cos). rho = F^H D for the M samples that
 * fhd_pack wrote into `packed` (same M), with the default paths
 * (FHD_GATHER_ALL: lines on the matrix cores in fp32-class split fp16, the
 * rest on the vector ALUs in fp32).
 *   packed       : fhd_packed_bytes(M) bytes written by fhd_pack (read only),
 *                  16-byte aligned
 *   x, y, z      : N fp32 values each (read only)
 *   rho_r, rho_i : N fp32 values each (written), not overlapping any input
 * M = 0 writes zeros; N = 0 does nothing. The per-voxel summation order is
 * fixed, so repeated calls give bitwise identical results. The library
 * allocates and frees a stream-ordered workspace on `stream`: the unit
 * classes, on the matrix-core paths the samples' cos / sin factor table
 * (16 KB per 32 samples: 49 MB at M = 100,000), and the partial sums
 * (2 x 4 bytes per voxel and part) when the voxels are too few to fill
 * the GPU in one pass over the samples.
 * Errors: FHD_ERR_INVALID_ARG, FHD_ERR_ALLOC, FHD_ERR_HIP.
 */
int fhd_gather(const void *packed, int M,
               const float *x, const float *y, const float *z,
               float *rho_r, float *rho_i, int N, void *stream);

/*
 * fhd_gather with a choice of paths: FHD_GATHER_ALL (identical to
 * fhd_gather), FHD_GATHER_VECTOR (every unit on the vector ALUs in fp32)
 * or FHD_GATHER_BF16X3 (lines on the matrix cores in split bf16). Other
 * arguments and errors as fhd_gather; any other `paths` is
 * FHD_ERR_INVALID_ARG.
 */
int fhd_gather_paths(const void *packed, int M,
                     const float *x, const float *y, const float *z,
                     float *rho_r, float *rho_i, int N, int paths, void *stream);

/*
 * Forward operator F (image to k-space; page "Case study -- iterative MRI
 * reconstruction", section 17.2, with F^H of section 17.3 its adjoint):
 *
 *     D_m = sum_{n < N} rho_n * exp(-i * 2*pi * (kx_m*x_n + ky_m*y_n + kz_m*z_n))
 *
 * for every sample m < M. Runs a per-voxel pre-pass (fhd_forward_pack) into
 * a stream-ordered workspace of fhd_packed_bytes(N) bytes, then the gather
 * kernel with one lane per sample (fhd_forward_gather), no atomics.
 *   kx, ky, kz         : M fp32 values each (read only)
 *   x, y, z, rho_r/_i  : N fp32 values each (read only)
 *   Dr, Di             : M fp32 values each (written), not overlapping any
 *                        input
 *   M = 0 does nothing; N = 0 writes zeros (an empty sum).
 * When every aligned pair of 4096-voxel units consists of lines of 128
 * voxels along x with one common step (same y and z bitwise, x_v = x_0 +
 * v dx rounded once; any x-fastest grid whose rows are a multiple of 128
 * voxels and whose voxel count is a multiple of 8192), F runs on the
 * matrix cores with fp32-class split-fp16 products (FHD_GATHER_ALL; each
 * line's operands scaled by its own power of two). When, beyond that, the
 * lines 2i + 1 of every unit are the lines 2i moved by one common offset
 * (bitwise equal differences of their first voxels' x, y, z; any such grid
 * with an even number of rows per slice, or rows of 256), F sums each such
 * line pair about its centre (one phasor per line pair and sample; each
 * tile of 16 line pairs scaled by one power of two). Units of lines of 64
 * voxels with one step take the same form where their lines come four by
 * four at offsets 0, d, e and e + d from the first, common to all units
 * (rows y .. y + 3 of a grid with rows of 64): one phasor per four lines.
 * Otherwise F runs on the vector ALUs in fp32 (the form fhd_forward_pack
 * / fhd_forward_gather always take). The choice is made on the device; the library allocates
 * its stream-ordered workspaces on `stream`.
 * Errors: FHD_ERR_INVALID_ARG, FHD_ERR_ALLOC, FHD_ERR_HIP.
 */
int fhd_forward(const float *kx, const float *ky, const float *kz,
                const float *x, const float *y, const float *z,
                const float *rho_r, const float *rho_i,
                float *Dr, float *Di, int M, int N, void *stream);

/*
 * fhd_forward with a choice of paths: FHD_GATHER_ALL (identical to
 * fhd_forward), FHD_GATHER_VECTOR (the vector form always) or
 * FHD_GATHER_BF16X3 (the line-pair or line form in split bf16 where it
 * applies). Any other value is FHD_ERR_INVALID_ARG; otherwise as
 * fhd_forward.
 */
int fhd_forward_paths(const float *kx, const float *ky, const float *kz,
                      const float *x, const float *y, const float *z,
                      const float *rho_r, const float *rho_i,
                      float *Dr, float *Di, int M, int N, int paths, void *stream);

/*
 * Pre-pass of F: packs the voxels and the image into `packed` in the record
 * format of fhd_pack (x, y, z, -arg(rho) in revolutions, |rho|), N padded to
 * a whole chunk; the size is fhd_packed_bytes(N).
 *   x, y, z, rho_r, rho_i : N fp32 values each (read only)
 *   packed                : device buffer, 16-byte aligned, packed_bytes >=
 *                           fhd_packed_bytes(N), not overlapping any input
 * N = 0 does nothing. Errors: FHD_ERR_INVALID_ARG, FHD_ERR_HIP.
 */
int fhd_forward_pack(const float *x, const float *y, const float *z,
                     const float *rho_r, const float *rho_i, int N,
                     void *packed, int64_t packed_bytes, void *stream);

/*
 * Gather of F over packed voxels (written by fhd_forward_pack with the same
 * N): D = F rho for the M samples.
 *   packed     : fhd_packed_bytes(N) bytes, 16-byte aligned (read only)
 *   kx, ky, kz : M fp32 values each (read only)
 *   Dr, Di     : M fp32 values each (written), not overlapping any input
 * M = 0 does nothing; N = 0 writes zeros. Repeated calls are bitwise
 * identical. Errors: FHD_ERR_INVALID_ARG, FHD_ERR_HIP.
 */
int fhd_forward_gather(const void *packed, int N,
                       const float *kx, const float *ky, const float *kz,
                       float *Dr, float *Di, int M, void *stream);

/*
 * Normal operator q = F^H F p, the product inside each conjugate-gradient
 * iteration (section 17.2; split by loop fission into F and F^H, section
 * 17.3.2). Runs F into a k-space temporary and F^H back, all in one
 * stream-ordered workspace of fhd_packed_bytes(N) + fhd_packed_bytes(M) +
 * 8*M bytes (plus the smaller ones fhd_forward and fhd_gather take). F and
 * F^H each take their matrix-core form (fp32-class split fp16) where
 * fhd_forward and fhd_gather would.
 *   kx, ky, kz       : M fp32 values each (read only)
 *   x, y, z, p_r/_i  : N fp32 values each (read only)
 *   q_r, q_i         : N fp32 values each (written), not overlapping any
 *                      input
 *   N = 0 does nothing; M = 0 writes zeros.
 * Errors: FHD_ERR_INVALID_ARG, FHD_ERR_ALLOC, FHD_ERR_HIP.
 */
int fhd_normal(const float *kx, const float *ky, const float *kz,
               const float *x, const float *y, const float *z,
               const float *p_r, const float *p_i,
               float *q_r, float *q_i, int M, int N, void *stream);

/* fhd_normal with a choice of paths for both F and F^H (as
 * fhd_forward_paths and fhd_gather_paths). */
int fhd_normal_paths(const float *kx, const float *ky, const float *kz,
                     const float *x, const float *y, const float *z,
                     const float *p_r, const float *p_i,
                     float *q_r, float *q_i, int M, int N, int paths, void *stream);

/*
 * F^H D for voxels on a Cartesian grid, as a complex matrix product on the
 * matrix cores (the exponential of section 17.3's F^H D equation factors
 * over the axes). Voxel n = ix + nx*(iy + ny*iz) has coordinates
 * (x0 + ix*dx, y0 + iy*dy, z0 + iz*dz), each computed in double and rounded
 * once to fp32; with explicit coordinate arrays holding those values, the
 * result equals fhd_compute's up to rounding.
 *   kx, ky, kz, Dr, Di : M fp32 values each (read only)
 *   nx, ny, nz >= 0    : grid size, nx*ny*nz < 2^31
 *   axis               : HOST array of 6 floats {x0, dx, y0, dy, z0, dz},
 *                        finite, read during the call
 *   precision          : FHD_GRID_FP32 or FHD_GRID_BF16X3 (about 1e-5
 *                        relative per term, within the same tolerance as
 *                        fp32 here, and several times faster)
 *   rho_r, rho_i       : nx*ny*nz fp32 values each (written), not
 *                        overlapping any input
 * Runs fhd_pack into a stream-ordered workspace, then fhd_grid_gather.
 * M = 0 writes zeros; an empty grid does nothing.
 * Errors: FHD_ERR_INVALID_ARG, FHD_ERR_ALLOC, FHD_ERR_HIP.
 */
int fhd_compute_grid(const float *kx, const float *ky, const float *kz,
                     const float *Dr, const float *Di, int M,
                     int nx, int ny, int nz, const float *axis, int precision,
                     float *rho_r, float *rho_i, void *stream);

/*
 * The matrix-core gather of fhd_compute_grid over k-space packed by
 * fhd_pack (same M; 16-byte aligned). Same grid arguments, precision and
 * outputs. Repeated calls are bitwise identical. Errors:
 * FHD_ERR_INVALID_ARG, FHD_ERR_ALLOC (split partial sums), FHD_ERR_HIP.
 */
int fhd_grid_gather(const void *packed, int M, int nx, int ny, int nz,
                    const float *axis, int precision, float *rho_r, float *rho_i,
                    void *stream);

/*
 * D = F rho (page "Case study -- iterative MRI reconstruction", section 17.2:
 * F maps the image to k-space, D_m = sum_n rho_n exp(-i 2 pi k_m . x_n))
 * for rho on the Cartesian grid of fhd_compute_grid (same voxel order and
 * coordinates), as a complex (ny*nz x nx) by (nx x M) matrix product on
 * the matrix cores followed by the (y, z) phases and a sum over rows.
 *   kx, ky, kz   : M fp32 values each (read only)
 *   nx, ny, nz   : grid size, nx*ny*nz < 2^31
 *   axis         : HOST array {x0, dx, y0, dy, z0, dz}, finite
 *   precision    : FHD_GRID_BF16X3 (the only mode of this call)
 *   rho_r, rho_i : nx*ny*nz fp32 values each (read only)
 *   Dr, Di       : M fp32 values each (written), not overlapping any input
 * Per-workgroup partial sums live in a stream-ordered workspace and are
 * added in a fixed order: repeated calls are bitwise identical. M = 0 does
 * nothing; an empty grid writes zeros.
 * Errors: FHD_ERR_INVALID_ARG, FHD_ERR_ALLOC, FHD_ERR_HIP.
 */
int fhd_forward_grid(const float *kx, const float *ky, const float *kz, int M,
                     int nx, int ny, int nz, const float *axis, int precision,
                     const float *rho_r, const float *rho_i, float *Dr, float *Di,
                     void *stream);

/*
 * Conjugate-gradient reconstruction (page "Case study -- iterative MRI
 * reconstruction", section 17.2 and its CG skeleton after section 17.3.6)
 * with the regulariser left out (the pages do not specify R or lambda):
 * solves F^H F rho = F^H D from rho = 0. Each iteration applies F^H F once
 * (fhd_normal) and two inner products (fp64 accumulation, fixed reduction
 * order: bitwise repeatable). The CG scalars stay in device memory: an
 * iteration is enqueued with no host round trip, the host checks the stop
 * flag once per 8 iterations, and reads the iteration count and residual
 * history back at the end, so this call synchronises `stream` and blocks
 * the calling thread.
 *   kx, ky, kz, Dr, Di : M fp32 values each (read only)
 *   x, y, z            : N fp32 values each (read only)
 *   rho_r, rho_i       : N fp32 values each (written: the last iterate),
 *                        not overlapping any input
 *   max_iter >= 0      : iteration limit
 *   tol >= 0           : stop once the squared residual norm ||r||^2 falls
 *                        below tol (absolute, as on the pages)
 *   iters_done         : host int, set to the iterations run
 *   residuals          : host array of max_iter + 1 floats or NULL; entry k
 *                        is ||r_k||^2 (entry 0 is ||F^H D||^2)
 * The workspace of fhd_cg_workspace_bytes(M, N, max_iter) bytes is
 * allocated and freed on `stream`. Errors: FHD_ERR_INVALID_ARG, FHD_ERR_ALLOC, FHD_ERR_HIP.
 */
int fhd_cg(const float *kx, const float *ky, const float *kz,
           const float *Dr, const float *Di,
           const float *x, const float *y, const float *z,
           float *rho_r, float *rho_i, int M, int N, int max_iter, float tol,
           int *iters_done, float *residuals, void *stream);

/* fhd_cg with a choice of paths for every F and F^H it applies
 * (FHD_GATHER_ALL, the default, FHD_GATHER_VECTOR or FHD_GATHER_BF16X3;
 * anything else is FHD_ERR_INVALID_ARG). */
int fhd_cg_paths(const float *kx, const float *ky, const float *kz,
                 const float *Dr, const float *Di,
                 const float *x, const float *y, const float *z,
                 float *rho_r, float *rho_i, int M, int N, int max_iter, float tol,
                 int *iters_done, float *residuals, int paths, void *stream);

/* Workspace bytes fhd_cg allocates for M samples, N voxels and max_iter
 * iterations (-1 if any is negative). */
int64_t fhd_cg_workspace_bytes(int M, int N, int max_iter);

/*
 * F^H F p on the Cartesian grid of fhd_compute_grid: fhd_forward_grid into a
 * stream-ordered workspace, then the grid F^H (loop fission, as fhd_normal;
 * section 17.3.2 names F^H F).
 *   kx, ky, kz : M fp32 (read only); nx, ny, nz, axis: as fhd_compute_grid
 *   precision  : FHD_GRID_BF16X3 (the only mode)
 *   p_r, p_i   : nx*ny*nz fp32 (read only)
 *   q_r, q_i   : nx*ny*nz fp32 (written), not overlapping any input
 * M = 0 writes zeros; an empty grid does nothing.
 * Errors: FHD_ERR_INVALID_ARG, FHD_ERR_ALLOC, FHD_ERR_HIP.
 */
int fhd_normal_grid(const float *kx, const float *ky, const float *kz, int M,
                    int nx, int ny, int nz, const float *axis, int precision,
                    const float *p_r, const float *p_i, float *q_r, float *q_i,
                    void *stream);

/*
 * fhd_cg with the voxels on the Cartesian grid of fhd_compute_grid and the
 * matrix-core operators (F^H D and F^H F as fhd_compute_grid and
 * fhd_normal_grid). Same iteration, scalars, stopping rule and outputs as
 * fhd_cg; rho_r, rho_i hold nx*ny*nz values. precision: FHD_GRID_BF16X3.
 * The workspace is fhd_cg_workspace_bytes(M, nx*ny*nz, max_iter) bytes,
 * stream-ordered; the call synchronises `stream`.
 * Errors: FHD_ERR_INVALID_ARG, FHD_ERR_ALLOC, FHD_ERR_HIP.
 */
int fhd_cg_grid(const float *kx, const float *ky, const float *kz,
                const float *Dr, const float *Di, int M,
                int nx, int ny, int nz, const float *axis, int precision,
                float *rho_r, float *rho_i, int max_iter, float tol,
                int *iters_done, float *residuals, void *stream);

/*
 * Launch shape of the gather kernel: voxels per lane, samples per packed
 * chunk and workgroup size (threads). Any pointer may be NULL.
 */
void fhd_gather_config(int *voxels_per_lane, int *samples_per_chunk, int *block_threads);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * fhd_compute_paths (same arguments, same results bit for bit) with every
 * temporary -- the packed k-space, the unit classes and the split partial
 * sums -- in one device array of FHD_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held from the library's first use of that GPU
 * until the process ends. The call allocates and frees nothing.
 *   - The workspace needed is about 20 bytes per sample (rounded up to 8
 *     samples), 8 bytes per 4096 voxels plus 272, and, when the voxels are
 *     too few to fill the GPU in one pass over the samples, 8 bytes per
 *     voxel for each partial sum: as many as the instance that takes most
 *     of an x-fastest grid needs to fill the GPU (4 at 128^3 voxels, 32 at
 *     64^3), the other instances' within the larger of that and 48 MiB;
 *     the call computes it exactly and returns FHD_ERR_INVALID_ARG, saying
 *     how many bytes it needed, when it exceeds the array. 128^3 voxels x
 *     100,000 samples needs about 66 MiB; 256^3 x 100,000 about 3 MiB.
 *   - Every call on one GPU uses that GPU's array: calls that overlap on
 *     one GPU (on different streams, or from different threads without
 *     ordering) race and give wrong results. Calls on one stream are
 *     ordered and safe. Nothing in the array needs clearing between calls.
 *   - The long-line and line-pair forms build their cos / sin factor
 *     operands inside each workgroup instead of from a per-call table
 *     (slower), with the same arithmetic: the results equal
 *     fhd_compute_paths' bit for bit except on grids where some quads of
 *     line pairs (or four-line groups, or unit pairs of 64-voxel line
 *     pairs) differ from the first one's step or offsets, which
 *     fhd_compute_paths sums in the next form down (long lines, 64-voxel
 *     line pairs or lines) and this entry point as they are (both within
 *     the same bound).
 * Errors: FHD_ERR_INVALID_ARG (also for a workspace beyond the array),
 * FHD_ERR_HIP.
 */
#define FHD_NOALLOC_SCRATCH_BYTES (128 * 1024 * 1024)
int fhd_compute_noalloc(const float *kx, const float *ky, const float *kz,
                        const float *Dr, const float *Di,
                        const float *x, const float *y, const float *z,
                        float *rho_r, float *rho_i, int M, int N, int paths,
                        void *stream);

/*
 * Measurement hook, not part of any computation. After this call, the
 * calling thread's next `count` launches of the library kernel named
 * `kernel` record events[2*i] on their stream just before launch i and
 * events[2*i + 1] just after it, so hipEventElapsedTime(events[2*i],
 * events[2*i + 1]) is that launch's duration on the GPU. Names are the
 * kernels' as a profiler lists them, with template arguments:
 * "fhd_gather_patch_kernel<true, true>" (quads of 128-voxel line pairs or
 * of four-line groups of 64-voxel lines, split fp16, B table) or "<false,
 * true>" (split bf16), "<true, false>"/"<false, false>" (B formed in the
 * workgroups), "fhd_gather_patch64_kernel<...>" (the same for unit pairs
 * of 64-voxel line pairs), "fhd_gather_long_lines_kernel<true>" (split
 * fp16) or "<false>" (split bf16), "fhd_gather_lines_kernel<true>"/"<false>",
 * "fhd_gather_kernel<16, true>" (one-step ramps) or "<16, false>",
 * "fhd_forward_pairs_kernel<true>"/"<false>" (line pairs),
 * "fhd_forward_lines_kernel<true>"/"<false>",
 * "fhd_forward_gather_kernel<2>", "fhd_grid_kernel",
 * "fhd_grid_bf16x3_kernel<4>"/"<2>", "fhd_forward_grid_bf16x3_kernel".
 *   kernel : NUL-terminated name (copied), or NULL to disarm
 *   events : 2*count hipEvent_t created by the caller (the handles are
 *            copied; the events must live until they have been recorded)
 *   count  : launches to record, >= 0 (0 disarms)
 * Launches past `count`, of other kernels or on other threads record
 * nothing. Errors: FHD_ERR_INVALID_ARG (count < 0, NULL events or a NULL
 * handle among them; the hook is then disarmed).
 */
int fhd_time_kernel(const char *kernel, void *const *events, int count);

/* Launches recorded on the calling thread since its last fhd_time_kernel. */
int fhd_timed_launches(void);

/*
 * Frees every workspace the library keeps (see the conventions above),
 * after waiting for all work on each device that holds one. The next call
 * on a stream allocates again. Not to be called while another thread is
 * inside a library call. Errors: FHD_ERR_HIP.
 */
int fhd_release_workspaces(void);

/* Static description of a status code. Never NULL. */
const char *fhd_status_string(int status);

/* Message for the calling thread's most recent failure ("" if none). */
const char *fhd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FHD_H */
