// fhd_internal.h -- shared pieces of libfhd.so's kernels and C ABI (not
// installed; the public interface is include/fhd.h).
//
// Both non-uniform DFT directions use one record format and one broadcast
// machine:
//
//  * A "packed" stream holds records of five fp32 fields -- three
//    coordinates, a phase offset in revolutions and an amplitude -- in
//    chunks of kChunk records, field-major inside a chunk
//    ([f0 x8][f1 x8][f2 x8][f3 x8][f4 x8], 160 B = ten float4). The tail
//    chunk is padded with amplitude-0 records, which add exactly 0.
//    F^H D streams k-space samples (kx, ky, kz, arg D / 2pi, |D|); the
//    forward F streams voxels (x, y, z, -arg rho / 2pi, |rho|).
//
//  * stream_chunks() walks a packed stream through LDS in stages of
//    kStageChunks chunks, double buffered: while a workgroup works on one
//    stage, the next one is copied straight from memory into the other
//    buffer (buffer_load ... lds, no registers held), completed before the
//    stage barrier. Every lane
//    then reads each chunk with same-address ds_read_b128, which the LDS
//    broadcasts, so the stream's values reach the FMAs in VGPRs (on gfx950
//    an FP32 FMA with an SGPR operand issues at half rate and never pairs).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "fhd.h"

namespace fhd {

constexpr int kBlock = 256;        // gather workgroup: 4 wave64
constexpr int kChunk = 8;          // records per packed chunk
constexpr int kFields = 5;         // three coordinates, phase offset, amplitude
constexpr int kChunkVec4 = kChunk * kFields / 4;        // 10 float4 per chunk
constexpr int kStageChunks = 64;   // chunks per LDS stage (512 records, 10 KB)
constexpr int kStageVec4 = kStageChunks * kChunkVec4;   // 640 float4
constexpr int kPackBlock = 256;

// Voxel units of the F^H D classification (fhd.hip, fhd_classify_kernel):
// 4096 consecutive voxels; class kClassLongPair marks both units of an
// aligned pair whose aligned runs of kLongLineVox voxels are lines along x
// of one step (same y and z bitwise, x_v = x_0 + v dx rounded once).
constexpr int kUnitVox = 4096;
constexpr int kLineVox = 64;
constexpr int kLongLineVox = 128;
enum : int { kClassGeneral = 0, kClassOneStep = 1, kClassLines = 2, kClassLongPair = 3 };

// Words the classification leaves after the unit classes ("info"): [0] 1
// if the first pair of units is of class kClassLongPair, [1] its lines'
// step (bits), [2] a flag the forward operator's line pre-pass sets, [3]
// unused, then kAmpSlots partial maxima of the packed sample amplitudes
// (bits), one per reduction workgroup (the largest amplitude is their
// maximum; see read_amp_shift).
constexpr int kAmpSlots = 64;
constexpr int kInfoWords = 4 + kAmpSlots;

static_assert(kBlock % 64 == 0, "workgroup must be whole wave64s");
static_assert(kChunk * kFields % 4 == 0, "chunks must be whole float4s");

inline int64_t packed_bytes_for(int64_t count)
{
    const int64_t chunks = (count + kChunk - 1) / kChunk;
    return chunks * kChunk * kFields * (int64_t)sizeof(float);
}

// Writes record r of a packed stream (one lane per padded record).
__device__ __forceinline__ void store_record(float *__restrict__ packed, int64_t r, float f0,
                                             float f1, float f2, float f3, float f4)
{
    float *c = packed + (r / kChunk) * (kFields * kChunk) + (r % kChunk);
    c[0 * kChunk] = f0;
    c[1 * kChunk] = f1;
    c[2 * kChunk] = f2;
    c[3 * kChunk] = f3;
    c[4 * kChunk] = f4;
}

// Unpacks one chunk's float4s (read from LDS) into per-field arrays.
__device__ __forceinline__ void load_chunk(const float4 *ch, float (&f)[kFields][kChunk])
{
#pragma unroll
    for (int q = 0; q < kChunkVec4; ++q) {
        const float4 t = ch[q];
        const int field = (4 * q) / kChunk, at = (4 * q) % kChunk;
        f[field][at + 0] = t.x;
        f[field][at + 1] = t.y;
        f[field][at + 2] = t.z;
        f[field][at + 3] = t.w;
    }
}

// Issues stage `st` of a packed stream of `total_vec4` float4 (starting at
// src; stages of STAGE_VEC4 float4) into `dst` with buffer_load ... lds, for
// a workgroup of BLOCK lanes:
// each wave's 64 lanes copy 64 consecutive float4 straight into LDS at the
// wave's base (lane l at base + l), with no registers in between. The
// buffer descriptor (SGPRs) starts at the stage and ends at the stream's
// end or the stage's, so a lane's offset is the same 32-bit value at every
// stage and reads past the end return zeros. Complete once vmcnt reaches 0.
template <int BLOCK = kBlock, int STAGE_VEC4 = kStageVec4>
__device__ __forceinline__ void issue_stage_load(const float4 *__restrict__ src, int64_t total_vec4,
                                                 int st, float4 *dst)
{
    static_assert(BLOCK % 64 == 0, "workgroup must be whole wave64s");
    constexpr int loads = (STAGE_VEC4 + BLOCK - 1) / BLOCK;
    // the wave's LDS base in a scalar register, so that the LDS addresses
    // (M0) are scalar arithmetic
    const int wave_base = __builtin_amdgcn_readfirstlane((int)threadIdx.x & ~63);
    const int64_t first = (int64_t)st * STAGE_VEC4;
    // callers pass st with total_vec4 - first > 0; the clamp to one stage
    // in 32-bit halves (scalar compares; 64-bit ordered compares would
    // take vector instructions)
    const uint64_t left = (uint64_t)(total_vec4 - first);
    unsigned left_hi = (unsigned)(left >> 32), left_lo = (unsigned)left;
    asm("" : "+s"(left_hi), "+s"(left_lo));   // kept apart (no 64-bit compare)
    const int bytes = (left_hi != 0u || left_lo >= (unsigned)STAGE_VEC4 ? STAGE_VEC4 : (int)left_lo) * 16;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)(src + first), (short)0, bytes, 0x00020000);
#pragma unroll
    for (int k = 0; k < loads; ++k) {
        const int i = k * BLOCK + threadIdx.x;
        if (i < STAGE_VEC4)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void *)(dst + k * BLOCK + wave_base), 16,
                (unsigned)i * 16u, 0, 0, 0);
    }
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads()
// it does not wait for outstanding global loads into registers. (A stage
// copy into LDS counts as an LDS write, so the compiler still waits for it
// here: issue one where that wait costs little.)
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Streams chunks [c_begin, c_end) of `src` through the workgroup's LDS
// stage buffers and calls body(chunks, count) for every STEP consecutive
// chunks of a stage, in order, in every lane: `chunks` points at the first
// of them in LDS and `count` (1..STEP) says how many are valid (fewer only
// at the end of the stream; the LDS beyond them holds stale data and must
// not be read). Every lane of the workgroup (BLOCK lanes) must call it (it
// holds workgroup barriers). Chunks past the end of `src` are never read.
template <int STEP, int BLOCK = kBlock, typename Body>
__device__ __forceinline__ void stream_chunk_groups(const float4 *__restrict__ src, int c_begin,
                                                    int c_end, float4 (*stage)[kStageVec4],
                                                    Body &&body)
{
    static_assert(kStageChunks % STEP == 0, "chunk groups tile a stage");
    const int nchunks = c_end > c_begin ? c_end - c_begin : 0;
    src += (int64_t)c_begin * kChunkVec4;
    const int64_t total_vec4 = (int64_t)nchunks * kChunkVec4;
    const int nstages = (nchunks + kStageChunks - 1) / kStageChunks;
    // stage st goes to stage[st & 1]
    if (nstages > 0) issue_stage_load<BLOCK>(src, total_vec4, 0, stage[0]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int st = 0; st < nstages; ++st) {
        // the next stage streams into the other buffer (last read before the
        // previous barrier) while this one is worked on
        if (st + 1 < nstages) issue_stage_load<BLOCK>(src, total_vec4, st + 1, stage[(st + 1) & 1]);
        const int chunks_here = min(kStageChunks, nchunks - st * kStageChunks);
        const float4 *buf = stage[st & 1];
        for (int c = 0; c < chunks_here; c += STEP) body(buf + c * kChunkVec4, min(STEP, chunks_here - c));
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
}

// stream_chunk_groups one chunk at a time: body(chunk).
template <typename Body>
__device__ __forceinline__ void stream_chunks(const float4 *__restrict__ src, int c_begin,
                                              int c_end, float4 (*stage)[kStageVec4], Body &&body)
{
    stream_chunk_groups<1>(src, c_begin, c_end, stage,
                           [&](const float4 *ch, int) { body(ch); });
}

// The hardware hands workgroup b of a launch to XCD b % kXcds (each XCD
// has its own L2). For a grid of `total` work units numbered split-major,
// xcd_unit gives workgroup b the unit that makes each XCD's workgroups a
// contiguous run of units -- so each XCD walks one split's part of the
// sample stream (two at a boundary) instead of all of them. A bijection of
// [0, total).
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_unit(int64_t b, int64_t total)
{
    const int64_t per = total / kXcds, rem = total % kXcds, k = b % kXcds;
    return k * per + (k < rem ? k : rem) + b / kXcds;
}

// Chunk range of split `s` when nchunks chunks are cut into `splits` parts
// of whole stages of STAGE_CHUNKS chunks.
template <int STAGE_CHUNKS = kStageChunks>
__device__ __forceinline__ void split_range(int nchunks, int splits, int s, int *c_begin,
                                            int *c_end)
{
    const int stages = (nchunks + STAGE_CHUNKS - 1) / STAGE_CHUNKS;
    const int per = (stages + splits - 1) / splits;   // stages per split
    const int b = s * per * STAGE_CHUNKS;
    *c_begin = min(b, nchunks);
    *c_end = min(b + per * STAGE_CHUNKS, nchunks);
}

// ---------------------------------------------------------------------------
// split-bf16 operands of the matrix cores
// ---------------------------------------------------------------------------
typedef float float16v __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), both rounded to
// nearest even: hi + lo carries 16 significant bits, x - (hi + lo) is
// within 2^-17 |x|. Two values per v_cvt_pk_bf16_f32, packed as one dword
// (element 2i in the low half). x - hi comes from v_dot2c_f32_bf16 as
// x + (-1) hi_0 + 0 hi_1 (or 0 hi_0 + (-1) hi_1): the products are exact
// and so is the sum, x - hi being an fp32 value, so this equals the
// subtraction of hi widened to fp32 in one instruction instead of two. The
// constant pairs stay in VGPRs: as an inline constant, -1.0 is not read by
// v_dot2c_f32_bf16 as the pair (-1, 0) the compiler encodes it for
// (measured: every low result wrong; register operands exact).
template <int E>
__device__ __forceinline__ void split_bf16(const float (&x)[E], unsigned (&hi)[E / 2],
                                           unsigned (&lo)[E / 2])
{
    unsigned c0 = 0x0000bf80u, c1 = 0xbf800000u;   // bf16 pairs (-1, 0) and (0, -1)
    asm("" : "+v"(c0));
    asm("" : "+v"(c1));
    const bf16x2 first = __builtin_bit_cast(bf16x2, c0), second = __builtin_bit_cast(bf16x2, c1);
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
        const bf16x2 h = __builtin_convertvector((float2v){x[2 * i], x[2 * i + 1]}, bf16x2);
        hi[i] = __builtin_bit_cast(unsigned, h);
        const float l0 = __builtin_amdgcn_fdot2_f32_bf16(h, first, x[2 * i], false);
        const float l1 = __builtin_amdgcn_fdot2_f32_bf16(h, second, x[2 * i + 1], false);
        lo[i] = __builtin_bit_cast(unsigned, __builtin_convertvector((float2v){l0, l1}, bf16x2));
    }
}

__device__ __forceinline__ bf16x8 as_bf16x8(const unsigned (&w)[4])
{
    return __builtin_bit_cast(bf16x8, (u32x4){w[0], w[1], w[2], w[3]});
}

// ---------------------------------------------------------------------------
// split-fp16 operands (the fp32-class form of the matrix-core products)
// ---------------------------------------------------------------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// x = hi + lo with hi = f16(x) and lo = f16(x - hi), both rounded to
// nearest even. For |x| in [2^-2, 2^15] both parts are normal fp16 numbers
// and x - (hi + lo) is within 2^-23 |x| (11 + 11 significant bits plus the
// sign of the remainder); below, lo is an fp16 subnormal and the error is
// at most 2^-25 in absolute terms (gfx950 keeps fp16 subnormals in
// v_cvt_pk_f16_f32 and in the f16 matrix products: measured). Callers keep
// |x| below 2^15 (fp16 overflows at 65520). x - hi comes from
// v_dot2c_f32_f16 exactly as in split_bf16 (the products with -1 and 0 are
// exact, and so is the sum).
template <int E>
__device__ __forceinline__ void split_f16(const float (&x)[E], unsigned (&hi)[E / 2],
                                          unsigned (&lo)[E / 2])
{
    unsigned c0 = 0x0000bc00u, c1 = 0xbc000000u;   // fp16 pairs (-1, 0) and (0, -1)
    asm("" : "+v"(c0));
    asm("" : "+v"(c1));
    const f16x2 first = __builtin_bit_cast(f16x2, c0), second = __builtin_bit_cast(f16x2, c1);
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
        const f16x2 h = __builtin_convertvector((float2v){x[2 * i], x[2 * i + 1]}, f16x2);
        hi[i] = __builtin_bit_cast(unsigned, h);
        const float l0 = __builtin_amdgcn_fdot2(h, first, x[2 * i], false);
        const float l1 = __builtin_amdgcn_fdot2(h, second, x[2 * i + 1], false);
        lo[i] = __builtin_bit_cast(unsigned, __builtin_convertvector((float2v){l0, l1}, f16x2));
    }
}

// The two-part split of the matrix-core line forms: fp16 (the default,
// fp32-class products) or bf16 (the opt-in three-product form with 16
// significant bits per operand).
template <bool F16, int E>
__device__ __forceinline__ void split_parts(const float (&x)[E], unsigned (&hi)[E / 2],
                                            unsigned (&lo)[E / 2])
{
    if constexpr (F16)
        split_f16<E>(x, hi, lo);
    else
        split_bf16<E>(x, hi, lo);
}

// One 16 x 16 x 32 product of split operands held as 4 dwords each (8
// two-byte elements), fp32 accumulation.
typedef float float4v __attribute__((ext_vector_type(4)));
template <bool F16>
__device__ __forceinline__ float4v mfma16(u32x4 a, u32x4 b, float4v c)
{
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One 32 x 32 x 16 product, as mfma16.
template <bool F16>
__device__ __forceinline__ float16v mfma32(u32x4 a, u32x4 b, float16v c)
{
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Power-of-two scaling of the amplitudes that enter the fp16 products: for
// a largest amplitude amax (bits as stored by the amplitude reduction),
// the shift s with amax 2^s in [2^14, 2^15), so that every scaled value
// stays below fp16's range limit and values down to 2^-16 amax keep the
// full 22-bit split. 0 for amax = 0 or not finite (the result is then 0,
// or not finite as the fp32 sum would be); a subnormal amax counts as
// 2^-126.
__device__ __forceinline__ int amp_shift(unsigned amax_bits)
{
    const int ex = (int)((amax_bits >> 23) & 0xffu);
    if (amax_bits == 0u || ex == 0xff) return 0;
    const int e = ex == 0 ? -126 : ex - 127;   // amax in [2^e, 2^(e+1))
    return 14 - e;
}

// An amplitude as it enters the products (scaled by 2^sh in the fp16
// form), and a product's sum as it leaves them (scaled back). Powers of two:
// exact unless the value leaves fp32's range.
template <bool F16>
__device__ __forceinline__ float scale_amp(float a, int sh)
{
    if constexpr (F16)
        return __builtin_ldexpf(a, sh);
    else
        return a;
}
template <bool F16>
__device__ __forceinline__ float unscale(float v, int sh)
{
    if constexpr (F16)
        return __builtin_ldexpf(v, -sh);
    else
        return v;
}

// The shift amp_shift() gives for the largest amplitude of the slots the
// classification filled (info + 4): every lane of the wave reads one slot
// and the wave takes the maximum. Uniform over the wave.
__device__ __forceinline__ int read_amp_shift(const int *__restrict__ info)
{
    static_assert(kAmpSlots == 64, "one slot per lane of a wave");
    unsigned m = (unsigned)info[4 + (threadIdx.x & 63)];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned t = (unsigned)__shfl_xor((int)m, o);
        m = t > m ? t : m;
    }
    return __builtin_amdgcn_readfirstlane(amp_shift(m));
}

// ---------------------------------------------------------------------------
// host side (abi_checks.hip)
// ---------------------------------------------------------------------------
struct Span {
    const void *p;
    int64_t bytes;
    const char *name;
    unsigned align = 4;   // required alignment in bytes
};

// Records msg as the calling thread's last error and returns status.
int fail(int status, const std::string &msg);
void clear_error();

// Whether `paths` is one of FHD_GATHER_ALL, FHD_GATHER_VECTOR,
// FHD_GATHER_BF16X3; fail_paths() records the error for one that is not.
inline bool valid_paths(int paths)
{
    return paths == FHD_GATHER_ALL || paths == FHD_GATHER_VECTOR || paths == FHD_GATHER_BF16X3;
}
int fail_paths();

// NULL and alignment of every span with bytes > 0; no HIP call.
int check_host_side(const Span *spans, int count);
// Spans [first_out, count) are outputs: none may overlap any other span.
int check_no_overlap(const Span *spans, int count, int first_out);
// Every span with bytes > 0 is device-accessible memory of the current
// device and, for device allocations, ends inside the allocation holding
// its first byte.
int check_device_spans(const Span *spans, int count);
// FHD_ERR_HIP with `what` if the last launch failed.
int launch_status(const char *what);

// Measurement hook (fhd_time_kernel): when the calling thread has armed it
// for `kernel`, timed_begin records the next start event on `stream` and
// returns its slot (else -1); timed_end records the matching stop event.
int timed_begin(const char *kernel, hipStream_t stream);
void timed_end(int slot, hipStream_t stream);
// Brackets one kernel launch in a scope: { TimedLaunch t(name, s); k<<<>>>(); }
struct TimedLaunch {
    int slot;
    hipStream_t stream;
    TimedLaunch(const char *kernel, hipStream_t s) : slot(timed_begin(kernel, s)), stream(s) {}
    ~TimedLaunch() { timed_end(slot, stream); }
    TimedLaunch(const TimedLaunch &) = delete;
    TimedLaunch &operator=(const TimedLaunch &) = delete;
};

// How many parts to cut a stream of `nchunks` chunks into, for a gather
// whose output needs `blocks` workgroups of which `per_cu` fit on a CU at
// once: below one round, enough parts to fill it (at least `granule`
// chunks per part); above, a few parts where that evens out a partly
// filled last round. `slack`: the fewest parts whose priced time is within
// this factor of the cheapest are taken (a part costs its workgroups'
// set-up and one more row of partial sums).
int split_count(int64_t blocks, int nchunks, int per_cu = 4, int granule = kStageChunks, double slack = 1.03);
// Compute units of the current device (cached per device); 0 on error.
int device_cus();

// out[i] = sum_{s < splits} part[s*n + i] in increasing s, for the real
// and the imaginary parts (stream-ordered launch, no checks). With a gate,
// only when lines_form_ran(gate) == gate_want.
int launch_reduce(const float *part_r, const float *part_i, int splits, int64_t n, float *out_r,
                  float *out_i, hipStream_t stream, const int *gate = nullptr, bool gate_want = true);

// Kernel launches without argument checks (callers have checked). A gather
// whose output is too small to fill the chip splits the stream, with a
// stream-ordered partial-sum workspace it allocates and frees itself.
// fhd.hip: adjoint F^H D
int launch_pack(const float *kx, const float *ky, const float *kz, const float *Dr, const float *Di,
                int M, float *packed, hipStream_t stream);
// Whether the forward operator's line-pair form ran (its line form then
// stands aside): info as launch_classify leaves it, with info[3] set by
// the line-pair pre-pass (which runs first on that path) when some unit
// breaks that form's rule.
__device__ __forceinline__ bool pairs_form_ran(const int *info) { return info[3] == 0; }
// Whether one of its matrix-core forms ran (and the vector form is to
// stand aside): the line-pair form, or the line form, info[2] set by the
// line pre-pass when some line breaks that form's rule.
__device__ __forceinline__ bool lines_form_ran(const int *info)
{
    return pairs_form_ran(info) || (info[0] != 0 && info[2] == 0);
}

// Classes of the ceil(N / kUnitVox) units into cls; info[0] = 1 if the
// first pair is of class kClassLongPair, info[1] its step's bits, info[2]
// = info[3] = 0 (stream-ordered; allow_lines = false gives no matrix-core
// class).
// With amp_slots, also the amplitude slots info[4 .. 4 + kAmpSlots) of
// the packed k-space of M samples (zeros when M = 0; info holds kInfoWords
// words). With patches (two int4 per unit pair), also each pair's
// line-pair record (the line-pair instance's classification).
int launch_classify(const float *x, const float *y, const float *z, int N, bool allow_lines, int *cls,
                    int *info, hipStream_t stream, bool amp_slots = false, const float *packed = nullptr,
                    int M = 0, int4 *patches = nullptr);
// paths: FHD_GATHER_ALL (lines on the matrix cores in split fp16, the
// rest on the vector ALUs), FHD_GATHER_BF16X3 (the same in split bf16) or
// FHD_GATHER_VECTOR (every unit on the vector-ALU paths). Takes its
// workspace stream-ordered from hipMallocAsync.
int launch_gather(const float *packed, int M, const float *x, const float *y, const float *z,
                  float *rho_r, float *rho_i, int N, hipStream_t stream, int paths = FHD_GATHER_ALL);

// The gather's launch shape and workspace for M samples and N > 0 voxels:
// the unit classes and info words, the long-line instance's B table (left
// out when with_table is false: its workgroups then form B themselves, with
// bitwise the same results), and the split partial sums. run_gather
// launches the gather into a caller's workspace of work_bytes() bytes,
// 256-byte aligned; nothing in it needs clearing first.
// A device buffer for one call's stream-ordered use on `stream`: the
// stream's kept buffer for `slot` (grown when too small), or, while the
// stream is being captured into a graph, a stream-ordered allocation that
// finish() (or the destructor) frees. From get() to finish() the call holds
// its stream's lock, so calls on one stream from several threads do not
// interleave their launches.
enum : int {
    kSlotGather = 0,      // classes, long-line table, partial sums of F^H D
    kSlotPacked,          // packed k-space of fhd_compute
    kSlotForward,         // classes, line tiles, partial sums of F
    kSlotForwardPacked,   // packed voxels of F's vector form
    kSlotForwardPart,     // partial sums of F's vector form
    kSlotNormal,          // packed voxels, packed samples and F p of F^H F
    kSlots
};
struct WorkspaceEntry;
class StreamBuffer {
public:
    StreamBuffer(hipStream_t stream, int slot);
    ~StreamBuffer();
    int get(size_t bytes, char **out);   // at most once per object
    int finish();
    StreamBuffer(const StreamBuffer &) = delete;
    StreamBuffer &operator=(const StreamBuffer &) = delete;

private:
    hipStream_t stream_;
    int slot_;
    char *async_ = nullptr;
    WorkspaceEntry *entry_ = nullptr;
};

// Each instance cuts the sample stream into its own number of splits (1:
// it writes rho itself); `splits` partial-sum rows of N serve them all.
struct GatherPlan {
    int paths = FHD_GATHER_ALL;
    int nchunks = 0, splits = 1;
    int s_long = 1, s_lines = 1, s_vec = 1;
    int64_t blocks = 0, pairs = 0, quads = 0, steps = 0;
    size_t patch_offset = 0, cls_bytes = 0, table_bytes = 0, patch_table_bytes = 0, part_bytes = 0;
    size_t work_bytes() const { return cls_bytes + table_bytes + patch_table_bytes + part_bytes; }
};
GatherPlan plan_gather(int M, int N, int paths, bool with_table);
int run_gather(const GatherPlan &g, char *work, const float *packed, int M, const float *x, const float *y,
               const float *z, float *rho_r, float *rho_i, int N, hipStream_t stream);
// fhd_forward.hip: forward F
// (with a gate: nothing when lines_form_ran(gate))
int launch_forward_pack(const float *x, const float *y, const float *z, const float *rho_r,
                        const float *rho_i, int N, float *packed, hipStream_t stream,
                        const int *gate = nullptr);
int launch_forward_gather(const float *packed, int N, const float *kx, const float *ky,
                          const float *kz, float *Dr, float *Di, int M, hipStream_t stream,
                          const int *gate = nullptr);
// D = F rho: on the matrix cores when every aligned pair of voxel units is
// lines of 128 voxels along x of one common step (decided on the device),
// else packed into vox (packed_bytes_for(N) bytes) for the vector gather.
// paths as for launch_gather (FHD_GATHER_VECTOR: the vector form always).
int launch_forward(const float *x, const float *y, const float *z, const float *rho_r,
                   const float *rho_i, int N, const float *kx, const float *ky, const float *kz,
                   float *Dr, float *Di, int M, float *vox, hipStream_t stream, int paths = FHD_GATHER_ALL);
// fhd_grid.hip: F^H D on a Cartesian grid (axis = x0, dx, y0, dy, z0, dz)
int launch_grid_gather(const float *packed, int M, int nx, int ny, int nz, const float *axis,
                       int precision, float *rho_r, float *rho_i, hipStream_t stream);
// D = F rho for rho on an nx x ny x nz grid (at least one voxel), split-bf16
// products only (precision FHD_GRID_BF16X3).
int launch_forward_grid(const float *rho_r, const float *rho_i, int nx, int ny, int nz,
                        const float *axis, int precision, const float *kx, const float *ky,
                        const float *kz, int M, float *Dr, float *Di, hipStream_t stream);

}  // namespace fhd
