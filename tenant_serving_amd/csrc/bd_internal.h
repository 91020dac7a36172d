// bd_internal.h -- internals shared by the translation units of libbitdelta.so.
//
// Workspace layouts, launch plans and small device helpers.  Every size a
// kernel assumes is computed here once and used both by the workspace queries
// and by the launches, so a plan that validates is a plan that fits.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bitdelta.h"

namespace bd {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Status word bits (first 4 bytes of every workspace).  ST_ENCODING: a delta product
// was asked of a prepared batch whose tokens were encoded for another scale mode.
enum : uint32_t { ST_NONFINITE = 1u, ST_USER_ID = 2u, ST_ENCODING = 4u };

// ---------------------------------------------------------------- compress
// Stream tiling: a wave covers one row segment of kSegCols columns per row
// (8 consecutive elements per lane, 16-byte loads for bf16), a block of 4
// waves covers `rows_per_block` rows of one segment.
constexpr int kSegCols = 512;
constexpr int kCompressThreads = 256;

struct CompressPlan {
    int64_t d_out = 0, d_in = 0, n = 0;
    int64_t n_seg = 0, rows_per_block = 0, n_rchunk = 0, n_blocks = 0;
    int mode = 0, group = 0, sdtype = 0;
    bool clip = false;
    double clip_k = 0.0;
    // workspace offsets (bytes)
    size_t off_status = 0, off_stats = 0, off_part_sum = 0, off_part_m2 = 0, off_part_abs = 0,
           off_flags = 0;  // one non-finite flag per block of the packing pass
    size_t total = 0;
};

// Returns BD_OK and fills `plan`, or the synchronous error for these params.
bd_status make_compress_plan(const bd_compress_params* p, int64_t d_out, int64_t d_in,
                             CompressPlan* plan);
hipError_t launch_compress(const CompressPlan& pl, const void* wf, const void* wb, int wdtype,
                           uint64_t* signs, void* scales, char* ws, hipStream_t s);

// INT8 base weights (bd_quantize_base) and the one-launch decode apply on them.
hipError_t launch_quantize_rows(const void* w, int wdtype, int64_t d_out, int64_t d_in, int8_t* q,
                                float* s, hipStream_t st);
bool q8_path_supported(int xdtype, int64_t T, int mode, int64_t d_in);
struct DeltaPlan;
hipError_t launch_decode_q8(int64_t T, int U, int64_t d_in, const DeltaPlan& dp, const void* x,
                            const int32_t* ids, const int8_t* wq, const float* wscale,
                            const uint64_t* signs, const void* scales, void* y, int ydtype, char* ws,
                            hipStream_t s);

// Per-layer axis choice (bd_select_axis): the compress plan's grid and clip passes, then
// one statistics pass (the ROW and COL absmean partials and sum d^2) and two reductions.
struct AxisPlan {
    CompressPlan c;
    size_t off_part = 0, off_rsq = 0, off_csq = 0, total = 0;
};
bd_status make_axis_plan(float clip_k, int64_t d_out, int64_t d_in, AxisPlan* plan);
hipError_t launch_select_axis(const AxisPlan& ap, const void* wf, const void* wb, int wdtype,
                              double* errors, int32_t* axis, char* ws, hipStream_t s);

// ------------------------------------------------------------------- apply
constexpr int kItemTokens = 32;   // max tokens of one (user, chunk) work item (<= 2 MFMA tiles)
constexpr int kMaxMats = 4;       // matrices of one grouped launch (they share X)
constexpr int kMaxGroupT = 8192;  // tokens the one-block grouping kernel sorts in LDS
constexpr int kMaxUsers = (1 << 17) - 1;

// Prepared batch (bd_batch_prepare): tokens grouped by user into work items; for
// bf16 inputs also the tiles of the delta products (bd_delta.hip): runs of at most
// 16 sorted positions that split no user of at most 16 tokens (their number, at
// most 2 ceil(T / 16) + 1, in meta[3]; start and length per tile), per tile
// kTileMetaInts ints of meta, per (tile, 512-column unit) kEncUnitBytes of encoded
// token operands.
constexpr int kTileMetaInts = 64;
constexpr int kEncUnitBytes = 13 * 1024;
struct BatchPlan {
    int64_t T = 0, d_in = 0;
    int32_t U = 0;
    int xdtype = 0;
    int64_t max_items = 0, ntiles = 0, nunit = 0;
    size_t off_meta = 0, off_perm = 0, off_user = 0, off_items = 0, off_tiles = 0, off_torder = 0,
           off_tpre = 0, off_tmeta = 0, off_enc = 0;
    size_t total = 0;
};

// One matrix's delta application on a prepared batch.  per_user: scales of one user;
// sstride / cstride: bytes from one user's (slot's) signs to the next and scale
// elements from one user's scales to the next, 0 for a dense bank (d_out d_in / 8 and
// per_user).
struct DeltaPlan {
    int64_t d_out = 0, per_user = 0;
    int mode = 0, group = 0, sdtype = 0;
    uint64_t sstride = 0;
    int64_t cstride = 0;
};
__host__ __device__ inline uint64_t sign_stride(uint64_t sstride, int64_t d_out, int64_t d_in) {
    return sstride ? sstride : (uint64_t)d_out * (uint64_t)(d_in / 8);
}
inline int64_t scale_stride(const DeltaPlan& dp) { return dp.cstride ? dp.cstride : dp.per_user; }

// One-pass path for decode batches of at most kDecodeMaxT bf16 tokens: the
// prepared batch (sorted tokens, user segments) and the fp8 encoding of X.
constexpr int kDecodeMaxT = 16;
struct DecodePlan {
    int64_t T = 0, d_in = 0, dpad = 0;
    size_t off_meta = 0, off_perm = 0, off_suser = 0, off_seg = 0;
    size_t off_xs = 0, off_x8 = 0, off_e8 = 0, total = 0;
};

// Single-launch decode path (MATRIX or ROW scales): the tokens of the batch, d_in
// padded to 512 columns, are staged in LDS, 32 bytes per padded column.
constexpr int64_t kFusedMaxDpad = 5120;

// bd_apply workspace = batch | fp32 Y (bf16 output only), or the decode plan's.
struct ApplyPlan {
    BatchPlan batch;
    DeltaPlan delta;
    int ydtype = 0;
    bool decode = false, fused = false;
    DecodePlan dec;
    size_t off_yf = 0, total = 0;
};

bd_status check_params(const bd_compress_params* p, int64_t d_out, int64_t d_in, int xdtype);
bd_status make_batch_plan(int64_t T, int32_t U, int64_t d_in, int xdtype, BatchPlan* plan);
bd_status make_delta_plan(const bd_compress_params* p, const BatchPlan& b, int64_t d_out,
                          DeltaPlan* plan);
// allow_decode = false: the prepared-batch plan even where the decode path applies.
bd_status make_apply_plan(const bd_compress_params* p, int64_t T, int32_t U, int64_t d_out,
                          int64_t d_in, int xdtype, int ydtype, ApplyPlan* plan,
                          bool allow_decode = true);
hipError_t launch_batch_prepare(const BatchPlan& pl, const void* x, const int32_t* ids,
                                char* batch, hipStream_t s);
hipError_t launch_base_gemm(const void* x, int xdtype, int64_t T, int64_t d_in, const void* wb,
                            int64_t d_out, float* y, hipStream_t s);
hipError_t launch_delta(const BatchPlan& bp, const DeltaPlan& dp, char* batch,
                        const void* x, const uint64_t* signs, const void* scales, float* y,
                        hipStream_t s);
hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s);
// bf16 delta products of a prepared batch (writes the batch's tile meta and encoded
// tokens, then adds into y).
hipError_t launch_tile_plan(const BatchPlan& bp, char* batch, hipStream_t s);
hipError_t launch_delta6(const BatchPlan& bp, const DeltaPlan& dp, char* batch, const void* x,
                         const uint64_t* signs, const void* scales, float* y, hipStream_t s);
// The two halves of launch_delta6: the tokens of x encoded into the batch (k_tile_encode;
// word kEncTagWord of the batch meta records which encoding), then the products on them.
constexpr int kEncTagWord = 4;
__host__ __device__ constexpr uint32_t enc_tag(bool grp, bool col) {
    return 0x454E4300u | (grp ? 1u : 0u) | (col ? 2u : 0u);
}
hipError_t launch_tile_encode(const BatchPlan& bp, const DeltaPlan& dp, char* batch,
                              const void* x, const void* scales, hipStream_t s);
hipError_t launch_delta6_encoded(const BatchPlan& bp, const DeltaPlan& dp, char* batch,
                                 const uint64_t* signs, const void* scales, float* y,
                                 hipStream_t s);
// The products of up to kMaxMats matrices of one scale mode on one encoded batch, in
// one launch (dp gives the mode, group size and scale dtype; each matrix its d_out).
struct DeltaMatArg {
    const uint64_t* signs;
    const void* scales;
    float* y;
    int64_t d_out;
    uint64_t sstride = 0;  // as DeltaPlan's; 0: dense bank
    int64_t cstride = 0;
};
hipError_t launch_delta6_set(const BatchPlan& bp, const DeltaPlan& dp, char* batch,
                             const DeltaMatArg* mats, int n, hipStream_t s);

// Tiled matrix-core GEMM for the base product of batches of more than kGemmMinT
// bf16 tokens (smaller batches take the streaming kernel of bd_apply.hip).
constexpr int64_t kGemmMinT = 64;
bool gemm_path_supported(int64_t T, int64_t d_in, int64_t d_out);
bool small_batch_gemm_supported(int64_t T, int64_t d_in, int64_t d_out);
hipError_t launch_small_batch_gemm(const void* x, int64_t T, int64_t d_in, const void* wb,
                                   int64_t d_out, float* y, hipStream_t s);
hipError_t launch_gemm(const void* x, int64_t T, int64_t d_in, const void* wb, int64_t d_out,
                       float* y, hipStream_t s);
// The base products of up to kMaxMats matrices that read the same X, in one launch
// (their row tiles back to back in one grid).
struct GemmMatArg {
    const void* w;
    float* y;
    int64_t d_out;
};
struct GemmMats {
    const uint16_t* w[kMaxMats];  // bf16 rows, or int8 rows for the INT8-base product
    const float* s[kMaxMats];     // INT8 base: the rows' scales
    float* part[kMaxMats];        // split K: the partial products, [S][T][N] per matrix
    float* y[kMaxMats];
    int N[kMaxMats];
    int rt_begin[kMaxMats + 1];
    int n;
};
// wscales (one per matrix, or null): the matrices hold INT8 codes with these row scales.
hipError_t launch_gemm_set(const void* x, int64_t T, int64_t d_in, const GemmMatArg* mats, int n,
                           hipStream_t s, const float* const* wscales = nullptr);
// The same with K split in S ordered parts where the large tiles would leave the chip
// idle: the partial products go to `ws` and a second launch sums them in split order
// (deterministic).  gemm_split_bytes: the workspace that split needs, 0 for no split.
size_t gemm_split_bytes(int64_t T, int64_t d_in, const int64_t* d_outs, int n);
hipError_t launch_gemm_set_split(const void* x, int64_t T, int64_t d_in, const GemmMatArg* mats,
                                 int n, char* ws, hipStream_t s,
                                 const float* const* wscales = nullptr);
// Y = s (.) (X Wq^T) for an INT8 base weight (per-row symmetric codes wq, row scales
// wscale): the same tiles, the codes widened to bf16 on their way into LDS (exact).
bool gemm_q8_supported(int64_t T, int64_t d_in, int64_t d_out);
hipError_t launch_gemm_q8(const void* x, int64_t T, int64_t d_in, const int8_t* wq,
                          const float* wscale, int64_t d_out, float* y, hipStream_t s);

bool decode_path_supported(int xdtype, int64_t T, int mode);
void make_decode_plan(int64_t T, int64_t d_in, DecodePlan* plan);
hipError_t launch_decode_prep(const DecodePlan& pl, int U, const DeltaPlan& dp, const void* x,
                              const int32_t* ids, const void* scales, char* ws, hipStream_t s);
hipError_t launch_decode_main(const DecodePlan& pl, const DeltaPlan& dp, const void* x,
                              const void* wb, const uint64_t* signs, const void* scales, void* y,
                              int ydtype, const char* ws, hipStream_t s);
bool fused_path_supported(int xdtype, int64_t T, int mode, int64_t d_in);
// Writes the status word at ws (bad user ids) and y; reads nothing else of ws.
hipError_t launch_decode_fused(int64_t T, int U, int64_t d_in, const DeltaPlan& dp, const void* x,
                               const int32_t* ids, const void* wb, const uint64_t* signs,
                               const void* scales, void* y, int ydtype, char* ws, hipStream_t s);

hipError_t launch_reconstruct(const uint64_t* signs, const void* scales, int mode, int group,
                              int sdtype, int64_t d_out, int64_t d_in, const void* wb, int wdtype,
                              void* out, int odtype, hipStream_t s);

// Zero `n` 32-bit words with a kernel (no memset node, so capture-safe).
hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s);

// ---------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// binary64 -> binary16, round to nearest even, from the bit fields.
__device__ __forceinline__ uint16_t f64_to_f16(double x) {
    uint64_t b = (uint64_t)__double_as_longlong(x);
    uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
    uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
    if (a > 0x7FF0000000000000ull) return 0x7E00u;
    if (a == 0x7FF0000000000000ull) return sign | 0x7C00u;
    int e = (int)(a >> 52) - 1023;
    if (e < -25) return sign;  // below half the smallest subnormal (also double subnormals)
    uint64_t mant = (a & 0x000FFFFFFFFFFFFFull) | 0x0010000000000000ull;  // 53 bits
    if (e >= -14) {
        uint64_t q = mant >> 42, rem = mant & ((1ull << 42) - 1), half = 1ull << 41;
        if (rem > half || (rem == half && (q & 1))) ++q;
        uint64_t r = ((uint64_t)(e + 15) << 10) + q - 1024;  // carry into the exponent is right
        if (r >= 0x7C00u) return sign | 0x7C00u;
        return sign | (uint16_t)r;
    }
    int sh = 28 - e;  // value / 2^-24 = mant * 2^(e-28); 43 <= sh <= 53
    uint64_t q = mant >> sh, rem = mant & ((1ull << sh) - 1), half = 1ull << (sh - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    return sign | (uint16_t)q;
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return (float)v;
}


// The fp6 e2m3 B operands of the block-scaled MFMA 16x16x128 for one lane's 32
// values (one 32-column block of one token): R[p] holds the bf16 values of
// columns 2p (low half) and 2p + 1 (high half).  k position j = 8 d + n carries
// column 4 n + d, the column whose sign bit the fp4 sign operand puts there.
// With E the exponent of the block's largest |x| (in [2^E, 2^(E+1))) and
// s = 2^(E-1): hi = fp6(x / s) and lo = fp6((x - hi) / (s / 32)), both rounded to
// nearest even; hi + lo equals x for every |x| >= s and is within 2^-10 of the
// block maximum otherwise.  code_hi / code_lo: the E8M0 scale codes of hi and lo.
// kone_lo / kone_hi: the bf16 pairs (1, 0) and (0, 1), passed in registers.
__device__ __forceinline__ void encode_fp6_block(const uint32_t* R, uint32_t kone_lo,
                                                 uint32_t kone_hi,
                                                 int __attribute__((ext_vector_type(6)))& h,
                                                 int __attribute__((ext_vector_type(6)))& l,
                                                 uint32_t& code_hi, uint32_t& code_lo) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x32 __attribute__((ext_vector_type(32)));
    typedef float f32x32 __attribute__((ext_vector_type(32)));
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    typedef unsigned int u32x16 __attribute__((ext_vector_type(16)));
    typedef int i32x6 __attribute__((ext_vector_type(6)));
    // block maximum of |x|: on the bf16 bits of non-negative values the integer
    // order is the numeric order
    u16x2 mx2 = {0, 0};
#pragma unroll
    for (int p = 0; p < 16; ++p)
        mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(u16x2, R[p] & 0x7FFF7FFFu));
    const uint32_t eb = (uint32_t)(mx2.x > mx2.y ? mx2.x : mx2.y) >> 7;  // biased exponent
    // s = 2^(eb - 128): code eb - 1; blocks below 2^-120 (zeros) take s = 1
    code_hi = eb >= 7u && eb <= 255u ? eb - 1u : 127u;
    code_lo = code_hi - 5u;
    const float sh = __uint_as_float(code_hi << 23), sl = __uint_as_float(code_lo << 23);
    // the values in k order: pair i = (column c, column c + 4), c = 8 (i % 4) + i / 4
    // (kept as scalars: each pair also feeds a dot product below)
    uint32_t V[16];
    u32x16 Vv;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int a = i & 3, d = i >> 2;
        const uint32_t r0 = R[4 * a + (d >> 1)], r1 = R[4 * a + (d >> 1) + 2];
        V[i] = __builtin_amdgcn_perm(r1, r0, (d & 1) ? 0x07060302u : 0x05040100u);
        Vv[i] = V[i];
    }
    h = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(__builtin_bit_cast(bf16x32, Vv), sh);
    // -hi, exact: the 32 fields with their sign bits (bit 6j + 5) flipped, widened
    const i32x6 sgn = {(int)0x20820820u, (int)0x08208208u, (int)0x82082082u,
                       (int)0x20820820u, (int)0x08208208u, (int)0x82082082u};
    f32x32 r = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(h ^ sgn, sh);
    // the exact residuals x - hi (the bf16 dot product picks one half of the pair),
    // accumulated onto -hi in place; each has at most 4 significant bits, so its bf16
    // form (the upper half of the fp32 word) is exact
    u32x16 W;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const bf16x2 pr = __builtin_bit_cast(bf16x2, V[i]);
        r[2 * i] = __builtin_amdgcn_fdot2_f32_bf16(pr, __builtin_bit_cast(bf16x2, kone_lo),
                                                   r[2 * i], false);
        r[2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, __builtin_bit_cast(bf16x2, kone_hi),
                                                       r[2 * i + 1], false);
        W[i] = __builtin_amdgcn_perm(__float_as_uint(r[2 * i + 1]), __float_as_uint(r[2 * i]),
                                     0x07060302u);
    }
    l = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(__builtin_bit_cast(bf16x32, W), sl);
}

}  // namespace bd
