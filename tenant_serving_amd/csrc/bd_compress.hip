// bd_compress.hip -- BitDelta compression on gfx950.
//
// One streaming pass reads W_fine and W_base once, forms the delta ([P1]
// "How BitDelta Works" step 1), optionally clamps it to mean +- k*std ([P1]
// "Outlier Clipping"), packs the signs with 64-lane ballots ([P2] "1.
// Mathematical Formulation": bit 1 <-> +1, zero -> +1) and accumulates
// |delta| per scale unit in binary64 ([P2] "2. Optimal L2 Norm
// Initialization", [P1] step 2, [P5] "Key Contributions" 1).  With clipping,
// two earlier passes compute the whole-matrix mean and the sum of squared
// deviations (binary64, deterministic block partials, no float atomics).
//
// Tiling: grid (segment, row chunk); a segment is 512 columns of a row, a
// wave owns one segment of a row at a time with 8 consecutive elements per
// lane (one 16-byte load per input for bf16).  Row r of a block's chunk goes
// to wave r % 4.  The 8 ballots of a segment give, for element j of every
// lane, a 64-bit mask; lanes 0..7 regroup them into the 8 canonical words of
// the segment with an 8x8 bit transpose.
#include "bd_internal.h"

namespace bd {
namespace {

constexpr int kUnroll = 4;  // rows whose loads are in flight together per wave

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename WT>
struct Elt;
template <>
struct Elt<uint16_t> {  // bf16: 16 bytes hold 8 elements
    static __device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
        u32x4 q = __builtin_nontemporal_load((const u32x4*)p);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
};
template <>
struct Elt<float> {
    static __device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
        f32x4 a = __builtin_nontemporal_load((const f32x4*)p);
        f32x4 b = __builtin_nontemporal_load((const f32x4*)(p + 4));
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

__device__ __forceinline__ double wave_sum(double v) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Transpose an 8x8 bit matrix held as bytes (row r = byte r): bit 8r+c -> bit 8c+r.
__device__ __forceinline__ uint64_t transpose8x8(uint64_t x) {
    uint64_t t;
    t = (x ^ (x >> 7)) & 0x00AA00AA00AA00AAull;
    x = x ^ t ^ (t << 7);
    t = (x ^ (x >> 14)) & 0x0000CCCC0000CCCCull;
    x = x ^ t ^ (t << 14);
    t = (x ^ (x >> 28)) & 0x00000000F0F0F0F0ull;
    x = x ^ t ^ (t << 28);
    return x;
}

struct Stats {   // clip statistics in the workspace
    double mu, sigma, lo, hi;
};

// Deterministic block reduction of one double per thread (fixed order).
__device__ __forceinline__ double block_sum(double v, double* sh) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) sh[w] = v;
    __syncthreads();
    double r = 0.0;
    if (threadIdx.x == 0)
        for (int i = 0; i < kCompressThreads / 64; ++i) r += sh[i];
    __syncthreads();
    return r;  // valid in thread 0
}

// PASS 0: sum of delta; PASS 1: sum of (delta - mu)^2; PASS 2: pack + scales; PASS 3:
// the statistics of the per-layer axis choice (sum d^2 per block, sum |d| per row and
// segment, sum |d| per column and row chunk, of the clipped delta), at
// part[0 .. n_blocks), part[n_blocks ..) and part[n_blocks + d_out n_seg ..).
template <typename WT, bool HAS_BASE, int PASS, int MODE, bool CLIP>
__global__ void __launch_bounds__(kCompressThreads)
k_compress(const WT* __restrict__ wf, const WT* __restrict__ wb, int64_t d_out, int64_t d_in,
           int64_t rows_per_block, int group, int sdtype, uint64_t* __restrict__ signs,
           void* __restrict__ scales, const Stats* __restrict__ st, double* __restrict__ part,
           uint32_t* __restrict__ flags) {
    __shared__ double sh[kCompressThreads / 64];
    constexpr bool kCol = (PASS == 2 && MODE == BD_SCALE_COL) || PASS == 3;
    __shared__ double colsh[kCol ? kCompressThreads / 64 : 1][kCol ? kSegCols : 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t seg = blockIdx.x, rc = blockIdx.y;
    const int64_t n_seg = gridDim.x;
    const int64_t c0 = seg * kSegCols + 8 * lane;
    const bool active = c0 < d_in;
    const int64_t r_begin = rc * rows_per_block;
    const int64_t r_end = r_begin + rows_per_block < d_out ? r_begin + rows_per_block : d_out;

    double mu = 0.0, lo = 0.0, hi = 0.0;
    if (PASS == 1) mu = st->mu;
    if (PASS >= 2 && CLIP) { lo = st->lo; hi = st->hi; }
    const int64_t n_blocks = n_seg * (int64_t)gridDim.y;

    double acc = 0.0;        // PASS 0/1 and MATRIX partial
    double colacc[8];        // COL partial
#pragma unroll
    for (int j = 0; j < 8; ++j) colacc[j] = 0.0;
    bool bad = false;

    for (int64_t r0 = r_begin + wave; r0 < r_end; r0 += 4 * kUnroll) {
        float f[kUnroll][8], b[kUnroll][8];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t r = r0 + 4 * u;
            if (active && r < r_end) {
                Elt<WT>::load8(wf + r * d_in + c0, f[u]);
                if (HAS_BASE) Elt<WT>::load8(wb + r * d_in + c0, b[u]);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) { f[u][j] = 0.f; b[u][j] = 0.f; }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t r = r0 + 4 * u;
            if (r >= r_end) break;  // wave-uniform
            float d[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) d[j] = HAS_BASE ? f[u][j] - b[u][j] : f[u][j];
            if (PASS == 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) acc += (double)d[j];
                continue;
            }
            if (PASS == 1) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    double e = (double)d[j] - mu;
                    acc += active ? e * e : 0.0;
                }
                continue;
            }
            if (PASS == 3) {
                double rs = 0.0;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    bad |= (__float_as_uint(d[j]) & 0x7F800000u) == 0x7F800000u;
                    double xv = (double)d[j];
                    if (CLIP) {
                        if (xv < lo) xv = lo;
                        if (xv > hi) xv = hi;
                    }
                    const double a = active ? fabs(xv) : 0.0;
                    acc += a * a;
                    rs += a;
                    colacc[j] += a;
                }
                rs = wave_sum(rs);
                if (lane == 0) part[n_blocks + r * n_seg + seg] = rs;
                continue;
            }
            // PASS 2: clamp, signs, |delta| partials
            double a[8];
            uint32_t byte = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                bad |= (__float_as_uint(d[j]) & 0x7F800000u) == 0x7F800000u;
                if (CLIP) {
                    double x = (double)d[j];
                    if (x < lo) x = lo;
                    if (x > hi) x = hi;
                    byte |= (uint32_t)!(x < 0.0) << j;
                    a[j] = fabs(x);
                } else {
                    byte |= (uint32_t)!(d[j] < 0.0f) << j;
                    a[j] = (double)fabsf(d[j]);
                }
            }
            if (!active) { byte = 0; }
            // signs: ballot per element position, regroup into canonical words
            uint64_t m[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) m[j] = __ballot((byte >> j) & 1u);
            if (lane < 8) {
                const int64_t word = seg * 8 + lane;
                if (word * 64 < d_in) {
                    uint64_t A = 0;
#pragma unroll
                    for (int j = 0; j < 8; ++j) A |= ((m[j] >> (8 * lane)) & 0xFFull) << (8 * j);
                    signs[r * (d_in / 64) + word] = transpose8x8(A);
                }
            }
            double rs = 0.0;
#pragma unroll
            for (int j = 0; j < 8; ++j) rs += a[j];
            if (!active) rs = 0.0;
            if (MODE == BD_SCALE_MATRIX) {
                acc += rs;
            } else if (MODE == BD_SCALE_GROUP) {
                const int L = group / 8;  // lanes per group (1..64)
                for (int off = 1; off < L; off <<= 1) rs += __shfl_xor(rs, off);
                if (active && (lane & (L - 1)) == 0) {
                    const int64_t gi = r * (d_in / group) + c0 / group;
                    const double v = rs / (double)group;
                    if (sdtype == BD_F16) ((uint16_t*)scales)[gi] = f64_to_f16(v);
                    else ((float*)scales)[gi] = (float)v;
                }
            } else if (MODE == BD_SCALE_ROW) {
                rs = wave_sum(rs);
                if (lane == 0) part[r * n_seg + seg] = rs;
            } else {  // COL
#pragma unroll
                for (int j = 0; j < 8; ++j) colacc[j] += active ? a[j] : 0.0;
            }
        }
    }

    // this block's non-finite flag (the call's status word is set from all of them by the
    // launch that finishes the scales, so nothing has to clear it first)
    if (PASS >= 2) {
        const int anybad = __syncthreads_or((int)bad);
        if (threadIdx.x == 0) flags[blockIdx.y * gridDim.x + blockIdx.x] = anybad ? 1u : 0u;
    }
    if (PASS < 2 || PASS == 3 || MODE == BD_SCALE_MATRIX) {
        const double tot = block_sum(acc, sh);
        if (threadIdx.x == 0) part[rc * n_seg + seg] = tot;
    }
    if (kCol) {
        double* pc = PASS == 3 ? part + n_blocks + d_out * n_seg : part;
#pragma unroll
        for (int j = 0; j < 8; ++j) colsh[wave][8 * lane + j] = colacc[j];
        __syncthreads();
        for (int c = threadIdx.x; c < kSegCols; c += kCompressThreads) {
            const int64_t col = seg * kSegCols + c;
            if (col < d_in) {
                double v = 0.0;
                for (int w = 0; w < kCompressThreads / 64; ++w) v += colsh[w][c];
                pc[rc * d_in + col] = v;
            }
        }
    }
}

// Clip bounds from the pass partials (one block).
template <int PASS>
__global__ void __launch_bounds__(256)
k_stats_finalize(const double* __restrict__ part, int64_t n_part, int64_t n, double k, Stats* st) {
    __shared__ double sh[256];
    double v = 0.0;
    for (int64_t i = threadIdx.x; i < n_part; i += 256) v += part[i];
    sh[threadIdx.x] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = 0.0;
        for (int i = 0; i < 256; ++i) s += sh[i];
        if (PASS == 0) {
            st->mu = s / (double)n;
        } else {
            const double sigma = sqrt(s / (double)(n - 1));
            st->sigma = sigma;
            st->lo = st->mu - k * sigma;
            st->hi = st->mu + k * sigma;
        }
    }
}

__device__ __forceinline__ void store_scale(void* scales, int sdtype, int64_t i, double v) {
    if (sdtype == BD_F16) ((uint16_t*)scales)[i] = f64_to_f16(v);
    else ((float*)scales)[i] = (float)v;
}

// The call's status word from the packing pass's block flags (one block of 256 threads;
// every thread must call it).
__device__ __forceinline__ void status_from_flags(const uint32_t* __restrict__ flags,
                                                  int64_t n_flags, uint32_t* __restrict__ status) {
    uint32_t any = 0u;
    for (int64_t i = threadIdx.x; i < n_flags; i += 256) any |= flags[i];
    const int bad = __syncthreads_or((int)any);
    if (threadIdx.x == 0) status[0] = bad ? ST_NONFINITE : 0u;
}

// GROUP scales are final after the packing pass: the status word only.
__global__ void __launch_bounds__(256)
k_status_finalize(const uint32_t* __restrict__ flags, int64_t n_flags, uint32_t* __restrict__ status) {
    status_from_flags(flags, n_flags, status);
}

// Scale finalisation for MATRIX (one block), ROW (thread per row), COL (thread per column);
// block 0 also sets the status word.
__global__ void __launch_bounds__(256)
k_scales_finalize(int mode, const double* __restrict__ part, int64_t n_seg, int64_t n_rchunk,
                  int64_t d_out, int64_t d_in, int sdtype, void* __restrict__ scales,
                  const uint32_t* __restrict__ flags, uint32_t* __restrict__ status) {
    if (blockIdx.x == 0) status_from_flags(flags, n_seg * n_rchunk, status);
    if (mode == BD_SCALE_MATRIX) {
        __shared__ double sh[256];
        const int64_t n_part = n_seg * n_rchunk;
        double v = 0.0;
        for (int64_t i = threadIdx.x; i < n_part; i += 256) v += part[i];
        sh[threadIdx.x] = v;
        __syncthreads();
        if (threadIdx.x == 0) {
            double s = 0.0;
            for (int i = 0; i < 256; ++i) s += sh[i];
            store_scale(scales, sdtype, 0, s / ((double)d_out * (double)d_in));
        }
        return;
    }
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (mode == BD_SCALE_ROW) {
        if (i >= d_out) return;
        double s = 0.0;
#pragma unroll 8
        for (int64_t c = 0; c < n_seg; ++c) s += part[i * n_seg + c];
        store_scale(scales, sdtype, i, s / (double)d_in);
    } else {  // COL
        if (i >= d_in) return;
        double s = 0.0;
#pragma unroll 8
        for (int64_t c = 0; c < n_rchunk; ++c) s += part[c * d_in + i];
        store_scale(scales, sdtype, i, s / (double)d_out);
    }
}

// Axis choice, step 1 (thread per row and per column): the squared sum of |d| of each
// row (over its segments) and of each column (over its row chunks), in a fixed order.
__global__ void __launch_bounds__(256)
k_axis_sums(const double* __restrict__ part, int64_t n_seg, int64_t n_rchunk, int64_t n_blocks,
            int64_t d_out, int64_t d_in, double* __restrict__ rsq, double* __restrict__ csq) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const double* prow = part + n_blocks;
    const double* pcol = prow + d_out * n_seg;
    // (unrolled so that the loads of a run go out together; the sum keeps its order)
    if (i < d_out) {
        double v = 0.0;
#pragma unroll 8
        for (int64_t c = 0; c < n_seg; ++c) v += prow[i * n_seg + c];
        rsq[i] = v * v;
    }
    if (i < d_in) {
        double v = 0.0;
#pragma unroll 8
        for (int64_t c = 0; c < n_rchunk; ++c) v += pcol[c * d_in + i];
        csq[i] = v * v;
    }
}

// Axis choice, step 2 (one block): for a unit of n deltas with absmean s = sum|d| / n,
// sum (|d| - s)^2 = sum d^2 - (sum |d|)^2 / n, so
//   err_row = sum d^2 - sum_rows (sum |d|)^2 / d_in,  err_col = sum d^2 - sum_cols (..)^2 / d_out;
// ROW when err_row <= err_col.  Every sum runs in a fixed order.
__global__ void __launch_bounds__(256)
k_axis_finalize(const double* __restrict__ part, int64_t n_blocks, const double* __restrict__ rsq,
                const double* __restrict__ csq, int64_t d_out, int64_t d_in,
                double* __restrict__ errors, int32_t* __restrict__ axis,
                const uint32_t* __restrict__ flags, uint32_t* __restrict__ status) {
    status_from_flags(flags, n_blocks, status);
    __shared__ double sh[3][256];
    double a = 0.0, b = 0.0, c = 0.0;
#pragma unroll 8
    for (int64_t i = threadIdx.x; i < n_blocks; i += 256) a += part[i];
#pragma unroll 8
    for (int64_t i = threadIdx.x; i < d_out; i += 256) b += rsq[i];
#pragma unroll 8
    for (int64_t i = threadIdx.x; i < d_in; i += 256) c += csq[i];
    sh[0][threadIdx.x] = a;
    sh[1][threadIdx.x] = b;
    sh[2][threadIdx.x] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        double ss = 0.0, R = 0.0, C = 0.0;
        for (int i = 0; i < 256; ++i) {
            ss += sh[0][i];
            R += sh[1][i];
            C += sh[2][i];
        }
        const double er = ss - R / (double)d_in, ec = ss - C / (double)d_out;
        if (errors) {
            errors[0] = er;
            errors[1] = ec;
        }
        if (axis) axis[0] = er <= ec ? BD_SCALE_ROW : BD_SCALE_COL;
    }
}

__global__ void k_zero_u32(uint32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

template <typename WT, bool HB>
hipError_t launch_typed(const CompressPlan& pl, const WT* wf, const WT* wb, uint64_t* signs,
                        void* scales, char* ws, hipStream_t s) {
    uint32_t* status = (uint32_t*)(ws + pl.off_status);
    Stats* st = (Stats*)(ws + pl.off_stats);
    double* psum = (double*)(ws + pl.off_part_sum);
    double* pm2 = (double*)(ws + pl.off_part_m2);
    double* pabs = (double*)(ws + pl.off_part_abs);
    uint32_t* flags = (uint32_t*)(ws + pl.off_flags);
    const dim3 grid((unsigned)pl.n_seg, (unsigned)pl.n_rchunk), block(kCompressThreads);
    if (pl.clip) {
        hipLaunchKernelGGL((k_compress<WT, HB, 0, 0, false>), grid, block, 0, s, wf, wb, pl.d_out,
                           pl.d_in, pl.rows_per_block, pl.group, pl.sdtype, signs, scales, st, psum,
                           flags);
        hipLaunchKernelGGL(k_stats_finalize<0>, dim3(1), dim3(256), 0, s, psum, pl.n_blocks, pl.n,
                           pl.clip_k, st);
        hipLaunchKernelGGL((k_compress<WT, HB, 1, 0, false>), grid, block, 0, s, wf, wb, pl.d_out,
                           pl.d_in, pl.rows_per_block, pl.group, pl.sdtype, signs, scales, st, pm2,
                           flags);
        hipLaunchKernelGGL(k_stats_finalize<1>, dim3(1), dim3(256), 0, s, pm2, pl.n_blocks, pl.n,
                           pl.clip_k, st);
    }
#define BD_PACK(MODE, CL)                                                                          \
    hipLaunchKernelGGL((k_compress<WT, HB, 2, MODE, CL>), grid, block, 0, s, wf, wb, pl.d_out,    \
                       pl.d_in, pl.rows_per_block, pl.group, pl.sdtype, signs, scales, st, pabs,  \
                       flags)
    switch (pl.mode) {
        case BD_SCALE_MATRIX: if (pl.clip) BD_PACK(BD_SCALE_MATRIX, true); else BD_PACK(BD_SCALE_MATRIX, false); break;
        case BD_SCALE_GROUP: if (pl.clip) BD_PACK(BD_SCALE_GROUP, true); else BD_PACK(BD_SCALE_GROUP, false); break;
        case BD_SCALE_ROW: if (pl.clip) BD_PACK(BD_SCALE_ROW, true); else BD_PACK(BD_SCALE_ROW, false); break;
        default: if (pl.clip) BD_PACK(BD_SCALE_COL, true); else BD_PACK(BD_SCALE_COL, false); break;
    }
#undef BD_PACK
    if (pl.mode != BD_SCALE_GROUP) {
        int64_t nthreads = pl.mode == BD_SCALE_MATRIX ? 256 : (pl.mode == BD_SCALE_ROW ? pl.d_out : pl.d_in);
        unsigned nb = pl.mode == BD_SCALE_MATRIX ? 1u : (unsigned)((nthreads + 255) / 256);
        hipLaunchKernelGGL(k_scales_finalize, dim3(nb), dim3(256), 0, s, pl.mode, pabs, pl.n_seg,
                           pl.n_rchunk, pl.d_out, pl.d_in, pl.sdtype, scales, flags, status);
    } else {
        hipLaunchKernelGGL(k_status_finalize, dim3(1), dim3(256), 0, s, flags, pl.n_blocks, status);
    }
    return hipGetLastError();
}

template <typename WT, bool HB>
hipError_t launch_axis_typed(const AxisPlan& ap, const WT* wf, const WT* wb, double* errors,
                             int32_t* axis, char* ws, hipStream_t s) {
    const CompressPlan& pl = ap.c;
    uint32_t* status = (uint32_t*)(ws + pl.off_status);
    Stats* st = (Stats*)(ws + pl.off_stats);
    double* psum = (double*)(ws + pl.off_part_sum);
    double* pm2 = (double*)(ws + pl.off_part_m2);
    double* part = (double*)(ws + ap.off_part);
    double* rsq = (double*)(ws + ap.off_rsq);
    double* csq = (double*)(ws + ap.off_csq);
    uint32_t* flags = (uint32_t*)(ws + pl.off_flags);
    const dim3 grid((unsigned)pl.n_seg, (unsigned)pl.n_rchunk), block(kCompressThreads);
    if (pl.clip) {
        hipLaunchKernelGGL((k_compress<WT, HB, 0, 0, false>), grid, block, 0, s, wf, wb, pl.d_out,
                           pl.d_in, pl.rows_per_block, 0, BD_F32, nullptr, nullptr, st, psum,
                           flags);
        hipLaunchKernelGGL(k_stats_finalize<0>, dim3(1), dim3(256), 0, s, psum, pl.n_blocks, pl.n,
                           pl.clip_k, st);
        hipLaunchKernelGGL((k_compress<WT, HB, 1, 0, false>), grid, block, 0, s, wf, wb, pl.d_out,
                           pl.d_in, pl.rows_per_block, 0, BD_F32, nullptr, nullptr, st, pm2,
                           flags);
        hipLaunchKernelGGL(k_stats_finalize<1>, dim3(1), dim3(256), 0, s, pm2, pl.n_blocks, pl.n,
                           pl.clip_k, st);
        hipLaunchKernelGGL((k_compress<WT, HB, 3, BD_SCALE_COL, true>), grid, block, 0, s, wf, wb,
                           pl.d_out, pl.d_in, pl.rows_per_block, 0, BD_F32, nullptr, nullptr, st,
                           part, flags);
    } else {
        hipLaunchKernelGGL((k_compress<WT, HB, 3, BD_SCALE_COL, false>), grid, block, 0, s, wf, wb,
                           pl.d_out, pl.d_in, pl.rows_per_block, 0, BD_F32, nullptr, nullptr, st,
                           part, flags);
    }
    const int64_t nmax = pl.d_out > pl.d_in ? pl.d_out : pl.d_in;
    hipLaunchKernelGGL(k_axis_sums, dim3((unsigned)((nmax + 255) / 256)), dim3(256), 0, s, part,
                       pl.n_seg, pl.n_rchunk, pl.n_blocks, pl.d_out, pl.d_in, rsq, csq);
    hipLaunchKernelGGL(k_axis_finalize, dim3(1), dim3(256), 0, s, part, pl.n_blocks, rsq, csq,
                       pl.d_out, pl.d_in, errors, axis, flags, status);
    return hipGetLastError();
}

}  // namespace

bd_status make_axis_plan(float clip_k, int64_t d_out, int64_t d_in, AxisPlan* ap) {
    if (!ap) return BD_ERR_INVALID_ARG;
    bd_compress_params p;
    p.bits = 1;
    p.mode = BD_SCALE_COL;  // the row chunks of the column partials
    p.group_size = 0;
    p.clip_k = clip_k;
    p.scale_dtype = BD_F32;
    AxisPlan q;
    const bd_status st = make_compress_plan(&p, d_out, d_in, &q.c);
    if (st != BD_OK) return st;
    size_t off = q.c.off_part_abs;  // the compress layout up to its partials, then ours
    q.off_part = off;
    off += align_up(sizeof(double) * (size_t)(q.c.n_blocks + d_out * q.c.n_seg +
                                              q.c.n_rchunk * d_in));
    q.off_rsq = off;
    off += align_up(sizeof(double) * (size_t)d_out);
    q.off_csq = off;
    off += align_up(sizeof(double) * (size_t)d_in);
    q.c.off_flags = off;  // (after ours: the compress layout's flags would overlap them)
    off += align_up(sizeof(uint32_t) * (size_t)q.c.n_blocks);
    q.total = off;
    *ap = q;
    return BD_OK;
}

hipError_t launch_select_axis(const AxisPlan& ap, const void* wf, const void* wb, int wdtype,
                              double* errors, int32_t* axis, char* ws, hipStream_t s) {
    if (wdtype == BD_BF16) {
        if (wb) return launch_axis_typed<uint16_t, true>(ap, (const uint16_t*)wf, (const uint16_t*)wb, errors, axis, ws, s);
        return launch_axis_typed<uint16_t, false>(ap, (const uint16_t*)wf, nullptr, errors, axis, ws, s);
    }
    if (wb) return launch_axis_typed<float, true>(ap, (const float*)wf, (const float*)wb, errors, axis, ws, s);
    return launch_axis_typed<float, false>(ap, (const float*)wf, nullptr, errors, axis, ws, s);
}

bd_status make_compress_plan(const bd_compress_params* p, int64_t d_out, int64_t d_in,
                             CompressPlan* pl) {
    if (!p || !pl) return BD_ERR_INVALID_ARG;
    if (p->bits != 1) return BD_ERR_UNSUPPORTED;
    if (p->mode < BD_SCALE_MATRIX || p->mode > BD_SCALE_COL) return BD_ERR_INVALID_ARG;
    if (p->scale_dtype != BD_F32 && p->scale_dtype != BD_F16) return BD_ERR_DTYPE;
    if (!(p->clip_k >= 0.0f) || p->clip_k > 1e30f) return BD_ERR_INVALID_ARG;  // rejects NaN too
    if (d_out <= 0 || d_in <= 0) return BD_ERR_SHAPE;
    if (d_in % 64 != 0) return BD_ERR_SHAPE;
    if (d_out > (int64_t)1 << 31 || d_in > (int64_t)1 << 31) return BD_ERR_SHAPE;
    if (p->mode == BD_SCALE_GROUP) {
        const int g = p->group_size;
        if (g < 8 || g > kSegCols || (g & (g - 1)) != 0) return BD_ERR_UNSUPPORTED;
        if (d_in % g != 0) return BD_ERR_SHAPE;
    }
    CompressPlan q;
    q.d_out = d_out;
    q.d_in = d_in;
    q.n = d_out * d_in;
    q.mode = p->mode;
    q.group = p->mode == BD_SCALE_GROUP ? p->group_size : 0;
    q.sdtype = p->scale_dtype;
    q.clip = p->clip_k > 0.0f;
    q.clip_k = (double)p->clip_k;
    if (q.clip && q.n < 2) return BD_ERR_SHAPE;
    q.n_seg = (d_in + kSegCols - 1) / kSegCols;
    // Column partials are written once per row chunk: use taller chunks there.
    q.rows_per_block = p->mode == BD_SCALE_COL ? 64 : 16;
    q.n_rchunk = (d_out + q.rows_per_block - 1) / q.rows_per_block;
    if (q.n_rchunk > 65535) {  // grid.y limit: grow the chunk instead
        q.rows_per_block = (d_out + 65534) / 65535;
        q.rows_per_block = (q.rows_per_block + 15) / 16 * 16;
        q.n_rchunk = (d_out + q.rows_per_block - 1) / q.rows_per_block;
    }
    q.n_blocks = q.n_seg * q.n_rchunk;
    size_t off = 0;
    q.off_status = off;
    off += kAlign;
    q.off_stats = off;
    off += align_up(sizeof(double) * 4);
    q.off_part_sum = off;
    off += q.clip ? align_up(sizeof(double) * (size_t)q.n_blocks) : 0;
    q.off_part_m2 = off;
    off += q.clip ? align_up(sizeof(double) * (size_t)q.n_blocks) : 0;
    q.off_part_abs = off;
    size_t nabs = 0;
    if (q.mode == BD_SCALE_MATRIX) nabs = (size_t)q.n_blocks;
    if (q.mode == BD_SCALE_ROW) nabs = (size_t)(d_out * q.n_seg);
    if (q.mode == BD_SCALE_COL) nabs = (size_t)(q.n_rchunk * d_in);
    off += align_up(sizeof(double) * nabs);
    q.off_flags = off;
    off += align_up(sizeof(uint32_t) * (size_t)q.n_blocks);
    q.total = off;
    *pl = q;
    return BD_OK;
}

hipError_t launch_compress(const CompressPlan& pl, const void* wf, const void* wb, int wdtype,
                           uint64_t* signs, void* scales, char* ws, hipStream_t s) {
    if (wdtype == BD_BF16) {
        if (wb) return launch_typed<uint16_t, true>(pl, (const uint16_t*)wf, (const uint16_t*)wb, signs, scales, ws, s);
        return launch_typed<uint16_t, false>(pl, (const uint16_t*)wf, nullptr, signs, scales, ws, s);
    }
    if (wb) return launch_typed<float, true>(pl, (const float*)wf, (const float*)wb, signs, scales, ws, s);
    return launch_typed<float, false>(pl, (const float*)wf, nullptr, signs, scales, ws, s);
}

hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t nb64 = (n + 255) / 256;
    unsigned nb = (unsigned)(nb64 < 4096 ? nb64 : 4096);
    hipLaunchKernelGGL(k_zero_u32, dim3(nb), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace bd
