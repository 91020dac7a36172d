// bd_apply.hip -- multi-tenant BitDelta apply on gfx950.
//
// y[t] = X[t] W_base^T + scale_u (.) (X[t] S_u^T), u = user of token t
// ([P2] "Systems Mechanics" 1: the shared base product is computed once for
// the batch, each request adds its own 1-bit delta product; 2: the bits cross
// HBM packed and are expanded on chip, no dense per-user weight).
//
// Kernels, in launch order (bf16 path):
//   k_group      one block: sorts (user, token) keys with a bitonic network in
//                LDS, so tokens of a user are contiguous and in token order;
//                emits work items of <= kItemTokens tokens of one user.
//   k_prep_x     gathers X rows in that order into a workspace copy whose
//                32-column blocks are permuted to the order in which the delta
//                kernel unpacks bit pairs (COL scales are applied here).
//   k_base_gemm  Y = X W_base^T with v_mfma_f32_16x16x32_bf16, fp32 out.
//   k_delta      per (64-row tile, work item): streams the user's packed
//                rows once, turns bits into +-1 bf16 MFMA operands in
//                registers, accumulates X S^T in fp32 and adds scale * sum
//                into Y.  Each Y element belongs to one item: no atomics.
// fp32 inputs take plain VALU kernels (reference-grade, fp32 FMA).
#include "bd_internal.h"

namespace bd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

constexpr int kGroupThreads = 1024;

// ------------------------------------------------------------------ group
// meta[0] status bits, meta[1] number of items, meta[2] number of tokens with
// a valid user.  items[i] = {user, first sorted position, token count, 0}.
__global__ void __launch_bounds__(kGroupThreads)
k_group(const int32_t* __restrict__ ids, int T, int U, int P, int32_t* __restrict__ perm,
        int4* __restrict__ items, uint32_t* __restrict__ meta) {
    extern __shared__ uint32_t keys[];  // P entries
    __shared__ int32_t sc[kGroupThreads];
    __shared__ int nvalid_sh;
    const int tid = threadIdx.x;
    bool badid = false;
    for (int i = tid; i < P; i += kGroupThreads) {
        uint32_t k = 0xFFFFFFFFu;
        if (i < T) {
            const int u = ids[i];
            uint32_t uu;
            if (u >= 0 && u < U) {
                uu = (uint32_t)u;
            } else {
                uu = (uint32_t)U;
                badid |= u != -1;
            }
            k = (uu << 14) | (uint32_t)i;
        }
        keys[i] = k;
    }
    if (badid) atomicOr(&meta[0], ST_USER_ID);
    if (tid == 0) nvalid_sh = T;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < P; i += kGroupThreads) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const uint32_t a = keys[i], b = keys[ixj];
                    const bool up = (i & k) == 0;
                    if ((a > b) == up) {
                        keys[i] = b;
                        keys[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < T; i += kGroupThreads) {
        const bool v = (keys[i] >> 14) < (uint32_t)U;
        const bool vprev = i == 0 || (keys[i - 1] >> 14) < (uint32_t)U;
        if (!v && vprev) nvalid_sh = i;
        if (v) perm[i] = (int32_t)(keys[i] & 0x3FFFu);
    }
    __syncthreads();
    const int nv = nvalid_sh;
    // items: every segment start emits ceil(len / kItemTokens) items
    auto seg_chunks = [&](int i, int* seg_end) -> int {
        const uint32_t u = keys[i] >> 14;
        if (i > 0 && (keys[i - 1] >> 14) == u) return 0;
        const uint32_t lim = (u + 1) << 14;
        int lo = i + 1, hi = nv;  // first position with key >= lim
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (keys[mid] < lim) lo = mid + 1;
            else hi = mid;
        }
        *seg_end = lo;
        return (lo - i + kItemTokens - 1) / kItemTokens;
    };
    const int per = (nv + kGroupThreads - 1) / kGroupThreads;
    const int lo = tid * per, hi = min(nv, lo + per);
    int local = 0, e;
    for (int i = lo; i < hi; ++i) local += seg_chunks(i, &e);
    sc[tid] = local;
    __syncthreads();
    for (int off = 1; off < kGroupThreads; off <<= 1) {  // inclusive scan
        const int v = tid >= off ? sc[tid - off] : 0;
        __syncthreads();
        sc[tid] += v;
        __syncthreads();
    }
    int base = sc[tid] - local;
    for (int i = lo; i < hi; ++i) {
        const int c = seg_chunks(i, &e);
        for (int q = 0; q < c; ++q) {
            const int b = i + q * kItemTokens;
            items[base + q] = make_int4((int)(keys[i] >> 14), b, min(kItemTokens, e - b), 0);
        }
        base += c;
    }
    if (tid == kGroupThreads - 1) {
        meta[1] = (uint32_t)sc[kGroupThreads - 1];
        meta[2] = (uint32_t)nv;
    }
}

// ----------------------------------------------------------------- prep X
// Xp[i][32c + 8q + 2j + h] = X[perm[i]][32c + 4q + j + 16h] (times the user's
// column scale in COL mode), for the nv tokens that have a user.
template <bool COL>
__global__ void __launch_bounds__(256)
k_prep_x(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
         const int4* __restrict__ items, const uint32_t* __restrict__ meta, int64_t T, int64_t d_in,
         const void* __restrict__ scales, int sdtype, int64_t per_user, const int32_t* __restrict__ ids,
         uint16_t* __restrict__ xp) {
    const int64_t nv = meta[2];
    const int64_t per_row = d_in / 8;  // 8 output elements per thread
    const int64_t total = nv * per_row;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = idx / per_row, r = idx % per_row;
        const int64_t blk = r / 4, q = r % 4;
        const int64_t t = perm[i];
        const uint16_t* src = x + t * d_in + blk * 32 + 4 * q;
        const u32x2 a = *(const u32x2*)src;          // k = 4q .. 4q+3
        const u32x2 b = *(const u32x2*)(src + 16);   // k = 4q+16 .. 4q+19
        u32x4 o;
        if (!COL) {
            o.x = (a.x & 0xFFFFu) | (b.x << 16);
            o.y = (a.x >> 16) | (b.x & 0xFFFF0000u);
            o.z = (a.y & 0xFFFFu) | (b.y << 16);
            o.w = (a.y >> 16) | (b.y & 0xFFFF0000u);
        } else {
            const int u = ids[t];
            const int64_t k0 = blk * 32 + 4 * q;
            float s[8];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int64_t s0 = (int64_t)u * per_user + k0 + jj, s1 = s0 + 16;
                if (sdtype == BD_F16) {
                    s[2 * jj] = f16_to_f32(((const uint16_t*)scales)[s0]);
                    s[2 * jj + 1] = f16_to_f32(((const uint16_t*)scales)[s1]);
                } else {
                    s[2 * jj] = ((const float*)scales)[s0];
                    s[2 * jj + 1] = ((const float*)scales)[s1];
                }
            }
            const float xa[4] = {bf16_lo(a.x), bf16_hi(a.x), bf16_lo(a.y), bf16_hi(a.y)};
            const float xb[4] = {bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y)};
            uint32_t w[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                w[jj] = (uint32_t)f32_to_bf16(xa[jj] * s[2 * jj]) |
                        ((uint32_t)f32_to_bf16(xb[jj] * s[2 * jj + 1]) << 16);
            o = u32x4{w[0], w[1], w[2], w[3]};
        }
        *(u32x4*)(xp + i * d_in + blk * 32 + 8 * q) = o;
    }
    (void)items;
    (void)T;
}

// -------------------------------------------------------------- base GEMM
// Block = 8 waves on one 16-row tile of W and NT 16-token tiles of X; wave w
// takes the 32-wide K steps w, w+8, ... and the 8 partial tiles are summed in
// LDS in wave order.
constexpr int kGemmWaves = 8;
constexpr int kGemmUnroll = 4;

template <int NT>
__global__ void __launch_bounds__(64 * kGemmWaves)
k_base_gemm(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ y,
            int64_t T, int64_t d_in, int64_t d_out) {
    __shared__ f32x4 red[kGemmWaves][NT][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int64_t r0 = (int64_t)blockIdx.x * 16, t0 = (int64_t)blockIdx.y * 16 * NT;
    const int64_t rowA = r0 + m < d_out ? r0 + m : d_out - 1;
    const uint16_t* wrow = w + rowA * d_in + 8 * g;
    const uint16_t* xrow[NT];
    bool tok_ok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int64_t t = t0 + 16 * nt + m;
        tok_ok[nt] = t < T;
        xrow[nt] = x + (tok_ok[nt] ? t : 0) * d_in + 8 * g;
    }
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t nsteps = d_in / 32;
    for (int64_t s = wv; s < nsteps; s += kGemmWaves * kGemmUnroll) {
        u32x4 A[kGemmUnroll], B[kGemmUnroll][NT];
#pragma unroll
        for (int u = 0; u < kGemmUnroll; ++u) {
            const int64_t st = s + (int64_t)u * kGemmWaves;
            const bool ok = st < nsteps;
            A[u] = ok ? __builtin_nontemporal_load((const u32x4*)(wrow + st * 32)) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                B[u][nt] = (ok && tok_ok[nt]) ? *(const u32x4*)(xrow[nt] + st * 32) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kGemmUnroll; ++u)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma_bf16(A[u], B[u][nt], acc[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) red[wv][nt][lane] = acc[nt];
    __syncthreads();
    if (wv != 0) return;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        f32x4 v = red[0][nt][lane];
        for (int q = 1; q < kGemmWaves; ++q) v += red[q][nt][lane];
        const int64_t t = t0 + 16 * nt + m;  // D column = lane % 16
        const int64_t o = r0 + 4 * g;        // D rows 4*(lane/16) .. +3
        if (t >= T) continue;
        float* dst = y + t * d_out + o;
        if (o + 3 < d_out && (d_out & 3) == 0) {
            *(f32x4*)dst = v;
        } else {
            for (int e = 0; e < 4; ++e)
                if (o + e < d_out) dst[e] = v[e];
        }
    }
}

// ------------------------------------------------------------ delta apply
// A operand of one MFMA step from a 32-bit word of packed signs: element pair
// j of step q takes bits (4q + j) and (4q + j + 16) into the two bf16 sign
// positions.  Bit 1 (+1) gives -1.0 and bit 0 gives +1.0, so the accumulator
// holds -(X S^T); the epilogue multiplies by -scale.
__device__ __forceinline__ u32x4 expand_pairs(uint32_t d, int q) {
    u32x4 a;
    a.x = ((d << (15 - 4 * q)) & 0x80008000u) | 0x3F803F80u;
    a.y = ((d << (14 - 4 * q)) & 0x80008000u) | 0x3F803F80u;
    a.z = ((d << (13 - 4 * q)) & 0x80008000u) | 0x3F803F80u;
    a.w = ((d << (12 - 4 * q)) & 0x80008000u) | 0x3F803F80u;
    return a;
}

__device__ __forceinline__ float load_scale(const void* s, int sdtype, int64_t i) {
    return sdtype == BD_F16 ? f16_to_f32(((const uint16_t*)s)[i]) : ((const float*)s)[i];
}

constexpr int kDeltaWaves = 4;  // 64 output rows per block

template <int MODE>
__global__ void __launch_bounds__(64 * kDeltaWaves)
k_delta(const uint16_t* __restrict__ xp, const uint64_t* __restrict__ signs,
        const void* __restrict__ scales, int sdtype, int64_t per_user, int group,
        const int4* __restrict__ items, const uint32_t* __restrict__ meta,
        const int32_t* __restrict__ perm, float* __restrict__ y, int64_t d_in, int64_t d_out) {
    const int item = blockIdx.y;
    if (item >= (int)meta[1]) return;
    const int4 it = items[item];
    const int u = it.x, b = it.y, n = it.z;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int64_t r0 = (int64_t)blockIdx.x * (16 * kDeltaWaves) + 16 * wv;
    if (r0 >= d_out) return;
    const int64_t wpr32 = d_in / 32;
    const int64_t rowA = r0 + m < d_out ? r0 + m : d_out - 1;
    const uint32_t* bits = (const uint32_t*)(signs + (int64_t)u * d_out * (d_in / 64)) + rowA * wpr32;
    const void* su = (const char*)scales + (size_t)u * per_user * (sdtype == BD_F16 ? 2 : 4);
    const int ntl = (n + 15) >> 4;

    const uint16_t* xr[4];
    bool tok_ok[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int slot = 16 * nt + m;
        tok_ok[nt] = slot < n;
        xr[nt] = xp + (int64_t)(b + (tok_ok[nt] ? slot : 0)) * d_in;
    }
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (MODE != BD_SCALE_GROUP) {
        // super-step of 512 columns: lane group g owns columns [kb+128g, kb+128g+128)
        for (int64_t kb = 0; kb < d_in; kb += 512) {
            const int64_t kg = kb + 128 * g;
            u32x4 D;
            if (kg + 128 <= d_in) {
                D = __builtin_nontemporal_load((const u32x4*)(bits + kg / 32));
            } else {
                D = u32x4{0, 0, 0, 0};
                for (int c = 0; c < 4; ++c)
                    if (kg + 32 * c < d_in) D[c] = bits[kg / 32 + c];
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t k0 = kg + 32 * c;
                const bool kok = k0 < d_in;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4 A = expand_pairs(D[c], q);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        if (nt < ntl) {
                            const u32x4 B = (kok && tok_ok[nt])
                                                ? *(const u32x4*)(xr[nt] + k0 + 8 * q)
                                                : u32x4{0, 0, 0, 0};
                            acc[nt] = mfma_bf16(A, B, acc[nt]);
                        }
                    }
                }
            }
        }
    } else {
        // GROUP (group = 128 * 2^a): every MFMA step stays inside one 128-column
        // block; partial sums are scaled when a group is complete.
        f32x4 accp[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) accp[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int64_t gpr = d_in / group;
        const int blocks_per_group = group / 128;
        const int64_t nblk = d_in / 128;
        for (int64_t G = 0; G < nblk; ++G) {
            const uint32_t dw = bits[G * 4 + g];
            const int64_t k0 = G * 128 + 32 * g;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 A = expand_pairs(dw, q);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    if (nt < ntl) {
                        const u32x4 B = tok_ok[nt] ? *(const u32x4*)(xr[nt] + k0 + 8 * q) : u32x4{0, 0, 0, 0};
                        accp[nt] = mfma_bf16(A, B, accp[nt]);
                    }
                }
            }
            if ((G + 1) % blocks_per_group == 0) {
                const int64_t gi = G / blocks_per_group;
                float sc[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    int64_t o = r0 + 4 * g + e;
                    o = o < d_out ? o : d_out - 1;
                    sc[e] = -load_scale(su, sdtype, o * gpr + gi);
                }
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    if (nt < ntl) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[nt][e] += accp[nt][e] * sc[e];
                        accp[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                }
            }
        }
    }

    // epilogue: Y[t][o] += factor * acc
    float f[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        int64_t o = r0 + 4 * g + e;
        o = o < d_out ? o : d_out - 1;
        if (MODE == BD_SCALE_MATRIX) f[e] = -load_scale(su, sdtype, 0);
        else if (MODE == BD_SCALE_ROW) f[e] = -load_scale(su, sdtype, o);
        else if (MODE == BD_SCALE_COL) f[e] = -1.0f;
        else f[e] = 1.0f;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        if (nt >= ntl) break;
        const int slot = 16 * nt + m;
        if (slot >= n) continue;
        const int64_t t = perm[b + slot];
        const int64_t o = r0 + 4 * g;
        float* dst = y + t * d_out + o;
        if (o + 3 < d_out && (d_out & 3) == 0) {
            f32x4 v = *(f32x4*)dst;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += acc[nt][e] * f[e];
            *(f32x4*)dst = v;
        } else {
            for (int e = 0; e < 4; ++e)
                if (o + e < d_out) dst[e] += acc[nt][e] * f[e];
        }
    }
}

__global__ void __launch_bounds__(256) k_cast_bf16(const float* __restrict__ src, uint16_t* __restrict__ dst, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = f32_to_bf16(src[i]);
}

// -------------------------------------------------------------- fp32 path
__global__ void __launch_bounds__(256)
k_base_f32(const float* __restrict__ x, const float* __restrict__ w, float* __restrict__ y,
           int64_t T, int64_t d_in, int64_t d_out) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= T * d_out) return;
    const int64_t t = idx / d_out, o = idx % d_out;
    float s = 0.f;
    for (int64_t k = 0; k < d_in; ++k) s = fmaf(x[t * d_in + k], w[o * d_in + k], s);
    y[idx] = s;
}

__global__ void __launch_bounds__(256)
k_delta_f32(const float* __restrict__ x, const int32_t* __restrict__ ids, int U,
            const uint64_t* __restrict__ signs, const void* __restrict__ scales, int sdtype,
            int64_t per_user, int mode, int group, float* __restrict__ y, int64_t T, int64_t d_in,
            int64_t d_out) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= T * d_out) return;
    const int64_t t = idx / d_out, o = idx % d_out;
    const int u = ids[t];
    if (u < 0 || u >= U) return;
    const uint64_t* row = signs + ((int64_t)u * d_out + o) * (d_in / 64);
    const void* su = (const char*)scales + (size_t)u * per_user * (sdtype == BD_F16 ? 2 : 4);
    const float* xt = x + t * d_in;
    float total = 0.f, part = 0.f;
    for (int64_t k = 0; k < d_in; ++k) {
        const bool pos = (row[k >> 6] >> (k & 63)) & 1ull;
        float xv = xt[k];
        if (mode == BD_SCALE_COL) xv *= load_scale(su, sdtype, k);
        part += pos ? xv : -xv;
        if (mode == BD_SCALE_GROUP && (k + 1) % group == 0) {
            total = fmaf(part, load_scale(su, sdtype, o * (d_in / group) + k / group), total);
            part = 0.f;
        }
    }
    if (mode == BD_SCALE_MATRIX) total = part * load_scale(su, sdtype, 0);
    else if (mode == BD_SCALE_ROW) total = part * load_scale(su, sdtype, o);
    else if (mode == BD_SCALE_COL) total = part;
    y[idx] += total;
}

__global__ void k_check_ids(const int32_t* __restrict__ ids, int64_t T, int U, uint32_t* meta) {
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < T;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int u = ids[i];
        bad |= (u < -1 || u >= U);
    }
    if (__ballot(bad) != 0ull && (threadIdx.x & 63) == 0) atomicOr(meta, ST_USER_ID);
}

unsigned grid_1d(int64_t n, int64_t per_block, int64_t cap = 65535) {
    int64_t g = (n + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (unsigned)g;
}

int pow2_at_least(int64_t n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

}  // namespace

bd_status make_apply_plan(const bd_compress_params* p, int64_t T, int32_t U, int64_t d_out,
                          int64_t d_in, int xdtype, int ydtype, ApplyPlan* pl) {
    if (!p || !pl) return BD_ERR_INVALID_ARG;
    if (p->bits != 1) return BD_ERR_UNSUPPORTED;
    if (p->mode < BD_SCALE_MATRIX || p->mode > BD_SCALE_COL) return BD_ERR_INVALID_ARG;
    if (p->scale_dtype != BD_F32 && p->scale_dtype != BD_F16) return BD_ERR_DTYPE;
    if (xdtype != BD_BF16 && xdtype != BD_F32) return BD_ERR_DTYPE;
    if (ydtype != BD_F32 && ydtype != BD_BF16) return BD_ERR_DTYPE;
    if (T < 0 || U < 0 || U > kMaxUsers) return BD_ERR_INVALID_ARG;
    if (d_out <= 0 || d_in <= 0 || d_in % 64 != 0) return BD_ERR_SHAPE;
    if (d_out > (int64_t)1 << 31 || d_in > (int64_t)1 << 31) return BD_ERR_SHAPE;
    if (p->mode == BD_SCALE_GROUP) {
        const int g = p->group_size;
        if (g < 8 || g > kSegCols || (g & (g - 1)) != 0) return BD_ERR_UNSUPPORTED;
        if (d_in % g != 0) return BD_ERR_SHAPE;
        // the MFMA path keeps each step inside one 128-column block
        if (xdtype == BD_BF16 && g < 128) return BD_ERR_UNSUPPORTED;
    }
    if (xdtype == BD_BF16 && T > kMaxGroupT) return BD_ERR_UNSUPPORTED;
    ApplyPlan q;
    q.T = T;
    q.U = U;
    q.d_in = d_in;
    q.d_out = d_out;
    q.mode = p->mode;
    q.group = p->mode == BD_SCALE_GROUP ? p->group_size : 0;
    q.sdtype = p->scale_dtype;
    q.xdtype = xdtype;
    q.ydtype = ydtype;
    const int64_t act = T < U ? T : U;
    q.max_items = act + T / kItemTokens + 1;
    size_t off = 0;
    q.off_status = off;
    off += kAlign;
    q.off_perm = off;
    off += align_up(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    q.off_items = off;
    off += align_up(sizeof(int4) * (size_t)q.max_items);
    q.off_xp = off;
    if (xdtype == BD_BF16) off += align_up(2 * (size_t)T * (size_t)d_in);
    q.off_yf = off;
    if (ydtype == BD_BF16) off += align_up(4 * (size_t)T * (size_t)d_out);
    q.total = off;
    *pl = q;
    return BD_OK;
}

hipError_t launch_apply(const ApplyPlan& pl, const void* x, const void* wb, const uint64_t* signs,
                        const void* scales, const int32_t* ids, void* y, char* ws, hipStream_t s) {
    uint32_t* meta = (uint32_t*)(ws + pl.off_status);
    hipError_t err = launch_zero_u32(meta, (int64_t)(kAlign / 4), s);
    if (err != hipSuccess || pl.T == 0) return err;
    const int64_t per_user =
        pl.mode == BD_SCALE_MATRIX ? 1
        : pl.mode == BD_SCALE_GROUP ? pl.d_out * (pl.d_in / pl.group)
        : pl.mode == BD_SCALE_ROW ? pl.d_out
                                  : pl.d_in;
    float* yacc = pl.ydtype == BD_F32 ? (float*)y : (float*)(ws + pl.off_yf);
    const int64_t n_out = pl.T * pl.d_out;

    if (pl.xdtype == BD_F32) {
        hipLaunchKernelGGL(k_check_ids, dim3(grid_1d(pl.T, 256, 1024)), dim3(256), 0, s, ids, pl.T,
                           pl.U, meta);
        hipLaunchKernelGGL(k_base_f32, dim3(grid_1d(n_out, 256, 1ll << 30)), dim3(256), 0, s,
                           (const float*)x, (const float*)wb, yacc, pl.T, pl.d_in, pl.d_out);
        hipLaunchKernelGGL(k_delta_f32, dim3(grid_1d(n_out, 256, 1ll << 30)), dim3(256), 0, s,
                           (const float*)x, ids, pl.U, signs, scales, pl.sdtype, per_user, pl.mode,
                           pl.group, yacc, pl.T, pl.d_in, pl.d_out);
    } else {
        int32_t* perm = (int32_t*)(ws + pl.off_perm);
        int4* items = (int4*)(ws + pl.off_items);
        uint16_t* xp = (uint16_t*)(ws + pl.off_xp);
        const int P = pow2_at_least(pl.T);
        hipLaunchKernelGGL(k_group, dim3(1), dim3(kGroupThreads), sizeof(uint32_t) * P, s, ids,
                           (int)pl.T, pl.U, P, perm, items, meta);
        const unsigned gp = grid_1d(pl.T * (pl.d_in / 8), 256, 8192);
        if (pl.mode == BD_SCALE_COL)
            hipLaunchKernelGGL(k_prep_x<true>, dim3(gp), dim3(256), 0, s, (const uint16_t*)x, perm,
                               items, meta, pl.T, pl.d_in, scales, pl.sdtype, per_user, ids, xp);
        else
            hipLaunchKernelGGL(k_prep_x<false>, dim3(gp), dim3(256), 0, s, (const uint16_t*)x, perm,
                               items, meta, pl.T, pl.d_in, scales, pl.sdtype, per_user, ids, xp);
        // base GEMM: tokens in tiles of 16 * NT
        const dim3 gb((unsigned)((pl.d_out + 15) / 16), 1);
        if (pl.T <= 16) {
            hipLaunchKernelGGL(k_base_gemm<1>, gb, dim3(64 * kGemmWaves), 0, s, (const uint16_t*)x,
                               (const uint16_t*)wb, yacc, pl.T, pl.d_in, pl.d_out);
        } else if (pl.T <= 32) {
            hipLaunchKernelGGL(k_base_gemm<2>, gb, dim3(64 * kGemmWaves), 0, s, (const uint16_t*)x,
                               (const uint16_t*)wb, yacc, pl.T, pl.d_in, pl.d_out);
        } else {
            const dim3 g4((unsigned)((pl.d_out + 15) / 16), (unsigned)((pl.T + 63) / 64));
            hipLaunchKernelGGL(k_base_gemm<4>, g4, dim3(64 * kGemmWaves), 0, s, (const uint16_t*)x,
                               (const uint16_t*)wb, yacc, pl.T, pl.d_in, pl.d_out);
        }
        const dim3 gd((unsigned)((pl.d_out + 16 * kDeltaWaves - 1) / (16 * kDeltaWaves)),
                      (unsigned)pl.max_items);
#define BD_DELTA(MODE)                                                                              \
    hipLaunchKernelGGL(k_delta<MODE>, gd, dim3(64 * kDeltaWaves), 0, s, xp, signs, scales,         \
                       pl.sdtype, per_user, pl.group, items, meta, perm, yacc, pl.d_in, pl.d_out)
        switch (pl.mode) {
            case BD_SCALE_MATRIX: BD_DELTA(BD_SCALE_MATRIX); break;
            case BD_SCALE_GROUP: BD_DELTA(BD_SCALE_GROUP); break;
            case BD_SCALE_ROW: BD_DELTA(BD_SCALE_ROW); break;
            default: BD_DELTA(BD_SCALE_COL); break;
        }
#undef BD_DELTA
    }
    if (pl.ydtype == BD_BF16)
        hipLaunchKernelGGL(k_cast_bf16, dim3(grid_1d(n_out, 256, 16384)), dim3(256), 0, s, yacc,
                           (uint16_t*)y, n_out);
    return hipGetLastError();
}

}  // namespace bd
