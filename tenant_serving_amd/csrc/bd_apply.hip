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
//                emits work items of <= kItemTokens tokens of one user (the tile
//                packing of bd_delta.hip reads them).
//   k_base_gemm  Y = X W_base^T with v_mfma_f32_16x16x32_bf16, fp32 out, for
//                16 < T <= 64 (larger batches: k_gemm, bd_gemm.hip).
// The delta products of bf16 batches are in bd_delta.hip; fp32 inputs take plain
// VALU kernels (reference-grade, fp32 FMA).
#include "bd_internal.h"

namespace bd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

constexpr int kGroupThreads = 1024;

// ------------------------------------------------------------------ group
// meta[0] status bits, meta[1] number of items, meta[2] number of tokens with
// a valid user.  items[i] = {user, first sorted position, token count, 0};
// suser[p] = user of sorted position p (p < meta[2]).
__global__ void __launch_bounds__(kGroupThreads)
k_group(const int32_t* __restrict__ ids, int T, int U, int P, int32_t* __restrict__ perm,
        int32_t* __restrict__ suser, int4* __restrict__ items, uint32_t* __restrict__ meta) {
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
    if (tid == 0) nvalid_sh = T;
    const int anybad = __syncthreads_or((int)badid);
    if (tid == 0) {  // the status word is owned by this kernel; no tokens are encoded yet
        meta[0] = anybad ? ST_USER_ID : 0u;
        meta[kEncTagWord] = 0u;
    }
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
        if (v) {
            perm[i] = (int32_t)(keys[i] & 0x3FFFu);
            suser[i] = (int32_t)(keys[i] >> 14);
        }
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

// Batches of at most 64 tokens: one wave, no barriers.  Lane l holds key l;
// a 64-lane bitonic network of shuffles sorts them, ballots find the segment
// starts and prefix counts place the items.  Same outputs as k_group.
__global__ void __launch_bounds__(64)
k_group_wave(const int32_t* __restrict__ ids, int T, int U, int32_t* __restrict__ perm,
             int32_t* __restrict__ suser, int4* __restrict__ items, uint32_t* __restrict__ meta) {
    const int l = threadIdx.x;
    uint32_t key = 0xFFFFFFFFu;
    bool bad = false;
    if (l < T) {
        const int u = ids[l];
        const bool ok = u >= 0 && u < U;
        bad = !ok && u != -1;
        key = ((ok ? (uint32_t)u : (uint32_t)U) << 14) | (uint32_t)l;
    }
    for (int k = 2; k <= 64; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint32_t other = __shfl_xor(key, j);
            const bool lower = (l & j) == 0;          // this lane keeps the smaller if ascending
            const bool asc = (l & k) == 0;
            const uint32_t mn = key < other ? key : other, mx = key < other ? other : key;
            key = (lower == asc) ? mn : mx;
        }
    }
    const uint32_t user = key >> 14;
    const bool valid = user < (uint32_t)U;
    const uint64_t vmask = __ballot(valid);
    const int nv = __popcll(vmask);  // valid keys sort first
    if (valid) {
        perm[l] = (int32_t)(key & 0x3FFFu);
        suser[l] = (int32_t)user;
    }
    const uint32_t prev = __shfl_up(user, 1);
    const bool start = valid && (l == 0 || prev != user);
    const uint64_t smask = __ballot(start);
    const uint64_t above = l == 63 ? 0ull : (smask >> (l + 1)) << (l + 1);
    const int next = above ? __ffsll((unsigned long long)above) - 1 : nv;
    const int len = start ? next - l : 0;
    const int nit = (len + kItemTokens - 1) / kItemTokens;  // 0, 1 or 2
    const uint64_t below = (1ull << l) - 1ull;
    const int base = __popcll(__ballot(nit >= 1) & below) + __popcll(__ballot(nit >= 2) & below);
    for (int q = 0; q < nit; ++q) {
        const int b = l + q * kItemTokens;
        items[base + q] = make_int4((int)user, b, min(kItemTokens, next - b), 0);
    }
    const int total = __popcll(__ballot(nit >= 1)) + __popcll(__ballot(nit >= 2));
    const bool anybad = __ballot(bad) != 0ull;
    if (l == 0) {
        meta[0] = anybad ? ST_USER_ID : 0u;
        meta[kEncTagWord] = 0u;
        meta[1] = (uint32_t)total;
        meta[2] = (uint32_t)nv;
    }
}

constexpr uint32_t kOOB = 0x80000000u;    // buffer offset past num_records: the load returns 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
    const int nrec = bytes > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// -------------------------------------------------------------- base GEMM
// Block = 8 waves on one 16-row tile of W and NT 16-token tiles of X; wave w
// takes the 32-wide K steps w, w+8, ... and the 8 partial tiles are summed in
// LDS in wave order.  Operands stream through a ring of 4 register slots, each
// reloaded in place after its MFMAs, so 3 steps of loads stay in flight; loads
// of absent tokens or steps past d_in are buffer loads out of range (zero).
constexpr int kGemmWaves = 8;

template <int NT>
__global__ void __launch_bounds__(64 * kGemmWaves)
k_base_gemm(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ y,
            int64_t T, int64_t d_in, int64_t d_out) {
    __shared__ f32x4 red[kGemmWaves][NT][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int64_t r0 = (int64_t)blockIdx.x * 16, t0 = (int64_t)blockIdx.y * 16 * NT;
    const int64_t rowA = r0 + m < d_out ? r0 + m : d_out - 1;
    // descriptors stay uniform (SGPRs); the lane's row lives in its 32-bit offset
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint64_t)d_out * d_in * 2);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint64_t)T * d_in * 2);
    const uint32_t woff = (uint32_t)((rowA * d_in + 8 * g) * 2);
    const int64_t nsteps = d_in / 32;
    uint32_t xoff[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int64_t t = t0 + 16 * nt + m;
        xoff[nt] = t < T ? (uint32_t)((t * d_in + 8 * g) * 2) : kOOB;
    }
    struct Slot {
        u32x4 a, b[NT];
    };
    auto load = [&](int64_t st) {
        Slot sl;
        const bool ok = st < nsteps;
        sl.a = buf_load16(wr, ok ? woff + (uint32_t)(st * 64) : kOOB);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            sl.b[nt] = buf_load16(xr, (ok && xoff[nt] != kOOB) ? xoff[nt] + (uint32_t)(st * 64) : kOOB);
        return sl;
    };
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto use = [&](const Slot& sl) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma_bf16(sl.a, sl.b[nt], acc[nt]);
    };
    constexpr int W = kGemmWaves;
    constexpr int R = NT <= 2 ? 8 : 4;  // ring depth: slots whose loads are in flight
    Slot ring[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        ring[r] = load(wv + r * W);
        __builtin_amdgcn_sched_barrier(0);
    }
    // steps past d_in load zeros, so the MFMAs run unconditionally (straight-line
    // code keeps the wait counters exact); scheduling barriers keep each slot's
    // reload after its MFMAs
    for (int64_t st = wv; st < nsteps; st += R * W) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            use(ring[r]);
            ring[r] = load(st + (R + r) * W);
            __builtin_amdgcn_sched_barrier(0);
        }
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

// Scale i of a user (fp32 or fp16 storage).
__device__ __forceinline__ float load_scale(const void* s, int sdtype, int64_t i) {
    return sdtype == BD_F16 ? f16_to_f32(((const uint16_t*)s)[i]) : ((const float*)s)[i];
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
            const uint64_t* __restrict__ signs, uint64_t sstride, const void* __restrict__ scales,
            int sdtype, int64_t cstride, int mode, int group, float* __restrict__ y, int64_t T,
            int64_t d_in, int64_t d_out) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= T * d_out) return;
    const int64_t t = idx / d_out, o = idx % d_out;
    const int u = ids[t];
    if (u < 0 || u >= U) return;
    const uint64_t* row = (const uint64_t*)((const char*)signs + (uint64_t)u * sstride) + o * (d_in / 64);
    const void* su = (const char*)scales + (size_t)u * cstride * (sdtype == BD_F16 ? 2 : 4);
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

// GROUP scales with groups of fewer than 128 columns on bf16 tokens (the matrix-core
// products cover 128 columns per group scale): one block per (sorted position, 256
// rows), one thread per row; the token's row of X comes through LDS in chunks of
// kSmallGroupChunk columns, each thread sums its signed values per group in fp32 and
// adds group sum * group scale.  Each (token, row) has one thread: a plain add into Y.
constexpr int kSmallGroupChunk = 4096;
__global__ void __launch_bounds__(256)
k_delta_small_group(const uint16_t* __restrict__ x, int64_t T, int64_t d_in,
                    const int32_t* __restrict__ perm, const int32_t* __restrict__ suser,
                    const uint32_t* __restrict__ meta, int U, const uint64_t* __restrict__ signs,
                    uint64_t sstride, const void* __restrict__ scales, int sdtype, int64_t cstride,
                    int group, float* __restrict__ y, int64_t d_out) {
    __shared__ float xs[kSmallGroupChunk];
    const int64_t p = blockIdx.y;
    if (p >= (int64_t)meta[2]) return;  // uniform: past the tokens with a valid user
    const int tok = perm[p], u = suser[p];
    if (tok < 0 || tok >= T || u < 0 || u >= U) return;  // uniform
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = o < d_out;
    const int64_t wpr = d_in / 64;
    const uint64_t* srow =
        (const uint64_t*)((const char*)signs + (uint64_t)u * sstride) + (live ? o : 0) * wpr;
    const void* su = (const char*)scales + (size_t)u * cstride * (sdtype == BD_F16 ? 2 : 4);
    const int64_t gpr = d_in / group;
    float total = 0.f;
    for (int64_t c0 = 0; c0 < d_in; c0 += kSmallGroupChunk) {
        const int64_t n = d_in - c0 < kSmallGroupChunk ? d_in - c0 : kSmallGroupChunk;
        __syncthreads();
        for (int64_t i = threadIdx.x; i < n; i += 256)
            xs[i] = __uint_as_float((uint32_t)x[(int64_t)tok * d_in + c0 + i] << 16);
        __syncthreads();
        if (!live) continue;
        for (int64_t w = 0; w < n / 64; ++w) {
            const uint64_t bits = srow[c0 / 64 + w];
            float part = 0.f;
            for (int k = 0; k < 64; ++k) {
                const float v = xs[64 * w + k];
                part += (bits >> k) & 1ull ? v : -v;
                if (((k + 1) & (group - 1)) == 0) {
                    const int64_t gi = (c0 + 64 * w + k) / group;
                    total = fmaf(part, load_scale(su, sdtype, o * gpr + gi), total);
                    part = 0.f;
                }
            }
        }
    }
    if (live) y[(int64_t)tok * d_out + o] += total;
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

bd_status check_params(const bd_compress_params* p, int64_t d_out, int64_t d_in, int xdtype) {
    if (!p) return BD_ERR_INVALID_ARG;
    if (p->bits != 1) return BD_ERR_UNSUPPORTED;
    if (p->mode < BD_SCALE_MATRIX || p->mode > BD_SCALE_COL) return BD_ERR_INVALID_ARG;
    if (p->scale_dtype != BD_F32 && p->scale_dtype != BD_F16) return BD_ERR_DTYPE;
    if (d_out <= 0 || d_out > (int64_t)1 << 31) return BD_ERR_SHAPE;
    if (p->mode == BD_SCALE_GROUP) {
        const int g = p->group_size;
        if (g < 8 || g > kSegCols || (g & (g - 1)) != 0) return BD_ERR_UNSUPPORTED;
        if (d_in % g != 0) return BD_ERR_SHAPE;
        (void)xdtype;  // bf16 groups under 128 columns: k_delta_small_group
    }
    return BD_OK;
}

bd_status make_batch_plan(int64_t T, int32_t U, int64_t d_in, int xdtype, BatchPlan* pl) {
    if (!pl) return BD_ERR_INVALID_ARG;
    if (xdtype != BD_BF16 && xdtype != BD_F32) return BD_ERR_DTYPE;
    if (T < 0 || U < 0 || U > kMaxUsers) return BD_ERR_INVALID_ARG;
    if (d_in <= 0 || d_in % 64 != 0 || d_in > (int64_t)1 << 31) return BD_ERR_SHAPE;
    if (xdtype == BD_BF16 && T > kMaxGroupT) return BD_ERR_UNSUPPORTED;
    // the delta kernel addresses X with 32-bit buffer offsets
    if (T * d_in * 2 >= ((int64_t)1 << 31)) return BD_ERR_UNSUPPORTED;
    BatchPlan q;
    q.T = T;
    q.U = U;
    q.d_in = d_in;
    q.xdtype = xdtype;
    const int64_t act = T < U ? T : U;
    q.max_items = act + T / kItemTokens + 1;
    const size_t Tn = (size_t)(T > 0 ? T : 1);
    size_t off = 0;
    q.off_meta = off;
    off += kAlign;
    q.off_perm = off;
    off += align_up(sizeof(int32_t) * Tn);
    q.off_user = off;
    off += align_up(sizeof(int32_t) * Tn);
    q.off_items = off;
    off += align_up(sizeof(int4) * (size_t)q.max_items);
    if (xdtype == BD_BF16) {
        q.ntiles = 2 * (int64_t)((Tn + 15) / 16) + 1;  // bound of the packed tiles
        q.nunit = 2 * ((d_in + 1023) / 1024);  // even: the delta steps take two units
        q.off_tiles = off;
        off += align_up(sizeof(int32_t) * ((size_t)q.ntiles + 1));
        q.off_torder = off;
        off += align_up(sizeof(int32_t) * (size_t)q.ntiles);
        q.off_tpre = off;
        off += align_up(sizeof(int32_t) * ((size_t)q.ntiles + 1));
        q.off_tmeta = off;
        off += align_up(sizeof(int32_t) * kTileMetaInts * (size_t)q.ntiles);
        q.off_enc = off;
        off += align_up((size_t)kEncUnitBytes * (size_t)q.ntiles * (size_t)q.nunit);
    }
    q.total = off;
    *pl = q;
    return BD_OK;
}

bd_status make_delta_plan(const bd_compress_params* p, const BatchPlan& b, int64_t d_out,
                          DeltaPlan* pl) {
    bd_status st = check_params(p, d_out, b.d_in, b.xdtype);
    if (st != BD_OK) return st;
    // the kernels address one user's bits and the base weight with 32-bit buffer offsets
    if (d_out * (b.d_in / 8) >= ((int64_t)1 << 31)) return BD_ERR_UNSUPPORTED;
    if (b.xdtype == BD_BF16 && d_out * b.d_in * 2 >= ((int64_t)1 << 31)) return BD_ERR_UNSUPPORTED;
    DeltaPlan q;
    q.d_out = d_out;
    q.mode = p->mode;
    q.group = p->mode == BD_SCALE_GROUP ? p->group_size : 0;
    q.sdtype = p->scale_dtype;
    q.per_user = q.mode == BD_SCALE_MATRIX ? 1
                 : q.mode == BD_SCALE_GROUP ? d_out * (b.d_in / q.group)
                 : q.mode == BD_SCALE_ROW ? d_out
                                          : b.d_in;
    *pl = q;
    return BD_OK;
}

bd_status make_apply_plan(const bd_compress_params* p, int64_t T, int32_t U, int64_t d_out,
                          int64_t d_in, int xdtype, int ydtype, ApplyPlan* pl, bool allow_decode) {
    if (!p || !pl) return BD_ERR_INVALID_ARG;
    if (ydtype != BD_F32 && ydtype != BD_BF16) return BD_ERR_DTYPE;
    ApplyPlan q;
    bd_status st = make_batch_plan(T, U, d_in, xdtype, &q.batch);
    if (st != BD_OK) return st;
    st = make_delta_plan(p, q.batch, d_out, &q.delta);
    if (st != BD_OK) return st;
    q.ydtype = ydtype;
    q.decode = allow_decode && decode_path_supported(xdtype, T, p->mode);
    q.fused = allow_decode && fused_path_supported(xdtype, T, p->mode, d_in);
    if (q.decode) {
        make_decode_plan(T, d_in, &q.dec);
        q.total = q.dec.total;
        *pl = q;
        return BD_OK;
    }
    size_t off = q.batch.total;
    q.off_yf = off;
    if (ydtype == BD_BF16) off += align_up(4 * (size_t)T * (size_t)d_out);
    q.total = off;
    *pl = q;
    return BD_OK;
}

hipError_t launch_batch_prepare(const BatchPlan& pl, const void* x, const int32_t* ids,
                                char* batch, hipStream_t s) {
    (void)x;
    uint32_t* meta = (uint32_t*)(batch + pl.off_meta);
    hipError_t err = hipSuccess;
    if (pl.T == 0 || pl.xdtype == BD_F32) err = launch_zero_u32(meta, (int64_t)(kAlign / 4), s);
    if (err != hipSuccess || pl.T == 0) return err;
    if (pl.xdtype == BD_F32) {  // fp32 path: no grouping, the delta kernel reads the ids
        hipLaunchKernelGGL(k_check_ids, dim3(grid_1d(pl.T, 256, 1024)), dim3(256), 0, s, ids, pl.T,
                           pl.U, meta);
        err = hipMemcpyAsync(batch + pl.off_user, ids, sizeof(int32_t) * pl.T,
                             hipMemcpyDeviceToDevice, s);
        return err != hipSuccess ? err : hipGetLastError();
    }
    if (pl.T <= 64) {
        hipLaunchKernelGGL(k_group_wave, dim3(1), dim3(64), 0, s, ids, (int)pl.T, pl.U,
                           (int32_t*)(batch + pl.off_perm), (int32_t*)(batch + pl.off_user),
                           (int4*)(batch + pl.off_items), meta);
    } else {
        const int P = pow2_at_least(pl.T);
        hipLaunchKernelGGL(k_group, dim3(1), dim3(kGroupThreads), sizeof(uint32_t) * P, s, ids,
                           (int)pl.T, pl.U, P, (int32_t*)(batch + pl.off_perm),
                           (int32_t*)(batch + pl.off_user), (int4*)(batch + pl.off_items), meta);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_tile_plan(pl, batch, s);
}

hipError_t launch_base_gemm(const void* x, int xdtype, int64_t T, int64_t d_in, const void* wb,
                            int64_t d_out, float* y, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (xdtype == BD_F32) {
        hipLaunchKernelGGL(k_base_f32, dim3(grid_1d(T * d_out, 256, 1ll << 30)), dim3(256), 0, s,
                           (const float*)x, (const float*)wb, y, T, d_in, d_out);
        return hipGetLastError();
    }
    if (gemm_path_supported(T, d_in, d_out)) return launch_gemm(x, T, d_in, wb, d_out, y, s);
    if (small_batch_gemm_supported(T, d_in, d_out))
        return launch_small_batch_gemm(x, T, d_in, wb, d_out, y, s);
    const dim3 gb((unsigned)((d_out + 15) / 16), 1);
    if (T <= 16) {
        hipLaunchKernelGGL(k_base_gemm<1>, gb, dim3(64 * kGemmWaves), 0, s, (const uint16_t*)x,
                           (const uint16_t*)wb, y, T, d_in, d_out);
    } else if (T <= 32) {
        hipLaunchKernelGGL(k_base_gemm<2>, gb, dim3(64 * kGemmWaves), 0, s, (const uint16_t*)x,
                           (const uint16_t*)wb, y, T, d_in, d_out);
    } else {
        const dim3 g4((unsigned)((d_out + 15) / 16), (unsigned)((T + 63) / 64));
        hipLaunchKernelGGL(k_base_gemm<4>, g4, dim3(64 * kGemmWaves), 0, s, (const uint16_t*)x,
                           (const uint16_t*)wb, y, T, d_in, d_out);
    }
    return hipGetLastError();
}

hipError_t launch_delta(const BatchPlan& bp, const DeltaPlan& dp, char* batch,
                        const void* x, const uint64_t* signs, const void* scales, float* y,
                        hipStream_t s) {
    if (bp.T == 0) return hipSuccess;
    if (bp.xdtype == BD_BF16 && dp.mode == BD_SCALE_GROUP && dp.group < 128) {
        const dim3 g((unsigned)((dp.d_out + 255) / 256), (unsigned)bp.T);
        hipLaunchKernelGGL(k_delta_small_group, g, dim3(256), 0, s, (const uint16_t*)x, bp.T,
                           bp.d_in, (const int32_t*)(batch + bp.off_perm),
                           (const int32_t*)(batch + bp.off_user),
                           (const uint32_t*)(batch + bp.off_meta), bp.U, signs,
                           sign_stride(dp.sstride, dp.d_out, bp.d_in), scales, dp.sdtype,
                           scale_stride(dp), dp.group, y, dp.d_out);
        return hipGetLastError();
    }
    if (bp.xdtype == BD_BF16) return launch_delta6(bp, dp, batch, x, signs, scales, y, s);
    const int32_t* row_user = (const int32_t*)(batch + bp.off_user);
    if (bp.xdtype == BD_F32) {
        hipLaunchKernelGGL(k_delta_f32, dim3(grid_1d(bp.T * dp.d_out, 256, 1ll << 30)), dim3(256), 0,
                           s, (const float*)x, row_user, bp.U, signs,
                           sign_stride(dp.sstride, dp.d_out, bp.d_in), scales, dp.sdtype,
                           scale_stride(dp), dp.mode, dp.group, y, bp.T, bp.d_in, dp.d_out);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;  // (unreachable: bf16 and fp32 are the only x dtypes)
}

hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_cast_bf16, dim3(grid_1d(n, 256, 16384)), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

}  // namespace bd
