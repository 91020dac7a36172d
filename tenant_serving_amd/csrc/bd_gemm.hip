// bd_gemm.hip -- the shared base product Y = X W_base^T for batches of many
// tokens (prefill chunks, large decode batches): a tiled bf16 GEMM on the
// gfx950 matrix cores ([P2] "Systems Mechanics" 1: one dense product of the
// whole batch with the shared base weight).
//
// Block tile: BR rows of W x BT tokens (128 x 256, 128 x 128, 64 x 128 or 64 x 64), 4 waves
// (2 x 2), each BR/2 x BT/2 =
// (BR/64) x (BT/64) tiles of v_mfma_f32_32x32x16_bf16 with the accumulators in
// AGPRs.  K advances BK columns per stage through a ring of NS LDS stages.
// Global -> LDS copies are buffer loads that write LDS directly (16 bytes per
// lane, 1 KB per instruction); each lane picks the global piece that belongs
// at its LDS slot; with BK = 64 a tile row is one 128-byte global piece, so the
// memory requests are whole 128-byte lines (half as many as with 64-byte rows,
// and the number of requests a CU keeps in flight is what bounds its fill rate).
// Chunks are swizzled within rows so that 16 lanes reading one chunk of 16
// consecutive rows hit 16 distinct bank groups.  Blocks that share a W tile sit on the same XCD
// (block id % 8): W crosses HBM once per XCD and the other token tiles of that
// row tile hit the XCD's L2.
#include "bd_internal.h"

namespace bd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kGemmK = 64;  // the K granularity every tile configuration needs
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
    const int nrec = bytes > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane.
// (A plain device function: the host pass of the kernel template never sees the
// LDS address-space cast.)
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, off, 0, 0, 0);
}

// Byte offset of 16-byte chunk c of row r in a tile of BK-column rows (CPR = BK / 8
// chunks per row): chunk c sits at slot c ^ ((r / (16 / CPR)) % CPR), so any 16
// consecutive rows read at one chunk land in 16 distinct bank groups.
template <int BK>
__device__ __forceinline__ uint32_t swz(int r, int c) {
    constexpr int CPR = BK / 8, RPG = 16 / CPR;
    return (uint32_t)(r * BK * 2 + 16 * (c ^ ((r / RPG) % CPR)));
}

}  // namespace

// Kernel templates live outside the anonymous namespace: the host compiler does
// not emit the launch stubs of internal-linkage kernel templates.
template <int BR, int BT, int BK, int NS>
__global__ void __launch_bounds__(256)
k_gemm(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ y,
       int T, int N, int K, int nrt, int ntt) {
    constexpr int MI = BR / 64, NJ = BT / 64;  // 32 x 32 tiles per wave
    constexpr int CPR = BK / 8, RPI = 64 / CPR;  // chunks per row, rows per copy instruction
    constexpr int kWBytes = BR * BK * 2, kXBytes = BT * BK * 2;
    constexpr int kStageBytes = kWBytes + kXBytes;
    constexpr int kWInst = kWBytes / 1024 / 4, kXInst = kXBytes / 1024 / 4;  // per wave
    static_assert(kWBytes % 4096 == 0 && kXBytes % 4096 == 0, "whole copy instructions per wave");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // block -> (row tile, token tile); the token tiles of one row tile share an XCD
    const int id = blockIdx.x;
    const int q = id >> 3;
    const int tt = q % ntt;
    const int rt = (q / ntt) * 8 + (id & 7);
    if (rt >= nrt) return;  // uniform
    const int r0 = rt * BR, t0 = tt * BT;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wv >> 1, wt = wv & 1;

    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(w, (uint64_t)N * K * 2);
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, (uint64_t)T * K * 2);

    // Loader: copy instruction i of a tile fills LDS bytes [1024 i, +1024): lane l
    // lands on row RPI i + l / CPR, slot l % CPR, i.e. the chunk whose swizzled slot
    // that is.  A row's BK columns are one contiguous global piece.
    uint32_t wsrc[kWInst], xsrc[kXInst];
#pragma unroll
    for (int j = 0; j < kWInst; ++j) {
        const int r = (wv * kWInst + j) * RPI + lane / CPR;
        const int c = (lane % CPR) ^ ((r / (16 / CPR)) % CPR);
        wsrc[j] = r0 + r < N ? (uint32_t)(((int64_t)(r0 + r) * K + 8 * c) * 2) : kOOB;
    }
#pragma unroll
    for (int j = 0; j < kXInst; ++j) {
        const int r = (wv * kXInst + j) * RPI + lane / CPR;
        const int c = (lane % CPR) ^ ((r / (16 / CPR)) % CPR);
        xsrc[j] = t0 + r < T ? (uint32_t)(((int64_t)(t0 + r) * K + 8 * c) * 2) : kOOB;
    }
    const int nk = K / BK;
    auto issue = [&](int s) {  // stage s into ring slot s % NS (zeros past K)
        char* base = smem + (s % NS) * kStageBytes;
        const bool ok = s < nk;
        const uint32_t kb = (uint32_t)s * BK * 2;
#pragma unroll
        for (int j = 0; j < kWInst; ++j)
            copy16_to_lds(wrs, base + (wv * kWInst + j) * 1024,
                          (ok && wsrc[j] != kOOB) ? wsrc[j] + kb : kOOB);
#pragma unroll
        for (int j = 0; j < kXInst; ++j)
            copy16_to_lds(xrs, base + kWBytes + (wv * kXInst + j) * 1024,
                          (ok && xsrc[j] != kOOB) ? xsrc[j] + kb : kOOB);
    };

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s);

    const int m32 = lane & 31, h = lane >> 5;
    for (int s = 0; s < nk; ++s) {
        // this wave's copies of stage s are done (NS - 2 younger stages in flight); the
        // barrier makes every wave's copies visible and frees the slot of stage s - 1
        constexpr int kAhead = (kWInst + kXInst) * (NS - 2);
        __builtin_amdgcn_s_waitcnt(0x0F70 | (kAhead & 0xF) | (((kAhead >> 4) & 3) << 14));
        __builtin_amdgcn_s_barrier();  // no fence: the explicit wait above covers the copies
        issue(s + NS - 1);
        const char* wt_base = smem + (s % NS) * kStageBytes;
        const char* xt_base = wt_base + kWBytes;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {  // 16 columns per step: lane half h takes chunk 2kk + h
            u32x4 A[MI], Bv[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i)
                A[i] = *(const u32x4*)(wt_base + swz<BK>(wr * (BR / 2) + 32 * i + m32, 2 * kk + h));
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                Bv[j] = *(const u32x4*)(xt_base + swz<BK>(wt * (BT / 2) + 32 * j + m32, 2 * kk + h));
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32(A[i], Bv[j], acc[i][j]);
        }
    }

    // D lane layout (32 x 32): column m32, register 4b + e holds row 8b + 4h + e
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int t = t0 + wt * (BT / 2) + 32 * j + m32;
        if (t >= T) continue;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int o = r0 + wr * (BR / 2) + 32 * i + 8 * b + 4 * h;
                float* dst = y + (int64_t)t * N + o;
                const f32x4 v = {acc[i][j][4 * b], acc[i][j][4 * b + 1], acc[i][j][4 * b + 2],
                                 acc[i][j][4 * b + 3]};
                if (o + 3 < N && (N & 3) == 0) {
                    *(f32x4*)dst = v;
                } else {
                    for (int e = 0; e < 4; ++e)
                        if (o + e < N) dst[e] = v[e];
                }
            }
        }
    }
}

namespace {

template <int BR, int BT, int BK, int NS>
hipError_t launch_tile(const void* x, int64_t T, int64_t d_in, const void* wb, int64_t d_out,
                       float* y, hipStream_t s) {
    const int nrt = (int)((d_out + BR - 1) / BR), ntt = (int)((T + BT - 1) / BT);
    const int nrt8 = (nrt + 7) / 8 * 8;
    const unsigned blocks = (unsigned)(nrt8 * ntt);
    constexpr int lds = NS * (BR + BT) * BK * 2;
    k_gemm<BR, BT, BK, NS><<<dim3(blocks), dim3(256), lds, s>>>(
        (const uint16_t*)x, (const uint16_t*)wb, y, (int)T, (int)d_out, (int)d_in, nrt, ntt);
    return hipGetLastError();
}

}  // namespace

// 17..64 tokens on a wide matrix: one 64-token tile per 64 rows copies the tokens once
// per 64 rows (the streaming kernel re-reads them from L2 for every 16 rows), and at
// >= 160 row tiles the grid still covers most of the chip.
bool small_batch_gemm_supported(int64_t T, int64_t d_in, int64_t d_out) {
    return T > 16 && T <= kGemmMinT && d_in % kGemmK == 0 && (d_out + 63) / 64 >= 160 &&
           T * d_in * 2 < ((int64_t)1 << 31) && d_out * d_in * 2 < ((int64_t)1 << 31);
}

hipError_t launch_small_batch_gemm(const void* x, int64_t T, int64_t d_in, const void* wb,
                                   int64_t d_out, float* y, hipStream_t s) {
    return launch_tile<64, 64, 64, 4>(x, T, d_in, wb, d_out, y, s);
}

bool gemm_path_supported(int64_t T, int64_t d_in, int64_t d_out) {
    return T > kGemmMinT && d_in % kGemmK == 0 && T * d_in * 2 < ((int64_t)1 << 31) &&
           d_out * d_in * 2 < ((int64_t)1 << 31) && d_out < ((int64_t)1 << 30);
}

// The largest tile that still yields enough blocks to cover the chip: 128 rows x 256
// tokens (most reuse per copied byte), 128 x 128, 64 x 128, else 64 x 64 (small
// matrices and batches, where idle CUs cost more than the extra copies).
hipError_t launch_gemm(const void* x, int64_t T, int64_t d_in, const void* wb, int64_t d_out,
                       float* y, hipStream_t s) {
    auto blocks = [&](int64_t br, int64_t bt) { return ((d_out + br - 1) / br) * ((T + bt - 1) / bt); };
    if (blocks(128, 256) >= 200) return launch_tile<128, 256, 64, 3>(x, T, d_in, wb, d_out, y, s);
    if (blocks(128, 128) >= 200) return launch_tile<128, 128, 64, 4>(x, T, d_in, wb, d_out, y, s);
    if (blocks(64, 128) >= 200) return launch_tile<64, 128, 64, 4>(x, T, d_in, wb, d_out, y, s);
    return launch_tile<64, 64, 64, 4>(x, T, d_in, wb, d_out, y, s);
}

}  // namespace bd
