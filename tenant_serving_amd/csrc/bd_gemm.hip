// bd_gemm.hip -- the shared base product Y = X W_base^T for batches of many
// tokens (prefill chunks, large decode batches): a tiled bf16 GEMM on the
// gfx950 matrix cores ([P2] "Systems Mechanics" 1: one dense product of the
// whole batch with the shared base weight).
//
// Block tile: BR rows of W x BT tokens (256 x 256 with 8 waves, two per SIMD, in 4 x 2;
// 128 x 256, 128 x 128, 64 x 128 or 64 x 64 with 4 waves in 2 x 2), each wave a block
// of (BR / (NW/2) / 32) x (BT / 64) tiles of v_mfma_f32_32x32x16_bf16.  K advances BK columns per stage through a ring of NS LDS stages.
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

#include <type_traits>

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

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Four int8 codes (one dword, low byte first) as two dwords of bf16 pairs: each code
// sign-extended and converted to fp32, whose upper half is its bf16 value (exact:
// |code| <= 128 needs 8 significant bits).  The sign extension is written with shifts:
// with the signed bit-field-extract builtin this compiler folded the extract into an
// unsigned byte conversion (v_cvt_f32_u32 with a sign-extended byte), which turns
// negative codes into values near 2^32.
__device__ __forceinline__ void widen_i8x4(uint32_t d, uint32_t& lo, uint32_t& hi) {
    const float f0 = (float)((int)(d << 24) >> 24);
    const float f1 = (float)((int)(d << 16) >> 24);
    const float f2 = (float)((int)(d << 8) >> 24);
    const float f3 = (float)((int)d >> 24);
    lo = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    hi = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
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
// Q8: W holds int8 codes with one scale per row (the INT8 base): each lane loads 16
// codes of a row into registers two stages ahead (two register sets, alternating), widens
// them to bf16 and writes the two chunks to their swizzled LDS slots after the products of
// the stage before; the epilogue multiplies each row by its scale.  Each stage's code
// loads go out before its token copies: vector loads complete in order, so waiting for
// the codes leaves the younger token copies in flight and the ring keeps its depth.
template <int BR, int BT, int BK, int NS, int NW, bool Q8>
__global__ void __launch_bounds__(64 * NW)
k_gemm(const uint16_t* __restrict__ x, const GemmMats gm, int T, int K, int ntt, int S, int kps) {
    // NW waves: NW / 2 along the rows, 2 along the tokens
    constexpr int NWR = NW / 2;
    constexpr int MI = BR / NWR / 32, NJ = BT / 64;  // 32 x 32 tiles per wave
    constexpr int CPR = BK / 8, RPI = 64 / CPR;  // chunks per row, rows per copy instruction
    constexpr int kWBytes = BR * BK * 2, kXBytes = BT * BK * 2;
    constexpr int kStageBytes = kWBytes + kXBytes;
    constexpr int kWInst = kWBytes / 1024 / NW, kXInst = kXBytes / 1024 / NW;  // per wave
    static_assert(kWBytes % (1024 * NW) == 0 && kXBytes % (1024 * NW) == 0,
                  "whole copy instructions per wave");
    static_assert(MI >= 1 && BR % (32 * NWR) == 0, "32-row tiles per wave");
    static_assert(!Q8 || (BR * BK) % (1024 * NW) == 0, "INT8 codes: whole loads per wave");
    constexpr int kQInst = Q8 ? BR * BK / (1024 * NW) : 1;  // 16-code loads per lane and stage
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // block -> (K part, row tile, token tile); the token tiles of one row tile share an
    // XCD.  Row tiles run over the matrices of the set back to back.  S > 1: K part sp
    // covers columns [sp kps, (sp + 1) kps) and writes its partial tile to part.
    const int per = (int)(gridDim.x / (unsigned)S);
    const int sp = (int)blockIdx.x / per;
    const int id = (int)blockIdx.x - sp * per;
    const int kbeg = sp * kps;
    const int q = id >> 3;
    const int tt = q % ntt;
    const int rtg = (q / ntt) * 8 + (id & 7);
    if (rtg >= gm.rt_begin[gm.n]) return;  // uniform
    int mi = 0;
#pragma unroll
    for (int j = 1; j < kMaxMats; ++j) mi += (j < gm.n && rtg >= gm.rt_begin[j]) ? 1 : 0;
    const uint16_t* const w = mi == 0 ? gm.w[0] : mi == 1 ? gm.w[1] : mi == 2 ? gm.w[2] : gm.w[3];
    float* const y = S > 1 ? (mi == 0 ? gm.part[0] : mi == 1 ? gm.part[1] : mi == 2 ? gm.part[2] : gm.part[3]) +
                                 (int64_t)sp * T * (mi == 0 ? gm.N[0] : mi == 1 ? gm.N[1] : mi == 2 ? gm.N[2] : gm.N[3])
                           : (mi == 0 ? gm.y[0] : mi == 1 ? gm.y[1] : mi == 2 ? gm.y[2] : gm.y[3]);
    const int N = mi == 0 ? gm.N[0] : mi == 1 ? gm.N[1] : mi == 2 ? gm.N[2] : gm.N[3];
    const float* const wsc = mi == 0 ? gm.s[0] : mi == 1 ? gm.s[1] : mi == 2 ? gm.s[2] : gm.s[3];
    const int rt = rtg - (mi == 0 ? gm.rt_begin[0] : mi == 1 ? gm.rt_begin[1]
                          : mi == 2 ? gm.rt_begin[2] : gm.rt_begin[3]);
    const int r0 = rt * BR, t0 = tt * BT;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wv >> 1, wt = wv & 1;

    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(w, (uint64_t)N * K * (Q8 ? 1 : 2));
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
    // Q8 loader: load j of lane l covers codes [16 c, 16 c + 16) of row r (g = 64 (wv
    // kQInst + j) + l, r = g / (BK / 16), c = g % (BK / 16)), bf16 chunks 2 c and 2 c + 1
    uint32_t qsrc[kQInst], qdst[kQInst];
    u32x4 qreg[2][kQInst];  // stage s's codes in set s % 2
#pragma unroll
    for (int j = 0; j < kQInst; ++j) {
        const int g = (wv * kQInst + j) * 64 + lane;
        const int r = g / (BK / 16), c = g % (BK / 16);
        qsrc[j] = Q8 && r0 + r < N ? (uint32_t)((int64_t)(r0 + r) * K + 16 * c) : kOOB;
        qdst[j] = (uint32_t)(r * 4096 + c);  // (row, code group), unpacked at the store
    }
    const int nk = kps / BK;  // stages of this block's K part
    auto qload = [&](int s, auto pc) {  // stage s's codes into set pc (zeros past K)
        constexpr int P = decltype(pc)::value;
#pragma unroll
        for (int j = 0; j < kQInst; ++j)
            qreg[P][j] = buf_load16(wrs, (s < nk && qsrc[j] != kOOB) ? qsrc[j] + (uint32_t)(kbeg + s * BK) : kOOB);
    };
    auto qstore = [&](int s, auto pc) {  // the codes of stage s (set pc), widened, into ring slot s % NS
        constexpr int P = decltype(pc)::value;
        char* base = smem + (s % NS) * kStageBytes;
#pragma unroll
        for (int j = 0; j < kQInst; ++j) {
            const int r = (int)(qdst[j] >> 12), c = (int)(qdst[j] & 4095u);
            uint32_t v[8];
            widen_i8x4(qreg[P][j].x, v[0], v[1]);
            widen_i8x4(qreg[P][j].y, v[2], v[3]);
            widen_i8x4(qreg[P][j].z, v[4], v[5]);
            widen_i8x4(qreg[P][j].w, v[6], v[7]);
            const u32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
            *(u32x4*)(base + swz<BK>(r, 2 * c)) = a;
            *(u32x4*)(base + swz<BK>(r, 2 * c + 1)) = b;
        }
    };
    auto issue = [&](int s) {  // stage s into ring slot s % NS (zeros past K)
        char* base = smem + (s % NS) * kStageBytes;
        const bool ok = s < nk;
        const uint32_t kb = (uint32_t)(kbeg + s * BK) * 2;
        if (!Q8) {
#pragma unroll
            for (int j = 0; j < kWInst; ++j)
                copy16_to_lds(wrs, base + (wv * kWInst + j) * 1024,
                              (ok && wsrc[j] != kOOB) ? wsrc[j] + kb : kOOB);
        }
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

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // The prologue issues in the loop's order, as if by stages t = -max(NS - 1, 2) .. -1
    // (stage t: stage t + 2's codes, then stage t + NS - 1's copies), so that the wait at the
    // top of every stage counts the same younger loads as in the loop.
#pragma unroll
    for (int t = -(NS - 1 > 2 ? NS - 1 : 2); t < 0; ++t) {
        if constexpr (Q8) {
            if (t + 2 == 0) qload(0, P0());
            if (t + 2 == 1) qload(1, P1());
        }
        if (t + NS - 1 >= 0) issue(t + NS - 1);
    }
    if constexpr (Q8) qstore(0, P0());

    const int m32 = lane & 31, h = lane >> 5;
    // stage s (parity pc: Q8 loads stage s + 2's codes into set pc and stores stage s + 1's
    // from the other set)
    auto stage = [&](int s, auto pc) {
        constexpr int P = decltype(pc)::value;
        // this wave's copies of stage s are done (NS - 2 younger stages in flight, each one
        // stage's token copies (bf16: and W copies; Q8: and the codes of a later stage));
        // the barrier makes every wave's copies visible and frees the slot of stage s - 1
        // (Q8: also this wave's LDS writes of the stage's codes)
        constexpr int kAhead = ((Q8 ? kQInst : kWInst) + kXInst) * (NS - 2);
        __builtin_amdgcn_s_waitcnt((Q8 ? 0x0070 : 0x0F70) | (kAhead & 0xF) |
                                   (((kAhead >> 4) & 3) << 14));
        __builtin_amdgcn_s_barrier();  // no fence: the explicit wait above covers the copies
        if constexpr (Q8) qload(s + 2, pc);  // (set P: stage s's codes were stored before)
        issue(s + NS - 1);
        const char* wt_base = smem + (s % NS) * kStageBytes;
        const char* xt_base = wt_base + kWBytes;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {  // 16 columns per step: lane half h takes chunk 2kk + h
            // the compiler's interleaving of LDS reads with the products (scheduling only)
            __builtin_amdgcn_iglp_opt(0);
            u32x4 A[MI], Bv[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i)
                A[i] = *(const u32x4*)(wt_base + swz<BK>(wr * (BR / NWR) + 32 * i + m32, 2 * kk + h));
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                Bv[j] = *(const u32x4*)(xt_base + swz<BK>(wt * (BT / 2) + 32 * j + m32, 2 * kk + h));
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32(A[i], Bv[j], acc[i][j]);
        }
        if constexpr (Q8) {
            if (s + 1 < nk) qstore(s + 1, std::integral_constant<int, 1 - P>());  // slot of stage s - 1: free
        }
    };
    for (int s = 0; s < nk; s += 2) {
        stage(s, P0());
        if (s + 1 < nk) stage(s + 1, P1());  // (uniform)
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
                const int o = r0 + wr * (BR / NWR) + 32 * i + 8 * b + 4 * h;
                float* dst = y + (int64_t)t * N + o;
                f32x4 v = {acc[i][j][4 * b], acc[i][j][4 * b + 1], acc[i][j][4 * b + 2],
                           acc[i][j][4 * b + 3]};
                if (Q8) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] *= o + e < N ? wsc[o + e] : 0.f;
                }
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

template <int BR, int BT, int BK, int NS, int NW = 4, bool Q8 = false>
hipError_t launch_tile(const void* x, int64_t T, int64_t d_in, const GemmMatArg* mats, int n,
                       hipStream_t s, const float* const* wscales = nullptr, int S = 1,
                       float* const* parts = nullptr) {
    GemmMats gm = {};
    gm.n = n;
    int rt = 0;
    for (int i = 0; i < n; ++i) {
        gm.w[i] = (const uint16_t*)mats[i].w;
        gm.s[i] = wscales ? wscales[i] : nullptr;
        gm.part[i] = parts ? parts[i] : nullptr;
        gm.y[i] = mats[i].y;
        gm.N[i] = (int)mats[i].d_out;
        gm.rt_begin[i] = rt;
        rt += (int)((mats[i].d_out + BR - 1) / BR);
    }
    for (int i = n; i <= kMaxMats; ++i) gm.rt_begin[i] = rt;
    const int ntt = (int)((T + BT - 1) / BT);
    const int nrt8 = (rt + 7) / 8 * 8;
    const unsigned blocks = (unsigned)(nrt8 * ntt * S);
    constexpr int lds = NS * (BR + BT) * BK * 2;
    k_gemm<BR, BT, BK, NS, NW, Q8><<<dim3(blocks), dim3(64 * NW), lds, s>>>(
        (const uint16_t*)x, gm, (int)T, (int)d_in, ntt, S, (int)(d_in / S));
    return hipGetLastError();
}

// y = the sum of the S partial products, in split order (grid.y: the matrix).
__global__ void __launch_bounds__(256)
k_split_reduce(const GemmMats gm, int64_t T, int S) {
    const int mi = (int)blockIdx.y;
    const int64_t n4 = T * (int64_t)gm.N[mi] / 4;  // (N % 4 == 0 on this path)
    const f32x4* part = (const f32x4*)gm.part[mi];
    f32x4* y = (f32x4*)gm.y[mi];
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        f32x4 v = part[i];
        for (int q = 1; q < S; ++q) v += part[(int64_t)q * n4 + i];
        y[i] = v;
    }
}

// K parts for the 256 x 256 tile: S in {2, 4, 8} when the grid would otherwise stay under
// 200 blocks, each part at least 1024 columns (16 stages), the split grid 192..320 blocks.
int choose_split(int64_t T, int64_t d_in, const int64_t* d_outs, int n) {
    if (T <= kGemmMinT) return 1;
    int64_t b = 0;
    for (int i = 0; i < n; ++i) {
        if (d_outs[i] % 4 != 0) return 1;
        b += (d_outs[i] + 255) / 256;
    }
    b *= (T + 255) / 256;
    if (b >= 200) return 1;
    for (int S = 8; S >= 2; S /= 2)
        if (d_in % (64 * S) == 0 && d_in / S >= 1024 && b * S >= 192 && b * S <= 320) return S;
    return 1;
}

// The product's tile and K split (bf16 and INT8 bases alike).  Measured at 512 tokens on one MI355X (one matrix
// per launch, HIP events; split times include the sum of the parts): 6144 x 4096 (q|k|v)
// 42 us on 128 x 128 tiles unsplit against 48 on 256 x 256 in 4 parts; 4096 x 4096 (o)
// 28 us on 64 x 64 tiles (two blocks per CU) against 31 on 64 x 128; 4096 x 14336 (down)
// 76 us on 128 x 256 in 4 parts against 82 on 256 x 256 in 8; 28672 x 4096 (gate|up) 123 us
// on 256 x 256 unsplit, the best; at 256 tokens 4096 x 14336 (the clipped MLP's down) 46 us
// on 128 x 128 in 4 parts against 73 on 64 x 64 (4096 x 4096 in 2 parts of 2048 columns
// does not pay: 32 us against 28).  Order: 256 x 256 when it fills the chip; 128 x 128 when
// its grid is one block per CU (192..256); with a workspace, 128 x 256 in 2..8 parts of at
// least 2048 columns (grid 192..320), 128 x 128 in parts of at least 3072 columns, then
// 256 x 256 in parts (choose_split); otherwise the largest unsplit tile that fills the chip.
enum { kT256x256, kT128x256, kT128x128, kT64x128, kT64x64 };
struct GemmPlan {
    int tile, S;
};
GemmPlan plan_gemm(int64_t T, int64_t d_in, const int64_t* d_outs, int n, bool split_ok) {
    auto blocks = [&](int64_t br, int64_t bt) {
        int64_t r = 0;
        for (int i = 0; i < n; ++i) r += (d_outs[i] + br - 1) / br;
        return r * ((T + bt - 1) / bt);
    };
    bool n4 = true;
    for (int i = 0; i < n; ++i) n4 = n4 && d_outs[i] % 4 == 0;  // (the parts' sum reads f32x4)
    if (blocks(256, 256) >= 200) return {kT256x256, 1};
    const int64_t b128 = blocks(128, 128);
    if (b128 >= 192 && b128 <= 256) return {kT128x128, 1};
    if (split_ok && n4 && T > kGemmMinT) {
        const int64_t b = blocks(128, 256);
        for (int S = 2; S <= 8; S *= 2)
            if (d_in % (64 * S) == 0 && d_in / S >= 2048 && b * S >= 192 && b * S <= 320) return {kT128x256, S};
        for (int S = 2; S <= 8; S *= 2)
            if (d_in % (64 * S) == 0 && d_in / S >= 3072 && b128 * S >= 192 && b128 * S <= 320) return {kT128x128, S};
        const int S = choose_split(T, d_in, d_outs, n);
        if (S > 1) return {kT256x256, S};
    }
    if (blocks(128, 256) >= 200) return {kT128x256, 1};
    if (b128 >= 200) return {kT128x128, 1};
    if (blocks(64, 64) >= 400) return {kT64x64, 1};
    if (blocks(64, 128) >= 200) return {kT64x128, 1};
    return {kT64x64, 1};
}

}  // namespace

size_t gemm_split_bytes(int64_t T, int64_t d_in, const int64_t* d_outs, int n) {
    const int S = plan_gemm(T, d_in, d_outs, n, true).S;  // (the INT8 product's too)
    if (S == 1) return 0;
    size_t b = 0;
    for (int i = 0; i < n; ++i) b += ((size_t)S * T * d_outs[i] * 4 + kAlign - 1) / kAlign * kAlign;
    return b;
}

hipError_t launch_gemm_set_split(const void* x, int64_t T, int64_t d_in, const GemmMatArg* mats,
                                 int n, char* ws, hipStream_t s, const float* const* wscales) {
    if (n < 1 || n > kMaxMats) return hipErrorInvalidValue;
    int64_t d_outs[kMaxMats];
    for (int i = 0; i < n; ++i) d_outs[i] = mats[i].d_out;
    const GemmPlan pl = plan_gemm(T, d_in, d_outs, n, ws != nullptr);
    const int S = pl.S;
    if (S == 1 || !ws) return launch_gemm_set(x, T, d_in, mats, n, s, wscales);
    float* parts[kMaxMats];
    size_t off = 0;
    int64_t nmax = 0;
    for (int i = 0; i < n; ++i) {
        parts[i] = (float*)(ws + off);
        off += ((size_t)S * T * d_outs[i] * 4 + kAlign - 1) / kAlign * kAlign;
        nmax = d_outs[i] > nmax ? d_outs[i] : nmax;
    }
    hipError_t e;
    if (wscales)
        e = pl.tile == kT128x256 ? launch_tile<128, 256, 64, 3, 4, true>(x, T, d_in, mats, n, s, wscales, S, parts)
            : pl.tile == kT128x128 ? launch_tile<128, 128, 64, 4, 4, true>(x, T, d_in, mats, n, s, wscales, S, parts)
                                   : launch_tile<256, 256, 64, 2, 8, true>(x, T, d_in, mats, n, s, wscales, S, parts);
    else
        e = pl.tile == kT128x256 ? launch_tile<128, 256, 64, 3>(x, T, d_in, mats, n, s, nullptr, S, parts)
            : pl.tile == kT128x128 ? launch_tile<128, 128, 64, 4>(x, T, d_in, mats, n, s, nullptr, S, parts)
                                   : launch_tile<256, 256, 64, 2, 8>(x, T, d_in, mats, n, s, nullptr, S, parts);
    if (e != hipSuccess) return e;
    GemmMats gm = {};
    gm.n = n;
    for (int i = 0; i < n; ++i) {
        gm.part[i] = parts[i];
        gm.y[i] = mats[i].y;
        gm.N[i] = (int)d_outs[i];
    }
    const int64_t n4 = T * nmax / 4;
    const unsigned gx = (unsigned)((n4 + 255) / 256 < 2048 ? (n4 + 255) / 256 : 2048);
    hipLaunchKernelGGL(k_split_reduce, dim3(gx, (unsigned)n), dim3(256), 0, s, gm, T, S);
    return hipGetLastError();
}

// 17..64 tokens on a wide matrix: one 64-token tile per 64 rows copies the tokens once
// per 64 rows (the streaming kernel re-reads them from L2 for every 16 rows), and at
// >= 160 row tiles the grid still covers most of the chip.
bool small_batch_gemm_supported(int64_t T, int64_t d_in, int64_t d_out) {
    return T > 16 && T <= kGemmMinT && d_in % kGemmK == 0 && (d_out + 63) / 64 >= 160 &&
           T * d_in * 2 < ((int64_t)1 << 31) && d_out * d_in * 2 < ((int64_t)1 << 31);
}

hipError_t launch_small_batch_gemm(const void* x, int64_t T, int64_t d_in, const void* wb,
                                   int64_t d_out, float* y, hipStream_t s) {
    const GemmMatArg m = {wb, y, d_out};
    return launch_tile<64, 64, 64, 4>(x, T, d_in, &m, 1, s);
}

bool gemm_path_supported(int64_t T, int64_t d_in, int64_t d_out) {
    return T > kGemmMinT && d_in % kGemmK == 0 && T * d_in * 2 < ((int64_t)1 << 31) &&
           d_out * d_in * 2 < ((int64_t)1 << 31) && d_out < ((int64_t)1 << 30);
}

// Without K parts: plan_gemm's unsplit tile (the largest that still covers the chip; small
// matrices and batches take small tiles, where idle CUs cost more than the extra copies).
// INT8 codes (wscales set): the same tiles and LDS rings.
hipError_t launch_gemm_set(const void* x, int64_t T, int64_t d_in, const GemmMatArg* mats, int n,
                           hipStream_t s, const float* const* wscales) {
    if (n < 1 || n > kMaxMats) return hipErrorInvalidValue;
    if (T == 0) return hipSuccess;
    int64_t d_outs[kMaxMats];
    for (int i = 0; i < n; ++i) d_outs[i] = mats[i].d_out;
    const int tile = plan_gemm(T, d_in, d_outs, n, false).tile;
    if (wscales) {
        const float* const* sc = wscales;
        switch (tile) {
            case kT256x256: return launch_tile<256, 256, 64, 2, 8, true>(x, T, d_in, mats, n, s, sc);
            case kT128x256: return launch_tile<128, 256, 64, 3, 4, true>(x, T, d_in, mats, n, s, sc);
            case kT128x128: return launch_tile<128, 128, 64, 4, 4, true>(x, T, d_in, mats, n, s, sc);
            case kT64x128: return launch_tile<64, 128, 64, 4, 4, true>(x, T, d_in, mats, n, s, sc);
            default: return launch_tile<64, 64, 64, 4, 4, true>(x, T, d_in, mats, n, s, sc);
        }
    }
    switch (tile) {
        case kT256x256: return launch_tile<256, 256, 64, 2, 8>(x, T, d_in, mats, n, s);
        case kT128x256: return launch_tile<128, 256, 64, 3>(x, T, d_in, mats, n, s);
        case kT128x128: return launch_tile<128, 128, 64, 4>(x, T, d_in, mats, n, s);
        case kT64x128: return launch_tile<64, 128, 64, 4>(x, T, d_in, mats, n, s);
        default: return launch_tile<64, 64, 64, 4>(x, T, d_in, mats, n, s);
    }
}

hipError_t launch_gemm(const void* x, int64_t T, int64_t d_in, const void* wb, int64_t d_out,
                       float* y, hipStream_t s) {
    const GemmMatArg m = {wb, y, d_out};
    return launch_gemm_set(x, T, d_in, &m, 1, s);
}

bool gemm_q8_supported(int64_t T, int64_t d_in, int64_t d_out) {
    return T >= 1 && d_in % kGemmK == 0 && T * d_in * 2 < ((int64_t)1 << 31) &&
           d_out * d_in < ((int64_t)1 << 31) && d_out < ((int64_t)1 << 30);
}

hipError_t launch_gemm_q8(const void* x, int64_t T, int64_t d_in, const int8_t* wq,
                          const float* wscale, int64_t d_out, float* y, hipStream_t s) {
    const GemmMatArg m = {wq, y, d_out};
    const float* sc[1] = {wscale};
    return launch_gemm_set(x, T, d_in, &m, 1, s, sc);
}

}  // namespace bd
