// bd_delta.hip -- the per-user delta products of a prepared batch of any size:
// Y[t] += scale_u (.) (X[t] S_u^T), u = user of token t ([P2] "Systems Mechanics"
// 1-2: each request adds its own 1-bit delta product; the bits cross HBM packed
// and are expanded on chip).
//
// The batch, sorted by user (k_group), is cut into tiles of 16 consecutive
// positions; a tile may hold tokens of several users and a user's tokens may span
// tiles.  Two kernels:
//   k_tile_encode  per (tile, 512-column unit): the tile's 16 tokens as the fp6
//                  e2m3 B operands of the gfx950 block-scaled MFMA 16x16x128, two
//                  parts per value (hi, lo) under one power-of-two scale per 32
//                  columns (the encoding of the decode path; COL scales are folded
//                  into the values first), and the tile's token and user lists.
//   k_delta6       per (64 output rows, range of tiles): for each tile and unit the
//                  tile's operands come into LDS (double-buffered copies shared by
//                  the block's four waves); every user of the tile then loads its
//                  16 B of sign bits per lane (a register ring keeps the next rows
//                  in flight), expands them to fp4 e2m1 +-1 A operands (two VALU
//                  ops per eight signs) and runs the four products twice (hi, lo).
//                  Other users' tokens of the tile enter with block scale 2^-127,
//                  so one accumulator per wave and tile collects every user's
//                  product in its own token columns.  GROUP: each product covers
//                  one 128-column group (the unit's group c at lane group g's
//                  32 columns), and its result is scaled by the group scale of
//                  each row before it is added.  The epilogue adds the tile's
//                  result into Y (each Y element belongs to exactly one tile).
#include "bd_internal.h"

namespace bd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x6 __attribute__((ext_vector_type(6)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past num_records: the load returns 0

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
// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, off, 0, 0, 0);
}

// D += A(fp4, 16 x 128) * B(fp6 e2m3, 128 x 16) * 2^(scale_b - 127), scale_b = byte SEL of sc.
template <int SEL>
__device__ __forceinline__ f32x4 mfma_f4f6(u32x4 a, i32x6 b, f32x4 c, uint32_t sc) {
    const i32x8 a8 = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const i32x8 b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, 4, 5, -1, -1);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 2, 0, 127, SEL, (int)sc);
}

// s_waitcnt with only the vector-memory count: vmcnt <= n (expcnt, lgkmcnt untouched).
#define BD_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 0xF) | ((((n) >> 4) & 3) << 14))

}  // namespace

// ------------------------------------------------------------ tile encoding
// Block (tile t, unit u), 4 waves: wave q encodes product q.  Lane (m, G) takes
// token m of the tile and the 32 columns of k-block G of product q: columns
// 512u + 128G + 32q, or 512u + 128q + 32G with the GROUP layout (product q = the
// unit's 128-column group q).  Unit (t, u) of `enc` (kEncUnitBytes): 1 KB chunks
// (q, c), c = 0..2, holding lane l's 16 bytes at 16 l: c = 0 hi[0..3], c = 1
// hi[4..5] lo[0..1], c = 2 lo[2..5]; then the codes, lane l at 16 l: byte q of
// dword 0 (hi) and dword 1 (lo).
template <bool GRP, bool COL>
__global__ void __launch_bounds__(256)
k_tile_encode(const uint16_t* __restrict__ x, int64_t T, int64_t d_in,
              const int32_t* __restrict__ perm, const int32_t* __restrict__ suser,
              const uint32_t* __restrict__ meta, const void* __restrict__ scales, int sdtype,
              int64_t per_user, int32_t* __restrict__ tmeta, char* __restrict__ enc) {
    const int t = blockIdx.x, u = blockIdx.y, nunit = gridDim.y;
    const int lane = threadIdx.x & 63;
    const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = lane & 15, G = lane >> 4;
    const int nv = (int)meta[2];
    const int p = 16 * t + m;
    const int tok = p < nv ? perm[p] : -1;
    const int usr = p < nv ? suser[p] : -1;
    if (u == 0 && q == 0) {
        // tile meta: tokens, their users, the distinct users in order, their number
        int32_t* tm = tmeta + (size_t)t * kTileMetaInts;
        if (lane < 16) {
            tm[lane] = tok;
            tm[16 + lane] = usr;
        }
        const int prev = __shfl(usr, (lane & 48) | ((m + 15) & 15));
        const bool start = lane < 16 && usr >= 0 && (m == 0 || prev != usr);
        const uint64_t smask = __ballot(start);
        const int j = __popcll(smask & ((1ull << lane) - 1ull));
        if (start) tm[32 + j] = usr;
        if (lane == 0) tm[48] = __popcll(smask);
    }
    if (16 * t >= nv) return;  // uniform: a tile past the valid tokens is skipped later

    const int64_t c0 = GRP ? 512 * (int64_t)u + 128 * q + 32 * G : 512 * (int64_t)u + 128 * G + 32 * q;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint64_t)T * (uint64_t)d_in * 2);
    uint32_t R[16];  // R[p]: columns c0 + 2p (low half) and c0 + 2p + 1 (high half)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t col = c0 + 8 * i;
        const bool ok = tok >= 0 && col < d_in;
        const u32x4 v = buf_load16(xr, ok ? (uint32_t)(((int64_t)tok * d_in + col) * 2) : kOOB);
        R[4 * i] = v.x;
        R[4 * i + 1] = v.y;
        R[4 * i + 2] = v.z;
        R[4 * i + 3] = v.w;
    }
    if (COL) {
        // x * (column scale of the token's user), rounded to bf16; zero for no user
        const size_t sb = sdtype == BD_F16 ? 2 : 4;
        const __amdgpu_buffer_rsrc_t sr =
            make_rsrc((const char*)scales + (usr >= 0 ? (size_t)usr * per_user * sb : 0),
                      usr >= 0 ? (uint64_t)per_user * sb : 0);
        float sc[32];
        if (sdtype == BD_F16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 h = buf_load16(sr, (uint32_t)((c0 + 8 * i) * 2));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sc[8 * i + 2 * e] = f16_to_f32((uint16_t)h[e]);
                    sc[8 * i + 2 * e + 1] = f16_to_f32((uint16_t)(h[e] >> 16));
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x4 f = buf_load16(sr, (uint32_t)((c0 + 4 * i) * 4));
#pragma unroll
                for (int e = 0; e < 4; ++e) sc[4 * i + e] = __uint_as_float(f[e]);
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i)
            R[i] = (uint32_t)f32_to_bf16(bf16_lo(R[i]) * sc[2 * i]) |
                   ((uint32_t)f32_to_bf16(bf16_hi(R[i]) * sc[2 * i + 1]) << 16);
    }
    uint32_t kb_lo, kb_hi;  // the bf16 pairs (1, 0) and (0, 1), in registers
    asm volatile("v_mov_b32 %0, 0x3f80" : "=v"(kb_lo));
    asm volatile("v_mov_b32 %0, 0x3f800000" : "=v"(kb_hi));
    i32x6 h, l;
    uint32_t ch, cl;
    encode_fp6_block(R, kb_lo, kb_hi, h, l, ch, cl);
    char* base = enc + ((size_t)t * nunit + u) * kEncUnitBytes;
    *(u32x4*)(base + (3 * q + 0) * 1024 + 16 * lane) =
        u32x4{(uint32_t)h[0], (uint32_t)h[1], (uint32_t)h[2], (uint32_t)h[3]};
    *(u32x4*)(base + (3 * q + 1) * 1024 + 16 * lane) =
        u32x4{(uint32_t)h[4], (uint32_t)h[5], (uint32_t)l[0], (uint32_t)l[1]};
    *(u32x4*)(base + (3 * q + 2) * 1024 + 16 * lane) =
        u32x4{(uint32_t)l[2], (uint32_t)l[3], (uint32_t)l[4], (uint32_t)l[5]};
    base[12 * 1024 + 16 * lane + q] = (char)ch;
    base[12 * 1024 + 16 * lane + 4 + q] = (char)cl;
}

// ------------------------------------------------------------ delta products
// Block (64 output rows, tiles [tpb y, tpb y + tpb)), 4 waves of 16 rows.  Per
// tile: for each unit u the block copies the tile's operands into LDS buffer u & 1
// (chunk i by wave i % 4) while the previous unit runs; a barrier per unit makes
// the copy visible and frees the other buffer.  The users of the tile form a ring
// sequence k = u * nusR + j (j < nusR, padded to a multiple of RB with zero
// loads), each slot holding L loads (the sign word(s), and for GROUP the row's
// group scales), issued RB slots ahead.  nusR >= RB keeps the copies of unit u + 1
// older than the last RB slots, so the wait vmcnt <= RB * L before each unit's
// barrier covers them.
template <int MODE, bool SF16>
__global__ void __launch_bounds__(256)
k_delta6(const uint64_t* __restrict__ signs, const void* __restrict__ scales, int64_t per_user,
         int bpg, const int32_t* __restrict__ tmeta, const char* __restrict__ enc,
         const uint32_t* __restrict__ meta, float* __restrict__ y, int64_t d_in, int64_t d_out,
         int nunit, int tpb) {
    constexpr bool GRP = MODE == BD_SCALE_GROUP;
    constexpr int RB = GRP ? 2 : 4;  // ring slots
    constexpr int L = GRP ? 8 : 1;   // loads per slot
    constexpr uint32_t SB = SF16 ? 2 : 4;  // bytes per scale
    __shared__ __attribute__((aligned(16))) char sbuf[2 * kEncUnitBytes];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = lane & 15, G = lane >> 4;
    const int64_t r0 = (int64_t)blockIdx.x * 64 + 16 * wv;
    const int64_t rowA = r0 + m < d_out ? r0 + m : d_out - 1;  // A operand row of this lane
    const int nv = (int)meta[2];
    const int ntv = (nv + 15) / 16;
    const int t0 = (int)blockIdx.y * tpb;
    const int t1 = t0 + tpb < ntv ? t0 + tpb : ntv;
    if (t0 >= t1) return;  // uniform over the block

    const int64_t bank_row = d_in / 8;
    const uint64_t user_bytes = (uint64_t)d_out * (uint64_t)bank_row;
    const int nrec_bits = user_bytes > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)user_bytes;
    const uint64_t sc_bytes = (uint64_t)per_user * SB;
    const int nrec_sc = sc_bytes > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)sc_bytes;
    const uint32_t brow = (uint32_t)(rowA * bank_row);
    const int64_t gpr = GRP ? d_in / (128 * (int64_t)bpg) : 1;  // groups per row
    // GROUP: this lane's scale rows 4G + e (clamped), as byte offsets of group 0
    uint32_t srow[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t ro = r0 + 4 * G + e < d_out ? r0 + 4 * G + e : d_out - 1;
        srow[e] = (uint32_t)(ro * gpr * SB);
    }
    const __amdgpu_buffer_rsrc_t er =
        make_rsrc(enc, (uint64_t)(t1 > 0 ? t1 : 1) * (uint64_t)nunit * kEncUnitBytes);
    uint32_t kmask, kone;  // operand constants in registers (gfx9 VOP3 takes no literal)
    asm volatile("v_mov_b32 %0, 0x88888888" : "=v"(kmask));
    asm volatile("s_mov_b32 %0, 0x22222222" : "=s"(kone));
    auto expand = [&](uint32_t wq) {
        u32x4 a;
        a.x = ((wq << 3) & kmask) | kone;
        a.y = ((wq << 2) & kmask) | kone;
        a.z = ((wq << 1) & kmask) | kone;
        a.w = (wq & kmask) | kone;
        return a;
    };
    // copies of the tile's operands for unit u into LDS buffer b (chunk i by wave i % 4)
    auto issue_enc = [&](int t, int u, int b) {
        const uint32_t src = (uint32_t)(((int64_t)t * nunit + u) * kEncUnitBytes) + 16 * lane;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = wv + 4 * i;
            if (c < kEncUnitBytes / 1024)  // uniform
                lds_copy16(er, sbuf + b * kEncUnitBytes + c * 1024, src + (uint32_t)c * 1024);
        }
    };
    struct Slot {
        uint32_t w[4];  // sign words (GROUP: one per group of the unit)
        u32x4 s[4];     // GROUP: the group scales of rows 4G + e, 4 (fp32) or 8 (fp16) from g0
    };

    for (int t = t0; t < t1; ++t) {
        const int32_t* tm = tmeta + (size_t)t * kTileMetaInts;
        const int nus = tm[48];  // >= 1 for a tile of valid tokens
        const int nusR = (nus + RB - 1) / RB * RB;
        const int tok = tm[m];            // token of this lane's column (or -1)
        const int tok_user = tm[16 + m];  // its user (or -1)
        const int tusers = tm[32 + (lane & 15)];  // lane j < nus: the tile's j-th user
        // lane j: base addresses of user j's bank and scales (read back with readlane)
        const uint64_t ub = (uint64_t)(const char*)signs +
                            (uint64_t)(uint32_t)(lane < nus ? tusers : 0) * user_bytes;
        const uint64_t sbp = (uint64_t)(const char*)scales +
                             (uint64_t)(uint32_t)(lane < nus ? tusers : 0) * sc_bytes;
        const uint32_t ub_lo = (uint32_t)ub, ub_hi = (uint32_t)(ub >> 32);
        const uint32_t sb_lo = (uint32_t)sbp, sb_hi = (uint32_t)(sbp >> 32);
        // slot sequence: unit lu, user lj (padded to nusR with zero loads), then zeros
        int lu = 0, lj = 0;
        uint32_t g0b = 0;  // GROUP: byte offset of the first group of unit lu
        auto load_slot = [&]() {
            Slot sl;
            const bool ok = lu < nunit && lj < nus;  // uniform
            const int jj = ok ? lj : 0;
            // (readlane returns int: widen through uint32_t, no sign extension)
            const uint64_t bb =
                ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(ub_hi, jj) << 32) |
                (uint64_t)(uint32_t)__builtin_amdgcn_readlane(ub_lo, jj);
            const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
                (void*)bb, (short)0, nrec_bits, 0x00020000);
            if (GRP) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    sl.w[c] = buf_load4(br, ok ? brow + (uint32_t)(64 * lu + 16 * c + 4 * G) : kOOB);
                const uint64_t sp =
                    ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(sb_hi, jj) << 32) |
                    (uint64_t)(uint32_t)__builtin_amdgcn_readlane(sb_lo, jj);
                const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)sp, (short)0, nrec_sc, 0x00020000);
#pragma unroll
                for (int e = 0; e < 4; ++e) sl.s[e] = buf_load16(sr, ok ? srow[e] + g0b : kOOB);
            } else {
                const u32x4 v = buf_load16(br, ok ? brow + (uint32_t)(64 * lu + 16 * G) : kOOB);
                sl.w[0] = v.x;
                sl.w[1] = v.y;
                sl.w[2] = v.z;
                sl.w[3] = v.w;
            }
            if (++lj == nusR) {
                lj = 0;
                ++lu;
                if (GRP) g0b = (uint32_t)((4 * (int64_t)lu) / bpg) * SB;
            }
            return sl;
        };
        // the previous tile's readers of both buffers are done before new copies land
        __builtin_amdgcn_s_barrier();
        issue_enc(t, 0, 0);
        Slot ring[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            ring[r] = load_slot();
            __builtin_amdgcn_sched_barrier(0);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
        int u = 0;
        do {
            BD_WAIT_VMCNT(RB * L);  // this wave's copies of unit u have landed
            __builtin_amdgcn_s_barrier();  // and every wave's; buffer (u + 1) & 1 is free
            if (u + 1 < nunit) issue_enc(t, u + 1, (u + 1) & 1);
            const char* sb = sbuf + (u & 1) * kEncUnitBytes;
            i32x6 hi[4], lo[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 c0 = *(const u32x4*)(sb + (3 * q + 0) * 1024 + 16 * lane);
                const u32x4 c1 = *(const u32x4*)(sb + (3 * q + 1) * 1024 + 16 * lane);
                const u32x4 c2 = *(const u32x4*)(sb + (3 * q + 2) * 1024 + 16 * lane);
                hi[q] = i32x6{(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w, (int)c1.x, (int)c1.y};
                lo[q] = i32x6{(int)c1.z, (int)c1.w, (int)c2.x, (int)c2.y, (int)c2.z, (int)c2.w};
            }
            const u32x4 cd = *(const u32x4*)(sb + 12 * 1024 + 16 * lane);
            // GROUP: the slot element of product c's group (relative to the unit's first)
            int gi[4];
            if (GRP) {
                const int64_t g0 = (4 * (int64_t)u) / bpg;
#pragma unroll
                for (int c = 0; c < 4; ++c) gi[c] = (int)((4 * (int64_t)u + c) / bpg - g0);
            }
            int j0 = 0;
            do {
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const int j = j0 + r;
                    const Slot sl = ring[r];
                    ring[r] = load_slot();
                    if (j < nus) {  // uniform
                        const int usr = __builtin_amdgcn_readlane(tusers, j);
                        const bool mine = tok_user == usr;
                        const uint32_t sh = mine ? cd.x : 0u, sl_ = mine ? cd.y : 0u;
                        if (GRP) {
#define BD_G(C)                                                                      \
    {                                                                                \
        const u32x4 a = expand(sl.w[C]);                                             \
        f32x4 tmp = {0.f, 0.f, 0.f, 0.f};                                            \
        tmp = mfma_f4f6<C>(a, hi[C], tmp, sh);                                       \
        tmp = mfma_f4f6<C>(a, lo[C], tmp, sl_);                                      \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) {                              \
            float sc;                                                                \
            if (SF16) {                                                              \
                const uint32_t raw = sl.s[e][gi[C] >> 1];                            \
                sc = f16_to_f32((uint16_t)(gi[C] & 1 ? raw >> 16 : raw));            \
            } else {                                                                 \
                sc = __uint_as_float(sl.s[e][gi[C]]);                                \
            }                                                                        \
            acc[e] -= sc * tmp[e];                                                   \
        }                                                                            \
    }
                            BD_G(0) BD_G(1) BD_G(2) BD_G(3)
#undef BD_G
                        } else {
                            const u32x4 a0 = expand(sl.w[0]), a1 = expand(sl.w[1]);
                            const u32x4 a2 = expand(sl.w[2]), a3 = expand(sl.w[3]);
                            acc = mfma_f4f6<0>(a0, hi[0], acc, sh);
                            acc2 = mfma_f4f6<0>(a0, lo[0], acc2, sl_);
                            acc = mfma_f4f6<1>(a1, hi[1], acc, sh);
                            acc2 = mfma_f4f6<1>(a1, lo[1], acc2, sl_);
                            acc = mfma_f4f6<2>(a2, hi[2], acc, sh);
                            acc2 = mfma_f4f6<2>(a2, lo[2], acc2, sl_);
                            acc = mfma_f4f6<3>(a3, hi[3], acc, sh);
                            acc2 = mfma_f4f6<3>(a3, lo[3], acc2, sl_);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                j0 += RB;
            } while (j0 < nusR);
            ++u;
        } while (u < nunit);
        // the ring's loads past the tile (zeros) land before the next tile's barrier
        BD_WAIT_VMCNT(0);

        // epilogue: Y[tok][rows] += f * sum; rows 4G + e of this wave's 16
        if (tok >= 0 && r0 < d_out) {
            const f32x4 v = acc + acc2;
            const size_t ubs = (size_t)tok_user * per_user;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t o = r0 + 4 * G + e;
                if (o >= d_out) continue;
                float f;
                if (MODE == BD_SCALE_MATRIX || MODE == BD_SCALE_ROW) {
                    const size_t i = ubs + (MODE == BD_SCALE_ROW ? (size_t)o : 0);
                    f = SF16 ? -f16_to_f32(((const uint16_t*)scales)[i]) : -((const float*)scales)[i];
                } else if (MODE == BD_SCALE_COL) {
                    f = -1.f;  // the scales are inside the encoded tokens
                } else {
                    f = 1.f;  // the group scales (negated) are applied per product
                }
                y[(int64_t)tok * d_out + o] += f * v[e];
            }
        }
    }
}

// ---------------------------------------------------------------- host side
hipError_t launch_delta6(const BatchPlan& bp, const DeltaPlan& dp, char* batch, const void* x,
                         const uint64_t* signs, const void* scales, float* y, hipStream_t s) {
    const uint32_t* meta = (const uint32_t*)(batch + bp.off_meta);
    const int32_t* perm = (const int32_t*)(batch + bp.off_perm);
    const int32_t* suser = (const int32_t*)(batch + bp.off_user);
    int32_t* tmeta = (int32_t*)(batch + bp.off_tmeta);
    char* enc = batch + bp.off_enc;
    const int ntiles = (int)bp.ntiles, nunit = (int)bp.nunit;
    const bool grp = dp.mode == BD_SCALE_GROUP, col = dp.mode == BD_SCALE_COL;
    const dim3 ge((unsigned)ntiles, (unsigned)nunit);
#define BD_ENC(G, C)                                                                           \
    hipLaunchKernelGGL((k_tile_encode<G, C>), ge, dim3(256), 0, s, (const uint16_t*)x, bp.T,   \
                       bp.d_in, perm, suser, meta, scales, dp.sdtype, dp.per_user, tmeta, enc)
    if (grp) BD_ENC(true, false);
    else if (col) BD_ENC(false, true);
    else BD_ENC(false, false);
#undef BD_ENC
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // enough blocks for four per CU: tiles per block from the row tiles and the tiles
    const int64_t rtiles = (dp.d_out + 63) / 64;
    int64_t tpb = rtiles * ntiles / 1024;
    tpb = tpb < 1 ? 1 : (tpb > ntiles ? ntiles : tpb);
    const dim3 gd((unsigned)rtiles, (unsigned)((ntiles + tpb - 1) / tpb));
    const int bpg = grp ? dp.group / 128 : 1;
#define BD_D6(MODE, F16)                                                                         \
    hipLaunchKernelGGL((k_delta6<MODE, F16>), gd, dim3(256), 0, s, signs, scales, dp.per_user,  \
                       bpg, (const int32_t*)tmeta, (const char*)enc, meta, y, bp.d_in, dp.d_out, \
                       nunit, (int)tpb)
    const bool f16 = dp.sdtype == BD_F16;
    switch (dp.mode) {
        case BD_SCALE_MATRIX:
            if (f16) BD_D6(BD_SCALE_MATRIX, true); else BD_D6(BD_SCALE_MATRIX, false);
            break;
        case BD_SCALE_GROUP:
            if (f16) BD_D6(BD_SCALE_GROUP, true); else BD_D6(BD_SCALE_GROUP, false);
            break;
        case BD_SCALE_ROW:
            if (f16) BD_D6(BD_SCALE_ROW, true); else BD_D6(BD_SCALE_ROW, false);
            break;
        default: BD_D6(BD_SCALE_COL, false); break;
    }
#undef BD_D6
    return hipGetLastError();
}

}  // namespace bd
