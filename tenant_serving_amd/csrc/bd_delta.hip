// bd_delta.hip -- the per-user delta products of a prepared batch of any size:
// Y[t] += scale_u (.) (X[t] S_u^T), u = user of token t ([P2] "Systems Mechanics"
// 1-2: each request adds its own 1-bit delta product; the bits cross HBM packed
// and are expanded on chip).
//
// The batch, sorted by user (k_group), is cut into tiles of at most 16 consecutive
// positions (k_tile_plan): users of at most 16 tokens are packed whole, so their
// sign rows are read once per tile range; a tile may hold several users.  Kernels:
//   k_tile_plan    one wave: greedy packing of the work items into tiles.
//   k_tile_encode  per (tile, 512-column unit): the tile's 16 tokens as the fp6
//                  e2m3 A operands of the gfx950 block-scaled MFMA 16x16x128, two
//                  parts per value (hi, lo) under one power-of-two scale per 32
//                  columns (the encoding of the decode path; COL scales are folded
//                  into the values first), and the tile's token and user lists.
//   k_delta6       per (64 output rows, range of tiles): for each tile and unit the
//                  tile's operands come into LDS (three buffers, copied two steps
//                  ahead, shared by the block's four waves); every user of the tile
//                  then loads its sign bits (16 B per lane) and scales, kept eight
//                  slots ahead in a register ring that runs across the block's
//                  tiles, expands the bits to fp4 e2m1 +-1 B operands (two VALU ops
//                  per eight signs) and runs the four products twice (hi, lo).
//                  Other users' tokens of the tile enter with block scale 2^-127,
//                  so one accumulator per wave and tile collects every user's
//                  product in its own token rows.  MATRIX / ROW: each user's sum is
//                  scaled when it is added; GROUP: each product covers one
//                  128-column group and is scaled by the row's group scale.  The
//                  tile's result is added into Y with one no-return atomic add per
//                  element (each Y element belongs to exactly one tile).
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

// D += A(fp6 e2m3, 16 x 128) * 2^(scale_a - 127) * B(fp4, 128 x 16), scale_a = byte SEL of sc.
template <int SEL>
__device__ __forceinline__ f32x4 mfma_f6f4(i32x6 a, u32x4 b, f32x4 c, uint32_t sc) {
    const i32x8 a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, 4, 5, -1, -1);
    const i32x8 b8 = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 2, 4, SEL, (int)sc, 0, 127);
}

// s_waitcnt with only the vector-memory count: vmcnt <= n (expcnt, lgkmcnt untouched).
#define BD_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 0xF) | ((((n) >> 4) & 3) << 14))

}  // namespace

// ------------------------------------------------------------ tile packing
// The work items of k_group (runs of <= 32 positions of one user, in position
// order) are packed into tiles of <= 16 positions: an item of c <= 16 positions
// joins the open tile if it fits and otherwise starts a new one (so a user of at
// most 16 tokens is never split); an item of 17..32 starts a tile of 16 and opens
// one with the rest.  Every tile but the last, together with the next, holds more
// than 16 positions: at most 2 ceil(T / 16) + 1 tiles.  One wave: the open tile's
// length is a short serial recurrence over the items (scalar, 64 per round); the
// tile starts are then written by the items' lanes.  tiles[t] = first position of
// tile t, tiles[ntiles] = number of valid positions, meta[3] = ntiles.
__global__ void __launch_bounds__(64)
k_tile_plan(const int4* __restrict__ items, uint32_t* __restrict__ meta, int32_t* __restrict__ tiles,
            int maxt) {
    const int lane = threadIdx.x;
    const int nit = (int)meta[1];
    int cl = 0, nt = 0;  // open tile length, tiles started (uniform)
    for (int b = 0; b < nit; b += 64) {
        const int4 it = b + lane < nit ? items[b + lane] : make_int4(0, 0, 0, 0);
        const int m = nit - b < 64 ? nit - b : 64;
        uint64_t smask = 0;  // item k starts a tile
        for (int k = 0; k < m; ++k) {
            const int c = __builtin_amdgcn_readlane(it.z, k);
            const int c0 = c > 16 ? 16 : c;
            const bool st = cl == 0 || cl + c0 > 16;
            smask |= (uint64_t)st << k;
            cl = c > 16 ? c - 16 : (st ? c : cl + c);
        }
        const bool st = (smask >> lane) & 1ull;
        const bool big = lane < m && it.z > 16;
        const uint64_t bmask = __ballot(big);
        const uint64_t below = (1ull << lane) - 1ull;
        const int idx = nt + __popcll(smask & below) + __popcll(bmask & below);
        if (lane < m) {
            if (st && idx < maxt) tiles[idx] = it.y;
            if (big && idx + (int)st < maxt) tiles[idx + (int)st] = it.y + 16;
        }
        nt += __popcll(smask) + __popcll(bmask);
    }
    nt = nt < maxt ? nt : maxt;
    if (lane == 0) {
        tiles[nt] = (int)meta[2];
        meta[3] = (uint32_t)nt;
    }
}

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
              const uint32_t* __restrict__ meta, const int32_t* __restrict__ tiles,
              const void* __restrict__ scales, int sdtype, int64_t per_user,
              int32_t* __restrict__ tmeta, char* __restrict__ enc) {
    const int t = blockIdx.x, u = blockIdx.y, nunit = gridDim.y;
    const int lane = threadIdx.x & 63;
    const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = lane & 15, G = lane >> 4;
    const int ntv = (int)meta[3];
    if (t >= ntv) return;  // uniform: no such tile in this batch
    const int ts = tiles[t], tl = tiles[t + 1] - ts;  // start, length
    const int p = ts + m;
    const int tok = m < tl ? perm[p] : -1;
    const int usr = m < tl ? suser[p] : -1;
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
        // (per-lane user: plain global loads, columns past d_in take scale 0)
        const size_t sb = sdtype == BD_F16 ? 2 : 4;
        const char* sp = (const char*)scales + (usr >= 0 ? (size_t)usr * per_user * sb : 0);
        float sc[32];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t col = c0 + 8 * i;
            const bool ok = usr >= 0 && col < d_in;
            if (sdtype == BD_F16) {
                const u32x4 h = ok ? *(const u32x4*)(sp + col * 2) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sc[8 * i + 2 * e] = f16_to_f32((uint16_t)h[e]);
                    sc[8 * i + 2 * e + 1] = f16_to_f32((uint16_t)(h[e] >> 16));
                }
            } else {
                const u32x4 f0 = ok ? *(const u32x4*)(sp + col * 4) : u32x4{0u, 0u, 0u, 0u};
                const u32x4 f1 = ok ? *(const u32x4*)(sp + col * 4 + 16) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sc[8 * i + e] = __uint_as_float(f0[e]);
                    sc[8 * i + 4 + e] = __uint_as_float(f1[e]);
                }
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
// Block (128 RT output rows, one tile), 8 waves of RT row tiles of 16 rows.  The
// work is a sequence of slots: step by step (two 512-column units, 2s and 2s + 1),
// user by user of the tile, two slots per user: its sign rows' 64 bytes of unit 2s
// and then of unit 2s + 1, so the two halves of every 128-byte line are read by
// consecutive loads of a wave (a row's next bytes come RT loads later).  Each wave
// keeps the loads of its next kRing slots in flight in a ring of registers: a slot's
// sign words are expanded first and only then reloaded, in place, with the slot
// kRing ahead (its scales likewise after their last use), so no register copy on a
// loop edge waits for a load in flight.  A step's encoded tokens (26 KB) come into
// LDS buffer s % 3, copied two steps ahead and shared by the 8 waves; the opening of
// step s waits until no more loads are in flight than were issued after that copy.
// Each slot reads its unit's operands from LDS (13 KB per wave and slot, read while
// the sign words are expanded).  Steps hold an even number of slots and kRing is
// even, so the unit of the slot at ring position r is r & 1.
// MFMA: A = the tile's 16 tokens (fp6 hi and lo; tokens of other users take block
// code 0, i.e. scale 2^-127), B = 16 sign rows (fp4 +-1); lane (j, g) of D holds
// tokens 4 g .. 4 g + 3 of output row j of the row tile.
constexpr int kNBuf = 3;                       // LDS buffers of step operands
constexpr int kStepBytes = 2 * kEncUnitBytes;  // two units
constexpr int kWaves = 4;  // (two blocks per CU: one block's start overlaps the other's work)

template <int MODE, bool SF16, int RT>
__global__ void __launch_bounds__(64 * kWaves)
k_delta6(const uint64_t* __restrict__ signs, const void* __restrict__ scales, int64_t per_user,
         int bsh, const int32_t* __restrict__ tmeta, const char* __restrict__ enc,
         const uint32_t* __restrict__ meta, float* __restrict__ y, int64_t d_in, int64_t d_out,
         int nunit) {
    // bsh: log2 of the group size / 128 (GROUP sizes are powers of two >= 128);
    // nunit: even (units past d_in are encoded as zeros)
    constexpr bool GRP = MODE == BD_SCALE_GROUP;
    constexpr bool COL = MODE == BD_SCALE_COL;
    constexpr int kRing = RT == 1 ? 8 : (GRP ? 4 : 6);              // slots in flight per wave
    // loads: RT sign loads per slot; GROUP one scale-window load per user and step (in
    // its second slot).  L: the fewest loads of a slot (the counted waits use it)
    constexpr int L = RT;
    constexpr int LMAX = RT + (GRP ? 1 : 0);
    constexpr uint32_t SB = SF16 ? 2 : 4;                            // bytes per scale
    static_assert((kRing - 1) * LMAX <= 63, "vmcnt range");
    static_assert(kRing % 2 == 0, "the unit of a ring position is its parity");
    __shared__ __attribute__((aligned(16))) char sbuf[kNBuf * kStepBytes];
    __shared__ int32_t smeta[kTileMetaInts];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, G = lane >> 4;
    const int64_t rw0 = (int64_t)blockIdx.x * (16 * kWaves * RT) + 16 * RT * wv;  // the wave's first row
    const int tile = blockIdx.y;
    if (tile >= (int)meta[3]) return;  // uniform: no such tile in this batch
    // (wave 0: a uniform branch, so the values around it stay scalar)
    if (wv == 0) smeta[lane] = tmeta[(size_t)tile * kTileMetaInts + lane];
    __syncthreads();
    const int nus = __builtin_amdgcn_readfirstlane(smeta[48]);  // >= 1
    const int S = nunit / 2;                                    // steps
    const int total = (2 * S * nus + kRing - 1) / kRing * kRing;  // slots, padded past the end

    const uint32_t bank_row = (uint32_t)(d_in / 8);
    const uint64_t user_bytes = (uint64_t)d_out * bank_row;
    const int nrec_bits = user_bytes > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)user_bytes;
    const uint64_t sc_bytes = (uint64_t)per_user * SB;
    const int nrec_sc = sc_bytes > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)sc_bytes;
    const uint32_t gpr = GRP ? (uint32_t)((d_in / 128) >> bsh) : 1u;  // groups per row
    uint32_t brow[RT], srow[RT];  // byte offsets of this lane's sign row and scale(s), per row tile
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int64_t r = rw0 + 16 * t + n;
        const uint32_t rowB = (uint32_t)(r < d_out ? r : d_out - 1);  // output row of B column n
        brow[t] = rowB * bank_row;
        srow[t] = GRP ? rowB * gpr * SB : (MODE == BD_SCALE_ROW ? rowB * SB : 0u);
    }
    const __amdgpu_buffer_rsrc_t er =
        make_rsrc(enc + (size_t)tile * nunit * kEncUnitBytes, (uint64_t)nunit * kEncUnitBytes);
    uint32_t kmask, kone;  // operand constants in registers (gfx9 VOP3 takes no literal)
    asm volatile("v_mov_b32 %0, 0x88888888" : "=v"(kmask));
    asm volatile("s_mov_b32 %0, 0x22222222" : "=s"(kone));
    auto expand = [&](uint32_t wq) __attribute__((always_inline)) {
        u32x4 a;
        a.x = ((wq << 3) & kmask) | kone;
        a.y = ((wq << 2) & kmask) | kone;
        a.z = ((wq << 1) & kmask) | kone;
        a.w = (wq & kmask) | kone;
        return a;
    };
    // the operands of step st into LDS buffer b (1 KB chunk i by wave i % 8)
    auto issue_enc = [&](int st, int b) __attribute__((always_inline)) {
        const uint32_t src = (uint32_t)st * kStepBytes + 16 * lane;
#pragma unroll
        for (int i = 0; i < (kStepBytes / 1024 + kWaves - 1) / kWaves; ++i) {
            const int c = wv + kWaves * i;
            if (c < kStepBytes / 1024)  // uniform
                lds_copy16(er, sbuf + b * kStepBytes + c * 1024, src + (uint32_t)c * 1024);
        }
    };
    // GROUP: per unit and row tile, each lane loads a 16-byte window of its row's
    // scales, starting at the unit's first group and moved back (never out of the
    // user's scales) so that it holds the groups of all four products
    const uint32_t swmax = sc_bytes >= 16 ? (uint32_t)sc_bytes - 16u : 0u;
    auto swin = [&](int u, int t) __attribute__((always_inline)) {
        uint32_t g0 = (4u * (uint32_t)u) >> bsh;
        g0 = g0 < gpr ? g0 : gpr - 1u;
        const uint32_t o = srow[t] + g0 * SB;
        return o < swmax ? o : swmax;
    };
    // lane j < nus: base addresses of user j's bank and scales (read back with readlane)
    uint32_t ub_lo, ub_hi, sb_lo, sb_hi;
    {
        const uint64_t usr = n < nus ? (uint64_t)(uint32_t)smeta[32 + n] : 0ull;
        const uint64_t ub = (uint64_t)(const char*)signs + usr * user_bytes;
        const uint64_t sbp = (uint64_t)(const char*)scales + usr * sc_bytes;
        ub_lo = (uint32_t)ub;
        ub_hi = (uint32_t)(ub >> 32);
        sb_lo = (uint32_t)sbp;
        sb_hi = (uint32_t)(sbp >> 32);
    }
    const int c_tuser = smeta[16 + n];  // lane n: user of token n (or -1)
    const int c_users = smeta[32 + n];  // lane j < nus: user j
    // (readlane returns int: widen through uint32_t, no sign extension)
    auto lbase = [&](uint32_t lo, uint32_t hi, int jj) __attribute__((always_inline)) {
        return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hi, jj) << 32) |
               (uint64_t)(uint32_t)__builtin_amdgcn_readlane(lo, jj);
    };

    // ---- loading side: slot (step ls, user lj, unit 2 ls + lh)
    int ls = 0, lj = 0, lh = 0;
    struct Slot {
        u32x4 w[RT];  // per row tile 16 bytes of sign words: 4 products
                      // (GROUP: group G's 4 k-blocks)
    };
    // GROUP: per user and step, one load of the scale windows of both row tiles and both
    // units: lane (j, g) takes row tile g % RT, unit g / RT; the slots read them with
    // ds_bpermute.  Entry i belongs to ring positions 2 i and 2 i + 1.
    u32x4 wring[GRP ? kRing / 2 : 1];
    auto issue_w = [&](Slot& sl, int t) __attribute__((always_inline)) {
        const bool ok = ls < S;                  // uniform
        const uint32_t oob = ok ? 0u : kOOB;     // (offsets stay below 2^31)
        const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
            (void*)lbase(ub_lo, ub_hi, lj), (short)0, nrec_bits, 0x00020000);
        sl.w[t] = buf_load16(br, (brow[t] + (uint32_t)(64 * (2 * ls + lh) + 16 * G)) | oob);
    };
    auto issue_s = [&](u32x4& sw) __attribute__((always_inline)) {
        // (called in the second slot of a pair: ls, lj are the pair's step and user)
        const bool ok = ls < S;                  // uniform
        const uint32_t oob = ok ? 0u : kOOB;
        const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)lbase(sb_lo, sb_hi, lj), (short)0, nrec_sc, 0x00020000);
        const int t = G % RT, hh = (G / RT) & 1;
        sw = buf_load16(sr, swin(2 * ls + hh, t) | oob);
    };
    auto l_advance = [&]() __attribute__((always_inline)) {
        lh ^= 1;
        if (lh == 0 && ++lj == nus) {
            lj = 0;
            ++ls;
        }
    };

    // ---- consumption side: step cs, slot q of the step (user q >> 1, unit 2 cs + (q & 1))
    int cs = 0, q = 0, bufc = 0, bufe = 2;
    issue_enc(0, 0);
    if (S > 1) issue_enc(1, 1);
    Slot ring[kRing];
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
#pragma unroll
        for (int t = 0; t < RT; ++t) issue_w(ring[r], t);
        if (GRP && (r & 1)) issue_s(wring[r / 2]);
        l_advance();
        // (in ring order: slot 0's loads must be the oldest when the loop starts)
        __builtin_amdgcn_sched_barrier(0);
    }
    // slots whose loads were issued; at that count the copies of steps cs and cs + 1 were issued
    int nslot = kRing, mark0 = 0, mark1 = 0;
    bool gfast[2] = {true, true};  // GROUP: the unit's four groups are its window's four words
    f32x4 acc[RT], acc2[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc2[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int k = 0; k < total; k += kRing) {
#pragma unroll
        for (int r = 0; r < kRing; ++r) {
            const int h = r & 1;  // the slot's unit within the step
            if (q == 0 && cs < S) {
                {
                    // wait until at most the loads issued after this step's copy
                    // (capped at kRing - 1 slots) are in flight
                    const int after = nslot - mark0;
                    if (after >= kRing - 1) {
                        BD_WAIT_VMCNT((kRing - 1) * L);
                    } else {
                        switch (after) {
                            case 0: BD_WAIT_VMCNT(0); break;
                            case 1: BD_WAIT_VMCNT(1 * L); break;
                            case 2: BD_WAIT_VMCNT(2 * L); break;
                            case 3: BD_WAIT_VMCNT(3 * L); break;
                            case 4: BD_WAIT_VMCNT(4 * L); break;
                            case 5: BD_WAIT_VMCNT(5 * L); break;
                            default: BD_WAIT_VMCNT(6 * L); break;
                        }
                    }
                }
                asm volatile("s_barrier" ::: "memory");
                if (cs + 2 < S) issue_enc(cs + 2, bufe);
                mark0 = mark1;
                mark1 = nslot;
#pragma unroll
                for (int uh = 0; uh < 2; ++uh) {
                    if (GRP) {
                        const int u = 2 * cs + uh;
                        bool moved = false;
#pragma unroll
                        for (int t = 0; t < RT; ++t) {
                            const uint32_t w0 = swin(u, t);
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                uint32_t g = (4u * (uint32_t)u + c) >> bsh;
                                g = g < gpr ? g : gpr - 1u;
                                moved |= (srow[t] + g * SB - w0) / SB != (uint32_t)c;
                            }
                        }
                        gfast[uh] = __ballot(moved) == 0ull;
                    }
                }
            }
            Slot& sl = ring[r];
            const bool live = cs < S;  // uniform
            // this slot's unit operands (hi, lo per product, block codes), from LDS (also
            // for the empty slots past the end: no value then merges at a branch)
            i32x6 hi[4], lo[4];
            uint32_t sh, sl_;
            {
                const char* sb = sbuf + bufc * kStepBytes + h * kEncUnitBytes;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const u32x4 c0 = *(const u32x4*)(sb + (3 * p + 0) * 1024 + 16 * lane);
                    const u32x4 c1 = *(const u32x4*)(sb + (3 * p + 1) * 1024 + 16 * lane);
                    const u32x4 c2 = *(const u32x4*)(sb + (3 * p + 2) * 1024 + 16 * lane);
                    hi[p] = i32x6{(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w, (int)c1.x, (int)c1.y};
                    lo[p] = i32x6{(int)c1.z, (int)c1.w, (int)c2.x, (int)c2.y, (int)c2.z, (int)c2.w};
                }
                const u32x4 cd = *(const u32x4*)(sb + 12 * 1024 + 16 * lane);
                const int usr = __builtin_amdgcn_readlane(c_users, q >> 1);
                const bool mine = c_tuser == usr;
                sh = mine ? cd.x : 0u;
                sl_ = mine ? cd.y : 0u;
            }
            // every row tile's sign words expanded first (materialised here, not sunk
            // into the branch below: the words must be dead before they are reloaded),
            // then all reloads, then the products of all row tiles
            u32x4 bx[RT][4];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                u32x4 wq = sl.w[t];
                if (GRP) {
                    // lane (j, g) holds group g's k-blocks 0..3; product c needs group c's
                    // k-block g: a 4 x 4 transpose over the lane groups
                    auto s32a = __builtin_amdgcn_permlane32_swap(wq.x, wq.z, false, false);
                    auto s32b = __builtin_amdgcn_permlane32_swap(wq.y, wq.w, false, false);
                    auto s16a = __builtin_amdgcn_permlane16_swap(s32a[0], s32b[0], false, false);
                    auto s16b = __builtin_amdgcn_permlane16_swap(s32a[1], s32b[1], false, false);
                    wq = u32x4{s16a[0], s16a[1], s16b[0], s16b[1]};
                }
                bx[t][0] = expand(wq.x);
                bx[t][1] = expand(wq.y);
                bx[t][2] = expand(wq.z);
                bx[t][3] = expand(wq.w);
                asm volatile("" ::"v"(bx[t][0]), "v"(bx[t][1]), "v"(bx[t][2]), "v"(bx[t][3]));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < RT; ++t) issue_w(sl, t);  // the slot kRing ahead, in place
            __builtin_amdgcn_sched_barrier(0);
            if (live) {
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    const u32x4 b0 = bx[t][0], b1 = bx[t][1], b2 = bx[t][2], b3 = bx[t][3];
                    if (GRP) {
                        // this lane's row, unit h, row tile t: the window of lane group t + RT h
                        const u32x4 swv = wring[r / 2];
                        const int src = 4 * (n + 16 * (t + RT * h));
                        u32x4 sv = {(uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)swv.x),
                                    (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)swv.y),
                                    (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)swv.z),
                                    (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)swv.w)};
                        if (!gfast[h]) {  // (rare: the last rows, or groups above 128)
                            const int u = 2 * cs + h;
                            const uint32_t w0 = swin(u, t);
                            auto pick = [&](int c) __attribute__((always_inline)) {
                                uint32_t g = (4u * (uint32_t)u + c) >> bsh;
                                g = g < gpr ? g : gpr - 1u;
                                const uint32_t i = (srow[t] + g * SB - w0) / SB;
                                if (SF16) {
                                    const uint32_t d = i < 4u ? (i < 2u ? sv.x : sv.y) : (i < 6u ? sv.z : sv.w);
                                    return i & 1u ? d >> 16 : d & 0xFFFFu;
                                }
                                return i < 2u ? (i == 0u ? sv.x : sv.y) : (i == 2u ? sv.z : sv.w);
                            };
                            sv = u32x4{pick(0), pick(1), pick(2), pick(3)};
                        } else if (SF16) {
                            sv = u32x4{sv.x & 0xFFFFu, sv.x >> 16, sv.y & 0xFFFFu, sv.y >> 16};
                        }
#define BD_G(C, B, SC)                                                 \
    {                                                                  \
        f32x4 tt = {0.f, 0.f, 0.f, 0.f};                               \
        tt = mfma_f6f4<C>(hi[C], B, tt, sh);                           \
        tt = mfma_f6f4<C>(lo[C], B, tt, sl_);                          \
        const float sc = SF16 ? f16_to_f32((uint16_t)(SC)) : __uint_as_float(SC); \
        acc[t] -= sc * tt;                                             \
    }
                        BD_G(0, b0, sv.x) BD_G(1, b1, sv.y) BD_G(2, b2, sv.z) BD_G(3, b3, sv.w)
#undef BD_G
                    } else {
                        // MATRIX, ROW and COL: the scale is applied per token at the end
                        acc[t] = mfma_f6f4<0>(hi[0], b0, acc[t], sh);
                        acc2[t] = mfma_f6f4<0>(lo[0], b0, acc2[t], sl_);
                        acc[t] = mfma_f6f4<1>(hi[1], b1, acc[t], sh);
                        acc2[t] = mfma_f6f4<1>(lo[1], b1, acc2[t], sl_);
                        acc[t] = mfma_f6f4<2>(hi[2], b2, acc[t], sh);
                        acc2[t] = mfma_f6f4<2>(lo[2], b2, acc2[t], sl_);
                        acc[t] = mfma_f6f4<3>(hi[3], b3, acc[t], sh);
                        acc2[t] = mfma_f6f4<3>(lo[3], b3, acc2[t], sl_);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (GRP && (r & 1)) issue_s(wring[r / 2]);  // the pair's windows, after their last use
            l_advance();
            ++nslot;
            if (++q == 2 * nus) {
                q = 0;
                ++cs;
                bufc = bufc == kNBuf - 1 ? 0 : bufc + 1;
                bufe = bufe == kNBuf - 1 ? 0 : bufe + 1;
            }
        }
    }
    // Y[token][row] += the tile's sum; one add per element (no-return atomics).  Token
    // row 4 g + e holds -X S^T of its own user: MATRIX and ROW scale it here by that
    // user's scale (the other users' products in it are 2^-127-scaled, below rounding)
    int tok[4], tus[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        tok[e] = smeta[4 * G + e];
        tus[e] = smeta[16 + 4 * G + e];
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int64_t o = rw0 + 16 * t + n;
        if (o < d_out) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (tok[e] < 0) continue;
                float f = 1.f;
                if (MODE == BD_SCALE_MATRIX || MODE == BD_SCALE_ROW) {
                    const size_t i = (size_t)tus[e] * per_user + (MODE == BD_SCALE_ROW ? (size_t)o : 0);
                    f = -(SF16 ? f16_to_f32(((const uint16_t*)scales)[i]) : ((const float*)scales)[i]);
                } else if (COL) {
                    f = -1.f;
                }
                const float v = GRP ? acc[t][e] : f * (acc[t][e] + acc2[t][e]);
                unsafeAtomicAdd(y + (int64_t)tok[e] * d_out + o, v);
            }
        }
    }
}

// ---------------------------------------------------------------- host side
hipError_t launch_tile_plan(const BatchPlan& bp, char* batch, hipStream_t s) {
    if (bp.xdtype != BD_BF16 || bp.T == 0) return hipSuccess;
    hipLaunchKernelGGL(k_tile_plan, dim3(1), dim3(64), 0, s, (const int4*)(batch + bp.off_items),
                       (uint32_t*)(batch + bp.off_meta), (int32_t*)(batch + bp.off_tiles),
                       (int)bp.ntiles);
    return hipGetLastError();
}

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
    const int32_t* tiles = (const int32_t*)(batch + bp.off_tiles);
#define BD_ENC(G, C)                                                                           \
    hipLaunchKernelGGL((k_tile_encode<G, C>), ge, dim3(256), 0, s, (const uint16_t*)x, bp.T,   \
                       bp.d_in, perm, suser, meta, tiles, scales, dp.sdtype, dp.per_user, tmeta, \
                       enc)
    if (grp) BD_ENC(true, false);
    else if (col) BD_ENC(false, true);
    else BD_ENC(false, false);
#undef BD_ENC
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // row tiles per wave: two (256 rows per block: fewer copies of the step operands
    // per sign byte; more do not fit the registers) when that still gives every CU a
    // block of work at the typical tile count, else one
    const int64_t ntyp = (bp.T + 15) / 16;  // tiles of a batch of small users, about
    const int rt = ((dp.d_out + 32 * kWaves - 1) / (32 * kWaves)) * ntyp >= 512 ? 2 : 1;
    // one tile per block (grid rows for the bound of tiles; blocks past the batch's
    // tiles exit at once): every block has the same work, whatever the tile count
    const int64_t rtiles = (dp.d_out + 16 * kWaves * rt - 1) / (16 * kWaves * rt);
    const dim3 gd((unsigned)rtiles, (unsigned)ntiles);
    int bsh = 0;
    while (grp && (128 << bsh) < dp.group) ++bsh;
#define BD_D6(MODE, F16, RT)                                                                      \
    hipLaunchKernelGGL((k_delta6<MODE, F16, RT>), gd, dim3(64 * kWaves), 0, s, signs, scales,     \
                       dp.per_user, bsh, (const int32_t*)tmeta, (const char*)enc, meta, y,        \
                       bp.d_in, dp.d_out, nunit)
#define BD_D6R2(MODE, F16)                             \
    do {                                               \
        if (rt == 2) BD_D6(MODE, F16, 2);              \
        else BD_D6(MODE, F16, 1);                      \
    } while (0)
    const bool f16 = dp.sdtype == BD_F16;
    switch (dp.mode) {
        case BD_SCALE_MATRIX:
            if (f16) BD_D6R2(BD_SCALE_MATRIX, true); else BD_D6R2(BD_SCALE_MATRIX, false);
            break;
        case BD_SCALE_GROUP:
            if (f16) BD_D6R2(BD_SCALE_GROUP, true); else BD_D6R2(BD_SCALE_GROUP, false);
            break;
        case BD_SCALE_ROW:
            if (f16) BD_D6R2(BD_SCALE_ROW, true); else BD_D6R2(BD_SCALE_ROW, false);
            break;
        default: BD_D6R2(BD_SCALE_COL, false); break;
    }
#undef BD_D6R2
#undef BD_D6
    return hipGetLastError();
}

}  // namespace bd
