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

#include <type_traits>

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
// The delta kernel's cost of a tile grows with its number of distinct users (one
// product pass and one bank stream per user), so the tiles are also listed by that
// number, largest first (torder, a counting sort, stable within a count): the grid
// starts the longest blocks first and the short ones fill the end.
constexpr int kMaxTilesLds = 2 * (kMaxGroupT / 16) + 1;
__global__ void __launch_bounds__(64)
k_tile_plan(const int4* __restrict__ items, const int32_t* __restrict__ suser,
            uint32_t* __restrict__ meta, int32_t* __restrict__ tiles,
            int32_t* __restrict__ torder, int32_t* __restrict__ tpre, int maxt) {
    __shared__ int32_t st[kMaxTilesLds + 1];
    __shared__ uint8_t snu[kMaxTilesLds];
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
            const bool stt = cl == 0 || cl + c0 > 16;
            smask |= (uint64_t)stt << k;
            cl = c > 16 ? c - 16 : (stt ? c : cl + c);
        }
        const bool stt = (smask >> lane) & 1ull;
        const bool big = lane < m && it.z > 16;
        const uint64_t bmask = __ballot(big);
        const uint64_t below = (1ull << lane) - 1ull;
        const int idx = nt + __popcll(smask & below) + __popcll(bmask & below);
        if (lane < m) {
            if (stt && idx < maxt) {
                tiles[idx] = it.y;
                st[idx] = it.y;
            }
            if (big && idx + (int)stt < maxt) {
                tiles[idx + (int)stt] = it.y + 16;
                st[idx + (int)stt] = it.y + 16;
            }
        }
        nt += __popcll(smask) + __popcll(bmask);
    }
    nt = nt < maxt ? nt : maxt;
    const int nv = (int)meta[2];
    if (lane == 0) {
        tiles[nt] = nv;
        st[nt] = nv;
        meta[3] = (uint32_t)nt;
    }
    __syncthreads();
    // distinct users of each tile: user changes over its (sorted) positions
    for (int t = lane; t < nt; t += 64) {
        const int a = st[t], e = st[t + 1];
        int cnt = 0, prev = -1;
        for (int q = a; q < e; ++q) {
            const int u = suser[q];
            cnt += u != prev;
            prev = u;
        }
        snu[t] = (uint8_t)cnt;
    }
    __syncthreads();
    // tpre[k]: the users of the tiles of rank < k (their sum in tpre[nt])
    int pos = 0, pre = 0;
    for (int v = 16; v >= 0; --v) {  // (a tile holds 1..16 positions; 0 keeps every tile ranked)
        for (int b = 0; b < nt; b += 64) {
            const int t = b + lane;
            const bool hit = t < nt && snu[t] == v;
            const uint64_t mk = __ballot(hit);
            const int below = __popcll(mk & ((1ull << lane) - 1ull));
            if (hit) {
                torder[pos + below] = t;
                tpre[pos + below] = pre + v * below;
            }
            pos += __popcll(mk);
            pre += v * __popcll(mk);
        }
    }
    if (lane == 0) tpre[nt] = pre;
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
k_tile_encode(const uint16_t* __restrict__ x, int64_t T, int U, int64_t d_in,
              const int32_t* __restrict__ perm, const int32_t* __restrict__ suser,
              const uint32_t* __restrict__ meta_r, const int32_t* __restrict__ tiles,
              const void* __restrict__ scales, int sdtype, int64_t per_user,
              int32_t* __restrict__ tmeta, char* __restrict__ enc, uint32_t* __restrict__ meta_w) {
    const int t = blockIdx.x, u = blockIdx.y, nunit = gridDim.y;
    const int lane = threadIdx.x & 63;
    const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = lane & 15, G = lane >> 4;
    // (the tag also for a batch without tiles: no token with a valid user)
    if (t == 0 && u == 0 && threadIdx.x == 0) meta_w[kEncTagWord] = enc_tag(GRP, COL);
    const int ntv = (int)meta_r[3];
    if (t >= ntv) return;  // uniform: no such tile in this batch
    const int ts = tiles[t], tl = tiles[t + 1] - ts;  // start, length
    const int p = ts + m;
    const int tok0 = m < tl ? perm[p] : -1;
    const int usr0 = m < tl ? suser[p] : -1;
    // (a batch prepared for other sizes: such tokens are encoded as absent)
    const bool okp = tok0 >= 0 && tok0 < T && usr0 >= 0 && usr0 < U;
    const int tok = okp ? tok0 : -1;
    const int usr = okp ? usr0 : -1;
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
// Block (16 kWaves RT output rows of one matrix of the set, one tile), kWaves waves of
// RT row tiles of 16 rows.  The work is a sequence of slots: step by step (two
// 512-column units, 2s and 2s + 1), user by user of the tile, two slots per user: its
// sign rows' 64 bytes of unit 2s and then of unit 2s + 1, so the two halves of every
// 128-byte line are read by consecutive loads of a wave (a row's next bytes come RT
// loads later).  Each wave keeps the loads of its next kRing slots in flight in a ring
// of registers: a slot's sign words are expanded first and only then reloaded, in
// place, with the slot kRing ahead (its scales likewise after their last use), so no
// register copy on a loop edge waits for a load in flight.  A step's encoded tokens
// (26 KB) come into LDS buffer s % 3, copied two steps ahead and shared by the block's
// waves; the opening of step s waits until no more loads are in flight than were
// issued after that copy.  Each slot reads its unit's operands from LDS (13 KB per
// wave and slot, read while the sign words are expanded).  Steps hold an even number
// of slots and kRing is even, so the unit of the slot at ring position r is r & 1.
// MFMA: A = the tile's 16 tokens (fp6 hi and lo; tokens of other users take block
// code 0, i.e. scale 2^-127), B = 16 sign rows (fp4 +-1); lane (j, g) of D holds
// tokens 4 g .. 4 g + 3 of output row j of the row tile.
// Grid: one block per (tile rank, row block), tile ranks in the order of k_tile_plan
// (most users first).  Block b runs on XCD b % 8 and takes, within its XCD's sequence,
// all of that XCD's row blocks of one tile rank before the next rank: consecutive
// tiles of one hot user (adjacent ranks) then re-read its sign rows from that XCD's L2.
constexpr int kNBuf = 3;                       // LDS buffers of step operands
constexpr int kStepBytes = 2 * kEncUnitBytes;  // two units
constexpr int kWaves = 4;  // 64 RT rows per block of 256 threads; two blocks per CU

// Up to kMaxMats matrices that read the same encoded batch (q, k and v; gate and up),
// their row blocks back to back: matrix m owns row blocks [rb_begin[m], rb_begin[m + 1]).
struct DeltaMats {
    const uint64_t* signs[kMaxMats];
    const void* scales[kMaxMats];
    float* y[kMaxMats];
    int64_t d_out[kMaxMats];
    int64_t per_user[kMaxMats];   // scales of one user
    uint64_t sstride[kMaxMats];   // bytes from one user's (slot's) signs to the next
    int64_t cstride[kMaxMats];    // scale elements from one user's scales to the next
    int rb_begin[kMaxMats + 1];
    int n;
};

// Values every lane of a wave holds alike, pinned to scalar registers: derived from a
// memory load or a select, the compiler cannot prove them uniform and would wrap every
// buffer load whose descriptor uses them in a loop over the lanes' distinct values.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni64(int64_t v) {
    const uint64_t u = (uint64_t)v;
    return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(u >> 32)) << 32) |
                     (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u));
}
template <typename P>
__device__ __forceinline__ P* uni_ptr(P* p) {
    return (P*)(uintptr_t)uni64((int64_t)(uintptr_t)p);
}

// Entry m of a kernel-argument array, chosen with scalar selects written out (a plain
// select chain is turned into an indexed load from a private copy of the arguments).
template <int K>
__device__ __forceinline__ uint64_t s_sel64(int m, uint64_t a, uint64_t b) {  // m == K ? a : b
    uint64_t r;
    const int ms = __builtin_amdgcn_readfirstlane(m);  // (an SGPR even when registers are short)
    asm volatile("s_cmp_eq_u32 %1, %4\n\ts_cselect_b64 %0, %2, %3"
                 : "=s"(r) : "s"(ms), "s"(a), "s"(b), "i"(K) : "scc");
    return r;
}
template <typename T>
__device__ __forceinline__ T pick_mat(const T (&a)[kMaxMats], int m) {
    static_assert(sizeof(T) == 8 && kMaxMats == 4, "64-bit entries, four matrices");
    uint64_t v = __builtin_bit_cast(uint64_t, a[0]);
    v = s_sel64<1>(m, __builtin_bit_cast(uint64_t, a[1]), v);
    v = s_sel64<2>(m, __builtin_bit_cast(uint64_t, a[2]), v);
    v = s_sel64<3>(m, __builtin_bit_cast(uint64_t, a[3]), v);
    return __builtin_bit_cast(T, v);
}
__device__ __forceinline__ int pick_rb(const int (&a)[kMaxMats + 1], int m) {
    uint64_t v = (uint64_t)(uint32_t)a[0];
    v = s_sel64<1>(m, (uint64_t)(uint32_t)a[1], v);
    v = s_sel64<2>(m, (uint64_t)(uint32_t)a[2], v);
    return (int)(uint32_t)s_sel64<3>(m, (uint64_t)(uint32_t)a[3], v);
}

// (two waves per SIMD: at most 256 registers each, so that two blocks share a CU)
template <int MODE, bool SF16, int RT>
__global__ void __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2)))
k_delta6(const DeltaMats dm, int bsh, const int32_t* __restrict__ tmeta,
         const int32_t* __restrict__ torder, const char* __restrict__ enc,
         uint32_t* __restrict__ meta, int64_t d_in, int nunit, int T, int U) {
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
    static_assert((kRing - 1) * LMAX <= 63 && kRing <= 16, "vmcnt range");
    static_assert(kRing % 2 == 0, "the unit of a ring position is its parity");
    __shared__ __attribute__((aligned(16))) char sbuf[kNBuf * kStepBytes];
    __shared__ int32_t smeta[kTileMetaInts];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, G = lane >> 4;
    // block -> (tile rank, row block of the matrix set)
    const int nrb = dm.rb_begin[kMaxMats];  // (entries past the set repeat the total)
    const int nrb8 = (nrb + 7) >> 3;
    const int bk = (int)blockIdx.x >> 3;
    const int rb = (bk % nrb8) * 8 + ((int)blockIdx.x & 7);
    const int trank = bk / nrb8;
    if (rb >= nrb || trank >= (int)meta[3]) return;  // uniform: no such row block or tile
    // The tile lists and operands exist only once the batch is encoded for this mode
    // (bd_batch_prepare clears the tag): nothing of them is read before this check.
    if (meta[kEncTagWord] != enc_tag(GRP, COL)) {
        if (threadIdx.x == 0) atomicOr(meta, ST_ENCODING);
        return;
    }
    const int tile = uni(torder[trank]);
    int mi = 0;
#pragma unroll
    for (int j = 1; j < kMaxMats; ++j) mi += (j < dm.n && rb >= dm.rb_begin[j]) ? 1 : 0;
    mi = uni(mi);
    const uint64_t* const signs = pick_mat(dm.signs, mi);
    const void* const scales = pick_mat(dm.scales, mi);
    float* const y = pick_mat(dm.y, mi);
    const int64_t d_out = pick_mat(dm.d_out, mi);
    const int64_t per_user = pick_mat(dm.per_user, mi);
    const uint64_t sstride = pick_mat(dm.sstride, mi);
    const int64_t cstride = pick_mat(dm.cstride, mi);
    const int rbl = rb - pick_rb(dm.rb_begin, mi);
    const int64_t rw0 = (int64_t)rbl * (16 * kWaves * RT) + 16 * RT * wv;  // the wave's first row
    // (wave 0: a uniform branch, so the values around it stay scalar)
    if (wv == 0) smeta[lane] = tmeta[(size_t)tile * kTileMetaInts + lane];
    __syncthreads();
    const int nus = __builtin_amdgcn_readfirstlane(smeta[48]);  // >= 1
    {
        // the tile's tokens, their users and its user list must fit this call's T and
        // n_users (a batch prepared for other sizes): checked before any becomes an address
        const int v = smeta[lane];
        const bool bad = lane < 16 ? v < -1 || v >= T
                         : lane < 32 ? v < -1 || v >= U
                         : lane < 48 ? (lane - 32 < nus && (v < 0 || v >= U))
                                     : lane == 48 && (v < 1 || v > 16);
        if (__ballot(bad) != 0ull) {  // uniform
            if (threadIdx.x == 0) atomicOr(meta, ST_ENCODING);
            return;
        }
    }
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
    // (ko = kone, or 0 for the empty slots past the end: their words load as 0, so their
    // operands are exact zeros and the products add nothing)
    auto expand = [&](uint32_t wq, uint32_t ko) __attribute__((always_inline)) {
        u32x4 a;
        a.x = ((wq << 3) & kmask) | ko;
        a.y = ((wq << 2) & kmask) | ko;
        a.z = ((wq << 1) & kmask) | ko;
        a.w = (wq & kmask) | ko;
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
        const uint64_t ub = (uint64_t)(const char*)signs + usr * sstride;
        const uint64_t sbp = (uint64_t)(const char*)scales + usr * (uint64_t)cstride * SB;
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
                        switch (after) {  // (after < kRing - 1 <= 15)
                            case 0: BD_WAIT_VMCNT(0); break;
                            case 1: BD_WAIT_VMCNT(1 * L); break;
                            case 2: BD_WAIT_VMCNT(2 * L); break;
                            case 3: BD_WAIT_VMCNT(3 * L); break;
                            case 4: BD_WAIT_VMCNT(4 * L); break;
                            case 5: BD_WAIT_VMCNT(5 * L); break;
                            case 6: BD_WAIT_VMCNT(6 * L); break;
                            case 7: BD_WAIT_VMCNT(7 * L); break;
                            case 8: BD_WAIT_VMCNT(8 * L); break;
                            case 9: BD_WAIT_VMCNT(9 * L); break;
                            case 10: BD_WAIT_VMCNT(10 * L); break;
                            case 11: BD_WAIT_VMCNT(11 * L); break;
                            case 12: BD_WAIT_VMCNT(12 * L); break;
                            case 13: BD_WAIT_VMCNT(13 * L); break;
                            default: BD_WAIT_VMCNT(14 * L); break;
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
            const uint32_t konel = cs < S ? kone : 0u;  // uniform (scalar select)
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
                // (an empty slot past the end may read a buffer never written: its block
                // codes are forced to 0, a finite scale, so its zero operands add exactly 0)
                const bool mine = cs < S && c_tuser == usr;
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
                bx[t][0] = expand(wq.x, konel);
                bx[t][1] = expand(wq.y, konel);
                bx[t][2] = expand(wq.z, konel);
                bx[t][3] = expand(wq.w, konel);
                asm volatile("" ::"v"(bx[t][0]), "v"(bx[t][1]), "v"(bx[t][2]), "v"(bx[t][3]));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < RT; ++t) issue_w(sl, t);  // the slot kRing ahead, in place
            __builtin_amdgcn_sched_barrier(0);
            // (no branch around the products: the accumulators then never merge at a
            // branch, which kept them moving between register files every slot)
            {
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    const u32x4 b0 = bx[t][0], b1 = bx[t][1], b2 = bx[t][2], b3 = bx[t][3];
                    if (GRP) {
                      // (GROUP: the empty slots past the end skip their products; without
                      // this branch the group-scale path needs more than 256 registers)
                      if (cs < S) {
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
                      }
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
                    const size_t i = (size_t)tus[e] * cstride + (MODE == BD_SCALE_ROW ? (size_t)o : 0);
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

// ------------------------------------------------ delta products, persistent
// The products of all units of d_in for MATRIX, ROW and COL scales, W units (one per
// wave) at a time: rows wider than W units are taken in groups of W, the block running
// its share of the items once per group (the sweep ring runs on from one group to the
// next, so no group waits for a new launch's start).
// Work item = (tile rank k, chunk c): 128 output rows (8 row tiles) of the matrix set
// for the 16 tokens of tile torder[k]; its cost is one sweep per user of the tile.
// One block per CU, W waves, wave w on unit g W + w in group g; the block takes the items whose
// first sweep falls in its equal share of all sweeps (tpre: sweeps of the ranks before
// k), tile-major, so it keeps one tile's operands for many chunks.  A wave loads its
// unit's encoded tokens when its tile changes (13 KB into registers: fp6 hi / lo of
// the four products and their block codes), then streams, sweep after sweep (one user
// of the item), the 8 row tiles' 16 sign rows x 64 bytes of its unit through a ring of
// two sweeps of loads in flight (16 bytes per lane, the B operand of the 4 products),
// running ahead across items and tiles.  Each row tile has its own accumulator over the
// item's users (other users' tokens carry block code 0, scale 2^-127).  At the end of
// an item the waves' partials (their units' shares) meet in LDS (double buffered, one
// barrier per item); wave w sums row tiles w, w + W, ... over the units in unit order,
// scales them per token (MATRIX / ROW: the scale of the token's user; COL: in the
// tokens) and adds them to y, one no-return atomic per element.  Every y element gets
// its addends (the base product, then one per group) in a fixed order: the result
// repeats bit for bit.
constexpr int kRT8 = 8;                // row tiles of a chunk: one sweep
constexpr int kChunkRows = 16 * kRT8;  // rows of a chunk
constexpr int kMaxW8 = 8;              // units (waves) per launch

typedef const __attribute__((address_space(4))) int32_t* cptr_i32;  // uniform: scalar loads
__device__ __forceinline__ int sload(const void* p, int64_t i) { return ((cptr_i32)p)[i]; }

// y[i] += v, no return, issued from asm: the compiler's own waits do not count it
__device__ __forceinline__ void atomic_add_nr(float* p, float v) {
    asm volatile("global_atomic_add_f32 %0, %1, off" ::"v"(p), "v"(v) : "memory");
}

template <int MODE, bool SF16, int RPW>
__global__ void __launch_bounds__(64 * kMaxW8)
k_delta8(const DeltaMats dm, const int32_t* __restrict__ tmeta,
         const int32_t* __restrict__ torder, const int32_t* __restrict__ tpre,
         const char* __restrict__ enc, uint32_t* __restrict__ meta, int64_t d_in, int nunit,
         int ngrp, int units, int T, int U) {
    // dm.rb_begin: first chunk of each matrix; RPW: row tiles each wave sums per item
    // (at least ceil(8 / W)); units: the units of d_in, taken W at a time in ngrp groups
    // (wave w of group g on unit g W + w; a wave whose unit is past them adds zeros)
    static_assert(MODE != BD_SCALE_GROUP, "GROUP scales take k_delta6");
    constexpr bool COL = MODE == BD_SCALE_COL;
    constexpr int RT = kRT8, D = 2 * RT;  // ring: two sweeps
    __shared__ __attribute__((aligned(16))) f32x4 part[2][RT][kMaxW8][64];
    __shared__ __attribute__((aligned(16))) float sF[kMaxMats][16];  // MATRIX: per matrix and token
    const int lane = threadIdx.x & 63;
    const int wv = uni((int)(threadIdx.x >> 6));
    const int W = uni((int)(blockDim.x >> 6));
    const int n = lane & 15, G = lane >> 4;
    if ((uint32_t)sload(meta, kEncTagWord) != enc_tag(false, COL)) {
        if (threadIdx.x == 0) atomicOr(meta, ST_ENCODING);
        return;
    }
    const int ntl = sload(meta, 3);
    const int C = dm.rb_begin[kMaxMats];  // chunks of the matrix set
    // tpre of the first 64 ranks in registers (lane = rank; one load for batches of up to
    // 63 tiles), the rest read where needed
    const int tp_l = lane <= ntl ? tpre[lane] : 0x7FFFFFFF;
    const int tot = sload(tpre, ntl);     // sweeps of one chunk over all tiles
    auto tpre_at = [&](int q) __attribute__((always_inline)) {
        return q < 64 ? __builtin_amdgcn_readlane(tp_l, q) : sload(tpre, q);
    };
    // ranks with users: torder lists them first and tpre rises over them
    int neff = __popcll(__ballot(lane < ntl && tp_l < tot));
    for (int b = 64; b < ntl; b += 64) {
        const int k = b + lane;
        neff += __popcll(__ballot(k < ntl && tpre[k] < tot));
    }
    neff = uni(neff);
    // The blocks split the launch's cost evenly: kCostSweep units per sweep and kCostEnd
    // per item end (the item's partial sums meet in LDS behind a barrier of the block's
    // waves and go to y: measured at a quarter to a third of a sweep), so a block of one-user
    // tiles, whose every sweep ends an item, takes fewer sweeps.  Sweeps run in the order
    // tile rank k, chunk c, user j of the tile; rank k starts at cost
    // C (kCostSweep tpre[k] + kCostEnd k) and each of its items costs
    // kCostSweep nu + kCostEnd (the last user's sweep carries the end).  locate: the sweep
    // whose cost range holds position w, as (k, c, j) and as a sweep index (tile k's
    // sweeps start at tpre[k] C); the end of the cost range gives the number of sweeps.
    // A block boundary may fall inside an item, at a user: each side then adds only its
    // own users' tokens.
    constexpr int kCostSweep = 8, kCostEnd = 2;
    const int64_t Wc = (int64_t)C * ((int64_t)kCostSweep * tot + (int64_t)kCostEnd * neff);
    auto locate = [&](int64_t w, int& kk, int& cc, int& jj) __attribute__((always_inline)) -> int64_t {
        kk = neff;
        cc = jj = 0;
        if (w >= Wc) return (int64_t)tot * C;  // (uniform)
        auto start = [&](int t, int q) { return (int64_t)C * ((int64_t)kCostSweep * t + (int64_t)kCostEnd * q); };
        int cnt = __popcll(__ballot(lane < neff && start(tp_l, lane) <= w));
        for (int b = 64; b < neff; b += 64) {
            const int q = b + lane;
            cnt += __popcll(__ballot(q < neff && start(tpre[q], q) <= w));
        }
        const int q = uni(cnt) - 1;  // (>= 0: rank 0 starts at 0)
        const int t0q = tpre_at(q);
        int nq = tpre_at(q + 1) - t0q;
        nq = nq < 1 ? 1 : nq;
        const int64_t rem = w - start(t0q, q);
        const int64_t isz = (int64_t)kCostSweep * nq + kCostEnd;
        kk = q;
        cc = (int)(rem / isz);
        const int r2 = (int)(rem - (int64_t)cc * isz) / kCostSweep;
        jj = r2 < nq - 1 ? r2 : nq - 1;
        return (int64_t)t0q * C + (int64_t)cc * nq + jj;
    };
    // share of block b: the workgroups of a launch go round-robin over the 8 XCDs (b on
    // XCD b % 8), so each XCD takes a contiguous run of shares and a tile's encoded
    // operands and split items stay within fewer L2s
    const int64_t nb = gridDim.x, bx = blockIdx.x;
    const int64_t sh = nb % 8 == 0 ? (bx % 8) * (nb / 8) + bx / 8 : bx;
    int sk0, sc0, sj0, ek, ec, ej;
    const int64_t s0 = locate(Wc * sh / nb, sk0, sc0, sj0);
    const int64_t s1 = locate(Wc * (sh + 1) / nb, ek, ec, ej);
    if (s1 <= s0) return;  // uniform: no sweeps
    sk0 = uni(sk0);
    sc0 = uni(sc0);
    sj0 = uni(sj0);

    // The block runs its share once per group of units; the sweep ring runs on across the
    // groups (the loader's unit is in each sweep's descriptor).  A y element gets one add
    // per group, from the same lane of the same wave and in group order (same-address
    // atomics of one thread are applied in program order), as from one launch per group.
    int u = wv;
    bool uact = u < units;  // uniform
    const int64_t nsw = s1 - s0;  // sweeps of the share, per group
    const uint32_t bank_row = (uint32_t)(d_in / 8);
    // a wave's 16 lanes of B column n read 16 bytes of row n at its unit's 64 (the unit's
    // column offset is in the descriptor); row tile r of a chunk 16 r rows further
    const uint32_t lane_off = (uint32_t)n * bank_row + 16u * (uint32_t)G;
    const uint32_t rstride = 16u * bank_row;
#define BD_VOFF(r) (lane_off + (uint32_t)(r) * rstride)

    // ---- loading side: item (kL, cL), user jL; scalar state, one descriptor per sweep
    int kL = sk0, cL = sc0, jL = sj0, gL = 0;
    int64_t leftL = nsw;  // sweeps of its group the loader has not issued
    const int tile0 = sload(torder, sk0);
    int nu0 = 1;
    {
        const int q = sload(tpre, sk0 + 1) - sload(tpre, sk0);
        nu0 = q < 1 ? 1 : (q > 16 ? 16 : q);
    }
    int tileL = tile0, nuL = nu0;
    auto lsweep = [&]() __attribute__((always_inline)) -> __amdgpu_buffer_rsrc_t {
        const bool live = leftL > 0;
        int mi = 0;
#pragma unroll
        for (int q = 1; q < kMaxMats; ++q) mi += (q < dm.n && cL >= dm.rb_begin[q]) ? 1 : 0;
        const int usr = live && (uint32_t)tileL < (uint32_t)ntl
                            ? sload(tmeta, (int64_t)tileL * kTileMetaInts + 32 + jL) : -1;
        const int uL = gL * W + wv;
        const bool ok = uL < units && (uint32_t)usr < (uint32_t)U;
        const uint64_t* sg = pick_mat(dm.signs, mi);
        const int64_t d_out = pick_mat(dm.d_out, mi);
        const int64_t row0 = (int64_t)(cL - pick_rb(dm.rb_begin, mi)) * kChunkRows;
        const uint64_t ucol = ok ? 64ull * (uint64_t)uL : 0ull;  // (< bank_row)
        const uint64_t base = (uint64_t)(uintptr_t)sg +
                              (uint64_t)(ok ? usr : 0) * pick_mat(dm.sstride, mi) +
                              (uint64_t)row0 * bank_row + ucol;
        const uint64_t rem = ok && row0 < d_out ? (uint64_t)(d_out - row0) * bank_row - ucol : 0ull;
        const int nrec = rem > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)rem;
        if (live) {
            --leftL;
            if (++jL == nuL) {  // next item
                jL = 0;
                if (leftL > 0 && ++cL == C) {
                    cL = 0;
                    ++kL;
                    tileL = sload(torder, kL);
                    const int nu = sload(tpre, kL + 1) - sload(tpre, kL);
                    nuL = nu < 1 ? 1 : (nu > 16 ? 16 : nu);
                }
            }
            if (leftL == 0 && gL + 1 < ngrp) {  // the share again, for the next group
                ++gL;
                kL = sk0;
                cL = sc0;
                jL = sj0;
                leftL = nsw;
                tileL = tile0;
                nuL = nu0;
            }
        }
        return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nrec, 0x00020000);
    };

    // ---- consuming side
    // tile state: operands, block codes, tokens and their factors, A c^T (see below)
    i32x6 hi[4], lo[4];
    uint32_t cdh = 0, cdl = 0;
    int trow = -1;  // lane l: word l of the tile's meta (tokens, their users, user list)
    bool tdead = true;
    int jt = -1;
    f32x4 ncor = {0.f, 0.f, 0.f, 0.f};
    // B operands straight from the sign words: dword d of a product's operand keeps bits
    // 4 k + d of the word in place (nibble k, bit d) over a constant pattern, so each
    // nibble is c_d + s (s = +1 for bit 0, -1 for bit 1; e2m1 1110/1111 = -4/-6,
    // 1100/1110 = -2/-4, 1000/1100 = -0/-2, 0010/1010 = 1/-1: c = -5, -3, -1, 0).  The
    // constant part, A (c_(k / 8))^T, is the same for every output row: computed once per
    // tile and the row tiles' sums start from its negative.
    uint32_t m0, m1, m2, m3, k0, k1, k2, k3;  // (gfx9 VOP3 takes no literal)
    asm volatile("v_mov_b32 %0, 0x11111111" : "=v"(m0));
    asm volatile("v_mov_b32 %0, 0x22222222" : "=v"(m1));
    asm volatile("v_mov_b32 %0, 0x44444444" : "=v"(m2));
    asm volatile("v_mov_b32 %0, 0x88888888" : "=v"(m3));
    asm volatile("s_mov_b32 %0, 0xEEEEEEEE" : "=s"(k0));
    asm volatile("s_mov_b32 %0, 0xCCCCCCCC" : "=s"(k1));
    asm volatile("s_mov_b32 %0, 0x88888888" : "=s"(k2));
    asm volatile("s_mov_b32 %0, 0x22222222" : "=s"(k3));
    int k = sk0, c = sc0, grp = 0;
    int64_t left = nsw;  // sweeps of the group not yet done
    int tile = -1, nu = 1, j = sj0, ja = sj0, ci = 0;  // ja: the item's first user here;
                                                     // ci: items done (LDS buffer parity)
    // A new tile in two parts.  tile_load issues the tile's loads: its meta (waited for:
    // the checks and the user of each token need it), the encoded operands and (MATRIX,
    // wave 0) the scale of each token's user in each matrix.  tile_finish uses them.  The
    // first tile's loads go out before the ring's, so its products wait only for them;
    // later tiles' loads are the youngest (their first use waits for every load in
    // flight; once or twice per block).
    uint64_t cdw = 0;
    int tv = -1;       // lane l: word l of the tile's meta
    bool tdead_n = true;
    uint32_t tfraw = 0;  // MATRIX: the scale of token lane % 16's user in matrix lane / 16
    bool tfok = false;
    auto tile_load = [&](int t, int nut) __attribute__((always_inline)) {
        const bool tok_ok = (uint32_t)t < (uint32_t)ntl;
        const int tt = tok_ok ? t : 0;
        const int v = tmeta[(size_t)tt * kTileMetaInts + lane];
        const __amdgpu_buffer_rsrc_t er = make_rsrc(
            enc + ((size_t)tt * nunit + (uact ? u : 0)) * kEncUnitBytes,
            uact && tok_ok ? (uint64_t)kEncUnitBytes : 0ull);  // (no unit: zeros)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const u32x4 c0 = buf_load16(er, (3 * p + 0) * 1024 + 16 * lane);
            const u32x4 c1 = buf_load16(er, (3 * p + 1) * 1024 + 16 * lane);
            const u32x4 c2 = buf_load16(er, (3 * p + 2) * 1024 + 16 * lane);
            hi[p] = i32x6{(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w, (int)c1.x, (int)c1.y};
            lo[p] = i32x6{(int)c1.z, (int)c1.w, (int)c2.x, (int)c2.y, (int)c2.z, (int)c2.w};
        }
        cdw = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(
                                               er, 12 * 1024 + 16 * lane, 0, 0));
        // the tile's tokens, their users and its user list must fit this call's T and
        // n_users, and its user count the plan's (a batch prepared for other sizes): a
        // tile that does not is flagged and adds nothing
        const bool bad = lane < 16 ? v < -1 || v >= T
                         : lane < 32 ? v < -1 || v >= U
                         : lane < 48 ? (lane - 32 < nut && (v < 0 || v >= U))
                                     : lane == 48 && v != nut;
        const bool dead = !tok_ok || __ballot(bad) != 0ull;  // uniform
        tv = v;
        tdead_n = dead;
        if constexpr (MODE == BD_SCALE_MATRIX) {
            // lane: matrix G, token n (raw bits: converted in tile_finish, so that nothing
            // here waits for the load; a lane with no token reads entry 0 of matrix 0)
            const int c_tuser = __shfl(v, 16 + n);
            const bool ok = G < dm.n && c_tuser >= 0 && !dead;
            typedef const __attribute__((address_space(1))) uint16_t* gh;
            typedef const __attribute__((address_space(1))) uint32_t* gw;
            // (pick_mat takes a uniform index: the lane's matrix is selected from the four)
            const void* const sp0 = pick_mat(dm.scales, 0);
            const void* sp = sp0;
            int64_t cs = pick_mat(dm.cstride, 0);
#pragma unroll
            for (int q = 1; q < kMaxMats; ++q) {
                const void* const spq = pick_mat(dm.scales, q);
                const int64_t csq = pick_mat(dm.cstride, q);
                if (G == q) {
                    sp = spq;
                    cs = csq;
                }
            }
            if (!ok) sp = sp0;
            const size_t i = ok ? (size_t)c_tuser * (size_t)cs : 0;
            tfraw = SF16 ? (uint32_t)((gh)sp)[i] : ((gw)sp)[i];
            tfok = ok;
        }
    };
    auto tile_finish = [&](int nut) __attribute__((always_inline)) {
        const int v = tv;
        const bool dead = tdead_n;
        if (dead && threadIdx.x == 0) atomicOr(meta, ST_ENCODING);
        trow = v;
        tdead = dead;
        const int c_tuser = __shfl(v, 16 + n);
        jt = -1;
        for (int q = 0; q < nut; ++q)
            if (__shfl(v, 32 + q) == c_tuser) jt = q;
        if constexpr (MODE == BD_SCALE_MATRIX) {
            // the scales into LDS (wave 0), after every wave is done with the last tile's
            __builtin_amdgcn_s_waitcnt(0xC07F);
            asm volatile("s_barrier" ::: "memory");
            if (wv == 0)
                sF[G][n] = !tfok ? 0.f : SF16 ? f16_to_f32((uint16_t)tfraw) : __uint_as_float(tfraw);
            __builtin_amdgcn_s_waitcnt(0xC07F);
            asm volatile("s_barrier" ::: "memory");
        }
        cdh = (uint32_t)cdw;
        cdl = (uint32_t)(cdw >> 32);
        // c = (-4, -3, -1, 0) + (-1, 0, 0, 0) in e2m1 (1110, 1101, 1010, 0000 and 1010):
        // two products per part, in the layout of the sign operands
        u32x4 c1, c2;
        asm volatile("v_mov_b32 %0, 0xEEEEEEEE" : "=v"(c1.x));
        asm volatile("v_mov_b32 %0, 0xDDDDDDDD" : "=v"(c1.y));
        asm volatile("v_mov_b32 %0, 0xAAAAAAAA" : "=v"(c1.z));
        c1.w = 0u;
        c2 = u32x4{c1.z, 0u, 0u, 0u};
        f32x4 t4 = {0.f, 0.f, 0.f, 0.f};
        t4 = mfma_f6f4<0>(hi[0], c1, t4, cdh);
        t4 = mfma_f6f4<0>(lo[0], c1, t4, cdl);
        t4 = mfma_f6f4<0>(hi[0], c2, t4, cdh);
        t4 = mfma_f6f4<0>(lo[0], c2, t4, cdl);
        t4 = mfma_f6f4<1>(hi[1], c1, t4, cdh);
        t4 = mfma_f6f4<1>(lo[1], c1, t4, cdl);
        t4 = mfma_f6f4<1>(hi[1], c2, t4, cdh);
        t4 = mfma_f6f4<1>(lo[1], c2, t4, cdl);
        t4 = mfma_f6f4<2>(hi[2], c1, t4, cdh);
        t4 = mfma_f6f4<2>(lo[2], c1, t4, cdl);
        t4 = mfma_f6f4<2>(hi[2], c2, t4, cdh);
        t4 = mfma_f6f4<2>(lo[2], c2, t4, cdl);
        t4 = mfma_f6f4<3>(hi[3], c1, t4, cdh);
        t4 = mfma_f6f4<3>(lo[3], c1, t4, cdl);
        t4 = mfma_f6f4<3>(hi[3], c2, t4, cdh);
        t4 = mfma_f6f4<3>(lo[3], c2, t4, cdl);
        ncor = -t4;
    };

    // item state: its matrix, first row, and the factors of its sums: MATRIX -(scale of
    // the token's user), ROW -(scale of the token's user at the row), COL -1 (its scales
    // are in the tokens); sign bit 1 is a positive delta, hence the minus
    // (the lane's tokens 4 G .. 4 G + 3 and their users, from the tile's meta)
    auto ltok = [&](int e) __attribute__((always_inline)) { return tdead ? -1 : __shfl(trow, 4 * G + e); };
    auto lusr = [&](int e) __attribute__((always_inline)) { return __shfl(trow, 16 + 4 * G + e); };
    // ROW: the factors of the wave's row tiles of the item (RPF of them, loaded in the
    // item's first sweep and used when its sums are added, an item later); with more than
    // two row tiles per wave the further ones load at the item's end instead
    constexpr int RPF = MODE == BD_SCALE_ROW && RPW == 2 ? 2 : 1;
    float fs[RPF][4];
#pragma unroll
    for (int t = 0; t < RPF; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) fs[t][e] = 1.f;
    bool fresh = false;
    int imi = 0;
    const void* isc = nullptr;
    int64_t ipu = 0;
    float* iy = nullptr;
    int64_t idout = 0, irow0 = 0;
    f32x4 acc[RT];
    // scale of token e of the lane at row tile r of the item, as loaded (its use
    // negates it: a use here would wait for every load in flight); every lane loads,
    // from entry 0 where it has no token
    // (called with every lane active: a lane shuffle reads 0 from inactive lanes)
    auto factor = [&](int r, int e) __attribute__((always_inline)) -> float {
        if constexpr (MODE == BD_SCALE_MATRIX || MODE == BD_SCALE_ROW) {
            const int te = ltok(e), ue = lusr(e);
            const int64_t o = irow0 + 16 * (int64_t)r + n;
            const bool ok = te >= 0 && (MODE == BD_SCALE_MATRIX || o < idout);
            const size_t i = ok ? (size_t)ue * ipu + (MODE == BD_SCALE_ROW ? (size_t)o : 0) : 0;
            typedef const __attribute__((address_space(1))) uint16_t* gh;  // global, not flat:
            typedef const __attribute__((address_space(1))) float* gf;     // counted waits
            if constexpr (SF16) return __builtin_bit_cast(float, (uint32_t)((gh)isc)[i]);  // raw half
            else return ((gf)isc)[i];
        } else {
            return 1.f;
        }
    };
    auto item_start = [&]() __attribute__((always_inline)) {
        int mi = 0;
#pragma unroll
        for (int q = 1; q < kMaxMats; ++q) mi += (q < dm.n && c >= dm.rb_begin[q]) ? 1 : 0;
        iy = pick_mat(dm.y, mi);
        idout = pick_mat(dm.d_out, mi);
        irow0 = (int64_t)(c - pick_rb(dm.rb_begin, mi)) * kChunkRows;
        isc = pick_mat(dm.scales, mi);
        ipu = pick_mat(dm.cstride, mi);
        imi = mi;
        fresh = true;  // (ROW: its factors load in its first sweep)
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r] = ncor;
    };
    // end of an item: the units' partials of each row tile meet in LDS (one barrier);
    // wave wv sums row tiles wv, wv + W, ... in unit order and adds them to y.  The sums
    // wait for the next item's first products (reduce_prev), whose latency they then
    // share; the LDS buffer is the other one's until the next item's barrier.
    bool pend = false;
    int ptk[4] = {-1, -1, -1, -1};
    float pfm[4] = {1.f, 1.f, 1.f, 1.f};
    float* py = nullptr;
    int64_t pdout = 0, prow0 = 0;
    int pci = 0;
    auto reduce_prev = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < RPW; ++t) {
            const int r = wv + t * W;
            if (r < RT) {  // uniform
                f32x4 v = part[pci & 1][r][0][lane];
                for (int q = 1; q < W; ++q) v += part[pci & 1][r][q][lane];
                // (ROW with more than two row tiles per wave: the further ones load their
                // factors here, before the next item changes the item state)
                float f[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[e] = MODE == BD_SCALE_MATRIX ? pfm[e]
                           : MODE == BD_SCALE_ROW ? (t < RPF ? fs[t < RPF ? t : 0][e] : factor(r, e)) : 1.f;
                    if (SF16 && MODE == BD_SCALE_ROW) f[e] = f16_to_f32((uint16_t)__builtin_bit_cast(uint32_t, f[e]));
                }
                const int64_t o = prow0 + 16 * (int64_t)r + n;
                if (o < pdout) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (ptk[e] >= 0) atomic_add_nr(py + (int64_t)ptk[e] * pdout + o, -(f[e] * v[e]));
                }
            }
        }
        pend = false;
    };
    // (users [jb, je) of the item's tile were done here: the sums of the other users'
    // tokens are another block's)
    auto item_end = [&](int jb, int je) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < RT; ++r) part[ci & 1][r][wv][lane] = acc[r];
        // this wave's partial writes have landed in LDS; then a bare barrier (a fence
        // would also wait for the sign loads in flight)
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
        asm volatile("s_barrier" ::: "memory");
#pragma unroll
        for (int e = 0; e < 4; ++e) ptk[e] = ltok(e);  // (every lane active)
        if (jb > 0 || je < nu) {  // uniform: part of the item's users
            int q_e[4] = {-1, -1, -1, -1};
            for (int q = 0; q < nu; ++q) {
                const int uq = __shfl(trow, 32 + q);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (lusr(e) == uq) q_e[e] = q;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (q_e[e] < jb || q_e[e] >= je) ptk[e] = -1;
        }
        if constexpr (MODE == BD_SCALE_MATRIX) {
            const f32x4 f4 = *(const f32x4*)&sF[imi][4 * G];
#pragma unroll
            for (int e = 0; e < 4; ++e) pfm[e] = f4[e];
        }
        py = iy;
        pdout = idout;
        prow0 = irow0;
        pci = ci;
        pend = true;
        ++ci;
        // ROW with more than two row tiles per wave: their factors follow the item state
        if constexpr (MODE == BD_SCALE_ROW && RPW > RPF) reduce_prev();
    };

    // the first tile's loads, the ring (the first two sweeps), then the first tile and item
    tile = tile0;
    nu = nu0;
    tile_load(tile, nu);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 ring[D];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const __amdgpu_buffer_rsrc_t br = lsweep();
#pragma unroll
        for (int r = 0; r < RT; ++r) ring[h * RT + r] = buf_load16(br, BD_VOFF(r));
    }
    __builtin_amdgcn_sched_barrier(0);
    tile_finish(nu);
    item_start();

    // one sweep (user j of the item) from ring half H; its slots reload with the sweep
    // two ahead
    auto sweep = [&](auto hc) __attribute__((always_inline)) {
        constexpr int H = decltype(hc)::value;
        // tokens of other users take block code 0
        const bool mine = jt == j;
        const uint32_t sh = mine ? cdh : 0u, sl = mine ? cdl : 0u;
        const __amdgpu_buffer_rsrc_t br = lsweep();
#pragma unroll
        for (int r = 0; r < RT; r += 2) {
            BD_WAIT_VMCNT(D - 2);  // row tiles r and r + 1 of this sweep have landed
            const u32x4 w0 = ring[H * RT + r], w1 = ring[H * RT + r + 1];
            u32x4 b0[4], b1[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                b0[p] = u32x4{(w0[p] & m0) | k0, (w0[p] & m1) | k1, (w0[p] & m2) | k2, (w0[p] & m3) | k3};
                b1[p] = u32x4{(w1[p] & m0) | k0, (w1[p] & m1) | k1, (w1[p] & m2) | k2, (w1[p] & m3) | k3};
            }
            asm volatile("" ::"v"(b0[0]), "v"(b0[1]), "v"(b0[2]), "v"(b0[3]), "v"(b1[0]),
                         "v"(b1[1]), "v"(b1[2]), "v"(b1[3]));
            __builtin_amdgcn_sched_barrier(0);
            ring[H * RT + r] = buf_load16(br, BD_VOFF(r));  // in place, after the words are expanded
            ring[H * RT + r + 1] = buf_load16(br, BD_VOFF(r + 1));
            __builtin_amdgcn_sched_barrier(0);
            if (left == 0) continue;  // (uniform: the block's items are done)
            f32x4 a = acc[r], b = acc[r + 1];
            a = mfma_f6f4<0>(hi[0], b0[0], a, sh);
            b = mfma_f6f4<0>(hi[0], b1[0], b, sh);
            a = mfma_f6f4<0>(lo[0], b0[0], a, sl);
            b = mfma_f6f4<0>(lo[0], b1[0], b, sl);
            a = mfma_f6f4<1>(hi[1], b0[1], a, sh);
            b = mfma_f6f4<1>(hi[1], b1[1], b, sh);
            a = mfma_f6f4<1>(lo[1], b0[1], a, sl);
            b = mfma_f6f4<1>(lo[1], b1[1], b, sl);
            a = mfma_f6f4<2>(hi[2], b0[2], a, sh);
            b = mfma_f6f4<2>(hi[2], b1[2], b, sh);
            a = mfma_f6f4<2>(lo[2], b0[2], a, sl);
            b = mfma_f6f4<2>(lo[2], b1[2], b, sl);
            a = mfma_f6f4<3>(hi[3], b0[3], a, sh);
            b = mfma_f6f4<3>(hi[3], b1[3], b, sh);
            a = mfma_f6f4<3>(lo[3], b0[3], a, sl);
            b = mfma_f6f4<3>(lo[3], b1[3], b, sl);
            acc[r] = a;
            acc[r + 1] = b;
            if (r == 0 && fresh) {  // uniform: the item's first sweep
                if (pend) reduce_prev();  // the previous item's sums
                // ROW: this item's factors of the wave's row tiles (used when its sums are
                // added, an item later)
                if constexpr (MODE == BD_SCALE_ROW) {
#pragma unroll
                    for (int t = 0; t < RPF; ++t)
                        if (wv + t * W < RT)  // uniform
#pragma unroll
                            for (int e = 0; e < 4; ++e) fs[t][e] = factor(wv + t * W, e);
                }
                fresh = false;
            }
        }
        if (left > 0) {  // uniform
            --left;
            if (++j == nu || left == 0) {  // the item, or this block's part of it, is done
                item_end(ja, j);
                j = ja = 0;
                const bool regroup = left == 0 && grp + 1 < ngrp;  // uniform: the share
                if (left > 0 || regroup) {                          // again, next units
                    bool newtile = regroup;
                    if (regroup) {
                        ++grp;
                        u = grp * W + wv;
                        uact = u < units;
                        left = nsw;
                        k = sk0;
                        c = sc0;
                        j = ja = sj0;
                        tile = tile0;
                        nu = nu0;
                    } else if (++c == C) {
                        c = 0;
                        ++k;
                        tile = sload(torder, k);
                        const int q = tpre_at(k + 1) - tpre_at(k);
                        nu = q < 1 ? 1 : (q > 16 ? 16 : q);
                        newtile = true;
                    }
                    if (newtile) {
                        tile_load(tile, nu);
                        tile_finish(nu);
                    }
                    item_start();
                }
            }
        }
    };
    // (one exit, both halves in every pass: the second half of the last pass only
    // keeps the ring's loads going; a mid-pass exit makes the compiler's own waits
    // count the ring short)
    do {
        sweep(std::integral_constant<int, 0>());
        sweep(std::integral_constant<int, 1>());
    } while (left > 0);
    if (pend) reduce_prev();
    BD_WAIT_VMCNT(0);  // (the ring's last loads, past the block's items, read nothing)
#undef BD_VOFF
}

// ---------------------------------------------------------------- host side
hipError_t launch_tile_plan(const BatchPlan& bp, char* batch, hipStream_t s) {
    if (bp.xdtype != BD_BF16 || bp.T == 0) return hipSuccess;
    hipLaunchKernelGGL(k_tile_plan, dim3(1), dim3(64), 0, s, (const int4*)(batch + bp.off_items),
                       (const int32_t*)(batch + bp.off_user), (uint32_t*)(batch + bp.off_meta),
                       (int32_t*)(batch + bp.off_tiles), (int32_t*)(batch + bp.off_torder),
                       (int32_t*)(batch + bp.off_tpre), (int)bp.ntiles);
    return hipGetLastError();
}

hipError_t launch_tile_encode(const BatchPlan& bp, const DeltaPlan& dp, char* batch,
                              const void* x, const void* scales, hipStream_t s) {
    uint32_t* meta = (uint32_t*)(batch + bp.off_meta);
    const int32_t* perm = (const int32_t*)(batch + bp.off_perm);
    const int32_t* suser = (const int32_t*)(batch + bp.off_user);
    int32_t* tmeta = (int32_t*)(batch + bp.off_tmeta);
    char* enc = batch + bp.off_enc;
    const dim3 ge((unsigned)bp.ntiles, (unsigned)bp.nunit);
    const int32_t* tiles = (const int32_t*)(batch + bp.off_tiles);
#define BD_ENC(G, C)                                                                           \
    hipLaunchKernelGGL((k_tile_encode<G, C>), ge, dim3(256), 0, s, (const uint16_t*)x, bp.T,   \
                       (int)bp.U, bp.d_in, perm, suser, meta, tiles, scales, dp.sdtype, scale_stride(dp), tmeta, \
                       enc, meta)
    if (dp.mode == BD_SCALE_GROUP) BD_ENC(true, false);
    else if (dp.mode == BD_SCALE_COL) BD_ENC(false, true);
    else BD_ENC(false, false);
#undef BD_ENC
    return hipGetLastError();
}

// Compute units of the current device (one persistent block each).
static int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
            v = 256;
        cus[dev] = v;
    }
    return cus[dev];
}

// Non-GROUP modes: one persistent launch (k_delta8), the units of d_in split into
// ceil(units / 8) groups of equal width, taken in unit order.
static hipError_t launch_delta8_set(const BatchPlan& bp, const DeltaPlan& dp, char* batch,
                                    const DeltaMatArg* mats, int n, hipStream_t s) {
    uint32_t* meta = (uint32_t*)(batch + bp.off_meta);
    const int32_t* tmeta = (const int32_t*)(batch + bp.off_tmeta);
    const int32_t* torder = (const int32_t*)(batch + bp.off_torder);
    const int32_t* tpre = (const int32_t*)(batch + bp.off_tpre);
    const char* enc = batch + bp.off_enc;
    const int nunit = (int)bp.nunit;
    const int units = (int)((bp.d_in + 511) / 512);  // units past d_in are zero operands
    const int nl = (units + kMaxW8 - 1) / kMaxW8;
    const int W = (units + nl - 1) / nl;
    DeltaMats dm = {};
    dm.n = n;
    int cb = 0;
    for (int i = 0; i < n; ++i) {
        dm.signs[i] = mats[i].signs;
        dm.scales[i] = mats[i].scales;
        dm.y[i] = mats[i].y;
        dm.d_out[i] = mats[i].d_out;
        dm.per_user[i] = dp.mode == BD_SCALE_MATRIX ? 1
                         : dp.mode == BD_SCALE_ROW ? mats[i].d_out
                                                   : bp.d_in;
        dm.sstride[i] = sign_stride(mats[i].sstride, mats[i].d_out, bp.d_in);
        dm.cstride[i] = mats[i].cstride ? mats[i].cstride : dm.per_user[i];
        dm.rb_begin[i] = cb;
        cb += (int)((mats[i].d_out + kChunkRows - 1) / kChunkRows);
    }
    for (int i = n; i <= kMaxMats; ++i) dm.rb_begin[i] = cb;
    const dim3 gd((unsigned)device_cus());
    const bool f16 = dp.sdtype == BD_F16;
    {
        // one launch: nl groups of W units (the last may hold fewer: its extra waves add 0)
#define BD_D8(MODE, F16, RPW)                                                                  \
    hipLaunchKernelGGL((k_delta8<MODE, F16, RPW>), gd, dim3(64 * W), 0, s, dm, tmeta, torder,  \
                       tpre, enc, meta, bp.d_in, nunit, nl, units, (int)bp.T, (int)bp.U)
#define BD_D8W(MODE, F16)                                      \
    do {                                                       \
        if (W == kMaxW8) BD_D8(MODE, F16, 1);                  \
        else if (W >= 4) BD_D8(MODE, F16, 2);                  \
        else if (W >= 2) BD_D8(MODE, F16, 4);                  \
        else BD_D8(MODE, F16, kRT8);                           \
    } while (0)
        switch (dp.mode) {
            case BD_SCALE_MATRIX:
                if (f16) BD_D8W(BD_SCALE_MATRIX, true); else BD_D8W(BD_SCALE_MATRIX, false);
                break;
            case BD_SCALE_ROW:
                if (f16) BD_D8W(BD_SCALE_ROW, true); else BD_D8W(BD_SCALE_ROW, false);
                break;
            default: BD_D8W(BD_SCALE_COL, false); break;
        }
#undef BD_D8W
#undef BD_D8
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// MATRIX / ROW / COL take the persistent kernel (k_delta8) for batches of many users with a
// few tokens each, when its groups of units are at least 7 wide; otherwise the per-tile
// kernel k_delta6.  Measured on one MI355X: the persistent kernel takes the 32-layer stack's
// delta phase (512 tokens, 128 users' banks) in 20.0 ms against 24.6; on the Qwen3-14B MLP
// batch (1144 tokens, 32 users, 8 prefill chunks of 128 tokens: a user's chunk fills 8
// tiles, which k_delta6 runs side by side, one tile per block) k_delta6 takes the step from
// 2054 to 1866 us; with fewer than 7 waves (rows of 5120 columns: two groups of 5 units) the
// persistent kernel's two-sweep ring keeps too few bytes in flight per CU.  The host knows
// only the batch's size and user count: the mean tokens per user decides.
static bool delta8_fits(const BatchPlan& bp) {
    const int64_t units = (bp.d_in + 511) / 512;
    const int64_t nl = (units + kMaxW8 - 1) / kMaxW8;
    return (units + nl - 1) / nl >= 7 && bp.T < 16 * (int64_t)bp.U;
}

hipError_t launch_delta6_set(const BatchPlan& bp, const DeltaPlan& dp, char* batch,
                             const DeltaMatArg* mats, int n, hipStream_t s) {
    if (n < 1 || n > kMaxMats) return hipErrorInvalidValue;
    if (dp.mode != BD_SCALE_GROUP && delta8_fits(bp)) return launch_delta8_set(bp, dp, batch, mats, n, s);
    uint32_t* meta = (uint32_t*)(batch + bp.off_meta);
    const int32_t* tmeta = (const int32_t*)(batch + bp.off_tmeta);
    const int32_t* torder = (const int32_t*)(batch + bp.off_torder);
    const char* enc = batch + bp.off_enc;
    const int ntiles = (int)bp.ntiles, nunit = (int)bp.nunit;
    const bool grp = dp.mode == BD_SCALE_GROUP;
    int64_t rows = 0;
    for (int i = 0; i < n; ++i) rows += mats[i].d_out;
    // row tiles per wave: two (fewer copies of the step operands per sign byte; more do
    // not fit the registers) when that still gives every CU blocks of work at the
    // typical tile count, else one
    const int64_t ntyp = (bp.T + 15) / 16;  // tiles of a batch of small users, about
    const int rt = ((rows + 32 * kWaves - 1) / (32 * kWaves)) * ntyp >= 512 ? 2 : 1;
    const int64_t rows_rb = 16 * kWaves * rt;
    DeltaMats dm = {};
    dm.n = n;
    int rb = 0;
    for (int i = 0; i < n; ++i) {
        dm.signs[i] = mats[i].signs;
        dm.scales[i] = mats[i].scales;
        dm.y[i] = mats[i].y;
        dm.d_out[i] = mats[i].d_out;
        dm.per_user[i] = dp.mode == BD_SCALE_MATRIX ? 1
                         : dp.mode == BD_SCALE_GROUP ? mats[i].d_out * (bp.d_in / dp.group)
                         : dp.mode == BD_SCALE_ROW ? mats[i].d_out
                                                   : bp.d_in;
        dm.sstride[i] = sign_stride(mats[i].sstride, mats[i].d_out, bp.d_in);
        dm.cstride[i] = mats[i].cstride ? mats[i].cstride : dm.per_user[i];
        dm.rb_begin[i] = rb;
        rb += (int)((mats[i].d_out + rows_rb - 1) / rows_rb);
    }
    for (int i = n; i <= kMaxMats; ++i) dm.rb_begin[i] = rb;
    const int64_t nrb8 = (rb + 7) / 8;
    const dim3 gd((unsigned)(nrb8 * 8 * ntiles));
    int bsh = 0;
    while (grp && (128 << bsh) < dp.group) ++bsh;
#define BD_D6(MODE, F16, RT)                                                                      \
    hipLaunchKernelGGL((k_delta6<MODE, F16, RT>), gd, dim3(64 * kWaves), 0, s, dm, bsh, tmeta,    \
                       torder, enc, meta, bp.d_in, nunit, (int)bp.T, (int)bp.U)
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

hipError_t launch_delta6_encoded(const BatchPlan& bp, const DeltaPlan& dp, char* batch,
                                 const uint64_t* signs, const void* scales, float* y,
                                 hipStream_t s) {
    const DeltaMatArg m = {signs, scales, y, dp.d_out, dp.sstride, dp.cstride};
    return launch_delta6_set(bp, dp, batch, &m, 1, s);
}

hipError_t launch_delta6(const BatchPlan& bp, const DeltaPlan& dp, char* batch, const void* x,
                         const uint64_t* signs, const void* scales, float* y, hipStream_t s) {
    hipError_t err = launch_tile_encode(bp, dp, batch, x, scales, s);
    if (err != hipSuccess) return err;
    return launch_delta6_encoded(bp, dp, batch, signs, scales, y, s);
}

}  // namespace bd
