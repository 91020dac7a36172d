// bd_decode.hip -- one-pass multi-tenant apply for decode-sized batches (T <= 16).
//
// y[t] = X[t] W_base^T + scale_u (.) (X[t] S_u^T) for every token of the batch
// in one kernel over the output rows ([P2] "Systems Mechanics" 1-2: one shared
// base product per batch, each request adds its user's 1-bit delta product,
// the bits cross HBM packed and are expanded on chip).
//
// One launch (MATRIX and ROW scales): k_decode_unit for rows of up to 4096
// columns (one wave per 512-column unit streams that unit's sign rows and W_base
// rows through one register ring), k_decode_fused for rows of up to 5120 (base
// and delta waves apart).  Every block stages the batch's tokens in LDS and
// encodes them itself, as two fp6 e2m3 parts per 32-column block (below); the
// delta products run the block-scaled MFMA with fp4 signs and fp6 tokens.
//
// Two launches (any row width, and COL scales):
//   k_decode_prep  sorts the (<= 16) tokens by user in one wave and encodes X
//                  for the delta products: every 32-column block of a token is
//                  scaled by a power of two (an MX block scale) and split into
//                  two OCP fp8 e4m3 parts, hi = fp8(x') and lo = fp8(x' - hi),
//                  which keeps about 8 significant bits, the precision of the
//                  bf16 input.
//   k_decode       one block per 16 output rows, 8 waves.  Base waves stream
//                  W_base rows (bf16 MFMA 16x16x32 against the bf16 tokens);
//                  delta waves stream the users' packed sign rows and run the
//                  gfx950 block-scaled MFMA 16x16x128 with the signs as fp4
//                  e2m1 +-1 operands and the encoded tokens as fp8 operands.
//                  The 16 tokens form one MFMA tile; for user u the tile's
//                  other tokens enter with block scale 2^-127 (E8M0 code 0),
//                  so one accumulator collects every user's product in its own
//                  token columns.  Partial tiles are summed in LDS in wave order
//                  and written once: no atomics, no read-modify-write of y.
//
// Sign bits to fp4: nibble = 0x2 | (bit << 3), i.e. +1.0 for a negative delta
// and -1.0 for a non-negative one, so the accumulator holds -(X S^T) and the
// epilogue multiplies by -scale.  Dword d of the A operand of a 32-bit sign
// word w is ((w << (3 - d)) & 0x88888888) | 0x22222222: its nibble n carries
// bit 4n + d.  The token encoding places column 4n + d of every 32-column
// block at MFMA k position 8d + n to match.
#include "bd_internal.h"

namespace bd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x6 __attribute__((ext_vector_type(6)));

constexpr int kDecodeWaves = 16;
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

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D += A(fp4, 16 x 128) * B(fp8 e4m3, 128 x 16) * 2^(scale_b - 127), scale_b = byte SEL of sc.
template <int SEL>
__device__ __forceinline__ f32x4 mfma_f4f8(u32x4 a, i32x8 b, f32x4 c, uint32_t sc) {
    const i32x8 a8 = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c, 4, 0, 0, 127, SEL, (int)sc);
}

__device__ __forceinline__ float load_scale(const void* s, int sdtype, int64_t i) {
    return sdtype == BD_F16 ? f16_to_f32(((const uint16_t*)s)[i]) : ((const float*)s)[i];
}

// ------------------------------------------------------------------- prep
// Every block, wave 0: bitonic sort of (user, token) keys over 64 lanes.  Tokens
// with a valid user come first, grouped by user in token order; the others (id
// -1 or out of range) follow.  Block 0 stores perm[p] = token at sorted position
// p, suser[p] = its user (or -1), seg[i] = {user, first position, count, 0} and
// the counts.  Then every thread encodes one (sorted position, 32-column block).
//
// Both operand buffers are stored in MFMA lane order, so every load of the apply
// kernel reads 1 KB contiguous (all blocks of that kernel read these buffers):
//  xs : bf16 B operand of the base product.  Step s (columns 32s .. 32s+31):
//       1 KB at s*1024, lane (m, g) = m + 16g holds columns 32s + 8g .. +7 of
//       the token at sorted position m (zero for m >= T).
//  x8 : fp8 B operands of the delta products, per chunk q (columns 128q ..
//       128q+127), part p (0 hi, 1 lo) and half h: 1 KB at ((q*2 + p)*2 + h)*1024,
//       lane (m, G) = m + 16G holding bytes 16h .. 16h+15 of that lane's 32-byte
//       operand.  The 32-column block kb of the chunk fills lane groups
//       G = 2 (kb % 2) + e, e = 0, 1, half h = kb / 2; byte b' of each 16-byte run
//       holds column 4 (b' % 8) + 2e + b' / 8 of the block: the column whose sign
//       bit the A operand puts at that k position.  Zero for positions without a
//       valid user and past d_in.
//  e8 : the blocks' scale codes, one dword per lane and 512-column unit u at
//       u*256 + 4 (m + 16 kb), byte q % 4 for chunk q = 4u + q % 4.
__global__ void __launch_bounds__(256)
k_decode_prep(const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, int T, int U,
              int64_t d_in, int64_t dpad, int col_mode, const void* __restrict__ scales, int sdtype,
              int64_t per_user, uint32_t* __restrict__ meta, int32_t* __restrict__ perm,
              int32_t* __restrict__ suser, int4* __restrict__ seg, uint16_t* __restrict__ xs,
              uint8_t* __restrict__ x8, uint8_t* __restrict__ e8) {
    __shared__ int32_t ptok[kDecodeMaxT], puser[kDecodeMaxT];
    if (threadIdx.x < 64) {
        const int l = threadIdx.x;
        uint32_t key = 0xFFFFFFFFu;
        bool bad = false;
        if (l < T) {
            const int u = ids[l];
            const bool ok = u >= 0 && u < U;
            bad = !ok && u != -1;
            key = ((ok ? (uint32_t)u : (uint32_t)U) << 6) | (uint32_t)l;
        }
        for (int k = 2; k <= 64; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                const uint32_t other = __shfl_xor(key, j);
                const bool lower = (l & j) == 0;
                const bool asc = (l & k) == 0;
                const uint32_t mn = key < other ? key : other, mx = key < other ? other : key;
                key = (lower == asc) ? mn : mx;
            }
        }
        const uint32_t user = key >> 6;
        const bool valid = l < T && user < (uint32_t)U;
        const int nv = __popcll(__ballot(valid));
        if (l < kDecodeMaxT) {
            ptok[l] = l < T ? (int32_t)(key & 63u) : -1;
            puser[l] = valid ? (int32_t)user : -1;
        }
        if (blockIdx.x == 0) {
            if (l < T) {
                perm[l] = (int32_t)(key & 63u);
                suser[l] = valid ? (int32_t)user : -1;
            }
            const uint32_t prev = __shfl_up(user, 1);
            const bool start = valid && (l == 0 || prev != user);
            const uint64_t smask = __ballot(start);
            const uint64_t above = l == 63 ? 0ull : (smask >> (l + 1)) << (l + 1);
            const int next = above ? __ffsll((unsigned long long)above) - 1 : nv;
            if (start) {
                const int idx = __popcll(smask & ((1ull << l) - 1ull));
                seg[idx] = make_int4((int)user, l, next - l, 0);
            }
            const bool anybad = __ballot(bad) != 0ull;
            if (l == 0) {
                meta[0] = anybad ? ST_USER_ID : 0u;
                meta[1] = (uint32_t)__popcll(smask);
                meta[2] = (uint32_t)nv;
            }
        }
    }
    __syncthreads();
    const int64_t nblk = dpad / 32;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < kDecodeMaxT * nblk;
         idx += (int64_t)gridDim.x * 256) {
        const int m = (int)(idx % kDecodeMaxT);
        const int64_t b = idx / kDecodeMaxT;
        const int64_t c0 = b * 32;
        const int tok = ptok[m], usr = puser[m];
        u32x4 raw[4] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u},
                        u32x4{0u, 0u, 0u, 0u}};
        if (tok >= 0 && c0 < d_in) {
            const u32x4* src = (const u32x4*)(x + tok * d_in + c0);
#pragma unroll
            for (int q = 0; q < 4; ++q) raw[q] = src[q];
        }
        if (c0 < d_in) {  // base operand, step b: lane group g takes columns 8g .. 8g+7
#pragma unroll
            for (int g = 0; g < 4; ++g) *(u32x4*)(xs + (b * 64 + m + 16 * g) * 8) = raw[g];
        }
        float v[32];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[8 * q + 2 * e] = usr >= 0 ? bf16_lo(raw[q][e]) : 0.f;
                v[8 * q + 2 * e + 1] = usr >= 0 ? bf16_hi(raw[q][e]) : 0.f;
            }
        }
        if (col_mode && usr >= 0 && c0 < d_in) {  // the user's column scales, folded into X
            const int64_t s0 = (int64_t)usr * per_user + c0;
#pragma unroll
            for (int c = 0; c < 32; ++c) v[c] *= load_scale(scales, sdtype, s0 + c);
        }
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < 32; ++c) amax = fmaxf(amax, fabsf(v[c]));
        // amax in [2^(E-1), 2^E): x' = x * 2^(8-E) puts the block maximum in [128, 256),
        // inside e4m3's range (448); the MFMA scale code 127 - (8-E) undoes it
        int code = 127, sh = 0;
        if (amax > 0.f) {
            int E;
            (void)frexpf(amax, &E);
            code = 119 + E;
            if (code < 0) code = 0;
            sh = 127 - code;
        }
        float hi[32], lo[32];
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            const float xsc = ldexpf(v[c], sh);
            const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(xsc, 0.f, 0, false);
            hi[c] = xsc;
            lo[c] = xsc - __builtin_amdgcn_cvt_f32_fp8(pk, 0);
        }
        const int64_t q = b / 4;
        const int kb = (int)(b % 4);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            u32x4 ph, pl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // bytes 4i .. 4i+3 of the run: b' = 4i + j, column 4 (b' % 8) + 2e + b' / 8
                const int base = 16 * (i & 1) + 2 * e + (i >> 1);
                int wh = __builtin_amdgcn_cvt_pk_fp8_f32(hi[base], hi[base + 4], 0, false);
                wh = __builtin_amdgcn_cvt_pk_fp8_f32(hi[base + 8], hi[base + 12], wh, true);
                int wl = __builtin_amdgcn_cvt_pk_fp8_f32(lo[base], lo[base + 4], 0, false);
                wl = __builtin_amdgcn_cvt_pk_fp8_f32(lo[base + 8], lo[base + 12], wl, true);
                ph[i] = (uint32_t)wh;
                pl[i] = (uint32_t)wl;
            }
            const int lane = m + 16 * (2 * (kb & 1) + e), h = kb >> 1;
            *(u32x4*)(x8 + (((q * 2 + 0) * 2 + h) * 64 + lane) * 16) = ph;
            *(u32x4*)(x8 + (((q * 2 + 1) * 2 + h) * 64 + lane) * 16) = pl;
        }
        e8[(q / 4) * 256 + 4 * (m + 16 * kb) + (q % 4)] = (uint8_t)code;
    }
}

// ------------------------------------------------------------------ apply
// Encoded tokens of one 512-column unit (4 chunks) for this lane.
struct Unit {
    i32x8 hi[4], lo[4];
    uint32_t e;
};

template <int MODE>
__global__ void __launch_bounds__(64 * kDecodeWaves)
k_decode(const uint16_t* __restrict__ x, int T, int64_t d_in, int64_t dpad,
         const uint16_t* __restrict__ w, int64_t d_out, const uint64_t* __restrict__ signs,
         uint64_t sstride, const void* __restrict__ scales, int sdtype, int64_t per_user,
         const uint32_t* __restrict__ meta, const int32_t* __restrict__ perm,
         const int32_t* __restrict__ suser, const int4* __restrict__ seg,
         const uint16_t* __restrict__ xs, const uint8_t* __restrict__ x8,
         const uint8_t* __restrict__ e8, void* __restrict__ y, int ydtype) {
    __shared__ f32x4 red_base[kDecodeWaves][64];   // per K slice of the base product
    __shared__ f32x4 red_delta[kDecodeWaves][64];  // per delta wave
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
    const int m = lane & 15, g = lane >> 4;
    const int nseg = (int)meta[1], nv = (int)meta[2];
    // waves split by HBM bytes per row: 2 d_in (base) against nseg d_in / 8 (delta)
    int nwb = kDecodeWaves;
    if (nseg > 0) {
        nwb = (16 * kDecodeWaves + (16 + nseg) / 2) / (16 + nseg);
        nwb = nwb < 1 ? 1 : (nwb > kDecodeWaves - 1 ? kDecodeWaves - 1 : nwb);
    }
    const int64_t r0 = (int64_t)blockIdx.x * 16;
    const int64_t rowA = r0 + m < d_out ? r0 + m : d_out - 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};

    if (wv < nwb) {
        // ---- base: the K steps of 32 columns form kDecodeWaves fixed slices (slice s =
        // steps s, s + kDecodeWaves, ...), each summed in step order and stored to LDS;
        // wave wv takes slices wv, wv + nwb, ...  The partition, and so the rounding, does
        // not depend on the batch's users.  Ring of 8 slots over the wave's steps.
        const int nsteps = (int)(d_in / 32);
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint64_t)d_out * d_in * 2);
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(xs, (uint64_t)nsteps * 1024);
        const uint32_t woff = (uint32_t)((rowA * d_in + 8 * g) * 2);
        const uint32_t xoff = (uint32_t)(lane * 16);
        const int spp = (nsteps + kDecodeWaves - 1) / kDecodeWaves;  // steps per slice
        const int nown = (kDecodeWaves - wv + nwb - 1) / nwb;          // slices of this wave
        const int total = nown * spp;
        struct Slot {
            u32x4 a, b;
        };
        // item i of the wave is step st(i) = wv + nwb * (i / spp) + kDecodeWaves * (i % spp);
        // the load stream (8 items ahead) and the compute stream each keep (slice, k)
        int ls = wv, lk = 0;   // next item to load
        auto load = [&](int i) {
            Slot sl;
            const int st = ls + kDecodeWaves * lk;
            const bool ok = i < total && st < nsteps;
            sl.a = buf_load16(wr, ok ? woff + (uint32_t)(st * 64) : kOOB);
            sl.b = buf_load16(xr, ok ? xoff + (uint32_t)(st * 1024) : kOOB);
            if (++lk == spp) {
                lk = 0;
                ls += nwb;
            }
            return sl;
        };
        constexpr int R = 8;
        Slot ring[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            ring[r] = load(r);
            __builtin_amdgcn_sched_barrier(0);
        }
        int cs = wv, ck = 0;  // slice and step of the item being summed
        for (int i0 = 0; i0 < total; i0 += R) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = i0 + r;
                acc = mfma_bf16(ring[r].a, ring[r].b, acc);
                ring[r] = load(i + R);
                if (++ck == spp) {  // uniform: the slice is complete
                    if (i < total) red_base[cs][lane] = acc;
                    acc = f32x4{0.f, 0.f, 0.f, 0.f};
                    ck = 0;
                    cs += nwb;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
        // ---- delta: 512-column units u = wd, wd + nwd, ...; every user of the batch.
        // Delta waves issue first: their operands gate the matrix-core work, while the
        // base waves only stream, so the delta loads should not queue behind them.
        __builtin_amdgcn_s_setprio(3);
        const int wd = wv - nwb, nwd = kDecodeWaves - nwb;
        const int nunit = (int)(dpad / 512);
        constexpr int RB = 8;  // bits ring depth (16 bytes per lane per slot)
        const int nsegR = (nseg + RB - 1) / RB * RB;
        const int64_t bank_row = d_in / 8;  // bytes of one packed row
        const uint64_t user_bytes = (uint64_t)d_out * (uint64_t)bank_row;
        const int lane_user = m < nv ? suser[m] : -1;    // user of this lane's token column
        const int utab = lane < nseg ? seg[lane].x : 0;  // lane j: user of segment j
        const __amdgpu_buffer_rsrc_t xr8 = make_rsrc(x8, (uint64_t)(dpad / 128) * 4096);
        const __amdgpu_buffer_rsrc_t er = make_rsrc(e8, (uint64_t)(dpad / 512) * 256);
        const uint32_t brow = (uint32_t)(rowA * bank_row + 16 * g);
        uint32_t kmask, kone;  // operand constants in registers (gfx9 VOP3 takes no literal)
        asm volatile("v_mov_b32 %0, 0x88888888" : "=v"(kmask));
        asm volatile("s_mov_b32 %0, 0x22222222" : "=s"(kone));

        auto load_unit = [&](int u) {
            Unit X;
            const bool ok = u < nunit;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t o = (uint32_t)(((4 * u + i) * 4) * 1024 + lane * 16);
                const u32x4 h0 = buf_load16(xr8, ok ? o : kOOB);
                const u32x4 h1 = buf_load16(xr8, ok ? o + 1024 : kOOB);
                const u32x4 l0 = buf_load16(xr8, ok ? o + 2048 : kOOB);
                const u32x4 l1 = buf_load16(xr8, ok ? o + 3072 : kOOB);
                X.hi[i] = i32x8{(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w,
                                (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
                X.lo[i] = i32x8{(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w,
                                (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
            }
            X.e = buf_load4(er, ok ? (uint32_t)(u * 256 + lane * 4) : kOOB);
            return X;
        };
        // 16 bytes of user j's row: columns [512u + 128g, +128) (4 words, one per chunk).
        // Always issued (out of range: a zero load), so the loads of the ring retire in
        // issue order on straight-line code and every wait is exact.
        auto load_bits = [&](int u, int j) {
            const bool ok = j < nseg && u < nunit;  // uniform
            const int usr = __builtin_amdgcn_readlane(utab, ok ? j : 0);
            const __amdgpu_buffer_rsrc_t br =
                make_rsrc((const char*)signs + (uint64_t)(uint32_t)usr * sstride, user_bytes);
            const bool in = ok && (int64_t)u * 512 + 128 * g < d_in;
            return buf_load16(br, in ? brow + (uint32_t)(u * 64) : kOOB);
        };
        auto item = [&](const Unit& X, int u, int j, u32x4 D) {
            // 4x4 transpose over the lane groups: lane group g gets word g of every chunk.
            // Done for every slot, so each slot's load is consumed at the same point on
            // every path and the waits stay exact; only the products are skipped.
            auto s32a = __builtin_amdgcn_permlane32_swap(D.x, D.z, false, false);
            auto s32b = __builtin_amdgcn_permlane32_swap(D.y, D.w, false, false);
            auto s16a = __builtin_amdgcn_permlane16_swap(s32a[0], s32b[0], false, false);
            auto s16b = __builtin_amdgcn_permlane16_swap(s32a[1], s32b[1], false, false);
            const uint32_t wd4[4] = {s16a[0], s16a[1], s16b[0], s16b[1]};
            if (j >= nseg || u >= nunit) return;  // uniform; no loads inside
            const int usr = __builtin_amdgcn_readlane(utab, j);
            const uint32_t sc = lane_user == usr ? X.e : 0u;
#define BD_CHUNK(I)                                                                   \
    {                                                                                 \
        const uint32_t wq = wd4[I];                                                   \
        u32x4 A;                                                                      \
        A.x = ((wq << 3) & kmask) | kone;                                             \
        A.y = ((wq << 2) & kmask) | kone;                                             \
        A.z = ((wq << 1) & kmask) | kone;                                             \
        A.w = (wq & kmask) | kone;                                                    \
        acc = mfma_f4f8<I>(A, X.hi[I], acc, sc);                                      \
        acc = mfma_f4f8<I>(A, X.lo[I], acc, sc);                                      \
    }
            BD_CHUNK(0) BD_CHUNK(1) BD_CHUNK(2) BD_CHUNK(3)
#undef BD_CHUNK
        };
        // Per unit: the encoded tokens first, then a ring of RB bit loads over the users
        // (slot r holds user j = r mod RB), so every wait in the user loop is exact.
        if (nseg > 0) {
            for (int u = wd; u < nunit; u += nwd) {
                const Unit X = load_unit(u);
                __builtin_amdgcn_sched_barrier(0);
                u32x4 ring[RB];
#pragma unroll
                for (int r = 0; r < RB; ++r) {  // in slot order: slot r retires before r + 1
                    ring[r] = load_bits(u, r);
                    __builtin_amdgcn_sched_barrier(0);
                }
                for (int j = 0; j < nsegR; j += RB) {
#pragma unroll
                    for (int r = 0; r < RB; ++r) {
                        item(X, u, j + r, ring[r]);
                        ring[r] = load_bits(u, j + r + RB);  // past the last user: a zero load
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
    }
    if (wv >= nwb) red_delta[wv - nwb][lane] = acc;
    __syncthreads();
    if (wv != 0) return;

    // ---- epilogue: base slices + factor * delta partials, each in a fixed order
    f32x4 vb = {0.f, 0.f, 0.f, 0.f}, vd = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < kDecodeWaves; ++q) vb += red_base[q][lane];
    for (int q = 0; q < kDecodeWaves - nwb; ++q) vd += red_delta[q][lane];
    if (m >= T) return;
    const int64_t o = r0 + 4 * g;
    float f[4] = {0.f, 0.f, 0.f, 0.f};
    if (m < nv) {
        const int64_t u = suser[m];
        const void* su = (const char*)scales + (size_t)u * per_user * (sdtype == BD_F16 ? 2 : 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t oe = o + e < d_out ? o + e : d_out - 1;
            if (MODE == BD_SCALE_MATRIX) f[e] = -load_scale(su, sdtype, 0);
            else if (MODE == BD_SCALE_ROW) f[e] = -load_scale(su, sdtype, oe);
            else f[e] = -1.0f;  // COL: the scales are folded into the encoded tokens
        }
    }
    f32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = vb[e] + f[e] * vd[e];
    const int64_t t = perm[m];
    if (ydtype == BD_F32) {
        float* dst = (float*)y + t * d_out + o;
        if (o + 3 < d_out && (d_out & 3) == 0) {
            *(f32x4*)dst = out;
        } else {
            for (int e = 0; e < 4; ++e)
                if (o + e < d_out) dst[e] = out[e];
        }
    } else {
        uint16_t* dst = (uint16_t*)y + t * d_out + o;
        if (o + 3 < d_out && (d_out & 3) == 0) {
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16(out[0]) | ((uint32_t)f32_to_bf16(out[1]) << 16);
            pk.y = (uint32_t)f32_to_bf16(out[2]) | ((uint32_t)f32_to_bf16(out[3]) << 16);
            *(uint2*)dst = pk;
        } else {
            for (int e = 0; e < 4; ++e)
                if (o + e < d_out) dst[e] = f32_to_bf16(out[e]);
        }
    }
}

// ------------------------------------------------------------ fused apply
// One launch for a whole decode batch (bf16 X, at most 16 tokens, MATRIX or ROW
// scales, d_in padded to 512 at most kFusedMaxDpad): every block stages the batch's
// tokens in LDS and encodes them for the delta products itself, so nothing has to
// run before it.  12 waves: 4 base waves stream W_base (bf16 MFMA against the
// tokens read from LDS), each over a quarter of the columns; 8 delta waves stream
// the users' packed rows (block-scaled MFMA, fp4 signs x fp6 e2m3 tokens: the fp6
// operand runs at 20 cycles per 16x16x128 product against 32 for fp8, and its
// 32-wide conversions take one instruction per block), each over its 512-column
// units.  The delta waves first copy the tokens into LDS (each its
// own units); one barrier then starts every wave's weight or sign-row stream.
//
// LDS: token row t (zeros past T and past d_in) at t * 2 dpad bytes; its 16-byte
// chunk c sits at slot (c & ~15) | ((c ^ t) & 15), so the 16 tokens read at one
// chunk index hit 16 distinct bank groups.  After the products the same memory
// holds the waves' partial tiles for the reduction.
constexpr int kFusedBaseWaves = 4, kFusedDeltaWaves = 8;
constexpr int kFusedWaves = kFusedBaseWaves + kFusedDeltaWaves;
constexpr int kFusedRedBytes = kFusedWaves * 64 * 16;
constexpr int kFusedMaxPieces = (int)(kFusedMaxDpad / 512);  // 1 KB pieces of a token row

typedef __attribute__((address_space(3))) void* lds_ptr;

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, off, 0, 0, 0);
}

__device__ __forceinline__ uint32_t xslot(int t, int c, uint32_t rowb) {
    return (uint32_t)t * rowb + 16u * (uint32_t)((c & ~15) | ((c ^ t) & 15));
}

// s_waitcnt with only the vector-memory count: vmcnt <= n (expcnt, lgkmcnt untouched).
#define BD_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 0xF) | ((((n) >> 4) & 3) << 14))

}  // namespace

// The tokens' delta operands for one 512-column unit, as fp6 e2m3 B operands: in
// the block-scaled 16x16x128 MFMA with 6-bit B values, lane (n, kb) supplies the 32
// k positions of k-block kb for token column n, packed in 6 dwords, and the scale of
// that block.
struct Unit6 {
    i32x6 hi[4], lo[4];
    uint32_t ehi, elo;  // byte q: scale codes of product q's hi and lo operands
};

// D += A(fp4, 16 x 128) * B(fp6 e2m3, 128 x 16) * 2^(scale_b - 127), scale_b = byte SEL of sc.
template <int SEL>
__device__ __forceinline__ f32x4 mfma_f4f6(u32x4 a, i32x6 b, f32x4 c, uint32_t sc) {
    const i32x8 a8 = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const i32x8 b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, 4, 5, -1, -1);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 2, 0, 127, SEL, (int)sc);
}

template <int SEL>
__device__ __forceinline__ f32x4 mfma_f4f6k(u32x4 a, i32x6 b, f32x4 c, uint32_t sc, uint32_t ka) {
    const i32x8 a8 = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const i32x8 b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, 4, 5, -1, -1);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 2, 0, (int)ka, SEL, (int)sc);
}

// Encodes, for lane (m, G), product q of unit u: the 32 columns 512 u + 128 G + 32 q
// of token m (the LDS chunks c0 .. c0 + 3, c0 = 64 u + 16 G + 4 q); see
// encode_fp6_block for the encoding.
__device__ __forceinline__ void encode6(const char* smem, uint32_t rowb, int c0, int m,
                                        uint32_t kone_lo, uint32_t kone_hi, i32x6& h, i32x6& l,
                                        uint32_t& code_hi, uint32_t& code_lo) {
    uint32_t R[16];  // R[p]: columns 2p (low half) and 2p + 1 (high half)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4 v = *(const u32x4*)(smem + xslot(m, c0 + i, rowb));
        R[4 * i] = v.x;
        R[4 * i + 1] = v.y;
        R[4 * i + 2] = v.z;
        R[4 * i + 3] = v.w;
    }
    encode_fp6_block(R, kone_lo, kone_hi, h, l, code_hi, code_lo);
}

__device__ __forceinline__ void fused_encode6(const char* smem, uint32_t rowb, int u, int lane,
                                              uint32_t kone_lo, uint32_t kone_hi, Unit6& X) {
    const int m = lane & 15, G = lane >> 4;
    X.ehi = 0u;
    X.elo = 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t ch, cl;
        encode6(smem, rowb, 64 * u + 16 * G + 4 * q, m, kone_lo, kone_hi, X.hi[q], X.lo[q], ch, cl);
        X.ehi |= ch << (8 * q);
        X.elo |= cl << (8 * q);
        __builtin_amdgcn_sched_barrier(0);  // one product at a time: bounded register use
    }
}

// Copies 1 KB pieces j0, j0 + step, ... (n of them, n <= NMAX) of every token row
// (piece j: columns [512 j, +512)) into LDS; all arguments wave-uniform.  The rows are
// taken in an order rotated by the block's place on its XCD, so the blocks of one XCD,
// which all copy the same activations, do not queue on the same lines at once.
template <int NMAX>
__device__ __forceinline__ void fused_stage(char* smem, uint32_t rowb, __amdgpu_buffer_rsrc_t xr,
                                            int T, int64_t d_in, int j0, int n, int step,
                                            int lane) {
    const int rot = (int)((blockIdx.x >> 3) & 15);
#pragma unroll
    for (int tt = 0; tt < kDecodeMaxT; ++tt) {
        const int t = (tt + rot) & 15;
        const int cl = (lane & 48) | ((lane & 15) ^ t);
#pragma unroll
        for (int k = 0; k < NMAX; ++k) {
            if (k < n) {  // uniform
                const int j = j0 + step * k;
                const int c = 64 * j + cl;
                const bool ok = t < T && (int64_t)c * 8 < d_in;
                lds_copy16(xr, smem + t * rowb + 1024 * j,
                           ok ? (uint32_t)(((int64_t)t * d_in + 8 * c) * 2) : kOOB);
            }
        }
    }
}

template <int MODE>
__global__ void __launch_bounds__(64 * kFusedWaves)
k_decode_fused(const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, int T, int U,
               int64_t d_in, int dpad, const uint16_t* __restrict__ w, int64_t d_out,
               const uint64_t* __restrict__ signs, uint64_t sstride, const void* __restrict__ scales,
               int sdtype, int64_t per_user, void* __restrict__ y, int ydtype,
               uint32_t* __restrict__ status) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
    const int m = lane & 15, g = lane >> 4;
    const uint32_t rowb = 2u * (uint32_t)dpad;
    const int64_t r0 = (int64_t)blockIdx.x * 16;
    const int64_t rowA = r0 + m < d_out ? r0 + m : d_out - 1;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint64_t)T * (uint64_t)d_in * 2);
    f32x4* red = (f32x4*)smem;  // after the products: [12 waves][64] partial tiles

    if (wv < kFusedBaseWaves) {
        // ---- base: wave wv takes the steps (32 columns) of columns [wv Kb, (wv+1) Kb),
        // Kb = dpad / 4, in order, into one accumulator; the partition does not depend on
        // the batch's users.  Ring of 16 W loads; the tokens come from LDS.
        const int spw = dpad / 128;  // steps per base wave (a multiple of 4)
        const int st0 = wv * spw;
        const int nsteps = (int)(d_in / 32);
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint64_t)d_out * (uint64_t)d_in * 2);
        const uint32_t woff = (uint32_t)((rowA * d_in + 8 * g) * 2);
        constexpr int R = 16;
        auto load = [&](int i) {
            const int st = st0 + i;
            const bool ok = i < spw && st < nsteps;
            return buf_load16(wr, ok ? woff + (uint32_t)(st * 64) : kOOB);
        };
        u32x4 ring[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            ring[r] = load(r);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_barrier();  // the tokens are in LDS
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        // token operand of step i (zero past the wave's steps), read one step ahead
        auto tok = [&](int i) {
            u32x4 b = {0u, 0u, 0u, 0u};
            if (i < spw)  // uniform
                b = *(const u32x4*)(smem + xslot(m, 4 * (st0 + i) + g, rowb));
            return b;
        };
        u32x4 bnext = tok(0);
        int i0 = 0;
        do {  // spw > 0: the ring is always consumed, so its loads stay above the barrier
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = i0 + r;
                const u32x4 b = bnext;
                bnext = tok(i + 1);
                acc = mfma_bf16(ring[r], b, acc);
                ring[r] = load(i + R);
                __builtin_amdgcn_sched_barrier(0);
            }
            i0 += R;
        } while (i0 < spw);
        // the token rows are no longer read: the partial tiles go to LDS
        __syncthreads();
        red[wv * 64 + lane] = acc;
        __syncthreads();
        return;
    }

    // ---- delta: 512-column units u = wd, wd + 8, ...; every user of the batch
    __builtin_amdgcn_s_setprio(3);
    const int wd = wv - kFusedBaseWaves;
    const int nunit = dpad / 512;
    const int nuw = wd < nunit ? (nunit - wd + kFusedDeltaWaves - 1) / kFusedDeltaWaves : 0;
    // the batch's user ids (scalar loads: their wait does not wait for the copies below)
    int sid[kDecodeMaxT];
#pragma unroll
    for (int j = 0; j < kDecodeMaxT; ++j) sid[j] = ids[j < T ? j : T - 1];  // in bounds
    fused_stage<(kFusedMaxPieces + kFusedDeltaWaves - 1) / kFusedDeltaWaves>(
        smem, rowb, xr, T, d_in, wd, nuw, kFusedDeltaWaves, lane);

    int uid = -1;
#pragma unroll
    for (int j = 0; j < kDecodeMaxT; ++j) uid = lane == j && j < T ? sid[j] : uid;
    // the users in order of first appearance (lane j of utab: the j-th)
    const bool valid = lane < T && uid >= 0 && uid < U;
    bool dup = false;
#pragma unroll
    for (int j = 0; j < kDecodeMaxT; ++j)
        dup |= (j < lane) & (__builtin_amdgcn_readlane(uid, j) == uid);
    const uint64_t fmask = __ballot(valid && !dup);
    const int nseg = __popcll(fmask);
    int utab = 0;
    {
        uint64_t mk = fmask;
        for (int j = 0; j < nseg; ++j) {
            const int src = __ffsll((unsigned long long)mk) - 1;
            mk &= mk - 1;
            const int us = __builtin_amdgcn_readlane(uid, src);
            if (lane == j) utab = us;
        }
    }
    const int tok_user = __shfl(valid ? uid : -1, m);  // user of this lane's token column
    uint32_t sraw[4] = {0u, 0u, 0u, 0u};  // epilogue wave: the scales of its outputs (bits)
    if (wd == 0) {
        if (blockIdx.x == 0) {
            const bool bad = lane < T && !valid && uid != -1;
            const bool anybad = __ballot(bad) != 0ull;
            if (lane == 0) status[0] = anybad ? ST_USER_ID : 0u;
        }
    }
    constexpr int RB = 8;
    const int nsegR = (nseg + RB - 1) / RB * RB;  // users padded: item (k, j) sits in slot j % RB
    const int64_t bank_row = d_in / 8;
    const uint64_t user_bytes = (uint64_t)d_out * (uint64_t)bank_row;
    const uint32_t brow = (uint32_t)(rowA * bank_row + 16 * g);
    uint32_t kmask, kone;  // operand constants in registers (gfx9 VOP3 takes no literal)
    asm volatile("v_mov_b32 %0, 0x88888888" : "=v"(kmask));
    asm volatile("s_mov_b32 %0, 0x22222222" : "=s"(kone));
    uint32_t kb_lo, kb_hi;  // the bf16 pairs (1, 0) and (0, 1), in registers as well
    asm volatile("v_mov_b32 %0, 0x3f80" : "=v"(kb_lo));
    asm volatile("v_mov_b32 %0, 0x3f800000" : "=v"(kb_hi));
    // this lane's offset in a user's bank for the wave's units (two at most)
    uint32_t uoff[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int u = wd + kFusedDeltaWaves * k;
        uoff[k] = (int64_t)u * 512 + 128 * g < d_in ? brow + (uint32_t)(u * 64) : kOOB;
    }
    int lk = 0, lj = 0;  // unit (of this wave) and user slot of the next load
    // 16 bytes of user lj's row: columns [512u + 128g, +128) (a word for each of the unit's
    // four products); always issued (a zero load for padding and past the end) so every
    // wait is exact
    auto load_bits = [&]() {
        const bool ok = lk < nuw && lj < nseg;  // uniform
        const int usr = __builtin_amdgcn_readlane(utab, ok ? lj : 0);
        const __amdgpu_buffer_rsrc_t br =
            make_rsrc((const char*)signs + (uint64_t)(uint32_t)usr * sstride, user_bytes);
        const u32x4 v = buf_load16(br, ok ? (lk == 0 ? uoff[0] : uoff[1]) : kOOB);
        if (++lj == nsegR) {
            lj = 0;
            ++lk;
        }
        return v;
    };
    u32x4 ring[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        ring[r] = load_bits();
        __builtin_amdgcn_sched_barrier(0);
    }
    BD_WAIT_VMCNT(RB);  // this wave's token copies have landed (the ring loads are younger)
    __builtin_amdgcn_s_barrier();  // and every delta wave's
    if (wd == 0 && tok_user >= 0 && m < T) {  // the epilogue's scales, used at the end
        const int64_t o = r0 + 4 * g;
        const int64_t s0 = (int64_t)tok_user * per_user;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t i =
                s0 + (MODE == BD_SCALE_MATRIX ? 0 : (o + e < d_out ? o + e : d_out - 1));
            sraw[e] = sdtype == BD_F16 ? (uint32_t)((const uint16_t*)scales)[i]
                                       : ((const uint32_t*)scales)[i];
        }
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    Unit6 X;
    // The fp4 operand of product q from word wq of a ring slot (word q of this lane's
    // load is k-group g of product q).  `one` is 0x22222222 (the magnitude 1.0) for a
    // user of the batch and 0 for a padding slot, whose load reads zeros: its operands
    // are then +0.0 and its products exactly 0.
    auto expand = [&](uint32_t wq, uint32_t one) {
        u32x4 a;
        a.x = ((wq << 3) & kmask) | one;
        a.y = ((wq << 2) & kmask) | one;
        a.z = ((wq << 1) & kmask) | one;
        a.w = (wq & kmask) | one;
        return a;
    };
    // Software pipeline: while the eight products of user j run (from Ac), the operands
    // of user j + 1 are expanded from the next ring slot into the other buffer (An),
    // which no product in flight reads, and that slot is refilled.  The buffers
    // alternate between users.  Products alternate between two accumulators, so two
    // consecutive ones never wait for each other.  At a unit's last user the next slot
    // (the next unit's first user) waits for the next unit.
    u32x4 A0[4], A1[4];
    f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
    int k_cur = 0;
    auto step = [&](int j, int r, bool next, u32x4* Ac, u32x4* An) {
        const int usr = __builtin_amdgcn_readlane(utab, j < nseg ? j : 0);
        const bool mine = k_cur < nuw && j < nseg && tok_user == usr;
        const uint32_t sh = mine ? X.ehi : 0u, sl = mine ? X.elo : 0u;
        const uint32_t onen = k_cur < nuw && j + 1 < nseg ? kone : 0u;
        const u32x4 Dn = ring[(r + 1) % RB];
        // (sched_barrier pins the order: two products, then one operand of the next
        // user, four times)
        acc = mfma_f4f6<0>(Ac[0], X.hi[0], acc, sh);
        acc2 = mfma_f4f6<0>(Ac[0], X.lo[0], acc2, sl);
        __builtin_amdgcn_sched_barrier(0);
        if (next) An[0] = expand(Dn[0], onen);
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma_f4f6<1>(Ac[1], X.hi[1], acc, sh);
        acc2 = mfma_f4f6<1>(Ac[1], X.lo[1], acc2, sl);
        __builtin_amdgcn_sched_barrier(0);
        if (next) An[1] = expand(Dn[1], onen);
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma_f4f6<2>(Ac[2], X.hi[2], acc, sh);
        acc2 = mfma_f4f6<2>(Ac[2], X.lo[2], acc2, sl);
        __builtin_amdgcn_sched_barrier(0);
        if (next) An[2] = expand(Dn[2], onen);
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma_f4f6<3>(Ac[3], X.hi[3], acc, sh);
        acc2 = mfma_f4f6<3>(Ac[3], X.lo[3], acc2, sl);
        __builtin_amdgcn_sched_barrier(0);
        if (next) {
            An[3] = expand(Dn[3], onen);
            ring[(r + 1) % RB] = load_bits();
        }
        // Ac stays allocated to the end of the step, so An never reuses the registers of
        // an operand that a product in flight still reads (that would stall the expansion)
        asm volatile("" ::"v"(Ac[0]), "v"(Ac[1]), "v"(Ac[2]), "v"(Ac[3]));
        __builtin_amdgcn_sched_barrier(0);
    };
    // do-while loops: every ring slot is consumed on every path, so no load is sunk
    // below a wait
    do {
        // encode this unit's tokens while its first users' rows are in flight
        if (k_cur < nuw && nseg > 0)
            fused_encode6(smem, rowb, wd + kFusedDeltaWaves * k_cur, lane, kb_lo, kb_hi, X);
        // the unit's first user: ring slot 0 (each unit takes nsegR slots, a multiple of RB)
        {
            const uint32_t one0 = k_cur < nuw && nseg > 0 ? kone : 0u;
            const u32x4 D0 = ring[0];
#pragma unroll
            for (int q = 0; q < 4; ++q) A0[q] = expand(D0[q], one0);
            ring[0] = load_bits();
        }
        int j0 = 0;
        do {
#pragma unroll
            for (int r = 0; r + 1 < RB; ++r) {  // RB is even: user r reads A0 for even r
                if (r & 1) step(j0 + r, r, true, A1, A0);
                else step(j0 + r, r, true, A0, A1);
            }
            if (j0 + RB < nsegR) step(j0 + RB - 1, RB - 1, true, A1, A0);  // uniform
            else step(j0 + RB - 1, RB - 1, false, A1, A0);
            j0 += RB;
        } while (j0 < nsegR);
        ++k_cur;
    } while (k_cur < nuw);
    acc += acc2;
    // the ring's last loads (past the end) land: no load of this wave stays in flight,
    // so the base waves' code, which the compiler may lay out after a join with this
    // path, starts without waits for it
    BD_WAIT_VMCNT(0);

    // ---- reduction: the token rows are no longer read; partial tiles go to LDS
    __syncthreads();
    red[wv * 64 + lane] = acc;
    __syncthreads();
    if (wd != 0) return;  // the first delta wave holds the factors
    f32x4 vb = {0.f, 0.f, 0.f, 0.f}, vd = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < kFusedBaseWaves; ++q) vb += red[q * 64 + lane];
    for (int q = kFusedBaseWaves; q < kFusedWaves; ++q) vd += red[q * 64 + lane];
    if (m >= T) return;
    const int64_t o = r0 + 4 * g;
    f32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // -scale (the fp4 operands carry -sign); 0 for tokens without a valid user
        const float f = tok_user < 0 ? 0.f
                        : sdtype == BD_F16 ? -f16_to_f32((uint16_t)sraw[e])
                                           : -__uint_as_float(sraw[e]);
        out[e] = vb[e] + f * vd[e];
    }
    if (ydtype == BD_F32) {
        float* dst = (float*)y + (int64_t)m * d_out + o;
        if (o + 3 < d_out && (d_out & 3) == 0) {
            *(f32x4*)dst = out;
        } else {
            for (int e = 0; e < 4; ++e)
                if (o + e < d_out) dst[e] = out[e];
        }
    } else {
        uint16_t* dst = (uint16_t*)y + (int64_t)m * d_out + o;
        if (o + 3 < d_out && (d_out & 3) == 0) {
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16(out[0]) | ((uint32_t)f32_to_bf16(out[1]) << 16);
            pk.y = (uint32_t)f32_to_bf16(out[2]) | ((uint32_t)f32_to_bf16(out[3]) << 16);
            *(uint2*)dst = pk;
        } else {
            for (int e = 0; e < 4; ++e)
                if (o + e < d_out) dst[e] = f32_to_bf16(out[e]);
        }
    }
}

// ------------------------------------------------------- one wave per unit
// One launch for decode batches whose rows have at most 512 * kUnitWaves columns
// (bf16 X, at most 16 tokens, MATRIX or ROW scales).  Wave w of a block owns the
// 512-column unit w of the block's 16 output rows, for the base and the delta
// product alike, so no wave waits for another before the final sum.
//  - Tokens: the wave copies its unit of every token row into its own 16 KB of
//    LDS (buffer loads that write LDS directly; rows in an order rotated by the
//    block's place on its XCD, so the blocks of one XCD, which all read the same
//    tokens, do not queue on the same lines at once) and encodes them from there
//    as soon as they land (fp6 hi/lo, the operands of k_decode_fused).
//  - One stream per wave: the sign rows of the batch's users in order of first
//    appearance (16 bytes of 16 rows per user, padded to a multiple of 8 users
//    with empty loads), then the unit's 16 steps of W_base rows, through an
//    8-slot register ring.  A CU keeps about 64 loads in flight, which is what 8
//    waves x 8 slots issue (16 slots, 128 loads, made every step several times
//    slower; 4 waves of two units with 16 slots each drew about 40% less memory
//    throughput per CU); a wave refills a slot as it consumes it, so its encoding
//    and its products overlap the CU's stream.  The two waves of a SIMD do not
//    progress evenly (whichever has the issue priority finishes about 4 us
//    earlier), which bounds the kernel rather than the memory system.
//  - Delta: for each user, eight block-scaled MFMAs 16x16x128 (fp4 signs x fp6
//    tokens), while the next slot's signs are expanded (as in k_decode_fused).
//  - Base: one bf16 MFMA 16x16x32 per step, the tokens read back from LDS.
// The partial tiles are summed in LDS in wave order, as in k_decode_fused, so the
// base sum does not depend on the users and y repeats bit for bit.
constexpr int kUnitWaves = 8;
constexpr int kUnitRing = 8;

// Q8: the base weight as INT8 rows with one fp32 scale per row (wq[o][i] * wscale[o]):
// half the base bytes.  A ring item then carries 16 columns per lane, two MFMA steps,
// whose codes are widened to bf16 exactly (|q| <= 127 has 7 significant bits); the
// base sum is multiplied by the row's scale in the epilogue.
template <int MODE, bool Q8>
__global__ void __launch_bounds__(64 * kUnitWaves)
k_decode_unit(const uint16_t* __restrict__ x, const int32_t* __restrict__ ids, int T, int U,
              int64_t d_in, const void* __restrict__ w, const float* __restrict__ wscale,
              int64_t d_out, const uint64_t* __restrict__ signs, uint64_t sstride,
              const void* __restrict__ scales, int sdtype, int64_t per_user, void* __restrict__ y,
              int ydtype,
              uint32_t* __restrict__ status) {
    __shared__ f32x4 red[2 * kUnitWaves * 64];  // base then delta partial tiles, wave order
    __shared__ __attribute__((aligned(16))) char xlds[kUnitWaves * 16384];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
    const int m = lane & 15, g = lane >> 4;
    const int64_t r0 = (int64_t)blockIdx.x * 16;
    const int64_t rowA = r0 + m < d_out ? r0 + m : d_out - 1;
    char* xs = xlds + wv * 16384;  // token t's unit at t * 1024; chunk c at slot xslot(t, c, 1024)

    // the batch's user ids (scalar loads, in flight beside the copies)
    int sid[kDecodeMaxT];
#pragma unroll
    for (int j = 0; j < kDecodeMaxT; ++j) sid[j] = ids[j < T ? j : T - 1];  // in bounds

    // ---- tokens of this wave's unit into LDS
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint64_t)T * (uint64_t)d_in * 2);
    {
        const int rot = (int)((blockIdx.x >> 3) & 15);
#pragma unroll
        for (int tt = 0; tt < kDecodeMaxT; ++tt) {
            const int t = (tt + rot) & 15;
            const int cl = (lane & 48) | ((lane & 15) ^ t);  // the chunk that belongs at slot lane
            const int64_t col = (int64_t)512 * wv + 8 * cl;
            const bool ok = t < T && col < d_in;
            lds_copy16(xr, xs + t * 1024, ok ? (uint32_t)(((int64_t)t * d_in + col) * 2) : kOOB);
        }
    }

    // ---- group the batch by user (every wave for itself): lane j of utab holds the
    // j-th distinct valid user in order of first appearance
    int uid = -1;
#pragma unroll
    for (int j = 0; j < kDecodeMaxT; ++j) uid = lane == j && j < T ? sid[j] : uid;
    const bool valid = lane < T && uid >= 0 && uid < U;
    bool dup = false;
#pragma unroll
    for (int j = 0; j < kDecodeMaxT; ++j)
        dup |= (j < lane) & (__builtin_amdgcn_readlane(uid, j) == uid);
    const uint64_t fmask = __ballot(valid && !dup);
    const int nseg = __popcll(fmask);
    int utab = 0;
    {
        uint64_t mk = fmask;
        for (int j = 0; j < nseg; ++j) {
            const int src = __ffsll((unsigned long long)mk) - 1;
            mk &= mk - 1;
            const int us = __builtin_amdgcn_readlane(uid, src);
            if (lane == j) utab = us;
        }
    }
    const int tok_user = __shfl(valid ? uid : -1, m);  // user of this lane's token column
    if (wv == 0 && blockIdx.x == 0) {
        const bool bad = lane < T && !valid && uid != -1;
        const bool anybad = __ballot(bad) != 0ull;
        if (lane == 0) status[0] = anybad ? ST_USER_ID : 0u;
    }

    // ---- the stream: item i < nsegR is the sign rows of user i (empty past nseg), item
    // nsegR + s the W_base step s (unit columns 32 s .. + 31; empty past 16)
    const int nsegR = (nseg + kUnitRing - 1) / kUnitRing * kUnitRing;
    const int64_t bank_row = d_in / 8;
    const uint64_t user_bytes = (uint64_t)d_out * (uint64_t)bank_row;
    constexpr int kWBytes = Q8 ? 1 : 2;  // bytes per base weight
    constexpr int kWItems = Q8 ? 8 : 16;  // base ring items per unit
    const uint64_t w_bytes = (uint64_t)d_out * (uint64_t)d_in * kWBytes;
    // lane (m, g): sign bytes of row rowA for columns 512 w + 128 g .. + 127 (word q: k-group
    // g of product q); W_base columns 512 w + 32 s + 8 g .. + 7 of row rowA (Q8: the INT8
    // codes of columns 512 w + 64 s + 16 g .. + 15, steps 2 s and 2 s + 1)
    const uint32_t soff = (int64_t)512 * wv + 128 * g < d_in
                              ? (uint32_t)(rowA * bank_row + 64 * wv + 16 * g)
                              : kOOB;
    const int64_t c0 = (int64_t)512 * wv + (Q8 ? 16 : 8) * g;
    const uint32_t woff = (uint32_t)((rowA * d_in + c0) * kWBytes);
    // (branch-free: a branch here splits the loop body into blocks, and the compiler then
    // gathers the products of a whole iteration at its end)
    const uint64_t wbase = (uint64_t)(uintptr_t)w;
    auto load_item = [&](int i) __attribute__((always_inline)) {
        const uint64_t msk = 0ull - (uint64_t)(i < nsegR);  // uniform: all ones for sign rows
        const int s = i - nsegR;
        const int usr = __builtin_amdgcn_readlane(utab, i < nseg ? i : 0);
        const uint64_t sbase = (uint64_t)(uintptr_t)signs + (uint64_t)(uint32_t)usr * sstride;
        const uint64_t base = wbase + ((sbase - wbase) & msk);
        const uint64_t bytes = w_bytes + ((user_bytes - w_bytes) & msk);
        const uint32_t so = i < nseg ? soff : kOOB;
        const bool okw = ((uint32_t)s < (uint32_t)kWItems) & (c0 + (Q8 ? 64 : 32) * s < d_in);
        const uint32_t wo = okw ? woff + 64u * (uint32_t)s : kOOB;  // no short-circuit branch
        const uint32_t off = wo + ((so - wo) & (uint32_t)msk);
        return buf_load16(make_rsrc((const void*)(uintptr_t)base, bytes), off);
    };
    u32x4 ring[kUnitRing];
#pragma unroll
    for (int r = 0; r < kUnitRing; ++r) {
        ring[r] = load_item(r);
        __builtin_amdgcn_sched_barrier(0);
    }
    BD_WAIT_VMCNT(kUnitRing);  // this wave's token copies have landed (the ring is younger)
    uint32_t sraw[4] = {0u, 0u, 0u, 0u};  // wave 0: the scales of its outputs (bits)
    float wsc[4] = {1.f, 1.f, 1.f, 1.f};  // wave 0, Q8: the rows' base scales
    if (Q8 && wv == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t o = r0 + 4 * g + e;
            wsc[e] = wscale[o < d_out ? o : d_out - 1];
        }
    }
    if (wv == 0 && tok_user >= 0 && m < T) {
        const int64_t o = r0 + 4 * g;
        const int64_t s0 = (int64_t)tok_user * per_user;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t i =
                s0 + (MODE == BD_SCALE_MATRIX ? 0 : (o + e < d_out ? o + e : d_out - 1));
            sraw[e] = sdtype == BD_F16 ? (uint32_t)((const uint16_t*)scales)[i]
                                       : ((const uint32_t*)scales)[i];
        }
    }

    // ---- encode the unit's tokens for the delta products (from LDS)
    uint32_t kb_lo, kb_hi;  // the bf16 pairs (1, 0) and (0, 1), in registers
    asm volatile("v_mov_b32 %0, 0x3f80" : "=v"(kb_lo));
    asm volatile("v_mov_b32 %0, 0x3f800000" : "=v"(kb_hi));
    Unit6 X6;
    if (nseg > 0) fused_encode6(xs, 1024u, 0, lane, kb_lo, kb_hi, X6);

    // ---- delta products, user by user (the k_decode_fused pipeline)
    uint32_t kmask, kone;  // operand constants in registers (gfx9 VOP3 takes no literal)
    asm volatile("v_mov_b32 %0, 0x88888888" : "=v"(kmask));
    asm volatile("s_mov_b32 %0, 0x22222222" : "=s"(kone));
    uint32_t ka;  // the A operands' block scale (2^0), kept in one register
    asm volatile("v_mov_b32 %0, 0x7f" : "=v"(ka));
    auto expand = [&](uint32_t wq, uint32_t one) {
        u32x4 a;
        a.x = ((wq << 3) & kmask) | one;
        a.y = ((wq << 2) & kmask) | one;
        a.z = ((wq << 1) & kmask) | one;
        a.w = (wq & kmask) | one;
        return a;
    };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
    u32x4 A0[4], A1[4];
    // user j's products from Ac while the next slot (user j + 1; zeros for padding) is
    // expanded into An and refilled with item j + 1 + kUnitRing
    auto step = [&](int j, int r, bool next, u32x4* Ac, u32x4* An)
                    __attribute__((always_inline)) {
        const int usr = __builtin_amdgcn_readlane(utab, j < nseg ? j : 0);
        const bool mine = j < nseg && tok_user == usr;
        const uint32_t sh = mine ? X6.ehi : 0u, sl = mine ? X6.elo : 0u;
        const uint32_t onen = j + 1 < nseg ? kone : 0u;
        const u32x4 Dn = ring[(r + 1) % kUnitRing];
        acc = mfma_f4f6k<0>(Ac[0], X6.hi[0], acc, sh, ka);
        acc2 = mfma_f4f6k<0>(Ac[0], X6.lo[0], acc2, sl, ka);
        __builtin_amdgcn_sched_barrier(0);
        if (next) An[0] = expand(Dn[0], onen);
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma_f4f6k<1>(Ac[1], X6.hi[1], acc, sh, ka);
        acc2 = mfma_f4f6k<1>(Ac[1], X6.lo[1], acc2, sl, ka);
        __builtin_amdgcn_sched_barrier(0);
        if (next) An[1] = expand(Dn[1], onen);
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma_f4f6k<2>(Ac[2], X6.hi[2], acc, sh, ka);
        acc2 = mfma_f4f6k<2>(Ac[2], X6.lo[2], acc2, sl, ka);
        __builtin_amdgcn_sched_barrier(0);
        if (next) An[2] = expand(Dn[2], onen);
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma_f4f6k<3>(Ac[3], X6.hi[3], acc, sh, ka);
        acc2 = mfma_f4f6k<3>(Ac[3], X6.lo[3], acc2, sl, ka);
        __builtin_amdgcn_sched_barrier(0);
        if (next) {
            An[3] = expand(Dn[3], onen);
            ring[(r + 1) % kUnitRing] = load_item(j + 1 + kUnitRing);
        }
        // Ac stays allocated to the end of the step: no expansion reuses the registers
        // of an operand that a product in flight still reads
        asm volatile("" ::"v"(Ac[0]), "v"(Ac[1]), "v"(Ac[2]), "v"(Ac[3]));
        __builtin_amdgcn_sched_barrier(0);
    };
    if (nsegR > 0) {  // uniform
        {
            const uint32_t one0 = nseg > 0 ? kone : 0u;
            const u32x4 D0 = ring[0];
#pragma unroll
            for (int q = 0; q < 4; ++q) A0[q] = expand(D0[q], one0);
            ring[0] = load_item(kUnitRing);
        }
        int j0 = 0;
        do {  // every slot is consumed at one fixed point on every path
#pragma unroll
            for (int r = 0; r + 1 < kUnitRing; ++r) {
                if (r & 1) step(j0 + r, r, true, A1, A0);
                else step(j0 + r, r, true, A0, A1);
            }
            if (j0 + kUnitRing < nsegR) step(j0 + kUnitRing - 1, kUnitRing - 1, true, A1, A0);
            else step(j0 + kUnitRing - 1, kUnitRing - 1, false, A1, A0);
            j0 += kUnitRing;
        } while (j0 < nsegR);
    }
    acc += acc2;

    // ---- base product: item nsegR + s in slot s % kUnitRing (nsegR is a multiple of it)
    f32x4 accb = {0.f, 0.f, 0.f, 0.f};
    auto tok = [&](int s) {  // B operand of step s: token m, columns 32 s + 8 g .. + 7
        return *(const u32x4*)(xs + xslot(m, 4 * s + g, 1024u));
    };
    if (Q8) {
        // item s: lane (m, g) holds the codes of columns 64 s + 16 g .. + 15 of row m; the
        // tokens of the same columns are LDS chunks 8 s + 2 g and 8 s + 2 g + 1
        // four codes -> two dwords of bf16 pairs (the upper halves of their exact fp32 values)
        auto widen = [&](uint32_t wd, uint32_t* out) {
            const float f0 = (float)(int8_t)(wd & 0xFFu), f1 = (float)(int8_t)((wd >> 8) & 0xFFu);
            const float f2 = (float)(int8_t)((wd >> 16) & 0xFFu), f3 = (float)(int8_t)(wd >> 24);
            out[0] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
            out[1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
        };
#pragma unroll
        for (int s = 0; s < kWItems; ++s) {
            const u32x4 b0 = *(const u32x4*)(xs + xslot(m, 8 * s + 2 * g, 1024u));
            const u32x4 b1 = *(const u32x4*)(xs + xslot(m, 8 * s + 2 * g + 1, 1024u));
            const u32x4 wq = ring[s % kUnitRing];
            uint32_t v[8];
            widen(wq.x, v);
            widen(wq.y, v + 2);
            widen(wq.z, v + 4);
            widen(wq.w, v + 6);
            const u32x4 a0 = {v[0], v[1], v[2], v[3]}, a1 = {v[4], v[5], v[6], v[7]};
            accb = mfma_bf16(a0, b0, accb);
            accb = mfma_bf16(a1, b1, accb);
            ring[s % kUnitRing] = load_item(nsegR + s + kUnitRing);  // empty past the unit
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        u32x4 bnext = tok(0);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const u32x4 b = bnext;
            if (s + 1 < 16) bnext = tok(s + 1);
            accb = mfma_bf16(ring[s % kUnitRing], b, accb);
            ring[s % kUnitRing] = load_item(nsegR + s + kUnitRing);  // empty past step 15
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    BD_WAIT_VMCNT(0);  // the empty loads past the end have landed

    // ---- reduction in wave order
    red[wv * 64 + lane] = accb;
    red[(kUnitWaves + wv) * 64 + lane] = acc;
    __syncthreads();
    if (wv != 0) return;  // wave 0 holds the factors
    f32x4 vb = {0.f, 0.f, 0.f, 0.f}, vd = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < kUnitWaves; ++q) vb += red[q * 64 + lane];
    for (int q = 0; q < kUnitWaves; ++q) vd += red[(kUnitWaves + q) * 64 + lane];
    if (m >= T) return;
    const int64_t o = r0 + 4 * g;
    f32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // -scale (the fp4 operands carry -sign); 0 for tokens without a valid user
        const float f = tok_user < 0 ? 0.f
                        : sdtype == BD_F16 ? -f16_to_f32((uint16_t)sraw[e])
                                           : -__uint_as_float(sraw[e]);
        out[e] = (Q8 ? wsc[e] * vb[e] : vb[e]) + f * vd[e];
    }
    if (ydtype == BD_F32) {
        float* dst = (float*)y + (int64_t)m * d_out + o;
        if (o + 3 < d_out && (d_out & 3) == 0) {
            *(f32x4*)dst = out;
        } else {
            for (int e = 0; e < 4; ++e)
                if (o + e < d_out) dst[e] = out[e];
        }
    } else {
        uint16_t* dst = (uint16_t*)y + (int64_t)m * d_out + o;
        if (o + 3 < d_out && (d_out & 3) == 0) {
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16(out[0]) | ((uint32_t)f32_to_bf16(out[1]) << 16);
            pk.y = (uint32_t)f32_to_bf16(out[2]) | ((uint32_t)f32_to_bf16(out[3]) << 16);
            *(uint2*)dst = pk;
        } else {
            for (int e = 0; e < 4; ++e)
                if (o + e < d_out) dst[e] = f32_to_bf16(out[e]);
        }
    }
}

bool decode_path_supported(int xdtype, int64_t T, int mode) {
    return xdtype == BD_BF16 && T >= 1 && T <= kDecodeMaxT && mode != BD_SCALE_GROUP;
}

void make_decode_plan(int64_t T, int64_t d_in, DecodePlan* pl) {
    DecodePlan q;
    q.T = T;
    q.d_in = d_in;
    q.dpad = (d_in + 511) / 512 * 512;
    size_t off = 0;
    q.off_meta = off;
    off += kAlign;
    q.off_perm = off;
    off += align_up(sizeof(int32_t) * kDecodeMaxT);
    q.off_suser = off;
    off += align_up(sizeof(int32_t) * kDecodeMaxT);
    q.off_seg = off;
    off += align_up(sizeof(int4) * kDecodeMaxT);
    q.off_xs = off;
    off += align_up((size_t)(d_in / 32) * 1024);
    q.off_x8 = off;
    off += align_up((size_t)(q.dpad / 128) * 4096);
    q.off_e8 = off;
    off += align_up((size_t)(q.dpad / 512) * 256);
    q.total = off;
    *pl = q;
}

hipError_t launch_decode_prep(const DecodePlan& pl, int U, const DeltaPlan& dp, const void* x,
                              const int32_t* ids, const void* scales, char* ws, hipStream_t s) {
    const int64_t work = kDecodeMaxT * (pl.dpad / 32);
    int64_t gp = (work + 255) / 256;
    gp = gp < 1 ? 1 : (gp > 1024 ? 1024 : gp);
    hipLaunchKernelGGL(k_decode_prep, dim3((unsigned)gp), dim3(256), 0, s, (const uint16_t*)x, ids,
                       (int)pl.T, U, pl.d_in, pl.dpad, dp.mode == BD_SCALE_COL ? 1 : 0, scales,
                       dp.sdtype, scale_stride(dp), (uint32_t*)(ws + pl.off_meta),
                       (int32_t*)(ws + pl.off_perm), (int32_t*)(ws + pl.off_suser),
                       (int4*)(ws + pl.off_seg), (uint16_t*)(ws + pl.off_xs),
                       (uint8_t*)(ws + pl.off_x8), (uint8_t*)(ws + pl.off_e8));
    return hipGetLastError();
}

hipError_t launch_decode_main(const DecodePlan& pl, const DeltaPlan& dp, const void* x,
                              const void* wb, const uint64_t* signs, const void* scales, void* y,
                              int ydtype, const char* ws, hipStream_t s) {
    const dim3 grid((unsigned)((dp.d_out + 15) / 16));
#define BD_DECODE(MODE)                                                                           \
    hipLaunchKernelGGL(k_decode<MODE>, grid, dim3(64 * kDecodeWaves), 0, s, (const uint16_t*)x,   \
                       (int)pl.T, pl.d_in, pl.dpad, (const uint16_t*)wb, dp.d_out, signs,          \
                       sign_stride(dp.sstride, dp.d_out, pl.d_in), scales, dp.sdtype,              \
                       scale_stride(dp), (const uint32_t*)(ws + pl.off_meta),                      \
                       (const int32_t*)(ws + pl.off_perm), (const int32_t*)(ws + pl.off_suser),    \
                       (const int4*)(ws + pl.off_seg), (const uint16_t*)(ws + pl.off_xs),          \
                       (const uint8_t*)(ws + pl.off_x8), (const uint8_t*)(ws + pl.off_e8), y,      \
                       ydtype)
    switch (dp.mode) {
        case BD_SCALE_MATRIX: BD_DECODE(BD_SCALE_MATRIX); break;
        case BD_SCALE_ROW: BD_DECODE(BD_SCALE_ROW); break;
        default: BD_DECODE(BD_SCALE_COL); break;
    }
#undef BD_DECODE
    return hipGetLastError();
}

bool fused_path_supported(int xdtype, int64_t T, int mode, int64_t d_in) {
    return xdtype == BD_BF16 && T >= 1 && T <= kDecodeMaxT &&
           (mode == BD_SCALE_MATRIX || mode == BD_SCALE_ROW) &&
           (d_in + 511) / 512 * 512 <= kFusedMaxDpad;
}

bool q8_path_supported(int xdtype, int64_t T, int mode, int64_t d_in) {
    return xdtype == BD_BF16 && T >= 1 && T <= kDecodeMaxT &&
           (mode == BD_SCALE_MATRIX || mode == BD_SCALE_ROW) &&
           (d_in + 511) / 512 * 512 <= 512 * kUnitWaves;
}

hipError_t launch_decode_q8(int64_t T, int U, int64_t d_in, const DeltaPlan& dp, const void* x,
                            const int32_t* ids, const int8_t* wq, const float* wscale,
                            const uint64_t* signs, const void* scales, void* y, int ydtype, char* ws,
                            hipStream_t s) {
    const dim3 grid((unsigned)((dp.d_out + 15) / 16));
#define BD_UNITQ(MODE)                                                                        \
    k_decode_unit<MODE, true><<<grid, dim3(64 * kUnitWaves), 0, s>>>(                         \
        (const uint16_t*)x, ids, (int)T, U, d_in, wq, wscale, dp.d_out, signs,                   \
        sign_stride(dp.sstride, dp.d_out, d_in), scales, dp.sdtype, scale_stride(dp), y, ydtype,  \
        (uint32_t*)ws)
    if (dp.mode == BD_SCALE_MATRIX) BD_UNITQ(BD_SCALE_MATRIX);
    else BD_UNITQ(BD_SCALE_ROW);
#undef BD_UNITQ
    return hipGetLastError();
}

hipError_t launch_decode_fused(int64_t T, int U, int64_t d_in, const DeltaPlan& dp, const void* x,
                               const int32_t* ids, const void* wb, const uint64_t* signs,
                               const void* scales, void* y, int ydtype, char* ws, hipStream_t s) {
    const int dpad = (int)((d_in + 511) / 512 * 512);
    const size_t lds = (size_t)32 * dpad > (size_t)kFusedRedBytes ? (size_t)32 * dpad
                                                                  : (size_t)kFusedRedBytes;
    const dim3 grid((unsigned)((dp.d_out + 15) / 16));
    if (dpad <= 512 * kUnitWaves) {
#define BD_UNIT(MODE)                                                                         \
    k_decode_unit<MODE, false><<<grid, dim3(64 * kUnitWaves), 0, s>>>(                        \
        (const uint16_t*)x, ids, (int)T, U, d_in, wb, nullptr, dp.d_out, signs,                  \
        sign_stride(dp.sstride, dp.d_out, d_in), scales, dp.sdtype, scale_stride(dp), y, ydtype,  \
        (uint32_t*)ws)
        if (dp.mode == BD_SCALE_MATRIX) BD_UNIT(BD_SCALE_MATRIX);
        else BD_UNIT(BD_SCALE_ROW);
#undef BD_UNIT
        return hipGetLastError();
    }
#define BD_FUSED(MODE)                                                                          \
    k_decode_fused<MODE><<<grid, dim3(64 * kFusedWaves), lds, s>>>(                             \
        (const uint16_t*)x, ids, (int)T, U, d_in, dpad, (const uint16_t*)wb, dp.d_out, signs,   \
        sign_stride(dp.sstride, dp.d_out, d_in), scales, dp.sdtype, scale_stride(dp), y, ydtype, \
        (uint32_t*)ws)
    if (dp.mode == BD_SCALE_MATRIX) BD_FUSED(BD_SCALE_MATRIX);
    else BD_FUSED(BD_SCALE_ROW);
#undef BD_FUSED
    return hipGetLastError();
}

}  // namespace bd
