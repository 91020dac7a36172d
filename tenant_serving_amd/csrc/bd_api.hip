// bd_api.hip -- the exported C ABI of libbitdelta.so (declared in
// include/bitdelta.h): argument validation, workspace checks, and the launch
// sequences on the caller's stream.  Validation happens entirely on the host
// before anything is enqueued, so every synchronous error leaves the stream
// untouched.
#include "bd_internal.h"

#include <mutex>

using namespace bd;

// Scratch of bd_apply_noalloc: the workspace of its launches, one copy per device for
// the life of the process (its device address is taken once per device below).
static __device__ __align__(256) char scratch[BD_NOALLOC_SCRATCH_BYTES];

namespace {

bool valid_wdtype(int d) { return d == BD_F32 || d == BD_BF16; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Device address of `scratch` on the current device (looked up on the first call per
// device, with that device current).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
bd_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BD_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return BD_ERR_DEVICE;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return BD_OK;
}

// *dst = *src (one word, device to device), or *dst = 0 without src
__global__ void k_copy_word(const uint32_t* src, uint32_t* dst) {
    if (threadIdx.x == 0) dst[0] = src ? src[0] : 0u;
}

// slot_ids[t] = the slot of token t's user: -1 stays -1 (base model only); an id outside
// [0, n_users), or a user without a slot (table value outside [0, n_slots)), becomes
// n_slots, which the apply reports as a bad user id (base product only).
__global__ void k_map_slots(const int32_t* __restrict__ ids, int64_t T,
                            const int32_t* __restrict__ slot_of_user, int32_t n_users,
                            int32_t n_slots, int32_t* __restrict__ slot_ids) {
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < T;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int32_t u = ids[t];
        int32_t k = -1;
        if (u != -1) {
            k = (uint32_t)u < (uint32_t)n_users ? slot_of_user[u] : n_slots;
            if ((uint32_t)k >= (uint32_t)n_slots) k = n_slots;
        }
        slot_ids[t] = k;
    }
}

}  // namespace

extern "C" {

int bd_abi_version(void) { return BD_ABI_VERSION; }

const char* bd_status_string(bd_status s) {
    switch (s) {
        case BD_OK: return "ok";
        case BD_ERR_INVALID_ARG: return "invalid argument";
        case BD_ERR_SHAPE: return "unsupported shape";
        case BD_ERR_DTYPE: return "unsupported dtype";
        case BD_ERR_UNSUPPORTED: return "unsupported parameter";
        case BD_ERR_WORKSPACE: return "workspace missing or too small";
        case BD_ERR_DEVICE: return "HIP error";
        case BD_ERR_NONFINITE: return "non-finite delta";
        case BD_ERR_USER_ID: return "user id out of range";
        case BD_ERR_BATCH: return "prepared batch encoded for another scale mode";
    }
    return "unknown status";
}

size_t bd_signs_bytes(int64_t d_out, int64_t d_in) {
    if (d_out <= 0 || d_in <= 0 || d_in % 64 != 0) return 0;
    return (size_t)d_out * (size_t)(d_in / 8);
}

int64_t bd_scales_count(const bd_compress_params* p, int64_t d_out, int64_t d_in) {
    CompressPlan pl;
    if (make_compress_plan(p, d_out, d_in, &pl) != BD_OK) return -1;
    switch (p->mode) {
        case BD_SCALE_MATRIX: return 1;
        case BD_SCALE_GROUP: return d_out * (d_in / p->group_size);
        case BD_SCALE_ROW: return d_out;
        default: return d_in;
    }
}

size_t bd_compress_workspace_bytes(const bd_compress_params* p, int64_t d_out, int64_t d_in) {
    CompressPlan pl;
    if (make_compress_plan(p, d_out, d_in, &pl) != BD_OK) return 0;
    return pl.total;
}

size_t bd_select_axis_workspace_bytes(int64_t d_out, int64_t d_in, float clip_k) {
    AxisPlan ap;
    if (make_axis_plan(clip_k, d_out, d_in, &ap) != BD_OK) return 0;
    return ap.total;
}

size_t bd_apply_workspace_bytes(const bd_compress_params* p, int64_t T, int32_t n_users,
                                int64_t d_out, int64_t d_in, bd_dtype x_dtype, bd_dtype y_dtype) {
    ApplyPlan pl;
    if (make_apply_plan(p, T, n_users, d_out, d_in, x_dtype, y_dtype, &pl) != BD_OK) return 0;
    return pl.total;
}

size_t bd_batch_workspace_bytes(int64_t T, int32_t n_users, int64_t d_in, bd_dtype x_dtype) {
    BatchPlan pl;
    if (make_batch_plan(T, n_users, d_in, x_dtype, &pl) != BD_OK) return 0;
    return pl.total;
}

bd_status bd_compress(const void* w_fine, const void* w_base, bd_dtype w_dtype, int64_t d_out,
                      int64_t d_in, const bd_compress_params* p, uint64_t* signs_out,
                      void* scales_out, void* workspace, size_t ws_bytes, void* stream) {
    if (!w_fine || !signs_out || !scales_out || !p) return BD_ERR_INVALID_ARG;
    if (!valid_wdtype(w_dtype)) return BD_ERR_DTYPE;
    CompressPlan pl;
    bd_status st = make_compress_plan(p, d_out, d_in, &pl);
    if (st != BD_OK) return st;
    if (!workspace || ws_bytes < pl.total || !aligned(workspace, kAlign)) return BD_ERR_WORKSPACE;
    // 16-byte vector loads of every row segment
    if (!aligned(w_fine, 16) || (w_base && !aligned(w_base, 16)) || !aligned(signs_out, 8))
        return BD_ERR_INVALID_ARG;
    hipError_t e = launch_compress(pl, w_fine, w_base, w_dtype, signs_out, scales_out,
                                   (char*)workspace, (hipStream_t)stream);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

bd_status bd_select_axis(const void* w_fine, const void* w_base, bd_dtype w_dtype, int64_t d_out,
                         int64_t d_in, float clip_k, double* errors, int32_t* axis,
                         void* workspace, size_t ws_bytes, void* stream) {
    if (!w_fine) return BD_ERR_INVALID_ARG;
    if (!valid_wdtype(w_dtype)) return BD_ERR_DTYPE;
    AxisPlan ap;
    bd_status st = make_axis_plan(clip_k, d_out, d_in, &ap);
    if (st != BD_OK) return st;
    if (!workspace || ws_bytes < ap.total || !aligned(workspace, kAlign)) return BD_ERR_WORKSPACE;
    if (!aligned(w_fine, 16) || (w_base && !aligned(w_base, 16)) || (errors && !aligned(errors, 8)) ||
        (axis && !aligned(axis, 4)))
        return BD_ERR_INVALID_ARG;
    hipError_t e = launch_select_axis(ap, w_fine, w_base, w_dtype, errors, axis, (char*)workspace,
                                      (hipStream_t)stream);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

bd_status bd_reconstruct(const uint64_t* signs, const void* scales, const bd_compress_params* p,
                         int64_t d_out, int64_t d_in, const void* w_base, bd_dtype w_dtype,
                         void* out, bd_dtype out_dtype, void* stream) {
    if (!signs || !scales || !out || !p) return BD_ERR_INVALID_ARG;
    if (w_base && !valid_wdtype(w_dtype)) return BD_ERR_DTYPE;
    if (out_dtype != BD_F32 && out_dtype != BD_BF16) return BD_ERR_DTYPE;
    CompressPlan pl;
    bd_status st = make_compress_plan(p, d_out, d_in, &pl);
    if (st != BD_OK) return st;
    hipError_t e = launch_reconstruct(signs, scales, p->mode, pl.group, p->scale_dtype, d_out, d_in,
                                      w_base, w_dtype, out, out_dtype, (hipStream_t)stream);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

bd_status bd_batch_prepare(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                           const int32_t* user_ids, int32_t n_users, void* batch,
                           size_t batch_bytes, void* stream) {
    BatchPlan bp;
    bd_status st = make_batch_plan(T, n_users, d_in, x_dtype, &bp);
    if (st != BD_OK) return st;
    if (!batch || batch_bytes < bp.total || !aligned(batch, kAlign)) return BD_ERR_WORKSPACE;
    if (T > 0 && (!x || !user_ids)) return BD_ERR_INVALID_ARG;
    if (T > 0 && (!aligned(x, 16) || !aligned(user_ids, 4))) return BD_ERR_INVALID_ARG;
    hipError_t e = launch_batch_prepare(bp, x, user_ids, (char*)batch, (hipStream_t)stream);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

bd_status bd_base_gemm(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                       const void* w_base, int64_t d_out, float* y, void* stream) {
    if (!valid_wdtype(x_dtype)) return BD_ERR_DTYPE;
    if (T < 0) return BD_ERR_INVALID_ARG;
    if (d_in <= 0 || d_in % 64 != 0 || d_out <= 0) return BD_ERR_SHAPE;
    if (x_dtype == BD_BF16 && (d_out * d_in * 2 >= ((int64_t)1 << 31) ||
                               T * d_in * 2 >= ((int64_t)1 << 31)))
        return BD_ERR_UNSUPPORTED;  // 32-bit buffer offsets
    if (T == 0) return BD_OK;
    if (!x || !w_base || !y) return BD_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(w_base, 16) || !aligned(y, 16)) return BD_ERR_INVALID_ARG;
    hipError_t e = launch_base_gemm(x, x_dtype, T, d_in, w_base, d_out, y, (hipStream_t)stream);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

bd_status bd_delta_apply(void* batch, size_t batch_bytes, const void* x, bd_dtype x_dtype,
                         int64_t T, int64_t d_in, int32_t n_users, int64_t d_out,
                         const uint64_t* signs_bank, const void* scales_bank,
                         const bd_compress_params* p, float* y, void* stream) {
    BatchPlan bp;
    DeltaPlan dp;
    bd_status st = make_batch_plan(T, n_users, d_in, x_dtype, &bp);
    if (st != BD_OK) return st;
    st = make_delta_plan(p, bp, d_out, &dp);
    if (st != BD_OK) return st;
    if (!batch || !aligned(batch, kAlign)) return BD_ERR_INVALID_ARG;
    if (batch_bytes < bp.total) return BD_ERR_WORKSPACE;
    if (T == 0) return BD_OK;
    if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return BD_ERR_INVALID_ARG;
    if (n_users > 0 && (!signs_bank || !scales_bank || !aligned(signs_bank, 16) ||
                        !aligned(scales_bank, 16)))
        return BD_ERR_INVALID_ARG;
    hipError_t e = launch_delta(bp, dp, (char*)batch, x, signs_bank, scales_bank, y,
                                (hipStream_t)stream);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

bd_status bd_batch_encode(void* batch, size_t batch_bytes, const void* x, bd_dtype x_dtype,
                          int64_t T, int64_t d_in, int32_t n_users, const void* scales_bank,
                          const bd_compress_params* p, void* stream) {
    // the shared encoding feeds the matrix-core products: groups of 128 columns or more
    if (p && p->mode == BD_SCALE_GROUP && p->group_size < 128) return BD_ERR_UNSUPPORTED;
    if (x_dtype != BD_BF16) return BD_ERR_DTYPE;
    BatchPlan bp;
    DeltaPlan dp;
    bd_status st = make_batch_plan(T, n_users, d_in, x_dtype, &bp);
    if (st != BD_OK) return st;
    st = make_delta_plan(p, bp, 1, &dp);
    if (st != BD_OK) return st;
    if (!batch || !aligned(batch, kAlign)) return BD_ERR_INVALID_ARG;
    if (batch_bytes < bp.total) return BD_ERR_WORKSPACE;
    if (T == 0) return BD_OK;
    if (!x || !aligned(x, 16)) return BD_ERR_INVALID_ARG;
    if (p->mode == BD_SCALE_COL && n_users > 0 && (!scales_bank || !aligned(scales_bank, 16)))
        return BD_ERR_INVALID_ARG;
    hipError_t e = launch_tile_encode(bp, dp, (char*)batch, x, scales_bank, (hipStream_t)stream);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

bd_status bd_delta_apply_encoded(void* batch, size_t batch_bytes, bd_dtype x_dtype, int64_t T,
                                 int64_t d_in, int32_t n_users, int64_t d_out,
                                 const uint64_t* signs_bank, const void* scales_bank,
                                 const bd_compress_params* p, float* y, void* stream) {
    // the shared encoding feeds the matrix-core products: groups of 128 columns or more
    if (p && p->mode == BD_SCALE_GROUP && p->group_size < 128) return BD_ERR_UNSUPPORTED;
    if (x_dtype != BD_BF16) return BD_ERR_DTYPE;
    BatchPlan bp;
    DeltaPlan dp;
    bd_status st = make_batch_plan(T, n_users, d_in, x_dtype, &bp);
    if (st != BD_OK) return st;
    st = make_delta_plan(p, bp, d_out, &dp);
    if (st != BD_OK) return st;
    if (!batch || !aligned(batch, kAlign)) return BD_ERR_INVALID_ARG;
    if (batch_bytes < bp.total) return BD_ERR_WORKSPACE;
    if (T == 0) return BD_OK;
    if (!y || !aligned(y, 16)) return BD_ERR_INVALID_ARG;
    if (n_users > 0 && (!signs_bank || !scales_bank || !aligned(signs_bank, 16) ||
                        !aligned(scales_bank, 16)))
        return BD_ERR_INVALID_ARG;
    hipError_t e = launch_delta6_encoded(bp, dp, (char*)batch, signs_bank, scales_bank, y,
                                         (hipStream_t)stream);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

size_t bd_base_gemm_n_workspace_bytes(bd_dtype x_dtype, int64_t T, int64_t d_in, int32_t n_mats,
                                      const int64_t* d_outs) {
    if (x_dtype != BD_BF16 || T <= 0 || n_mats < 1 || n_mats > kMaxMats || !d_outs || d_in <= 0 ||
        d_in % 64 != 0)
        return 0;
    for (int i = 0; i < n_mats; ++i)
        if (!gemm_path_supported(T, d_in, d_outs[i])) return 0;
    return gemm_split_bytes(T, d_in, d_outs, n_mats);
}

bd_status bd_base_gemm_n(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                         int32_t n_mats, const void* const* w_bases, const int64_t* d_outs,
                         float* const* ys, void* workspace, size_t ws_bytes, void* stream) {
    if (!valid_wdtype(x_dtype)) return BD_ERR_DTYPE;
    if (T < 0 || n_mats < 1 || n_mats > kMaxMats || !w_bases || !d_outs || !ys)
        return BD_ERR_INVALID_ARG;
    if (d_in <= 0 || d_in % 64 != 0) return BD_ERR_SHAPE;
    for (int i = 0; i < n_mats; ++i) {
        if (d_outs[i] <= 0) return BD_ERR_SHAPE;
        if (x_dtype == BD_BF16 && (d_outs[i] * d_in * 2 >= ((int64_t)1 << 31) ||
                                   T * d_in * 2 >= ((int64_t)1 << 31)))
            return BD_ERR_UNSUPPORTED;  // 32-bit buffer offsets
    }
    if (T == 0) return BD_OK;
    if (!x || !aligned(x, 16)) return BD_ERR_INVALID_ARG;
    for (int i = 0; i < n_mats; ++i)
        if (!w_bases[i] || !ys[i] || !aligned(w_bases[i], 16) || !aligned(ys[i], 16))
            return BD_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    bool tiled = x_dtype == BD_BF16;
    for (int i = 0; i < n_mats; ++i) tiled = tiled && gemm_path_supported(T, d_in, d_outs[i]);
    hipError_t e = hipSuccess;
    if (tiled) {
        GemmMatArg m[kMaxMats];
        for (int i = 0; i < n_mats; ++i) m[i] = GemmMatArg{w_bases[i], ys[i], d_outs[i]};
        const size_t need = gemm_split_bytes(T, d_in, d_outs, n_mats);
        if (need > 0 && workspace) {
            if (ws_bytes < need || !aligned(workspace, kAlign)) return BD_ERR_WORKSPACE;
            e = launch_gemm_set_split(x, T, d_in, m, n_mats, (char*)workspace, s);
        } else {
            e = launch_gemm_set(x, T, d_in, m, n_mats, s);
        }
    } else {
        for (int i = 0; i < n_mats && e == hipSuccess; ++i)
            e = launch_base_gemm(x, x_dtype, T, d_in, w_bases[i], d_outs[i], ys[i], s);
    }
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

bd_status bd_base_gemm_q8_n(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                            int32_t n_mats, const int8_t* const* wqs,
                            const float* const* wscales, const int64_t* d_outs,
                            float* const* ys, void* workspace, size_t ws_bytes, void* stream) {
    if (x_dtype != BD_BF16) return BD_ERR_DTYPE;
    if (T < 0 || n_mats < 1 || n_mats > kMaxMats || !wqs || !wscales || !d_outs || !ys)
        return BD_ERR_INVALID_ARG;
    if (d_in <= 0 || d_in % 64 != 0) return BD_ERR_SHAPE;
    for (int i = 0; i < n_mats; ++i) {
        if (d_outs[i] <= 0) return BD_ERR_SHAPE;
        if (T > 0 && !gemm_q8_supported(T, d_in, d_outs[i])) return BD_ERR_UNSUPPORTED;
    }
    if (T == 0) return BD_OK;
    if (!x || !aligned(x, 16)) return BD_ERR_INVALID_ARG;
    for (int i = 0; i < n_mats; ++i)
        if (!wqs[i] || !wscales[i] || !ys[i] || !aligned(wqs[i], 16) || !aligned(wscales[i], 4) ||
            !aligned(ys[i], 16))
            return BD_ERR_INVALID_ARG;
    GemmMatArg m[kMaxMats];
    for (int i = 0; i < n_mats; ++i) m[i] = GemmMatArg{wqs[i], ys[i], d_outs[i]};
    // split exactly where bd_base_gemm_n_workspace_bytes (bf16 shapes) asks for room
    const size_t need = bd_base_gemm_n_workspace_bytes(BD_BF16, T, d_in, n_mats, d_outs);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (need > 0 && workspace) {
        if (ws_bytes < need || !aligned(workspace, kAlign)) return BD_ERR_WORKSPACE;
        e = launch_gemm_set_split(x, T, d_in, m, n_mats, (char*)workspace, s, wscales);
    } else {
        e = launch_gemm_set(x, T, d_in, m, n_mats, s, wscales);
    }
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

bd_status bd_delta_apply_encoded_n(void* batch, size_t batch_bytes, bd_dtype x_dtype, int64_t T,
                                   int64_t d_in, int32_t n_users, int32_t n_mats,
                                   const int64_t* d_outs, const uint64_t* const* signs_banks,
                                   const void* const* scales_banks, const bd_compress_params* p,
                                   float* const* ys, void* stream) {
    // the shared encoding feeds the matrix-core products: groups of 128 columns or more
    if (p && p->mode == BD_SCALE_GROUP && p->group_size < 128) return BD_ERR_UNSUPPORTED;
    if (x_dtype != BD_BF16) return BD_ERR_DTYPE;
    if (n_mats < 1 || n_mats > kMaxMats || !d_outs || !signs_banks || !scales_banks || !ys)
        return BD_ERR_INVALID_ARG;
    BatchPlan bp;
    bd_status st = make_batch_plan(T, n_users, d_in, x_dtype, &bp);
    if (st != BD_OK) return st;
    DeltaPlan dp;
    DeltaMatArg m[kMaxMats];
    for (int i = 0; i < n_mats; ++i) {
        st = make_delta_plan(p, bp, d_outs[i], &dp);
        if (st != BD_OK) return st;
        m[i] = DeltaMatArg{signs_banks[i], scales_banks[i], ys[i], d_outs[i]};
    }
    if (!batch || !aligned(batch, kAlign)) return BD_ERR_INVALID_ARG;
    if (batch_bytes < bp.total) return BD_ERR_WORKSPACE;
    if (T == 0) return BD_OK;
    for (int i = 0; i < n_mats; ++i) {
        if (!ys[i] || !aligned(ys[i], 16)) return BD_ERR_INVALID_ARG;
        if (n_users > 0 && (!signs_banks[i] || !scales_banks[i] || !aligned(signs_banks[i], 16) ||
                            !aligned(scales_banks[i], 16)))
            return BD_ERR_INVALID_ARG;
    }
    hipError_t e = launch_delta6_set(bp, dp, (char*)batch, m, n_mats, (hipStream_t)stream);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

bd_status bd_quantize_base(const void* w, bd_dtype w_dtype, int64_t d_out, int64_t d_in,
                           int8_t* q_out, float* scales_out, void* stream) {
    if (!w || !q_out || !scales_out) return BD_ERR_INVALID_ARG;
    if (!valid_wdtype(w_dtype)) return BD_ERR_DTYPE;
    if (d_out <= 0 || d_in <= 0 || d_out > ((int64_t)1 << 31) - 1 || d_in > (int64_t)1 << 31)
        return BD_ERR_SHAPE;
    hipError_t e = launch_quantize_rows(w, w_dtype, d_out, d_in, q_out, scales_out,
                                        (hipStream_t)stream);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

size_t bd_apply_q8_workspace_bytes(const bd_compress_params* p, int64_t T, int32_t n_users,
                                   int64_t d_out, int64_t d_in, bd_dtype x_dtype,
                                   bd_dtype y_dtype) {
    if (!p) return 0;
    ApplyPlan pl;
    const bool dec = q8_path_supported(x_dtype, T, p->mode, d_in);
    if (make_apply_plan(p, T, n_users, d_out, d_in, x_dtype, y_dtype, &pl, dec) != BD_OK) return 0;
    return pl.total;
}

bd_status bd_apply_q8(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in, const int8_t* wq,
                      const float* wscales, int64_t d_out, const uint64_t* signs_bank,
                      const void* scales_bank, const bd_compress_params* p, int32_t n_users,
                      const int32_t* user_ids, void* y, bd_dtype y_dtype, void* workspace,
                      size_t ws_bytes, void* stream) {
    if (!p) return BD_ERR_INVALID_ARG;
    const bool dec = q8_path_supported(x_dtype, T, p->mode, d_in);
    ApplyPlan pl;
    bd_status st = make_apply_plan(p, T, n_users, d_out, d_in, x_dtype, y_dtype, &pl, dec);
    if (st != BD_OK) return st;
    if (T == 0) return BD_OK;
    if (x_dtype != BD_BF16 || (!dec && !gemm_q8_supported(T, d_in, d_out)))
        return BD_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < pl.total || !aligned(workspace, kAlign)) return BD_ERR_WORKSPACE;
    if (!x || !wq || !wscales || !y || !user_ids) return BD_ERR_INVALID_ARG;
    if (n_users > 0 && (!signs_bank || !scales_bank)) return BD_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(wscales, 4) || !aligned(y, 16) ||
        !aligned(user_ids, 4) || (signs_bank && !aligned(signs_bank, 16)) ||
        (scales_bank && !aligned(scales_bank, 16)))
        return BD_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    if (dec) {
        hipError_t e = launch_decode_q8(T, n_users, d_in, pl.delta, x, user_ids, wq, wscales,
                                        signs_bank, scales_bank, y, y_dtype, ws, s);
        return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
    }
    hipError_t e = launch_batch_prepare(pl.batch, x, user_ids, ws, s);
    float* yacc = y_dtype == BD_F32 ? (float*)y : (float*)(ws + pl.off_yf);
    if (e == hipSuccess) e = launch_gemm_q8(x, T, d_in, wq, wscales, d_out, yacc, s);
    if (e == hipSuccess)
        e = launch_delta(pl.batch, pl.delta, ws, x, signs_bank, scales_bank, yacc, s);
    if (e == hipSuccess && y_dtype == BD_BF16)
        e = launch_cast_bf16(yacc, (uint16_t*)y, T * d_out, s);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

}  // extern "C"

// bd_apply on a workspace of ws_bytes (the caller's, or the no-allocation scratch).
// sstride / cstride: bytes and scale elements from one user's bank to the next (0: dense).
static bd_status apply_on(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                          const void* w_base, int64_t d_out, const uint64_t* signs_bank,
                          const void* scales_bank, const bd_compress_params* p, int32_t n_users,
                          const int32_t* user_ids, void* y, bd_dtype y_dtype, void* workspace,
                          size_t ws_bytes, void* stream, uint64_t sstride = 0,
                          int64_t cstride = 0) {
    if (!p) return BD_ERR_INVALID_ARG;
    ApplyPlan pl;
    bd_status st = make_apply_plan(p, T, n_users, d_out, d_in, x_dtype, y_dtype, &pl);
    if (st != BD_OK) return st;
    pl.delta.sstride = sstride;
    pl.delta.cstride = cstride;
    if (!workspace || ws_bytes < pl.total || !aligned(workspace, kAlign)) return BD_ERR_WORKSPACE;
    if (T > 0) {
        if (!x || !w_base || !y || !user_ids) return BD_ERR_INVALID_ARG;
        if (n_users > 0 && (!signs_bank || !scales_bank)) return BD_ERR_INVALID_ARG;
        if (!aligned(x, 16) || !aligned(w_base, 16) || !aligned(y, 16) || !aligned(user_ids, 4) ||
            (signs_bank && !aligned(signs_bank, 16)) || (scales_bank && !aligned(scales_bank, 16)))
            return BD_ERR_INVALID_ARG;
    }
    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    if (pl.fused) {
        hipError_t e = launch_decode_fused(T, n_users, d_in, pl.delta, x, user_ids, w_base,
                                           signs_bank, scales_bank, y, y_dtype, ws, s);
        return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
    }
    if (pl.decode) {
        hipError_t e = launch_decode_prep(pl.dec, n_users, pl.delta, x, user_ids, scales_bank, ws, s);
        if (e == hipSuccess)
            e = launch_decode_main(pl.dec, pl.delta, x, w_base, signs_bank, scales_bank, y,
                                   y_dtype, ws, s);
        return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
    }
    hipError_t e = launch_batch_prepare(pl.batch, x, user_ids, ws, s);
    if (e != hipSuccess || T == 0) return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
    float* yacc = y_dtype == BD_F32 ? (float*)y : (float*)(ws + pl.off_yf);
    e = launch_base_gemm(x, x_dtype, T, d_in, w_base, d_out, yacc, s);
    if (e == hipSuccess)
        e = launch_delta(pl.batch, pl.delta, ws, x, signs_bank, scales_bank, yacc, s);
    if (e == hipSuccess && y_dtype == BD_BF16)
        e = launch_cast_bf16(yacc, (uint16_t*)y, T * d_out, s);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

extern "C" {

bd_status bd_apply(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in, const void* w_base,
                   int64_t d_out, const uint64_t* signs_bank, const void* scales_bank,
                   const bd_compress_params* p, int32_t n_users, const int32_t* user_ids, void* y,
                   bd_dtype y_dtype, void* workspace, size_t ws_bytes, void* stream) {
    return apply_on(x, x_dtype, T, d_in, w_base, d_out, signs_bank, scales_bank, p, n_users,
                    user_ids, y, y_dtype, workspace, ws_bytes, stream);
}

size_t bd_apply_paged_workspace_bytes(const bd_compress_params* p, int64_t T, int32_t n_slots,
                                      int64_t d_out, int64_t d_in, bd_dtype x_dtype,
                                      bd_dtype y_dtype) {
    const size_t w = bd_apply_workspace_bytes(p, T, n_slots, d_out, d_in, x_dtype, y_dtype);
    if (w == 0 || T < 0) return 0;
    return w + ((size_t)T * 4 + kAlign - 1) / kAlign * kAlign;
}

bd_status bd_apply_paged(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                         const void* w_base, int64_t d_out, const uint64_t* signs_pool,
                         const void* scales_pool, uint64_t signs_stride, uint64_t scales_stride,
                         int32_t n_slots, const bd_compress_params* p,
                         const int32_t* slot_of_user, int32_t n_users, const int32_t* user_ids,
                         void* y, bd_dtype y_dtype, void* workspace, size_t ws_bytes,
                         void* stream) {
    if (!p) return BD_ERR_INVALID_ARG;
    const size_t need = bd_apply_paged_workspace_bytes(p, T, n_slots, d_out, d_in, x_dtype, y_dtype);
    if (need == 0) {  // invalid sizes or parameters: the plain call names the error
        ApplyPlan pl;
        const bd_status st = make_apply_plan(p, T, n_slots, d_out, d_in, x_dtype, y_dtype, &pl);
        return st != BD_OK ? st : BD_ERR_INVALID_ARG;
    }
    if (n_users < 0) return BD_ERR_INVALID_ARG;
    const size_t esz = p->scale_dtype == BD_F16 ? 2 : 4;
    const uint64_t sbytes = (uint64_t)d_out * (uint64_t)(d_in / 8);
    const uint64_t cbytes = (uint64_t)bd_scales_count(p, d_out, d_in) * esz;
    if ((signs_stride != 0 && (signs_stride < sbytes || signs_stride % 16 != 0)) ||
        (scales_stride != 0 && (scales_stride < cbytes || scales_stride % 16 != 0)))
        return BD_ERR_INVALID_ARG;
    if (!workspace || ws_bytes < need || !aligned(workspace, kAlign)) return BD_ERR_WORKSPACE;
    if (T > 0 && (!user_ids || (n_users > 0 && !slot_of_user) || !aligned(user_ids, 4) ||
                  (slot_of_user && !aligned(slot_of_user, 4))))
        return BD_ERR_INVALID_ARG;
    const size_t w = need - ((size_t)T * 4 + kAlign - 1) / kAlign * kAlign;
    int32_t* slot_ids = (int32_t*)((char*)workspace + w);
    if (T > 0) {
        hipLaunchKernelGGL(k_map_slots, dim3((unsigned)((T + 255) / 256 < 1024 ? (T + 255) / 256 : 1024)),
                           dim3(256), 0, (hipStream_t)stream, user_ids, T, slot_of_user, n_users,
                           n_slots, slot_ids);
        if (hipGetLastError() != hipSuccess) return BD_ERR_DEVICE;
    }
    return apply_on(x, x_dtype, T, d_in, w_base, d_out, signs_pool, scales_pool, p, n_slots,
                    slot_ids, y, y_dtype, workspace, w, stream, signs_stride,
                    (int64_t)(scales_stride / esz));
}

bd_status bd_apply_noalloc(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                           const void* w_base, int64_t d_out, const uint64_t* signs_bank,
                           const void* scales_bank, const bd_compress_params* p,
                           int32_t n_users, const int32_t* user_ids, void* y, bd_dtype y_dtype,
                           uint32_t* status, void* stream) {
    if (!p) return BD_ERR_INVALID_ARG;
    if (status && !aligned(status, 4)) return BD_ERR_INVALID_ARG;
    const size_t need = bd_apply_workspace_bytes(p, T, n_users, d_out, d_in, x_dtype, y_dtype);
    if (need > (size_t)BD_NOALLOC_SCRATCH_BYTES) return BD_ERR_WORKSPACE;  // (0: invalid sizes,
                                                                           // reported below)
    void* ws = nullptr;
    bd_status st = scratch_address(&ws);
    if (st != BD_OK) return st;
    st = apply_on(x, x_dtype, T, d_in, w_base, d_out, signs_bank, scales_bank, p, n_users,
                  user_ids, y, y_dtype, ws, BD_NOALLOC_SCRATCH_BYTES, stream);
    if (st != BD_OK || !status) return st;
    // the call's status word (its launches rewrite word 0 of the workspace; none for T == 0)
    hipLaunchKernelGGL(k_copy_word, dim3(1), dim3(64), 0, (hipStream_t)stream,
                       T > 0 ? (const uint32_t*)ws : (const uint32_t*)nullptr, status);
    return hipGetLastError() == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

// Shared validation of the two decode-path entry points.
static bd_status decode_plans(const bd_compress_params* p, int64_t T, int32_t n_users,
                              int64_t d_out, int64_t d_in, bd_dtype x_dtype, ApplyPlan* pl) {
    if (!p) return BD_ERR_INVALID_ARG;
    bd_status st = make_apply_plan(p, T, n_users, d_out, d_in, x_dtype, BD_F32, pl);
    if (st != BD_OK) return st;
    return pl->decode ? BD_OK : BD_ERR_UNSUPPORTED;
}

bd_status bd_decode_prepare(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                            const int32_t* user_ids, int32_t n_users, const void* scales_bank,
                            const bd_compress_params* p, void* workspace, size_t ws_bytes,
                            void* stream) {
    ApplyPlan pl;
    bd_status st = decode_plans(p, T, n_users, 1, d_in, x_dtype, &pl);
    if (st != BD_OK) return st;
    if (!workspace || ws_bytes < pl.dec.total || !aligned(workspace, kAlign))
        return BD_ERR_WORKSPACE;
    if (!x || !user_ids || !aligned(x, 16) || !aligned(user_ids, 4)) return BD_ERR_INVALID_ARG;
    if (p->mode == BD_SCALE_COL && n_users > 0 && (!scales_bank || !aligned(scales_bank, 16)))
        return BD_ERR_INVALID_ARG;
    pl.delta.per_user = d_in;  // COL: one scale per input column
    hipError_t e = launch_decode_prep(pl.dec, n_users, pl.delta, x, user_ids, scales_bank,
                                      (char*)workspace, (hipStream_t)stream);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

bd_status bd_decode_apply(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                          const void* w_base, int64_t d_out, const uint64_t* signs_bank,
                          const void* scales_bank, const bd_compress_params* p, int32_t n_users,
                          void* y, bd_dtype y_dtype, const void* workspace, size_t ws_bytes,
                          void* stream) {
    ApplyPlan pl;
    bd_status st = decode_plans(p, T, n_users, d_out, d_in, x_dtype, &pl);
    if (st != BD_OK) return st;
    if (y_dtype != BD_F32 && y_dtype != BD_BF16) return BD_ERR_DTYPE;
    if (!workspace || ws_bytes < pl.dec.total || !aligned(workspace, kAlign))
        return BD_ERR_WORKSPACE;
    if (!x || !w_base || !y || !aligned(x, 16) || !aligned(w_base, 16) || !aligned(y, 16))
        return BD_ERR_INVALID_ARG;
    if (n_users > 0 && (!signs_bank || !scales_bank || !aligned(signs_bank, 16) ||
                        !aligned(scales_bank, 16)))
        return BD_ERR_INVALID_ARG;
    hipError_t e = launch_decode_main(pl.dec, pl.delta, x, w_base, signs_bank, scales_bank, y,
                                      y_dtype, (const char*)workspace, (hipStream_t)stream);
    return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
}

bd_status bd_device_status(const void* workspace, void* stream) {
    if (!workspace) return BD_ERR_INVALID_ARG;
    uint32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost,
                                  (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return BD_ERR_DEVICE;
    if (word & ST_NONFINITE) return BD_ERR_NONFINITE;
    if (word & ST_USER_ID) return BD_ERR_USER_ID;
    if (word & ST_ENCODING) return BD_ERR_BATCH;
    return BD_OK;
}

}  // extern "C"
