// bd_api.hip -- the exported C ABI of libbitdelta.so (declared in
// include/bitdelta.h): argument validation, workspace checks, and the launch
// sequences on the caller's stream.  Validation happens entirely on the host
// before anything is enqueued, so every synchronous error leaves the stream
// untouched.
#include "bd_internal.h"

using namespace bd;

namespace {

bool valid_wdtype(int d) { return d == BD_F32 || d == BD_BF16; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

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

size_t bd_apply_workspace_bytes(const bd_compress_params* p, int64_t T, int32_t n_users,
                                int64_t d_out, int64_t d_in, bd_dtype x_dtype, bd_dtype y_dtype) {
    ApplyPlan pl;
    if (make_apply_plan(p, T, n_users, d_out, d_in, x_dtype, y_dtype, &pl) != BD_OK) return 0;
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

bd_status bd_apply(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in, const void* w_base,
                   int64_t d_out, const uint64_t* signs_bank, const void* scales_bank,
                   const bd_compress_params* p, int32_t n_users, const int32_t* user_ids, void* y,
                   bd_dtype y_dtype, void* workspace, size_t ws_bytes, void* stream) {
    if (!p) return BD_ERR_INVALID_ARG;
    ApplyPlan pl;
    bd_status st = make_apply_plan(p, T, n_users, d_out, d_in, x_dtype, y_dtype, &pl);
    if (st != BD_OK) return st;
    if (!workspace || ws_bytes < pl.total || !aligned(workspace, kAlign)) return BD_ERR_WORKSPACE;
    if (T == 0) {
        hipError_t e = launch_zero_u32((uint32_t*)workspace, (int64_t)(kAlign / 4), (hipStream_t)stream);
        return e == hipSuccess ? BD_OK : BD_ERR_DEVICE;
    }
    if (!x || !w_base || !y || !user_ids) return BD_ERR_INVALID_ARG;
    if (n_users > 0 && (!signs_bank || !scales_bank)) return BD_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(w_base, 16) || !aligned(y, 16) || !aligned(user_ids, 4) ||
        (signs_bank && !aligned(signs_bank, 16)))
        return BD_ERR_INVALID_ARG;
    hipError_t e = launch_apply(pl, x, w_base, signs_bank, scales_bank, user_ids, y,
                                (char*)workspace, (hipStream_t)stream);
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
    return BD_OK;
}

}  // extern "C"
