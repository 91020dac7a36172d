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

bd_status bd_delta_apply(void* batch, const void* x, bd_dtype x_dtype, int64_t T,
                         int64_t d_in, int32_t n_users, int64_t d_out, const uint64_t* signs_bank,
                         const void* scales_bank, const bd_compress_params* p, float* y,
                         void* stream) {
    BatchPlan bp;
    DeltaPlan dp;
    bd_status st = make_batch_plan(T, n_users, d_in, x_dtype, &bp);
    if (st != BD_OK) return st;
    st = make_delta_plan(p, bp, d_out, &dp);
    if (st != BD_OK) return st;
    if (!batch || !aligned(batch, kAlign)) return BD_ERR_INVALID_ARG;
    if (T == 0) return BD_OK;
    if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return BD_ERR_INVALID_ARG;
    if (n_users > 0 && (!signs_bank || !scales_bank || !aligned(signs_bank, 16) ||
                        !aligned(scales_bank, 16)))
        return BD_ERR_INVALID_ARG;
    hipError_t e = launch_delta(bp, dp, (char*)batch, x, signs_bank, scales_bank, y,
                                (hipStream_t)stream);
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

bd_status bd_apply_q8(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in, const int8_t* wq,
                      const float* wscales, int64_t d_out, const uint64_t* signs_bank,
                      const void* scales_bank, const bd_compress_params* p, int32_t n_users,
                      const int32_t* user_ids, void* y, bd_dtype y_dtype, void* workspace,
                      size_t ws_bytes, void* stream) {
    if (!p) return BD_ERR_INVALID_ARG;
    ApplyPlan pl;
    bd_status st = make_apply_plan(p, T, n_users, d_out, d_in, x_dtype, y_dtype, &pl);
    if (st != BD_OK) return st;
    if (T == 0) return BD_OK;
    if (!q8_path_supported(x_dtype, T, p->mode, d_in)) return BD_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < pl.total || !aligned(workspace, kAlign)) return BD_ERR_WORKSPACE;
    if (!x || !wq || !wscales || !y || !user_ids) return BD_ERR_INVALID_ARG;
    if (n_users > 0 && (!signs_bank || !scales_bank)) return BD_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(wscales, 4) || !aligned(y, 16) ||
        !aligned(user_ids, 4) || (signs_bank && !aligned(signs_bank, 16)) ||
        (scales_bank && !aligned(scales_bank, 16)))
        return BD_ERR_INVALID_ARG;
    hipError_t e = launch_decode_q8(T, n_users, d_in, pl.delta, x, user_ids, wq, wscales,
                                    signs_bank, scales_bank, y, y_dtype, (char*)workspace,
                                    (hipStream_t)stream);
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
    return BD_OK;
}

}  // extern "C"
