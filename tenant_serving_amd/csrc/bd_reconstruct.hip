// bd_reconstruct.hip -- dense reconstruction of a packed delta.
//
// out[o][i] = (W_base[o][i] if given) + sign(o,i) * scale(o,i) ([P1] "How
// BitDelta Works" step 4 "Reconstruction" and step 5 "Serving"), added in
// fp32 and rounded once to the output dtype.  Off the serving hot path (the
// apply never builds this); used for checks and for merging a hot user's
// weight.  Each thread writes 8 consecutive columns.
#include "bd_internal.h"

namespace bd {
namespace {

__device__ __forceinline__ float scale_at(const void* s, int sdtype, int mode, int group,
                                          int64_t d_in, int64_t o, int64_t i) {
    int64_t idx = 0;
    if (mode == BD_SCALE_GROUP) idx = o * (d_in / group) + i / group;
    else if (mode == BD_SCALE_ROW) idx = o;
    else if (mode == BD_SCALE_COL) idx = i;
    return sdtype == BD_F16 ? f16_to_f32(((const uint16_t*)s)[idx]) : ((const float*)s)[idx];
}

__global__ void __launch_bounds__(256)
k_reconstruct(const uint64_t* __restrict__ signs, const void* __restrict__ scales, int mode,
              int group, int sdtype, int64_t d_out, int64_t d_in, const void* __restrict__ wb,
              int wdtype, void* __restrict__ out, int odtype) {
    const int64_t per_row = d_in / 8;
    const int64_t total = d_out * per_row;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t o = idx / per_row, i0 = (idx % per_row) * 8;
        const uint32_t byte = (uint32_t)(signs[o * (d_in / 64) + i0 / 64] >> (i0 % 64)) & 0xFFu;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float s = scale_at(scales, sdtype, mode, group, d_in, o, i0 + j);
            float d = ((byte >> j) & 1u) ? s : -s;
            if (wb) {
                const int64_t e = o * d_in + i0 + j;
                const float b = wdtype == BD_BF16 ? __uint_as_float((uint32_t)((const uint16_t*)wb)[e] << 16)
                                                  : ((const float*)wb)[e];
                d = b + d;
            }
            v[j] = d;
        }
        if (odtype == BD_BF16) {
            uint16_t* dst = (uint16_t*)out + o * d_in + i0;
#pragma unroll
            for (int j = 0; j < 8; ++j) dst[j] = f32_to_bf16(v[j]);
        } else {
            float* dst = (float*)out + o * d_in + i0;
#pragma unroll
            for (int j = 0; j < 8; ++j) dst[j] = v[j];
        }
    }
}

}  // namespace

hipError_t launch_reconstruct(const uint64_t* signs, const void* scales, int mode, int group,
                              int sdtype, int64_t d_out, int64_t d_in, const void* wb, int wdtype,
                              void* out, int odtype, hipStream_t s) {
    const int64_t total = d_out * (d_in / 8);
    int64_t nb = (total + 255) / 256;
    if (nb > 65535) nb = 65535;
    hipLaunchKernelGGL(k_reconstruct, dim3((unsigned)nb), dim3(256), 0, s, signs, scales, mode,
                       group, sdtype, d_out, d_in, wb, wdtype, out, odtype);
    return hipGetLastError();
}

}  // namespace bd

namespace bd {
namespace {

__device__ __forceinline__ float load_w(const uint16_t* p, int64_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);  // bf16 -> fp32, exact
}
__device__ __forceinline__ float load_w(const float* p, int64_t i) { return p[i]; }

// INT8 base weights, one block per row: s = max |w| / 127 and q = round-half-even(w / s)
// clamped to [-127, 127], both divisions in binary32 (correctly rounded); a zero row
// gets s = 0 and q = 0.
template <typename WT>
__global__ void __launch_bounds__(256)
k_quantize_rows(const WT* __restrict__ w, int64_t d_in, int8_t* __restrict__ q,
                float* __restrict__ s) {
    __shared__ float sh[256];
    const int64_t o = blockIdx.x;
    const WT* row = w + o * d_in;
    float m = 0.f;
    bool bad = false;
    for (int64_t i = threadIdx.x; i < d_in; i += 256) {
        const float a = fabsf(load_w(row, i));
        bad |= !(a <= 3.402823466e38f);  // NaN or Inf
        m = fmaxf(m, a);
    }
    sh[threadIdx.x] = m;
    const bool anybad = __syncthreads_or((int)bad) != 0;
    for (int k = 128; k > 0; k >>= 1) {
        if ((int)threadIdx.x < k) sh[threadIdx.x] = fmaxf(sh[threadIdx.x], sh[threadIdx.x + k]);
        __syncthreads();
    }
    // a row holding a NaN or Inf weight has no INT8 codes: scale NaN and codes 0, so
    // that its outputs are NaN rather than finite and wrong
    const float so = anybad ? __builtin_nanf("") : sh[0] / 127.0f;
    if (threadIdx.x == 0) s[o] = so;
    for (int64_t i = threadIdx.x; i < d_in; i += 256) {
        float r = so > 0.f ? rintf(load_w(row, i) / so) : 0.f;
        r = fminf(fmaxf(r, -127.f), 127.f);
        q[o * d_in + i] = (int8_t)r;
    }
}

}  // namespace

hipError_t launch_quantize_rows(const void* w, int wdtype, int64_t d_out, int64_t d_in, int8_t* q,
                                float* s, hipStream_t st) {
    if (wdtype == BD_BF16)
        hipLaunchKernelGGL(k_quantize_rows<uint16_t>, dim3((unsigned)d_out), dim3(256), 0, st,
                           (const uint16_t*)w, d_in, q, s);
    else
        hipLaunchKernelGGL(k_quantize_rows<float>, dim3((unsigned)d_out), dim3(256), 0, st,
                           (const float*)w, d_in, q, s);
    return hipGetLastError();
}

}  // namespace bd
