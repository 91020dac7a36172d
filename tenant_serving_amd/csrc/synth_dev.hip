// synth_dev.hip -- device side of the seeded synthetic input generator.
//
// Evaluates the element recipes of synth_core.h on the GPU (built with
// -ffp-contract=off, like the host side), so large workloads are generated in
// HBM without a host round trip while staying bit-identical to the host fills
// that feed the CPU oracle.  dtype: 0 = fp32, 1 = bf16.  Returns 0 on success,
// a hipError_t value otherwise.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "synth_core.h"

namespace {

__global__ void __launch_bounds__(256) k_fill_normal(void* dst, int dtype, uint64_t key, uint64_t start,
                                                     uint64_t n, double sigma) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
        float v = syn_normal_value(key, start + j, sigma);
        if (dtype == 1) ((uint16_t*)dst)[j] = syn_f32_to_bf16(v);
        else ((float*)dst)[j] = v;
    }
}

__global__ void __launch_bounds__(256) k_fill_fine(void* dst, int dtype, const void* wbase, uint64_t key,
                                                   uint64_t okey, uint64_t start, uint64_t n, double b,
                                                   uint64_t thresh, double omag) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
        double p = syn_perturb(key, okey, start + j, b, thresh, omag);
        if (dtype == 1) {
            float wb = syn_bf16_to_f32(((const uint16_t*)wbase)[j]);
            ((uint16_t*)dst)[j] = syn_f32_to_bf16(syn_fine_value(wb, p));
        } else {
            float wb = ((const float*)wbase)[j];
            ((float*)dst)[j] = syn_fine_value(wb, p);
        }
    }
}

unsigned grid_for(uint64_t n) {
    uint64_t g = (n + 255) / 256;
    if (g > 65536) g = 65536;
    if (g == 0) g = 1;
    return (unsigned)g;
}

}  // namespace

extern "C" int bds_dev_fill_normal(void* dst, int dtype, uint64_t key, uint64_t start, uint64_t n,
                                   double sigma, void* stream) {
    if (n == 0) return 0;
    if (!dst || (dtype != 0 && dtype != 1)) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_fill_normal, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, dst, dtype,
                       key, start, n, sigma);
    return (int)hipGetLastError();
}

extern "C" int bds_dev_fill_fine(void* dst, int dtype, const void* wbase, uint64_t key, uint64_t okey,
                                 uint64_t start, uint64_t n, double b, uint64_t thresh, double omag,
                                 void* stream) {
    if (n == 0) return 0;
    if (!dst || !wbase || (dtype != 0 && dtype != 1)) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_fill_fine, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, dst, dtype,
                       wbase, key, okey, start, n, b, thresh, omag);
    return (int)hipGetLastError();
}
