/*
 * synth_host.c -- host side of the seeded synthetic input generator.
 *
 * Built with gcc (no HIP) into libbdsynth_host.so.  Fills host buffers with
 * the element recipes of synth_core.h; the device generator (synth_dev.hip)
 * evaluates the same recipes from the same header, so a tensor, or any row
 * range of it, is bit-identical on both sides.
 *
 * dtype: 0 = fp32, 1 = bf16 (stored as uint16).  Element index of a buffer
 * element j is start + j, so callers can fill any contiguous slice.
 */
#include <stddef.h>
#include <stdint.h>
#include "synth_core.h"

uint64_t bds_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, uint64_t d) {
    return syn_key(seed, a, b, c, d);
}

uint64_t bds_draw(uint64_t key, uint64_t i) { return syn_draw(key, i); }

double bds_uniform(uint64_t key, uint64_t i) { return syn_uniform(key, i); }

double bds_laplace(uint64_t key, uint64_t i) { return syn_laplace(key, i); }

double bds_normal(uint64_t key, uint64_t i) { return syn_normal(key, i); }

void bds_fill_normal(void* dst, int dtype, uint64_t key, uint64_t start, uint64_t n, double sigma) {
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)n; ++j) {
        float v = syn_normal_value(key, start + (uint64_t)j, sigma);
        if (dtype == 1) ((uint16_t*)dst)[j] = syn_f32_to_bf16(v);
        else ((float*)dst)[j] = v;
    }
}

/* dst[j] = round(wbase[j] + perturbation(start + j)); wbase in the same dtype. */
void bds_fill_fine(void* dst, int dtype, const void* wbase, uint64_t key, uint64_t okey,
                   uint64_t start, uint64_t n, double b, uint64_t outlier_thresh53,
                   double outlier_mag) {
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)n; ++j) {
        uint64_t i = start + (uint64_t)j;
        double p = syn_perturb(key, okey, i, b, outlier_thresh53, outlier_mag);
        if (dtype == 1) {
            float wb = syn_bf16_to_f32(((const uint16_t*)wbase)[j]);
            ((uint16_t*)dst)[j] = syn_f32_to_bf16(syn_fine_value(wb, p));
        } else {
            float wb = ((const float*)wbase)[j];
            ((float*)dst)[j] = syn_fine_value(wb, p);
        }
    }
}
