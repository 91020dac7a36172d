/*
 * synth_core.h -- seeded, counter-based synthetic input generator.
 *
 * This header is the ONE definition of the synthetic workload values.  It is
 * compiled twice: by gcc into the host generator (synth_host.c) and by hipcc
 * into the device generator (synth_dev.hip).  It holds none of the BitDelta
 * arithmetic (no delta, sign, scale, clip or apply): only random draws and the
 * rounding of a drawn value to a storage dtype, so that the host side (which
 * feeds the CPU oracle) and the device side (which feeds the GPU library)
 * produce bit-identical tensors without either copying data from the other.
 *
 * Bit-exactness rests on three rules that both compilers honour:
 *   - integer hashing only (SplitMix64) for the random bits;
 *   - every floating-point step is a single IEEE binary64 +, -, * or / in a
 *     fixed order (correctly rounded on both sides); both builds pass
 *     -ffp-contract=off, so no step is fused into an FMA;
 *   - the narrowing to fp32 / bf16 is explicit round-to-nearest-even.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used in its counter form:
 * draw(key, i) = mix64(key + (i + 1) * golden_gamma).
 */
#ifndef TS_SYNTH_CORE_H
#define TS_SYNTH_CORE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYN_FN __host__ __device__ static inline
#else
#define SYN_FN static inline
#endif

#if defined(__clang__)
#define SYN_NO_CONTRACT _Pragma("clang fp contract(off)")
#else
#define SYN_NO_CONTRACT
#endif

#define SYN_GAMMA 0x9E3779B97F4A7C15ULL

/* SplitMix64 finaliser (the published mixing function). */
SYN_FN uint64_t syn_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* i-th 64-bit draw of stream `key`. */
SYN_FN uint64_t syn_draw(uint64_t key, uint64_t i) {
    return syn_mix64(key + (i + 1ULL) * SYN_GAMMA);
}

/* Stream key for one tensor: seed, then up to four small tags. */
SYN_FN uint64_t syn_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, uint64_t d) {
    uint64_t k = syn_mix64(seed + 0x5EEDULL * SYN_GAMMA);
    k = syn_mix64(k ^ (a + 1ULL) * 0xD6E8FEB86659FD93ULL);
    k = syn_mix64(k ^ (b + 1ULL) * 0xC2B2AE3D27D4EB4FULL);
    k = syn_mix64(k ^ (c + 1ULL) * 0x165667B19E3779F9ULL);
    k = syn_mix64(k ^ (d + 1ULL) * 0x27D4EB2F165667C5ULL);
    return k;
}

SYN_FN uint64_t syn_f64_bits(double x) { uint64_t u; __builtin_memcpy(&u, &x, 8); return u; }
SYN_FN double syn_bits_f64(uint64_t u) { double x; __builtin_memcpy(&x, &u, 8); return x; }
SYN_FN uint32_t syn_f32_bits(float x) { uint32_t u; __builtin_memcpy(&u, &x, 4); return u; }

/* Approximately standard normal: centred Irwin-Hall sum of eight 16-bit
 * uniforms, scaled to unit variance (support +-4.9).  The sum is exact; the
 * only rounding is the final multiply by sqrt(3/2). */
SYN_FN double syn_normal(uint64_t key, uint64_t i) {
    SYN_NO_CONTRACT
    uint64_t r0 = syn_draw(key, 2ULL * i), r1 = syn_draw(key, 2ULL * i + 1ULL);
    uint64_t s = 0;
    for (int j = 0; j < 4; ++j) s += ((r0 >> (16 * j)) & 0xFFFFULL) + ((r1 >> (16 * j)) & 0xFFFFULL);
    double u = ((double)s + 4.0) / 65536.0 - 4.0;   /* exact: multiple of 2^-16, |u| < 4 */
    return u * 1.2247448713915890491;               /* sqrt(3/2) */
}

/* Natural log of a in [2^-52, 1], written out from frexp and the atanh series
 * log(m) = 2*atanh((m-1)/(m+1)); the series is cut after z^19 (|z| < 0.172,
 * truncation < 1e-17).  Only IEEE binary64 ops, in a fixed order. */
SYN_FN double syn_log(double a) {
    SYN_NO_CONTRACT
    uint64_t bits = syn_f64_bits(a);
    int e = (int)((bits >> 52) & 0x7FFULL) - 1022;                  /* a normal, > 0 */
    double m = syn_bits_f64((bits & 0x000FFFFFFFFFFFFFULL) | (1022ULL << 52)); /* [0.5,1) */
    if (m < 0.70710678118654752440) { m = m * 2.0; e -= 1; }
    double z = (m - 1.0) / (m + 1.0);
    double w = z * z;
    double p = 1.0 / 19.0;
    p = p * w + 1.0 / 17.0;
    p = p * w + 1.0 / 15.0;
    p = p * w + 1.0 / 13.0;
    p = p * w + 1.0 / 11.0;
    p = p * w + 1.0 / 9.0;
    p = p * w + 1.0 / 7.0;
    p = p * w + 1.0 / 5.0;
    p = p * w + 1.0 / 3.0;
    p = p * w + 1.0;
    return (double)e * 0.69314718055994530942 + (2.0 * z) * p;
}

/* Laplace(0, 1) by inverse CDF from one 52-bit uniform; every step before the
 * log is exact. */
SYN_FN double syn_laplace(uint64_t key, uint64_t i) {
    SYN_NO_CONTRACT
    uint64_t k = syn_draw(key, i) >> 12;                  /* 52 bits */
    double u = ((double)k + 0.5) * (1.0 / 4503599627370496.0); /* (0,1), exact */
    double v = u - 0.5;
    double a = 1.0 - 2.0 * (v < 0.0 ? -v : v);             /* (0,1], exact */
    double mag = -syn_log(a);
    return v < 0.0 ? -mag : mag;
}

/* 53-bit uniform in [0,1). */
SYN_FN double syn_uniform(uint64_t key, uint64_t i) {
    return (double)(syn_draw(key, i) >> 11) * (1.0 / 9007199254740992.0);
}

/* Round-to-nearest-even narrowing (inputs here are always finite). */
SYN_FN float syn_to_f32(double x) { return (float)x; }
SYN_FN uint16_t syn_f32_to_bf16(float f) {
    uint32_t u = syn_f32_bits(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
SYN_FN float syn_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16; float f; __builtin_memcpy(&f, &u, 4); return f;
}

/* ---- the workload's element recipes ------------------------------------ */

/* Element i of a normal tensor N(0, sigma^2) stored as bf16 (dtype 1) or fp32 (0). */
SYN_FN float syn_normal_value(uint64_t key, uint64_t i, double sigma) {
    SYN_NO_CONTRACT
    return syn_to_f32(sigma * syn_normal(key, i));
}

/* Perturbation added to the base weight at element i: Laplace(0, b), and with
 * probability outlier_p (compared as an exact 53-bit integer threshold) the
 * element is replaced by +-outlier_mag with a fair sign. */
SYN_FN double syn_perturb(uint64_t key, uint64_t okey, uint64_t i, double b,
                          uint64_t outlier_thresh53, double outlier_mag) {
    SYN_NO_CONTRACT
    if (outlier_thresh53 != 0ULL) {
        uint64_t q = syn_draw(okey, i);
        if ((q >> 11) < outlier_thresh53) return (q & 1ULL) ? outlier_mag : -outlier_mag;
    }
    return b * syn_laplace(key, i);
}

/* Fine-tuned weight at element i: (wbase + perturbation) computed in binary64,
 * rounded to fp32 (and then to bf16 for bf16 storage). */
SYN_FN float syn_fine_value(float wbase, double pert) {
    SYN_NO_CONTRACT
    return syn_to_f32((double)wbase + pert);
}

#endif /* TS_SYNTH_CORE_H */
