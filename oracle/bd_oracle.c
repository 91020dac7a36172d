/*
 * bd_oracle.c -- plain, slow, CPU reference of the BitDelta hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header or constant with the GPU library (tenant_serving_amd/csrc) and
 * includes nothing from it.  Every step is written out from the method's
 * definition in the order the source pages give it, in binary64 unless a
 * step says otherwise; there is no blocking, fusion or reordering.
 *
 * Sources (web pages on BitDelta):
 *  [P1] "BitDelta (ZIP-7) - Per-User Personalization Without LoRA"
 *       (hanzoskills.com/bitdelta), section "How BitDelta Works" steps 1-5
 *       and "Safety Benefits / 1. Outlier Clipping".
 *  [P2] "BitDelta Guide: 1-Bit Delta Quantization for LLM Serving"
 *       (aifetchly blog), sections "1. Mathematical Formulation",
 *       "2. Optimal L2 Norm Initialization", "Systems Mechanics" 1-2.
 *  [P5] "Per-Axis Weight Deltas for Frequent Model Updates" (ai.info summary
 *       of arXiv 2512.19720), "Key Contributions" 1 and the implementation
 *       details under "Methodology in Plain English".
 *
 * Readings where the pages are silent or disagree (each is listed with its
 * reason in the design notes of the repository):
 *  - sign(0) is +1: the bit is !(delta < 0), so -0.0 and +0.0 map to +1;
 *  - delta is one IEEE binary32 subtraction of the widened inputs;
 *  - clip statistics are whole-matrix mean and unbiased (n-1) std, in
 *    binary64, applied before sign and scale;
 *  - scales are absmean over their unit accumulated in binary64 and rounded
 *    once: fp32 for MATRIX and GROUP, fp16 for ROW (one per output row) and
 *    COL (one per input column);
 *  - groups are g consecutive elements along the input axis (g | d_in);
 *  - packed words are uint64, bit k of word w of row o holds column 64w+k,
 *    bit value 1 meaning +1;
 *  - apply: user id -1 (or any id outside [0, n_users)) gets the base term
 *    only.
 *
 * dtypes: 0 = fp32 (float), 1 = bf16 (uint16 bit pattern), 2 = fp16 (uint16).
 * scale modes: 0 MATRIX, 1 GROUP, 2 ROW, 3 COL.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { O_F32 = 0, O_BF16 = 1, O_F16 = 2 };

/* Threads the parallel loops of orc_apply may use. */
int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
enum { O_MATRIX = 0, O_GROUP = 1, O_ROW = 2, O_COL = 3 };

/* ------------------------------------------------------------ conversions */

/* bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 one. */
static float o_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float o_load(const void* p, int dtype, int64_t i) {
    if (dtype == O_BF16) return o_bf16_to_f32(((const uint16_t*)p)[i]);
    return ((const float*)p)[i];
}

/* binary64 -> IEEE binary16, round to nearest even, written from the format's
 * definition (1 sign, 5 exponent bits with bias 15, 10 fraction bits). */
uint16_t orc_f64_to_f16(double x) {
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (isnan(x)) return 0x7E00u;
    if (a >= 65520.0) return sign | 0x7C00u; /* at or past the midpoint 65504..65536 */
    if (a < 6.103515625e-05) {               /* below 2^-14: subnormal grid 2^-24 */
        double q = rint(a * 16777216.0);     /* exact scaling, RNE */
        return sign | (uint16_t)q;           /* q == 1024 is the smallest normal */
    }
    int e;
    double m = frexp(a, &e);                 /* a = m * 2^e, m in [0.5, 1) */
    double q = rint(ldexp(m, 11));           /* 11 significant bits, RNE */
    if (q == 2048.0) { q = 1024.0; e += 1; }
    int E = e - 1 + 15;
    if (E >= 31) return sign | 0x7C00u;
    return (uint16_t)(sign | (uint16_t)(E << 10) | (uint16_t)((int)q - 1024));
}

double orc_f16_to_f64(uint16_t h) {
    int s = (h >> 15) & 1, E = (h >> 10) & 31, f = h & 1023;
    double v;
    if (E == 0) v = ldexp((double)f, -24);
    else if (E == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), E - 25);
    return s ? -v : v;
}

/* ---------------------------------------------------------------- O1 delta */

/* [P1] step 1 "Delta Computation", [P2] "1. Mathematical Formulation":
 * delta = W_fine - W_base, elementwise.  One binary32 subtraction of the
 * widened inputs.  wb == NULL means wf already holds the delta. */
void orc_delta(const void* wf, const void* wb, int dtype, int64_t n, float* delta) {
    for (int64_t i = 0; i < n; ++i) {
        float f = o_load(wf, dtype, i);
        delta[i] = wb ? f - o_load(wb, dtype, i) : f;
    }
}

/* Number of non-finite deltas (NaN or Inf inputs). */
int64_t orc_count_nonfinite(const float* delta, int64_t n) {
    int64_t c = 0;
    for (int64_t i = 0; i < n; ++i) c += !isfinite(delta[i]);
    return c;
}

/* ----------------------------------------------------------- O2 clipping */

/* [P1] "Outlier Clipping": mean = delta.mean(), std = delta.std(),
 * clamp(delta, mean - k*std, mean + k*std); default k = 3.  Two passes in
 * binary64, sample (n-1) standard deviation.  out = {mu, sigma, lo, hi}. */
void orc_clip_stats(const float* delta, int64_t n, double k, double* out) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += (double)delta[i];
    double mu = s / (double)n;
    double m2 = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double d = (double)delta[i] - mu;
        m2 += d * d;
    }
    double sigma = sqrt(m2 / (double)(n - 1));
    out[0] = mu;
    out[1] = sigma;
    out[2] = mu - k * sigma;
    out[3] = mu + k * sigma;
}

/* dc = clamp(delta, lo, hi) in binary64, or the delta itself when clip == 0. */
void orc_clamp(const float* delta, int64_t n, int clip, double lo, double hi, double* dc) {
    for (int64_t i = 0; i < n; ++i) {
        double d = (double)delta[i];
        if (clip) {
            if (d < lo) d = lo;
            if (d > hi) d = hi;
        }
        dc[i] = d;
    }
}

/* ------------------------------------------------------- O3/O4 signs, bits */

int64_t orc_words_per_row(int64_t d_in) { return (d_in + 63) / 64; }

/* [P2] "1. Mathematical Formulation": Sign(delta) in {-1,+1}, one bit per
 * weight, bit 1 <-> +1; [P2] "Systems Mechanics 2" and [P5] implementation
 * details: bits packed along the input axis.  Zero maps to +1. */
void orc_pack_signs(const double* dc, int64_t d_out, int64_t d_in, uint64_t* words) {
    int64_t wpr = orc_words_per_row(d_in);
    for (int64_t o = 0; o < d_out; ++o) {
        for (int64_t w = 0; w < wpr; ++w) {
            uint64_t word = 0;
            for (int64_t k = 0; k < 64; ++k) {
                int64_t i = 64 * w + k;
                if (i < d_in && !(dc[o * d_in + i] < 0.0)) word |= (uint64_t)1 << k;
            }
            words[o * wpr + w] = word;
        }
    }
}

/* ------------------------------------------------------------- O5 scales */

int64_t orc_scales_count(int mode, int64_t d_out, int64_t d_in, int64_t g) {
    switch (mode) {
        case O_MATRIX: return 1;
        case O_GROUP: return d_out * (d_in / g);
        case O_ROW: return d_out;
        case O_COL: return d_in;
    }
    return -1;
}

static void o_store_scale(void* scales, int sdtype, int64_t idx, double v) {
    if (sdtype == O_F16) ((uint16_t*)scales)[idx] = orc_f64_to_f16(v);
    else ((float*)scales)[idx] = (float)v;
}

/* Absmean over each scale unit: [P2] "2. Optimal L2 Norm Initialization"
 * (alpha = mean |delta| over the matrix minimises ||delta - alpha Sign||_F^2),
 * [P1] step 2 "Group Quantization" (per group of g elements), [P5] "Key
 * Contributions" 1 (one value per output row, 1 x d_out, or per input column,
 * d_in x 1).  The per-axis values are the same closed form restricted to the
 * axis.  Sum in binary64 in index order, divide, round once. */
void orc_absmean_scales(const double* dc, int64_t d_out, int64_t d_in, int mode, int64_t g,
                        int sdtype, void* scales) {
    if (mode == O_MATRIX) {
        double s = 0.0;
        for (int64_t i = 0; i < d_out * d_in; ++i) s += fabs(dc[i]);
        o_store_scale(scales, sdtype, 0, s / (double)(d_out * d_in));
    } else if (mode == O_GROUP) {
        int64_t gpr = d_in / g;
        for (int64_t o = 0; o < d_out; ++o)
            for (int64_t j = 0; j < gpr; ++j) {
                double s = 0.0;
                for (int64_t k = 0; k < g; ++k) s += fabs(dc[o * d_in + j * g + k]);
                o_store_scale(scales, sdtype, o * gpr + j, s / (double)g);
            }
    } else if (mode == O_ROW) {
        for (int64_t o = 0; o < d_out; ++o) {
            double s = 0.0;
            for (int64_t i = 0; i < d_in; ++i) s += fabs(dc[o * d_in + i]);
            o_store_scale(scales, sdtype, o, s / (double)d_in);
        }
    } else if (mode == O_COL) {
        for (int64_t i = 0; i < d_in; ++i) {
            double s = 0.0;
            for (int64_t o = 0; o < d_out; ++o) s += fabs(dc[o * d_in + i]);
            o_store_scale(scales, sdtype, i, s / (double)d_out);
        }
    }
}

/* Whole compression of one matrix: O1, O2 (when clip_k > 0), O3-O5.
 * stats (may be NULL) receives {mu, sigma, lo, hi} (zeros without clip).
 * Returns the number of non-finite deltas, or -1 on allocation failure. */
int64_t orc_compress(const void* wf, const void* wb, int dtype, int64_t d_out, int64_t d_in,
                     int mode, int64_t g, double clip_k, int sdtype, uint64_t* words,
                     void* scales, double* stats) {
    int64_t n = d_out * d_in;
    float* delta = (float*)malloc(sizeof(float) * (size_t)n);
    double* dc = (double*)malloc(sizeof(double) * (size_t)n);
    if (!delta || !dc) {
        free(delta);
        free(dc);
        return -1;
    }
    orc_delta(wf, wb, dtype, n, delta);
    int64_t bad = orc_count_nonfinite(delta, n);
    double st[4] = {0.0, 0.0, 0.0, 0.0};
    int clip = clip_k > 0.0;
    if (clip) orc_clip_stats(delta, n, clip_k, st);
    orc_clamp(delta, n, clip, st[2], st[3], dc);
    orc_pack_signs(dc, d_out, d_in, words);
    orc_absmean_scales(dc, d_out, d_in, mode, g, sdtype, scales);
    if (stats) memcpy(stats, st, sizeof st);
    free(delta);
    free(dc);
    return bad;
}

/* ------------------------------------------------- O7 per-layer axis choice */

/* [P5] "Key Contributions" 1-2: one scale vector per layer, per output row or per
 * input column, the axis chosen per layer.  The page keeps the axis with the lower
 * validation loss; without data this reading keeps the axis whose absmean
 * reconstruction s * sign(d) is closer to the (clipped, as in compression) delta in
 * the Frobenius norm.  The errors are summed element by element over both
 * reconstructions, in binary64:
 *     err_row = sum_o sum_i (dc[o][i] - srow[o] * sign(dc[o][i]))^2,  srow[o] = mean_i |dc[o][i]|
 *     err_col = sum_o sum_i (dc[o][i] - scol[i] * sign(dc[o][i]))^2,  scol[i] = mean_o |dc[o][i]|
 * with sign(0) = +1.  Ties keep ROW.  out = {err_row, err_col, axis (2 ROW, 3 COL)}.
 * Returns the number of non-finite deltas, or -1 on allocation failure. */
int64_t orc_select_axis(const void* wf, const void* wb, int dtype, int64_t d_out, int64_t d_in,
                        double clip_k, double* out) {
    int64_t n = d_out * d_in;
    float* delta = (float*)malloc(sizeof(float) * (size_t)n);
    double* dc = (double*)malloc(sizeof(double) * (size_t)n);
    double* srow = (double*)calloc((size_t)d_out, sizeof(double));
    double* scol = (double*)calloc((size_t)d_in, sizeof(double));
    if (!delta || !dc || !srow || !scol) {
        free(delta);
        free(dc);
        free(srow);
        free(scol);
        return -1;
    }
    orc_delta(wf, wb, dtype, n, delta);
    int64_t bad = orc_count_nonfinite(delta, n);
    double st[4] = {0.0, 0.0, 0.0, 0.0};
    int clip = clip_k > 0.0;
    if (clip) orc_clip_stats(delta, n, clip_k, st);
    orc_clamp(delta, n, clip, st[2], st[3], dc);
    for (int64_t o = 0; o < d_out; ++o)
        for (int64_t i = 0; i < d_in; ++i) {
            srow[o] += fabs(dc[o * d_in + i]);
            scol[i] += fabs(dc[o * d_in + i]);
        }
    for (int64_t o = 0; o < d_out; ++o) srow[o] /= (double)d_in;
    for (int64_t i = 0; i < d_in; ++i) scol[i] /= (double)d_out;
    double er = 0.0, ec = 0.0;
    for (int64_t o = 0; o < d_out; ++o)
        for (int64_t i = 0; i < d_in; ++i) {
            double d = dc[o * d_in + i];
            double sg = d < 0.0 ? -1.0 : 1.0;
            double a = d - srow[o] * sg, b = d - scol[i] * sg;
            er += a * a;
            ec += b * b;
        }
    out[0] = er;
    out[1] = ec;
    out[2] = er <= ec ? (double)O_ROW : (double)O_COL;
    free(delta);
    free(dc);
    free(srow);
    free(scol);
    return bad;
}

/* -------------------------------------------------------- O6 reconstruct */

static double o_scale_at(const void* scales, int mode, int64_t g, int sdtype, int64_t d_in,
                         int64_t o, int64_t i) {
    int64_t idx = 0;
    switch (mode) {
        case O_MATRIX: idx = 0; break;
        case O_GROUP: idx = o * (d_in / g) + i / g; break;
        case O_ROW: idx = o; break;
        case O_COL: idx = i; break;
    }
    if (sdtype == O_F16) return orc_f16_to_f64(((const uint16_t*)scales)[idx]);
    return (double)((const float*)scales)[idx];
}

static double o_sign_at(const uint64_t* words, int64_t wpr, int64_t o, int64_t i) {
    return ((words[o * wpr + i / 64] >> (i % 64)) & 1) ? 1.0 : -1.0;
}

/* [P1] step 4 "Reconstruction": reconstructed = signs * scales; [P1] step 5
 * "Serving": user weight = base + signs * scales.  out[o][i] in binary64;
 * wb == NULL gives the reconstructed delta alone. */
void orc_reconstruct(const uint64_t* words, const void* scales, int mode, int64_t g, int sdtype,
                     int64_t d_out, int64_t d_in, const void* wb, int wdtype, double* out) {
    int64_t wpr = orc_words_per_row(d_in);
    for (int64_t o = 0; o < d_out; ++o)
        for (int64_t i = 0; i < d_in; ++i) {
            double d = o_sign_at(words, wpr, o, i) * o_scale_at(scales, mode, g, sdtype, d_in, o, i);
            out[o * d_in + i] = wb ? (double)o_load(wb, wdtype, o * d_in + i) + d : d;
        }
}

/* ------------------------------------------------------------- O7 apply */

/* [P2] "Systems Mechanics 1": Y_i = W_base X_i + Delta_hat_i X_i for each
 * request i with its own delta; the plain definition is
 * y[t][o] = sum_i x[t][i] * (W_base[o][i] + Delta_hat_{u(t)}[o][i]).
 *
 * The caller passes only the output rows it wants: wb is [n_rows][d_in] (the
 * base rows), words_bank is [n_users][n_rows][wpr] (those rows of each
 * user's signs) and scales_bank per user holds MATRIX: 1, GROUP:
 * [n_rows][d_in/g], ROW: [n_rows], COL: [d_in] values.  y, y_base and y_delta
 * are [T][n_rows] binary64 (y_base / y_delta may be NULL). */
void orc_apply(const void* x, int xdtype, int64_t T, int64_t d_in, const void* wb, int wdtype,
               int64_t n_rows, const uint64_t* words_bank, const void* scales_bank, int mode,
               int64_t g, int sdtype, int32_t n_users, const int32_t* user_ids, double* y,
               double* y_base, double* y_delta) {
    int64_t wpr = orc_words_per_row(d_in);
    int64_t spu = orc_scales_count(mode, n_rows, d_in, g);
    size_t ssz = (sdtype == O_F16) ? 2 : 4;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        int32_t u = user_ids[t];
        int has = u >= 0 && u < n_users;
        const uint64_t* wu = has ? words_bank + (int64_t)u * n_rows * wpr : NULL;
        const void* su = has ? (const void*)((const char*)scales_bank + (size_t)u * spu * ssz) : NULL;
        for (int64_t o = 0; o < n_rows; ++o) {
            double full = 0.0, base = 0.0, delta = 0.0;
            for (int64_t i = 0; i < d_in; ++i) {
                double xv = (double)o_load(x, xdtype, t * d_in + i);
                double wv = (double)o_load(wb, wdtype, o * d_in + i);
                double dv = has ? o_sign_at(wu, wpr, o, i) * o_scale_at(su, mode, g, sdtype, d_in, o, i) : 0.0;
                full += xv * (wv + dv);
                base += xv * wv;
                delta += xv * dv;
            }
            y[t * n_rows + o] = full;
            if (y_base) y_base[t * n_rows + o] = base;
            if (y_delta) y_delta[t * n_rows + o] = delta;
        }
    }
}

/* ---------------------------------------------- O8 quantized base weights */

/* [P2] "Systems Mechanics" (production notes): the 1-bit delta applied on an INT8
 * base.  The page names no quantizer; this reading is symmetric per output row:
 * s[o] = max_i |w[o][i]| / 127 and q[o][i] = round-half-even(w[o][i] / s[o]) clamped
 * to [-127, 127], both divisions in binary32 (a zero row gets s = 0 and q = 0). */
void orc_quantize_rows(const void* w, int dtype, int64_t d_out, int64_t d_in, int8_t* q,
                       float* s) {
    for (int64_t o = 0; o < d_out; ++o) {
        float m = 0.0f;
        int finite = 1;
        for (int64_t i = 0; i < d_in; ++i) {
            float a = fabsf(o_load(w, dtype, o * d_in + i));
            if (!isfinite(a)) finite = 0;
            if (a > m) m = a;
        }
        /* a row holding a NaN or Inf weight has no INT8 codes: scale NaN, codes 0, so
         * that its outputs are NaN rather than finite and wrong */
        float so = finite ? m / 127.0f : NAN;
        s[o] = so;
        for (int64_t i = 0; i < d_in; ++i) {
            float v = so > 0.0f ? o_load(w, dtype, o * d_in + i) / so : 0.0f;
            float r = rintf(v);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[o * d_in + i] = (int8_t)r;
        }
    }
}

/* The apply of orc_apply with the base weight given as (q, s): for every token t and
 * row o, base = s[o] * sum_i x[t][i] q[o][i], delta as in orc_apply, y = base + delta,
 * in binary64. */
void orc_apply_q8(const void* x, int xdtype, int64_t T, int64_t d_in, const int8_t* q,
                  const float* s, int64_t n_rows, const uint64_t* words_bank,
                  const void* scales_bank, int mode, int64_t g, int sdtype, int32_t n_users,
                  const int32_t* user_ids, double* y, double* y_base, double* y_delta) {
    int64_t wpr = orc_words_per_row(d_in);
    int64_t spu = orc_scales_count(mode, n_rows, d_in, g);
    size_t ssz = (sdtype == O_F16) ? 2 : 4;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        int32_t u = user_ids[t];
        int has = u >= 0 && u < n_users;
        const uint64_t* wu = has ? words_bank + (int64_t)u * n_rows * wpr : NULL;
        const void* su = has ? (const void*)((const char*)scales_bank + (size_t)u * spu * ssz) : NULL;
        for (int64_t o = 0; o < n_rows; ++o) {
            double base = 0.0, delta = 0.0;
            for (int64_t i = 0; i < d_in; ++i) {
                double xv = (double)o_load(x, xdtype, t * d_in + i);
                base += xv * (double)q[o * d_in + i];
                if (has) delta += xv * o_sign_at(wu, wpr, o, i) * o_scale_at(su, mode, g, sdtype, d_in, o, i);
            }
            base *= (double)s[o];
            y[t * n_rows + o] = base + delta;
            if (y_base) y_base[t * n_rows + o] = base;
            if (y_delta) y_delta[t * n_rows + o] = delta;
        }
    }
}
