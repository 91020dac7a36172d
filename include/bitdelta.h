/*
 * bitdelta.h -- C ABI of libbitdelta.so: BitDelta compression of fine-tune
 * deltas and multi-tenant application of many users' 1-bit deltas on one
 * shared base weight, on AMD Instinct MI355X (gfx950).
 *
 * The operations are those described on the pages
 *  [P1] "BitDelta (ZIP-7) - Per-User Personalization Without LoRA"
 *       (hanzoskills.com/bitdelta), "How BitDelta Works" steps 1-5,
 *       "Safety Benefits / 1. Outlier Clipping" and "Production Serving";
 *  [P2] "BitDelta Guide: 1-Bit Delta Quantization for LLM Serving"
 *       (aifetchly blog), "1. Mathematical Formulation", "2. Optimal L2 Norm
 *       Initialization", "Systems Mechanics: Fused 1-Bit GEMM and
 *       Multi-Tenant Serving Runtimes" 1-3;
 *  [P5] "Per-Axis Weight Deltas for Frequent Model Updates" (ai.info summary
 *       of arXiv 2512.19720), "Key Contributions" 1 and 4 and the implementation
 *       details under "Methodology in Plain English".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Weights use the nn.Linear layout W[d_out][d_in], row-major; activations
 *    X[T][d_in]; outputs Y[T][d_out].
 *  - Every pointer except the host-side `params` structs is a DEVICE pointer
 *    owned by the caller.  The library never allocates, frees or keeps device
 *    memory (the one exception: the static scratch of bd_apply_noalloc); scratch
 *    space is the caller's `workspace`, sized by the *_workspace_bytes queries.
 *  - `stream` is a hipStream_t passed as an opaque pointer (NULL = the null
 *    stream).  All work is enqueued on it; no entry point synchronises except
 *    bd_device_status.  Calls are re-entrant: no global mutable state.
 *  - Argument and shape errors are returned synchronously before anything is
 *    enqueued.  Data-dependent errors (non-finite delta, out-of-range user id)
 *    are recorded in a status word inside the workspace and read back with
 *    bd_device_status after the call.
 *  - Sign convention: bit 1 <-> +1, bit 0 <-> -1 ([P2] "1. Mathematical
 *    Formulation"); a zero delta (+0 or -0) maps to +1, i.e. the bit is
 *    !(delta < 0).
 *  - Packed signs: uint64 signs[d_out][d_in/64]; bit k of word w of row o is
 *    the sign of column 64*w + k (bits packed along the input axis, [P2]
 *    "Systems Mechanics 2", [P5] implementation details).
 */
#ifndef BITDELTA_H
#define BITDELTA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BD_ABI_VERSION 3

typedef enum {
    BD_OK = 0,
    BD_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad enum value */
    BD_ERR_SHAPE = 2,       /* d_in % 64 != 0, d_in % group_size != 0, too few elements to clip */
    BD_ERR_DTYPE = 3,       /* dtype not accepted for that argument */
    BD_ERR_UNSUPPORTED = 4, /* bits != 1, group_size not a power of two in [8, 512] */
    BD_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the query returns */
    BD_ERR_DEVICE = 6,      /* a HIP call or launch failed */
    BD_ERR_NONFINITE = 7,   /* (async) a delta was NaN or Inf */
    BD_ERR_USER_ID = 8,     /* (async) a user id outside [-1, n_users) */
    BD_ERR_BATCH = 9        /* (async) delta products asked of a prepared batch whose tokens
                               were encoded for another scale mode (bd_batch_encode) */
} bd_status;

typedef enum { BD_F32 = 0, BD_BF16 = 1, BD_F16 = 2 } bd_dtype;

/* Scale unit of the absmean magnitude.
 *  MATRIX: one value for the whole matrix ([P2] "2. Optimal L2 Norm
 *          Initialization": alpha = mean |delta|).
 *  GROUP:  one value per group of `group_size` consecutive elements along the
 *          input axis, stored [d_out][d_in/group_size] ([P1] step 2 "Group
 *          Quantization").
 *  ROW:    one value per output row, [d_out] (the 1 x d_out vector of [P5]
 *          "Key Contributions" 1).
 *  COL:    one value per input column, [d_in] (the d_in x 1 vector). */
typedef enum {
    BD_SCALE_MATRIX = 0,
    BD_SCALE_GROUP = 1,
    BD_SCALE_ROW = 2,
    BD_SCALE_COL = 3
} bd_scale_mode;

typedef struct {
    int32_t bits;        /* must be 1 */
    int32_t mode;        /* bd_scale_mode */
    int32_t group_size;  /* GROUP only: power of two in [8, 512], divides d_in */
    float clip_k;        /* 0: no clipping; > 0: clamp delta to mean +- clip_k * std first */
    int32_t scale_dtype; /* BD_F32 or BD_F16 */
} bd_compress_params;

/* ---------------------------------------------------------------- queries */

int bd_abi_version(void);
const char* bd_status_string(bd_status s);

/* Bytes of one matrix's packed signs: d_out * d_in / 8 (d_in % 64 == 0), or 0
 * for invalid sizes. */
size_t bd_signs_bytes(int64_t d_out, int64_t d_in);

/* Number of scale values of one matrix for params p (MATRIX 1, GROUP
 * d_out*d_in/group_size, ROW d_out, COL d_in); -1 if p is invalid. */
int64_t bd_scales_count(const bd_compress_params* p, int64_t d_out, int64_t d_in);

/* Workspace bytes bd_compress needs for this shape (0 if invalid). */
size_t bd_compress_workspace_bytes(const bd_compress_params* p, int64_t d_out, int64_t d_in);

/* Workspace bytes bd_select_axis needs for this shape and clip_k (0 if invalid). */
size_t bd_select_axis_workspace_bytes(int64_t d_out, int64_t d_in, float clip_k);

/* Workspace bytes bd_apply needs (0 if invalid). */
size_t bd_apply_workspace_bytes(const bd_compress_params* p, int64_t T, int32_t n_users,
                                int64_t d_out, int64_t d_in, bd_dtype x_dtype, bd_dtype y_dtype);

/* ------------------------------------------------------------ compression */

/* Compress one user's fine-tune delta of one matrix.
 *
 * Computes delta = W_fine - W_base ([P1] step 1, [P2] "1. Mathematical
 * Formulation") as one binary32 subtraction of the widened inputs; when
 * p->clip_k > 0 clamps it to [mu - k*sigma, mu + k*sigma] with the
 * whole-matrix mean and unbiased standard deviation computed in binary64 in
 * two passes ([P1] "Outlier Clipping"); writes the packed signs of the clamped
 * delta ([P1] step 3, [P2] Sign) and the absmean of |clamped delta| over each
 * scale unit, accumulated in binary64 and rounded once to p->scale_dtype
 * ([P2] "2. Optimal L2 Norm Initialization", [P1] step 2, [P5] "Key
 * Contributions" 1).
 *
 *  w_fine, w_base : [d_out][d_in] of w_dtype (BD_F32 or BD_BF16); w_base may
 *                   be NULL, then w_fine already holds the delta.
 *  signs_out      : bd_signs_bytes(d_out, d_in) bytes, layout above.
 *  scales_out     : bd_scales_count(p, ...) values of p->scale_dtype.
 *  workspace      : >= bd_compress_workspace_bytes(p, d_out, d_in) bytes,
 *                   256-byte aligned; its status word is reset by the call.
 * Requires d_in % 64 == 0, d_out >= 1; with clipping d_out*d_in >= 2.
 * A NaN/Inf delta sets BD_ERR_NONFINITE in the status word (outputs are then
 * unspecified). */
bd_status bd_compress(const void* w_fine, const void* w_base, bd_dtype w_dtype, int64_t d_out,
                      int64_t d_in, const bd_compress_params* p, uint64_t* signs_out,
                      void* scales_out, void* workspace, size_t ws_bytes, void* stream);

/* Per-layer choice between per-row and per-column scales, without data.
 *
 * [P5] "Key Contributions" 1-2 store one scale vector per layer, either per
 * output row or per input column, and keep, per layer, the axis whose model
 * has the lower validation loss.  Without data this call keeps the axis whose
 * absmean reconstruction s (.) sign(delta) is closer to the delta in the
 * Frobenius norm, over the same delta and clipping bd_compress uses.  For a
 * unit (row or column) of n deltas with absmean s = sum|d| / n the squared
 * error is sum d^2 - (sum |d|)^2 / n, so one pass over the delta gives both:
 *     err_row = sum d^2 - sum over rows    (sum |d|)^2 / d_in
 *     err_col = sum d^2 - sum over columns (sum |d|)^2 / d_out
 * and the axis is BD_SCALE_ROW when err_row <= err_col, else BD_SCALE_COL.
 * Every sum is binary64 in a fixed order, so repeated calls agree bit for bit.
 *
 *  w_fine, w_base, w_dtype, d_out, d_in : as in bd_compress.
 *  clip_k    : as bd_compress_params.clip_k (0 = no clipping).
 *  errors    : device double[2] = {err_row, err_col}, or NULL.
 *  axis      : device int32 = BD_SCALE_ROW or BD_SCALE_COL, or NULL.
 *  workspace : >= bd_select_axis_workspace_bytes(d_out, d_in, clip_k) bytes,
 *              256-byte aligned; its status word is reset by the call.
 * Same shape rules as bd_compress.  A NaN/Inf delta sets BD_ERR_NONFINITE in
 * the status word (the errors are then NaN and the axis BD_SCALE_COL). */
bd_status bd_select_axis(const void* w_fine, const void* w_base, bd_dtype w_dtype, int64_t d_out,
                         int64_t d_in, float clip_k, double* errors, int32_t* axis,
                         void* workspace, size_t ws_bytes, void* stream);

/* -------------------------------------------------------- reconstruction */

/* Dense reconstruction ([P1] step 4 "Reconstruction", step 5 "Serving"):
 * out[o][i] = (w_base ? w_base[o][i] : 0) + sign(o,i) * scale(o,i), summed in
 * fp32 and rounded once to out_dtype (BD_F32 or BD_BF16).  w_base (of
 * w_dtype, BD_F32 or BD_BF16) may be NULL.  Not on the serving hot path: the
 * apply below never materialises this. */
bd_status bd_reconstruct(const uint64_t* signs, const void* scales, const bd_compress_params* p,
                         int64_t d_out, int64_t d_in, const void* w_base, bd_dtype w_dtype,
                         void* out, bd_dtype out_dtype, void* stream);

/* ------------------------------------------------------------------ apply */

/* Multi-tenant forward of one linear layer ([P2] "Systems Mechanics" 1-2):
 *     y[t] = X[t] . W_base^T + scale_u (.) (X[t] . S_u^T),   u = user_ids[t],
 * with the base product computed once for the whole batch and each user's
 * packed signs streamed from HBM and expanded on chip, never materialising a
 * dense per-user weight.  The scale enters per mode: MATRIX/ROW multiply the
 * signed sum, GROUP multiplies each group's partial sum, COL scales X before
 * the signed sum.
 *
 *  x           : [T][d_in] of x_dtype (BD_BF16, or BD_F32 with fp32 w_base).
 *  w_base      : [d_out][d_in], same dtype as x.
 *  signs_bank  : [n_users][d_out][d_in/64] uint64, one bd_compress output per
 *                user, back to back.
 *  scales_bank : [n_users][bd_scales_count(p, d_out, d_in)] of p->scale_dtype.
 *  user_ids    : device int32[T]; -1 = base model only; any other id outside
 *                [0, n_users) also gets the base term only and sets
 *                BD_ERR_USER_ID in the status word.
 *  y           : [T][d_out] of y_dtype (BD_F32, or BD_BF16 rounded once from
 *                the fp32 result).
 *  workspace   : >= bd_apply_workspace_bytes(...) bytes, 256-byte aligned.
 * Accumulation is fp32.  T == 0 is a no-op.  bf16 inputs: T <= 8192 tokens
 * per call (BD_ERR_UNSUPPORTED otherwise).  The matrix-core delta products scale
 * whole 128-column products: bf16 GROUP scales with groups of 8..64 columns take a
 * plain kernel instead (one thread per token and row summing each group in fp32;
 * correct at any size, several times slower than groups of 128 or more).
 * bf16 batches of 1..16 tokens with MATRIX, ROW or COL scales take the decode path:
 * for MATRIX or ROW scales and d_in <= 5120 one launch that writes only y and the
 * status word (the workspace is NOT left prepared for bd_decode_apply; callers
 * that share one batch across matrices call bd_decode_prepare themselves), else
 * bd_decode_prepare + bd_decode_apply on the workspace.  The one-launch kernels
 * encode the tokens differently from bd_decode_prepare, so the two agree within
 * the bf16 tolerance, not bit for bit.  Every other batch is computed as
 * bd_batch_prepare + bd_base_gemm + bd_delta_apply (+ a cast for bf16 y) on one
 * workspace. */
bd_status bd_apply(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in, const void* w_base,
                   int64_t d_out, const uint64_t* signs_bank, const void* scales_bank,
                   const bd_compress_params* p, int32_t n_users, const int32_t* user_ids, void* y,
                   bd_dtype y_dtype, void* workspace, size_t ws_bytes, void* stream);

/* bd_apply on banks held in a resident pool of slots: the deltas of a bounded set of
 * users stay in HBM while the rest wait in host memory and are swapped in per
 * request ([P2] "Systems Mechanics" 3, dynamic hot-swapping: deltas cached in the
 * GPU's spare memory or streamed from host memory; [P1] "Production Serving": the
 * base model stays on the GPU, the deltas in CPU memory; [P5] "Key Contributions" 4:
 * a user's packed delta of a module moves in one transfer).  A module's slot holds
 * each of its matrices' signs and scales at fixed offsets, so one copy fills a slot
 * and the banks of one matrix are strided through the pool.
 *
 *  signs_pool    : signs of slot 0 of this matrix; slot k's at signs_pool +
 *                  k * signs_stride bytes ([d_out][d_in/64] uint64 each).
 *  scales_pool   : scales of slot 0; slot k's at scales_pool + k * scales_stride
 *                  bytes (bd_scales_count values of p->scale_dtype each).
 *  signs_stride, scales_stride : bytes between slots, multiples of 16 and at least
 *                  one slot's signs / scales; 0 = a dense bank ([n_slots][...]).
 *  n_slots       : slots of the pool.
 *  slot_of_user  : device int32[n_users], the slot of each user, or -1 for a user
 *                  without one (not resident).
 *  user_ids      : device int32[T] user ids as for bd_apply (-1: base model only).
 *                  A token whose user has no slot, or whose id is outside
 *                  [-1, n_users), gets the base product only and sets
 *                  BD_ERR_USER_ID in the status word.
 *  workspace     : >= bd_apply_paged_workspace_bytes(...) bytes, 256-byte aligned.
 * The slot of every token's user is looked up once per call (one small launch); the
 * call is then bd_apply over the slots, with every other argument, result and error
 * as for bd_apply.  The pool, table and ids are only read: filling slots and the
 * table (and not overwriting a slot that an earlier call on another stream still
 * reads) is the caller's. */
size_t bd_apply_paged_workspace_bytes(const bd_compress_params* p, int64_t T, int32_t n_slots,
                                      int64_t d_out, int64_t d_in, bd_dtype x_dtype,
                                      bd_dtype y_dtype);
bd_status bd_apply_paged(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                         const void* w_base, int64_t d_out, const uint64_t* signs_pool,
                         const void* scales_pool, uint64_t signs_stride, uint64_t scales_stride,
                         int32_t n_slots, const bd_compress_params* p,
                         const int32_t* slot_of_user, int32_t n_users, const int32_t* user_ids,
                         void* y, bd_dtype y_dtype, void* workspace, size_t ws_bytes,
                         void* stream);

/* bd_apply for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): no workspace
 * argument and no allocation of any kind.  The launches use a scratch array of the
 * library, BD_NOALLOC_SCRATCH_BYTES per device (held by every device the library runs
 * on until the process ends); a call whose bd_apply workspace would be larger
 * (bd_apply_workspace_bytes) returns BD_ERR_WORKSPACE and enqueues nothing.  Every
 * call on one device shares that device's scratch: calls that overlap on one device
 * (other streams, other host threads) race and give undefined results; calls in
 * order on one stream are safe.  status (device uint32, may be NULL) receives the
 * call's status word as written to a workspace by bd_apply (read it as bd_device_status
 * would: bit 0 non-finite, bit 1 user id, bit 2 batch); other arguments, results and
 * errors as for
 * bd_apply. */
#define BD_NOALLOC_SCRATCH_BYTES (8u << 20)
bd_status bd_apply_noalloc(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                           const void* w_base, int64_t d_out, const uint64_t* signs_bank,
                           const void* scales_bank, const bd_compress_params* p,
                           int32_t n_users, const int32_t* user_ids, void* y, bd_dtype y_dtype,
                           uint32_t* status, void* stream);

/* The three phases of bd_apply, for callers that apply many matrices to one
 * batch (e.g. q, k and v read the same X and the same user ids): prepare the
 * batch once, then run the shared base product and the per-user delta product
 * of each matrix ([P2] "Systems Mechanics" 1: Y = Y_base + Y_delta). */

/* ------------------------------------------------- INT8 base weights */

/* INT8 base weights for the apply below ([P2] "Production Engineering" 3, Quantized
 * Base Model Compatibility: the 1-bit delta on top of an INT8-quantized base).  The pages name no quantizer; this one is
 * symmetric per output row: scales_out[o] = max_i |w[o][i]| / 127 and
 * q_out[o][i] = round-half-even(w[o][i] / scales_out[o]) clamped to [-127, 127],
 * both divisions in binary32 (a zero row gets scale 0 and codes 0; a row holding a
 * NaN or Inf weight gets scale NaN and codes 0, so that its outputs are NaN).
 *  w          : [d_out][d_in] of w_dtype (BD_F32 or BD_BF16).
 *  q_out      : [d_out][d_in] int8.   scales_out : [d_out] fp32. */
bd_status bd_quantize_base(const void* w, bd_dtype w_dtype, int64_t d_out, int64_t d_in,
                           int8_t* q_out, float* scales_out, void* stream);

/* bd_apply with the base weight given as INT8 rows (bd_quantize_base):
 *     y[t] = wscales (.) (X[t] . wq^T) + scale_u (.) (X[t] . S_u^T),
 * bf16 X only (BD_ERR_UNSUPPORTED for fp32).  Decode batches (1..16 tokens, MATRIX or
 * ROW scales, d_in <= 4096) take one launch; every other batch (any scale mode, up
 * to 8192 tokens, d_in a multiple of 64) the prepared-batch path of bd_apply with the
 * base product on the matrix cores from the codes.  The base weight crosses HBM at
 * one byte per element; its codes are widened to bf16 exactly on chip and each row's
 * sum is scaled once.  workspace: >= bd_apply_q8_workspace_bytes(...) bytes; other
 * arguments and the status word as for bd_apply. */
size_t bd_apply_q8_workspace_bytes(const bd_compress_params* p, int64_t T, int32_t n_users,
                                   int64_t d_out, int64_t d_in, bd_dtype x_dtype,
                                   bd_dtype y_dtype);
bd_status bd_apply_q8(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in, const int8_t* wq,
                      const float* wscales, int64_t d_out, const uint64_t* signs_bank,
                      const void* scales_bank, const bd_compress_params* p, int32_t n_users,
                      const int32_t* user_ids, void* y, bd_dtype y_dtype, void* workspace,
                      size_t ws_bytes, void* stream);

/* Workspace of a prepared batch: the grouping of the tokens by user and, for
 * bf16 inputs, room for the tokens encoded as delta-product operands. */
size_t bd_batch_workspace_bytes(int64_t T, int32_t n_users, int64_t d_in, bd_dtype x_dtype);

/* Groups the T tokens by user id (tokens of one user contiguous, in token
 * order, cut into work items of at most 32 tokens) into `batch` (caller-owned
 * device memory of >= bd_batch_workspace_bytes, 256-byte aligned).  Its first
 * word is the status word (BD_ERR_USER_ID for an id outside [-1, n_users)).
 * x is not read for bf16 inputs (it may be NULL); the grouping depends only on
 * the ids. */
bd_status bd_batch_prepare(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                           const int32_t* user_ids, int32_t n_users, void* batch,
                           size_t batch_bytes, void* stream);

/* Shared base product y[T][d_out] = X . W_base^T in fp32 (overwrites y); bf16
 * inputs run on the matrix cores, fp32 inputs on the vector ALUs. */
bd_status bd_base_gemm(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                       const void* w_base, int64_t d_out, float* y, void* stream);

/* Per-user delta product added into y: y[t] += scale_u (.) (X[t] . S_u^T) for
 * every token of the prepared batch whose user is valid.  `batch` (batch_bytes
 * long, >= bd_batch_workspace_bytes) must come from bd_batch_prepare with the
 * same user ids, x_dtype, T, d_in and n_users; x is [T][d_in] (any activation
 * tensor of that batch, e.g. the input of q, k or v); y is fp32 [T][d_out].  For
 * bf16 inputs the call is bd_batch_encode followed by bd_delta_apply_encoded:
 * it first writes this x (times the column scales, for COL) into `batch` as
 * tiles of 16 user-sorted tokens encoded as fp6 e2m3 operands, so calls on one
 * batch must not overlap; the grouping itself is left unchanged.  (bf16 GROUP
 * scales with groups under 128 columns: the plain kernel of bd_apply, no encoding;
 * bd_batch_encode and bd_delta_apply_encoded(_n) return BD_ERR_UNSUPPORTED for
 * them.) */
bd_status bd_delta_apply(void* batch, size_t batch_bytes, const void* x, bd_dtype x_dtype,
                         int64_t T, int64_t d_in, int32_t n_users, int64_t d_out,
                         const uint64_t* signs_bank, const void* scales_bank,
                         const bd_compress_params* p, float* y, void* stream);

/* The two halves of bd_delta_apply for bf16 inputs, so that matrices reading the
 * same activations (q, k and v; gate and up) share one encoding of them.
 *
 * bd_batch_encode writes x [T][d_in] bf16 into the prepared `batch` as the
 * delta-product operands: per tile of 16 user-sorted tokens and 512-column unit,
 * two fp6 e2m3 parts per value under one power-of-two scale per 32 columns (the
 * hi part is x rounded to 3 fraction bits under the block's scale, the lo part
 * the rounded residual; together they keep the bf16 value exactly for every
 * element of at least a quarter of its block's largest magnitude).  The column
 * order depends on p->mode (GROUP or not); for COL, x is first multiplied by the
 * column scales of each token's user (scales_bank, rounded to bf16), so a COL
 * encoding belongs to one matrix's scales.  Other modes do not read scales_bank
 * (it may be NULL).  Overwrites the previous encoding of the batch.
 *
 * bd_delta_apply_encoded adds y[t] += scale_u (.) (X[t] . S_u^T) for one matrix
 * from the batch's current encoding ([P2] "Systems Mechanics" 1-2).  p->mode must
 * be the mode the batch was encoded for (GROUP / COL / the others): otherwise
 * nothing is added and the batch's status word reports BD_ERR_BATCH. */
bd_status bd_batch_encode(void* batch, size_t batch_bytes, const void* x, bd_dtype x_dtype,
                          int64_t T, int64_t d_in, int32_t n_users, const void* scales_bank,
                          const bd_compress_params* p, void* stream);
bd_status bd_delta_apply_encoded(void* batch, size_t batch_bytes, bd_dtype x_dtype, int64_t T,
                                 int64_t d_in, int32_t n_users, int64_t d_out,
                                 const uint64_t* signs_bank, const void* scales_bank,
                                 const bd_compress_params* p, float* y, void* stream);

/* Grouped forms for matrices that read the same activations (q, k and v; gate and
 * up), up to 4 per call: one launch each instead of one per matrix, so small
 * matrices (k and v) share the grid with large ones.  Results equal, bit for bit,
 * n_mats calls of bd_base_gemm / bd_delta_apply_encoded with the same arguments
 * (bd_base_gemm_n without a workspace: with one, K may be split, below).
 *  n_mats      : 1..4.
 *  d_outs      : host int64[n_mats], the output rows of each matrix.
 *  w_bases     : host array of n_mats device pointers, [d_outs[i]][d_in] each.
 *  signs_banks, scales_banks : host arrays of n_mats device pointers, each as for
 *                bd_delta_apply_encoded with d_out = d_outs[i].
 *  ys          : host array of n_mats device pointers, fp32 [T][d_outs[i]] each.
 * bd_base_gemm_n falls back to one launch per matrix for batches the tiled GEMM
 * does not take (T <= 64, fp32).  Where no tile gives the chip a full grid with K
 * whole (few rows and tokens: down_proj at 512 tokens) and `workspace` is given, K
 * is split into 2, 4 or 8 ordered parts whose partial products go to the workspace
 * and are summed by a second launch in part order, so y repeats bit for bit;
 * workspace NULL (or bd_base_gemm_n_workspace_bytes == 0): no split.
 *  workspace   : >= bd_base_gemm_n_workspace_bytes(...) bytes, 256-byte aligned,
 *                or NULL. */
size_t bd_base_gemm_n_workspace_bytes(bd_dtype x_dtype, int64_t T, int64_t d_in, int32_t n_mats,
                                      const int64_t* d_outs);
bd_status bd_base_gemm_n(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                         int32_t n_mats, const void* const* w_bases, const int64_t* d_outs,
                         float* const* ys, void* workspace, size_t ws_bytes, void* stream);
bd_status bd_delta_apply_encoded_n(void* batch, size_t batch_bytes, bd_dtype x_dtype, int64_t T,
                                   int64_t d_in, int32_t n_users, int32_t n_mats,
                                   const int64_t* d_outs, const uint64_t* const* signs_banks,
                                   const void* const* scales_banks, const bd_compress_params* p,
                                   float* const* ys, void* stream);

/* bd_base_gemm_n on INT8 base weights (bd_quantize_base; [P2] "Production
 * Engineering" 3): ys[i][t] = wscales[i] (.) (X[t] . wqs[i]^T) for up to 4 matrices
 * that read the same bf16 activations, so that an INT8-based stack groups its
 * matrices as the bf16 one does.  Same tiles as bd_apply_q8's base product (the
 * codes widened to bf16 exactly on chip, each row's sum scaled once), K split as in
 * bd_base_gemm_n: the workspace is sized by bd_base_gemm_n_workspace_bytes with
 * x_dtype BD_BF16 and these shapes, NULL for no split.
 *  x       : bf16 [T][d_in], 1 <= T, d_in a multiple of 64.
 *  wqs     : host array of n_mats device pointers, int8 [d_outs[i]][d_in] each.
 *  wscales : host array of n_mats device pointers, fp32 [d_outs[i]] each.
 *  ys      : host array of n_mats device pointers, fp32 [T][d_outs[i]] each.
 * Errors: BD_ERR_DTYPE (x not bf16), BD_ERR_SHAPE, BD_ERR_UNSUPPORTED (32-bit offsets
 * exceeded), BD_ERR_INVALID_ARG (null or misaligned pointer), BD_ERR_WORKSPACE;
 * nothing is launched on an error. */
bd_status bd_base_gemm_q8_n(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                            int32_t n_mats, const int8_t* const* wqs,
                            const float* const* wscales, const int64_t* d_outs,
                            float* const* ys, void* workspace, size_t ws_bytes, void* stream);

/* The two-launch form of bd_apply's decode path (what bd_apply runs for COL scales
 * and rows wider than 5120 columns), callable on its own: bf16 x and
 * w_base, 1 <= T <= 16, MATRIX, ROW or COL scales (BD_ERR_UNSUPPORTED for any
 * other batch).  Same formula as bd_apply ([P2] "Systems Mechanics" 1-2).
 *
 * bd_decode_prepare sorts the tokens by user and encodes x for the delta
 * products (per 32-column block a power-of-two scale and two fp8 e4m3 parts,
 * about 8 significant bits, the precision of bf16) into `workspace`:
 * caller-owned device memory of >= bd_apply_workspace_bytes(p, T, n_users,
 * d_out, d_in, BD_BF16, y_dtype) bytes, 256-byte aligned, whose first word is
 * the status word (BD_ERR_USER_ID for an id outside [-1, n_users)).  For COL
 * scales the users' column scales (scales_bank) are folded into the encoding;
 * other modes do not read scales_bank here (it may be NULL).
 *
 * bd_decode_apply computes y[T][d_out] (y_dtype BD_F32 or BD_BF16, written,
 * not accumulated) for one matrix from a prepared workspace.  One prepared
 * workspace serves every matrix that reads the same x and user ids with the
 * same p->mode (for COL, the same column scales), e.g. q, k and v; the
 * workspace size does not depend on d_out.  Arguments as for bd_apply. */
bd_status bd_decode_prepare(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                            const int32_t* user_ids, int32_t n_users, const void* scales_bank,
                            const bd_compress_params* p, void* workspace, size_t ws_bytes,
                            void* stream);
bd_status bd_decode_apply(const void* x, bd_dtype x_dtype, int64_t T, int64_t d_in,
                          const void* w_base, int64_t d_out, const uint64_t* signs_bank,
                          const void* scales_bank, const bd_compress_params* p, int32_t n_users,
                          void* y, bd_dtype y_dtype, const void* workspace, size_t ws_bytes,
                          void* stream);

/* ------------------------------------------------------- status read-back */

/* Synchronises `stream`, then returns the status recorded in the workspace (or
 * prepared batch) of the last bd_compress / bd_apply / bd_batch_prepare that
 * used it (BD_OK, BD_ERR_NONFINITE, BD_ERR_USER_ID or BD_ERR_BATCH), or
 * BD_ERR_DEVICE if the copy fails. */
bd_status bd_device_status(const void* workspace, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BITDELTA_H */
