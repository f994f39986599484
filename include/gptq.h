/*
 * gptq.h — C ABI of the GPTQ layer quantizer for AMD Instinct MI355X (gfx950).
 *
 * The method (sources cited by page title and section):
 *   - "Warum Geometrie Gewichte nicht komprimiert" (CHMC article, nonndazone.ru),
 *     Methodik, Schritt 2: the layer Hessian is built from the calibration
 *     activations X of the layer, damped by lambda*mean(diag H)*I, inverted via
 *     the Cholesky decomposition; columns are visited in act-order (descending
 *     diag H); each column is rounded to its group's grid and its error,
 *     divided by the factor's diagonal entry, is subtracted from the later
 *     columns through the factor's row. Schritt 3 / Tabelle 1: GPTQ stores
 *     integer codes plus per-group scales, groups along input channels.
 *   - "The Geometry of LLM Quantization: GPTQ as Babai's Nearest Plane
 *     Algorithm" (gist.science), 2.1-2.3: the sweep is Babai's nearest-plane
 *     algorithm on the lattice of the Hessian; act-order is the pivot order.
 *
 * Conventions used by every entry point:
 *   - All array arguments are DEVICE pointers (HIP global memory) owned by the
 *     caller; the library allocates no device memory. Scratch space comes from
 *     a caller workspace whose size the *_workspace_bytes() calls return.
 *   - Matrices are row-major with an explicit leading dimension (elements).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *     is enqueued on it in order; see each call for where it synchronizes.
 *   - Arguments are validated on the host first; an invalid call returns
 *     GPTQ_EINVAL / GPTQ_EWORKSPACE before anything is enqueued.
 *   - Fp16 values (weights, scales, zero points) travel as uint16_t bit
 *     patterns (IEEE binary16).
 *   - No exception crosses the ABI. Calls on different streams with disjoint
 *     buffers are independent and may come from different host threads. The
 *     optional profiler (gptq_profile_*) is the only state kept across calls:
 *     a process-wide switch and one shared record, both guarded, so it is
 *     thread-safe too.
 */
#ifndef GPTQ_H
#define GPTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_EINVAL = 1,      /* null pointer, negative size, bits/group size out of range   */
  GPTQ_ENOTSPD = 2,     /* damped Hessian not positive definite (pivot <= 0 or NaN)    */
  GPTQ_EHIP = 3,        /* a HIP runtime call or kernel launch failed                   */
  GPTQ_EWORKSPACE = 4,  /* workspace pointer null or smaller than required              */
  GPTQ_ENONFINITE = 5   /* NaN/Inf weight, or a group scale beyond the fp16 range       */
} gptq_status;

/* flags */
#define GPTQ_FLAG_ACT_ORDER 1u          /* gptq_prepare_hinv: visit columns by descending diag H */
#define GPTQ_FLAG_HESSIAN_OVERWRITE 2u  /* gptq_hessian_accumulate: S = X^T X instead of S += */
#define GPTQ_FLAG_NO_SYNC 4u            /* prepare / quantize: return after enqueueing; the
                                           device-side status stays in the workspace, read
                                           it with gptq_workspace_status */
#define GPTQ_FLAG_MIN_PIVOT 8u          /* gptq_prepare_hinv: min-pivot order instead of
                                           act-order (exclusive with GPTQ_FLAG_ACT_ORDER) */
#define GPTQ_FLAG_NO_CLIP 16u           /* gptq_quantize_layer: levels not clamped to the grid
                                           (the no-clipping regime of Satz 5); stored codes
                                           saturate to [0, 255] */
#define GPTQ_FLAG_HESSIAN_SPLIT8 32u    /* gptq_hessian_accumulate: X^T X from int8 digit
                                           slices on the int8 matrix cores (see Step 1) */
#define GPTQ_FLAG_FACTOR_FORM 64u       /* prepare / quantize: the factor of H itself in
                                           place of U beyond U's diagonal blocks (see
                                           Steps 2-3), no full triangular inverse */

/* ---------------------------------------------------------------------------
 * Step 1 — Hessian statistics.  CHMC article, Schritt 2 (H from the layer's
 * calibration activations). Accumulates the unnormalised sum
 *     S[i x i] += X^T X,   X = n_tokens x in_features fp32, row stride ldx,
 * or S = X^T X with flags & GPTQ_FLAG_HESSIAN_OVERWRITE (S's old contents are
 * then never read; with n_tokens == 0 S is set to zero). S is fp64 and
 * symmetric: both triangles are written, and when accumulating S must be
 * symmetric on entry (as every call leaves it; the lower triangle is
 * rewritten from the upper one). The products of two fp32 values are
 * formed exactly (fp64), only the sums round. Call it once per token chunk
 * (the first with the overwrite flag, or on a zeroed S) and keep the running
 * token count; the normalisation (2/n) is applied by gptq_prepare_hinv.
 * Other flag bits are rejected (GPTQ_EINVAL).
 * ws may be NULL (ws_bytes 0): the call is then done without token splitting.
 * With ws of gptq_hessian_workspace_bytes(in_features, n_tokens) bytes the
 * token range is split across more workgroups and reduced in a fixed order
 * (results are bitwise reproducible either way for a given ws choice).
 * in_features == 0, or n_tokens == 0 without the overwrite flag, is a no-op.
 * Asynchronous on `stream`.
 *
 * With GPTQ_FLAG_HESSIAN_SPLIT8 the products are formed on the int8 matrix
 * cores instead (error-free slicing of a matrix product into integer slice
 * products, after Ozaki, Ogita, Oishi and Rump). Per call, column f of X
 * gets the scale 2^e_f, the smallest power of two above max_k |x_kf|, and
 * each value is rounded to the nearest multiple of 2^(e_f - 30) (ties to
 * even); that fixed-point value m 2^(e_f - 30) is cut into four signed int8
 * digits, m = d0 2^24 + d1 2^16 + d2 2^8 + d3 (d1..d3 in [-128, 127]), and
 * the digit-pair products of orders a + b <= 4 (13 of the 16) are summed
 * exactly in int32, then in fp64. The result is X~^T X~ for the rounded X~
 * (|x~ - x| <= 2^(e_f - 31)) less its digit orders 5 and 6
 * (2^(e_f + e_g - 60) (2^8 (D2^T D3 + D3^T D2) + D3^T D3), under
 * 2^(e_f + e_g - 36.99) per token), up to the fp64 additions. A column holding NaN or Inf gives NaN in its row and
 * column of S. The workspace is then required: ws_bytes >=
 * gptq_hessian_split8_workspace_bytes(in_features, n_tokens), else
 * GPTQ_EWORKSPACE (it holds the digit planes, 4 * in_features * n_tokens
 * bytes rounded up to tiles, and any token-split partial tiles). A call whose
 * tiles and token splits would exceed one launch grid (2^31 - 1 workgroups)
 * is rejected with GPTQ_EINVAL.
 * ------------------------------------------------------------------------- */
size_t gptq_hessian_workspace_bytes(int64_t in_features, int64_t n_tokens);
size_t gptq_hessian_split8_workspace_bytes(int64_t in_features, int64_t n_tokens);
gptq_status gptq_hessian_accumulate(double* S, int64_t in_features,
                                    const float* X, int64_t n_tokens, int64_t ldx,
                                    uint32_t flags, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Steps 2-3 — damping, act-order, factor of the inverse.  CHMC article,
 * Schritt 2 (H = X^T X/n + lambda*mean(diag H)*I, H^-1 via Cholesky,
 * act-order); The Geometry of LLM Quantization 2.3 (act-order pivoting).
 *   H  = (2/n_tokens_total) * S + damp * mean(diag((2/n) S)) * I
 *   perm (out, int32[i]) = stable order of descending diag H when
 *        flags & GPTQ_FLAG_ACT_ORDER; with GPTQ_FLAG_MIN_PIVOT the min-pivot
 *        order of The Geometry of LLM Quantization 2.3: the LDL of H that
 *        takes the smallest diagonal of the current Schur complement as the
 *        next pivot (ties: the higher index), visited in the reverse of that
 *        elimination order; else the identity;
 *        perm[k] = original column visited k-th.
 *   U  (out, fp32 [i x i], row-major, ld = in_features) = the upper triangular
 *        factor with U^T U = (H[perm][:,perm])^-1, zeros below the diagonal.
 * Computed in fp64 (one Cholesky of the order-reversed permuted Hessian and
 * one triangular inverse), stored as fp32. S is read, never written.
 * With GPTQ_FLAG_FACTOR_FORM the output in U is instead the matrix M that
 * gptq_quantize_layer takes with the same flag (The Geometry of LLM
 * Quantization 2.2: the nearest-plane step needs a triangular factor of the
 * lattice's Gram matrix, here H itself):
 *   M[j][k] = U[j][k]  for j <= k in the same 128-wide block of sweep
 *                      positions (blocks start at 0; the last may be short),
 *   M[j][k] = (R U)[j][k] over k's block, i.e. sum of R[j][l] U[l][k] for l in
 *                      k's block, for k in a later block; R = U^-1 is the
 *                      upper triangular factor with R R^T = H[perm][:,perm],
 *   0 below the diagonal. R is the order-reversed Cholesky factor of the
 * permuted H, so only the 128 x 128 diagonal blocks are inverted: no full
 * triangular inverse runs (each tile beyond them is one 128 x 128 product).
 * The flag combines with either order.
 * All work is enqueued on `stream`.
 * Workspace: gptq_prepare_workspace_bytes(in_features) bytes.
 * Synchronizes `stream` once at the end to read the factorisation status;
 * returns GPTQ_ENOTSPD if a pivot is <= 0 or not finite (U is then garbage).
 * With GPTQ_FLAG_NO_SYNC it returns after enqueueing (argument errors are
 * still returned at once) and the status is read by gptq_workspace_status.
 * The min-pivot search of up to 8192 features runs as one cooperative launch
 * per 128 pivots whose workgroups wait for each other with bounded waits: if
 * one of them waits for about a second (the device held by other work), the
 * call reports GPTQ_ENOTSPD as well. Where a cooperative launch of that size
 * is not possible, and above 8192 features, it runs as one launch per pivot.
 * ------------------------------------------------------------------------- */
size_t gptq_prepare_workspace_bytes(int64_t in_features);
gptq_status gptq_prepare_hinv(const double* S, int64_t in_features, int64_t n_tokens_total,
                              double damp, uint32_t flags, int32_t* perm, float* U,
                              void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Steps 4-6 — the column sweep.  CHMC article, Schritt 2 (per column:
 * round to the group grid, err = (col - q)/U[j,j], later columns -= err *
 * U[j, j+1:]); the lazy form applies the update of a 128-column block to the
 * columns after it only when they are reached (same sums, other order).
 *   W     fp16 [rows x cols], leading dimension ldw (>= cols), original order.
 *   U     fp32 [cols x cols] from gptq_prepare_hinv (sweep order); with
 *         GPTQ_FLAG_FACTOR_FORM the matrix M that gptq_prepare_hinv returns
 *         with that flag (U's diagonal blocks, R U over each block beyond).
 *   perm  int32[cols] from gptq_prepare_hinv, or NULL for the identity.
 *   bits  2..8; group_size one of 16, 32, 64, 128 (groups = group_size
 *         consecutive columns in sweep order; the last may be shorter).
 * Grid of a group (asymmetric min-max), taken when the sweep reaches the
 * group's first column from the current, error-updated values v:
 *   scale = fp16_rne((max(0,max v) - min(0,min v)) / (2^bits - 1)),
 *   zero  = clamp(rint(-min(0,min v)/scale), 0, 2^bits - 1);
 *   scale 1 / zero 0 when max == min or the scale rounds to 0.
 *   code  = clamp(rint(v/scale) + zero, 0, 2^bits - 1)   (round half even).
 * Outputs:
 *   codes    uint8 [rows x cols], ld = cols, ORIGINAL column order.
 *   scales   fp16 [rows x ceil(cols/group_size)], ld = ceil(cols/gs), group g
 *            covers sweep positions [g*gs, (g+1)*gs).
 *   zeros    fp16, same layout (integer values).
 *   g_idx    int32[cols] or NULL: g_idx[perm[k]] = k / group_size.
 *   row_loss fp64[rows]: sum_j e_j^2, e_j = (v_j - dequant_j)/U[j,j]; equals
 *            (w-q) H (w-q)^T for the damped, permuted H.
 * Workspace: gptq_quantize_workspace_bytes(rows, cols, group_size) bytes.
 * perm must be a permutation of 0..cols-1 (checked on the device: GPTQ_EINVAL).
 * flags: 0, GPTQ_FLAG_NO_SYNC, GPTQ_FLAG_NO_CLIP (The Geometry of LLM
 * Quantization 2.3, the no-clipping regime of Satz 5: code = rint(v/scale) +
 * zero without the clamp; the errors, the propagation and row_loss use that
 * unclamped code, the stored byte is it saturated to [0, 255]),
 * GPTQ_FLAG_FACTOR_FORM (the same sweep, carried differently: since the
 * scaled errors are E = (W - Q) R, R = U^-1, the sum over the earlier blocks
 * E[:, :j0] U[:j0, blk] equals (Q - W)[:, :j0] M[:j0, blk], formed from the
 * residuals q - w of the original weights; results agree with the plain
 * form up to rounding). Synchronizes
 * `stream` at the end unless
 * GPTQ_FLAG_NO_SYNC; returns GPTQ_ENONFINITE if a weight is NaN/Inf or a
 * scale overflows fp16 (outputs are then unspecified).
 * rows == 0 or cols == 0 is a no-op.
 * ------------------------------------------------------------------------- */
size_t gptq_quantize_workspace_bytes(int64_t rows, int64_t cols, int group_size);
gptq_status gptq_quantize_layer(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw,
                                const float* U, const int32_t* perm, int bits, int group_size,
                                uint32_t flags, uint8_t* codes, uint16_t* scales,
                                uint16_t* zeros, int32_t* g_idx, double* row_loss,
                                void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * gptq_quantize_layer_noalloc — for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): gptq_quantize_layer with the same arguments, flags,
 * outputs and statuses, minus the workspace. Its scratch is one fixed array
 * of the library in device memory, 64 MiB per device, which each device
 * holds from the first call there until the process ends; the call itself
 * allocates nothing.
 *   - A layer whose workspace (gptq_quantize_workspace_bytes) exceeds 64 MiB
 *     is rejected with GPTQ_EWORKSPACE before anything is enqueued (896 x
 *     4864 at groups of 128 fits; 9728 x 896 does not).
 *   - `stream` must belong to the current device (else GPTQ_EINVAL).
 *   - Every call on a device shares that device's array and leaves its
 *     contents there; each call clears what it needs cleared, so calls one
 *     after the other are fine, but calls that overlap in time on one device
 *     (other streams, other host threads) race and give wrong results.
 * ------------------------------------------------------------------------- */
gptq_status gptq_quantize_layer_noalloc(const uint16_t* W, int64_t rows, int64_t cols,
                                        int64_t ldw, const float* U, const int32_t* perm,
                                        int bits, int group_size, uint32_t flags,
                                        uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                                        int32_t* g_idx, double* row_loss, void* stream);

/* ---------------------------------------------------------------------------
 * SSQR — The Geometry of LLM Quantization, section 3 ("Skalengerechte SpQR":
 * outliers that would overflow the grid are kept as sparse floating-point
 * values; a binary search on the scales meets a target outlier density).
 * The page prints no rule; the one taken here:
 *   step_g = fp16(alpha * (xmax - xmin) / maxq) for every group (xmin/xmax as
 *   in the plain grid), zero point = that of the unscaled grid (so the grid
 *   shrinks about 0 for alpha < 1); a weight whose level rint(v/step) + zero
 *   falls outside [0, maxq] is an outlier: it is kept as fp16(v) (its current,
 *   error-updated value) and only that fp16 rounding error propagates; its
 *   stored code is the clamped level. alpha = 1 is the min-max grid.
 * gptq_quantize_layer_ssqr: as gptq_quantize_layer (same workspace), plus
 *   alpha       in (0, 16], else GPTQ_EINVAL;
 *   outlier_mask (out, u8 [rows x cols], original column order): 1 = outlier;
 *   outlier_vals (out, fp16 bits [rows x cols]): fp16(v) at outliers, 0 else;
 *   n_outliers  (host, may be NULL): the count, read after a synchronize
 *               (GPTQ_EINVAL with GPTQ_FLAG_NO_SYNC).
 *   GPTQ_FLAG_NO_CLIP is not accepted (the rule above replaces clipping).
 * gptq_ssqr_search: bisection on alpha in [alpha_lo, alpha_hi] (0 < lo < hi
 *   <= 16) for the smallest alpha whose outlier fraction (count / (rows *
 *   cols)) is at most target (in [0, 1]): alpha_hi is tried first and, if it
 *   already exceeds the target, returned; else iters (<= 60) midpoints are
 *   tried, keeping hi at the passing ones. Each probe is one full sweep into
 *   the output buffers, synchronized to read its count; on return they hold
 *   the sweep at *alpha_out (host), and *n_outliers (host, may be NULL) its
 *   count. flags must be 0.
 * ------------------------------------------------------------------------- */
gptq_status gptq_quantize_layer_ssqr(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw,
                                     const float* U, const int32_t* perm, int bits,
                                     int group_size, uint32_t flags, double alpha,
                                     uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                                     int32_t* g_idx, double* row_loss, uint8_t* outlier_mask,
                                     uint16_t* outlier_vals, uint64_t* n_outliers, void* ws,
                                     size_t ws_bytes, void* stream);
gptq_status gptq_ssqr_search(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw,
                             const float* U, const int32_t* perm, int bits, int group_size,
                             uint32_t flags, double target, int iters, double alpha_lo,
                             double alpha_hi, double* alpha_out, uint8_t* codes,
                             uint16_t* scales, uint16_t* zeros, int32_t* g_idx,
                             double* row_loss, uint8_t* outlier_mask, uint16_t* outlier_vals,
                             uint64_t* n_outliers, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * gptq_ssqr_outliers_csr — the storage of SSQR's outliers (The Geometry of LLM
 * Quantization, section 3: the weights that would overflow the grid are kept
 * sparse, in floating point). Compacts the dense outlier_mask / outlier_vals
 * of a gptq_quantize_layer_ssqr or gptq_ssqr_search call into compressed
 * sparse rows:
 *   mask     (in, u8 [rows x cols], device, contiguous): nonzero = outlier;
 *   vals     (in, fp16 bits [rows x cols], device, contiguous);
 *   row_ptr  (out, int64 [rows + 1], device): row r's entries are
 *            [row_ptr[r], row_ptr[r + 1]); row_ptr[rows] = their count;
 *   col_idx  (out, int32 [capacity], device): columns, increasing in a row;
 *   csr_vals (out, fp16 bits [capacity], device): vals at those columns;
 *   capacity entries the caller provides (the n_outliers of the SSQR call
 *            suffices); when the count exceeds it, row_ptr is still written,
 *            col_idx / csr_vals are left untouched and the call returns
 *            GPTQ_EINVAL (without GPTQ_FLAG_NO_SYNC; with it, compare
 *            row_ptr[rows] with capacity afterwards);
 *   flags    0 or GPTQ_FLAG_NO_SYNC; nnz (host, may be NULL, must be NULL
 *            with GPTQ_FLAG_NO_SYNC): the count, read after a synchronize.
 *   Needs no workspace. rows, cols >= 0, cols < 2^31.
 * ------------------------------------------------------------------------- */
gptq_status gptq_ssqr_outliers_csr(const uint8_t* mask, const uint16_t* vals, int64_t rows,
                                   int64_t cols, int64_t* row_ptr, int32_t* col_idx,
                                   uint16_t* csr_vals, int64_t capacity, uint32_t flags,
                                   int64_t* nnz, void* stream);

/* ---------------------------------------------------------------------------
 * HPTQ — The Geometry of LLM Quantization, section 3 (Huffman-coded PTQ:
 * inliers and outliers in one unbounded integer grid, the integers Huffman
 * coded to meet a compression budget). The page prints no rule; the one
 * taken here:
 *   step_g = fp16(alpha * (xmax - xmin) / maxq) (xmin/xmax and maxq = 2^bits
 *   - 1 as in the plain grid), level k = rint(v / step) relative to 0, no
 *   zero point and no clipping (the no-clipping sweep on this grid);
 *   bits per weight = (the total length of a Huffman code for all levels of
 *   the call, one codebook, a single distinct level costing 1 bit per weight,
 *   + 16 per group step) / (rows * cols).
 * gptq_quantize_layer_hptq: as gptq_quantize_layer (same workspace), with
 *   alpha   in (0, 16], else GPTQ_EINVAL;
 *   levels  (out, int16 [rows x cols], original column order): k; a level
 *           beyond the int16 range is reported as GPTQ_ENONFINITE;
 *   scales  (out, fp16 [rows x ceil(cols/gs)], groups in sweep order): steps;
 *   zeros   (out, same shape): 0 for every group;
 *   bpw     (host, may be NULL): bits per weight, read after a synchronize
 *           (GPTQ_EINVAL with GPTQ_FLAG_NO_SYNC).
 * gptq_hptq_search: bisection on alpha in [alpha_lo, alpha_hi] (0 < lo < hi
 *   <= 16) for the smallest alpha whose bits per weight are at most budget
 *   (> 0), in the probe order of gptq_ssqr_search; on return the outputs hold
 *   the sweep at *alpha_out (host) and *bpw_out (host, may be NULL) its bits
 *   per weight. flags must be 0.
 * ------------------------------------------------------------------------- */
gptq_status gptq_quantize_layer_hptq(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw,
                                     const float* U, const int32_t* perm, int bits,
                                     int group_size, uint32_t flags, double alpha,
                                     int16_t* levels, uint16_t* scales, uint16_t* zeros,
                                     int32_t* g_idx, double* row_loss, double* bpw, void* ws,
                                     size_t ws_bytes, void* stream);
gptq_status gptq_hptq_search(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw,
                             const float* U, const int32_t* perm, int bits, int group_size,
                             uint32_t flags, double budget, int iters, double alpha_lo,
                             double alpha_hi, double* alpha_out, int16_t* levels,
                             uint16_t* scales, uint16_t* zeros, int32_t* g_idx,
                             double* row_loss, double* bpw_out, void* ws, size_t ws_bytes,
                             void* stream);

/* ---------------------------------------------------------------------------
 * Status of the last gptq_prepare_hinv / gptq_quantize_layer call that used
 * workspace `ws` (a device pointer): synchronizes `stream` (the stream of that
 * call), then reads the status word the call left at the start of `ws`.
 * ------------------------------------------------------------------------- */
gptq_status gptq_workspace_status(const void* ws, void* stream);

/* ---------------------------------------------------------------------------
 * Utilities.
 * gptq_status_string: static, never NULL.
 * gptq_fp16_round_host: HOST function (host pointers); rounds each double to
 *   the nearest-even binary16 with the same routine the kernels use for group
 *   scales (no double rounding through fp32). Returns GPTQ_EINVAL on NULL.
 * gptq_version: ABI version number (currently 1).
 * gptq_last_error_string: text of the last HIP runtime error that made a call
 *   of this thread return GPTQ_EHIP ("no error" if none); static storage.
 * ------------------------------------------------------------------------- */
const char* gptq_status_string(gptq_status status);
const char* gptq_last_error_string(void);
gptq_status gptq_fp16_round_host(const double* in, uint16_t* out, int64_t n);
int gptq_version(void);

/* ---------------------------------------------------------------------------
 * HPTQ code stream — the stored form of HPTQ's levels (The Geometry of LLM
 * Quantization, section 3: the integer levels are Huffman-coded).
 * gptq_hptq_encode: levels (in, int16 [rows x cols], device, row-major, e.g.
 *   the levels of gptq_quantize_layer_hptq) as one bit stream, rows in order,
 *   each row's levels in column order:
 *   - code lengths: a Huffman code of the call's level histogram (the two
 *     lightest subtrees merged first; ties to the subtree made earlier, the
 *     leaves in increasing level order); a single distinct level costs 1 bit;
 *   - codes: the canonical code of those lengths (levels ordered by length,
 *     then value; the first code 0, each next one the previous plus one,
 *     shifted left by the growth in length), most significant bit first;
 *   - bit b of the stream is bit 31 - b % 32 of words[b / 32];
 *   code_len (out, host [65536], may be NULL): the length of level v at
 *     v + 32768, 0 for levels that do not occur;
 *   words (out, device uint32 [capacity_words]); row_bit (out, device int64
 *     [rows + 1]): the stream position of each row's first code, row_bit[rows]
 *     = *total_bits (out, host). A capacity below ceil(total / 32) words is
 *     GPTQ_EINVAL with row_bit and *total_bits still set; a code longer than 63
 *     bits is GPTQ_EINVAL. Synchronizes `stream`.
 * gptq_hptq_decode: the inverse (one device thread per row): words [nwords],
 *   row_bit and code_len from gptq_hptq_encode; levels (out, device int16
 *   [rows x cols]). A stream that does not decode is GPTQ_EINVAL.
 *   Synchronizes `stream`.
 * Workspace (both): gptq_hptq_code_workspace_bytes() bytes (about 1 MB).
 * ------------------------------------------------------------------------- */
size_t gptq_hptq_code_workspace_bytes(void);
gptq_status gptq_hptq_encode(const int16_t* levels, int64_t rows, int64_t cols,
                             uint8_t* code_len, uint32_t* words, int64_t capacity_words,
                             int64_t* row_bit, int64_t* total_bits, void* ws, size_t ws_bytes,
                             void* stream);
gptq_status gptq_hptq_decode(const uint32_t* words, int64_t nwords, const int64_t* row_bit,
                             int64_t rows, int64_t cols, const uint8_t* code_len,
                             int16_t* levels, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * CHMC frontend — CHMC article, "Methodik. Was ist CHMC", Schritt 1-3: the
 * weight is split into a low-rank part, kept as two fp16 factors, and a
 * residual quantized by the GPTQ sweep with one grid per group of output
 * channels (rows) and column.
 *   energies  c_j = S_jj / n + 0.05 * mean_k(S_kk / n) (activation energy,
 *             damped by 5 % of its mean);
 *   low rank  of W~ = W diag(sqrt c) by randomized subspace iteration
 *             (Halko, Martinsson and Tropp 2011, Algorithm 4.4) from the
 *             caller's sketch omega with 5 power iterations, then the SVD of
 *             the r x i projection: W~ ~ Ul diag(s) V^T;
 *             A = fp16(Ul diag(s)) [rows x r], B = fp16(V^T diag(1/sqrt c)) [r x cols];
 *   residual  R = W - A B (fp64 from the fp16 factors), swept in the order
 *             perm with the factor U of gptq_prepare_hinv: column j gets, per
 *             group of group_size rows, the min-max asymmetric grid of the
 *             group's current values (fp16 scale, integer zero point), and its
 *             scaled errors propagate along row j of U.
 * gptq_chmc_rank: the largest r whose factors (16 r (rows + cols) bits),
 *   bits-bit codes, one 16-bit scale per row group and column and that
 *   group's zero point (an integer in [0, 2^bits - 1], counted at bits bits)
 *   fit bpw_target bits per weight: floor((bpw rows cols - bits rows cols -
 *   (16 + bits) ceil(rows/gs) cols) / (16 (rows + cols))), clamped to
 *   [0, min(rows, cols, 64)] (64 is the largest rank gptq_chmc_layer takes; a
 *   smaller rank stays under the budget); 0 for invalid arguments.
 * gptq_chmc_workspace_bytes: workspace for gptq_chmc_layer (0 if rank is not
 *   in [0, 64] or a size is not positive): about 3 rows*cols fp64 matrices.
 * gptq_chmc_layer:
 *   W       (in, fp16 bits, device, [rows x cols] row stride ldw >= cols);
 *   S       (in, fp64, device, [cols x cols]) the Hessian sum X^T X over
 *           n_tokens (> 0) tokens (only its diagonal is read here);
 *   U, perm (in, device) from gptq_prepare_hinv: U fp32 [cols x cols] upper,
 *           sweep order; perm int32 [cols] a permutation (NULL = identity);
 *           a perm that is not one is reported as GPTQ_EINVAL;
 *   omega   (in, fp64, device, [cols x rank] row-major) the Gaussian sketch;
 *   rank    in [0, min(64, rows, cols)] (0: no low-rank part; omega, A, B
 *           may then be NULL); bits in [2, 8]; group_size 32, 64 or 128;
 *   flags   0, GPTQ_FLAG_NO_SYNC, GPTQ_FLAG_FACTOR_FORM (U is then the
 *           factor-form matrix of gptq_prepare_hinv with that flag, and the
 *           residual sweep forms its update sums from the residuals q - r of
 *           the residual matrix's entries, as gptq_quantize_layer does);
 *   A       (out, fp16 bits [rows x rank]), B (out, fp16 bits [rank x cols]);
 *           each component is determined up to a common sign of its column
 *           of A and row of B;
 *   codes   (out, u8 [rows x cols], original column order);
 *   scales, zeros (out, fp16 bits [ceil(rows/group_size) x cols], original
 *           column order): the grid of each row group and column;
 *   row_loss (out, fp64 [rows]): sum over columns of the squared scaled
 *           errors of the residual sweep.
 *   u_stream (may be NULL): a HIP stream on which U and perm are still being
 *           produced (gptq_prepare_hinv enqueued there before this call).
 *           The frontend, which reads only W, diag S and omega, starts at
 *           once on `stream`; the permutation check and the sweep wait for
 *           the work enqueued on u_stream up to this call. NULL: U and perm
 *           are ready in stream order. S must be complete in `stream` order
 *           either way.
 *   Returns GPTQ_ENOTSPD when the sketch loses rank (the weighted W has
 *   rank below r), GPTQ_ENONFINITE for a NaN/Inf weight or energy or an
 *   fp16 overflow of a scale; with GPTQ_FLAG_NO_SYNC the status is read later
 *   with gptq_workspace_status. Calls on one workspace must not overlap.
 * ------------------------------------------------------------------------- */
int gptq_chmc_rank(int64_t rows, int64_t cols, int bits, int group_size, double bpw_target);
size_t gptq_chmc_workspace_bytes(int64_t rows, int64_t cols, int rank);
gptq_status gptq_chmc_layer(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw,
                            const double* S, int64_t n_tokens, const float* U,
                            const int32_t* perm, const double* omega, int rank, int bits,
                            int group_size, uint32_t flags, uint16_t* A, uint16_t* B,
                            uint8_t* codes, uint16_t* scales, uint16_t* zeros, double* row_loss,
                            void* ws, size_t ws_bytes, void* stream, void* u_stream);

/* ---------------------------------------------------------------------------
 * Optional kernel timing (process-wide, thread-safe). gptq_profile_enable
 * takes a bit mask of kernel ids (bit k = kernel id k; 0 turns timing off,
 * 0xFFFFFFFF times every kernel). Each launch of a selected kernel is then
 * bracketed by two HIP events recorded on the stream it is launched on.
 * gptq_profile_read synchronizes on the recorded events, adds their durations
 * per kernel class and clears the record.
 *   kernel ids: 0 .. gptq_profile_kernel_count()-1; names via
 *   gptq_profile_kernel_name(id) (static string, NULL for a bad id).
 *   totals_ms / launches: host arrays of gptq_profile_kernel_count() entries.
 * ------------------------------------------------------------------------- */
gptq_status gptq_profile_enable(uint32_t kernel_mask);
int gptq_profile_kernel_count(void);
const char* gptq_profile_kernel_name(int id);
gptq_status gptq_profile_read(double* totals_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* GPTQ_H */
