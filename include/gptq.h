/*
 * gptq.h -- C ABI of libgptq_mi355x.so, GPTQ's per-layer quantization solver
 * written for AMD MI355X (gfx950).
 *
 * The method (sources cited by page title and section):
 *   "GPTQ量化算法深度解析：从Hessian曲率到大模型单卡部署" (sheratonhq.com)
 *     §2.2  OBS-style compensation of a column's quantization error into the
 *           columns not yet quantized;
 *     §2.4  fixed column order, lazy batch updates per block, Cholesky form;
 *     §3.1  per layer: H = 2XX^T + lambda*I, Cholesky, blocks of 128 columns
 *           (per column: scale, round, accumulate the error; one update of the
 *           later columns per block), save codes + scale/zero;
 *     §3.3  group size, desc_act (act-order), damp_percent (default 0.01).
 *   "通义千问1.5-1.8B-Chat-GPTQ-Int4模型压缩技术解析" (deepseek.csdn.net) §2.1-2.2:
 *     min/max range split into 2^b levels; scale and zero point per group.
 *   ai.lansai.wang GPTQ guide, field table ("bits、group_size、sym 与 desc_act
 *     分别影响什么"): bits, group_size, sym, desc_act, damp_percent.
 *   "gptq-for-llama" article (ainews.cool), "工程细节": 4-bit codes packed
 *     four to a 16-bit integer.
 *
 * Conventions shared by every entry point
 *   - All array pointers are DEVICE pointers owned by the caller; the library
 *     allocates no memory and keeps no state between calls.
 *   - Matrices are row-major.  W is d_out x d_in (row = output channel);
 *     X is n_tok x d_in (row = token).
 *   - Work is enqueued on `stream` (0 = the null stream).  Calls are
 *     asynchronous unless their comment says "synchronous".
 *   - Errors are returned as gptq_status; nothing is thrown across the ABI.
 *     Arguments are validated before anything is enqueued; on a non-OK
 *     return from validation no device memory has been touched.
 *   - The solver computes in float64 (codes are decided in float64, the
 *     precision of the reference oracle); the Hessian's token products are
 *     accumulated in float32 over runs of 256 tokens and summed in float64,
 *     and its diagonal in float64.
 *   - Calls that share a workspace must not overlap.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GPTQ_OK = 0,
    GPTQ_ERR_INVALID_ARG = 1,  /* null pointer, bad size, unsupported bits, bad group/block */
    GPTQ_ERR_NOT_PD = 2,       /* damped Hessian not positive definite (pivot <= 0) */
    GPTQ_ERR_NONFINITE = 3,    /* NaN/Inf found in H (hence in X) or in W */
    GPTQ_ERR_WORKSPACE = 4,    /* workspace pointer null or smaller than the query says */
    GPTQ_ERR_HIP = 5,          /* a HIP runtime call failed */
    GPTQ_ERR_UNSUPPORTED = 6   /* valid request this build does not implement */
} gptq_status;

typedef enum { GPTQ_F32 = 0, GPTQ_F16 = 1, GPTQ_BF16 = 2 } gptq_dtype;

/* Quantizer configuration (the quantize_config fields of the ai.lansai.wang
 * field table; defaults per "GPTQ量化算法深度解析" §3.3). */
typedef struct {
    int32_t bits;        /* 2, 3, 4 or 8: codes take values 0 .. 2^bits - 1 */
    int32_t group_size;  /* > 0: columns per (scale, zero); <= 0: one group per row */
    int32_t sym;         /* 0: asymmetric range with zero point; 1: symmetric */
    int32_t act_order;   /* 0: natural column order; 1: descending diag(H) (desc_act) */
    int32_t block_size;  /* B, columns per lazy-update block (128); 1..128 in this build
                            (larger: GPTQ_ERR_UNSUPPORTED).  Any B gives the codes of
                            the per-column sweep, also when B and group_size do not
                            divide one another (a group that begins inside a block
                            and runs past its end sees its later columns with the
                            block's pending compensation applied) */
    int32_t static_groups; /* 0: groups of group_size consecutive SWEEP-order columns,
                            each group's (scale, zero) taken when the sweep reaches
                            its first column from the compensated values; 1: groups
                            of group_size consecutive ORIGINAL columns (g_idx[j] =
                            j / group_size, no gather at inference), every group's
                            (scale, zero) taken before the sweep from W as given;
                            act_order then only orders the sweep.  The option the
                            desc_act row of the ai.lansai.wang field table points
                            at (order vs. compatibility and execution cost; act-
                            order's inference gather: "GPTQ量化算法深度解析" §3.3).
                            Same as 0 when group_size <= 0 */
    double  damp;        /* lambda = damp * mean(diag H) is added to diag H (0.01) */
} gptq_config;

/* Fills *cfg with bits 4, group 128, asymmetric, natural order, block 128,
 * dynamic groups, damp 0.01. */
void gptq_config_default(gptq_config* cfg);

/* ------------------------------------------------------------------------
 * Step 1 -- Hessian accumulation ("GPTQ量化算法深度解析" §3.1 step 1).
 *
 *   H[i][j] += 2 * sum_t X[t][i] * X[t][j]     for i <= j (upper triangle)
 *
 * H: d_in x d_in float64, row stride d_in.  Only entries with i <= j are
 * read or written; the strict lower triangle is left untouched.  The caller
 * zeroes H before the first call; repeated calls over token chunks sum up.
 * X: n_tok x d_in of x_dtype with row stride ld_x elements (ld_x >= d_in).
 * Token products are exact in float32 for bf16/fp16 inputs; they are summed
 * in float32 over runs of 256 tokens, the runs in float64 over windows of
 * up to 32768 tokens, and each window is added to H in float64 in token
 * order (every entry within 32 * 2^-24 * 2 * sum_t |X[t][i] X[t][j]| of the
 * exact sum); the diagonal is summed from exact float64 squares.  fp32
 * inputs are accumulated in float64 throughout.  Deterministic
 * (bit-reproducible).
 * NaN/Inf in X propagate into diag(H) and are reported by gptq_prepare_hinv.
 * workspace: gptq_hessian_workspace(n_tok, d_in) bytes, which covers both
 * uses (the query does not know X's alignment): float64 partial tiles of
 * shorter windows when the layer has fewer than 256 tiles of 256 x 128
 * (d_in below about 4000), and a zero-padded aligned copy of up to 64 MiB
 * of tokens when the rows are not 16-byte aligned (d_in or ld_x not a
 * multiple of 8, or X misaligned).  Aligned rows of a wide layer use none
 * of it.  May be NULL for fp32 inputs or n_tok = 0.  Calls on one
 * workspace must not overlap.
 * ------------------------------------------------------------------------ */
size_t gptq_hessian_workspace(int64_t n_tok, int64_t d_in);
gptq_status gptq_hessian_accumulate(double* H, const void* X, gptq_dtype x_dtype,
                                    int64_t n_tok, int64_t d_in, int64_t ld_x,
                                    void* workspace, size_t ws_bytes, hipStream_t stream);

/* Measurement variant of gptq_hessian_accumulate: the same kernels in the
 * same launch configuration on the same stream, with HIP events recorded
 * around each launch of the Hessian product kernel (up to one window of
 * tiles per launch).
 * Synchronous.  On OK, *syrk_ms (host) holds the mean duration of those
 * launches in milliseconds and *n_launches (host) their number.  Returns
 * GPTQ_ERR_INVALID_ARG for null output pointers, otherwise as
 * gptq_hessian_accumulate, or GPTQ_ERR_HIP if an event call fails. */
gptq_status gptq_hessian_accumulate_timed(double* H, const void* X, gptq_dtype x_dtype,
                                          int64_t n_tok, int64_t d_in, int64_t ld_x,
                                          void* workspace, size_t ws_bytes, hipStream_t stream,
                                          double* syrk_ms, int64_t* n_launches);

/* Allocation-free variant of gptq_hessian_accumulate, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments and result as
 * gptq_hessian_accumulate, minus the workspace: its scratch memory is a
 * fixed device array of GPTQ_NOALLOC_SCRATCH_BYTES bytes inside the library
 * (one per GPU, held until the process ends).  Narrow layers then sum fewer,
 * longer token windows per partial tile (results agree with
 * gptq_hessian_accumulate to float64 rounding; identical when its plan fits
 * the array); inputs whose rows are not 16-byte aligned are copied in
 * chunks of at most a quarter of the array.  Calls nothing that allocates.
 * Returns GPTQ_ERR_WORKSPACE if such a copied chunk of 256 tokens does not
 * fit (misaligned rows wider than 32768 elements), GPTQ_ERR_HIP if the
 * array's address cannot be obtained.  All calls on one GPU share its
 * array: calls that overlap on one GPU race. */
#define GPTQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gptq_status gptq_hessian_accumulate_noalloc(double* H, const void* X, gptq_dtype x_dtype,
                                            int64_t n_tok, int64_t d_in, int64_t ld_x,
                                            hipStream_t stream);

/* ------------------------------------------------------------------------
 * Step 2 -- column order, damping, Cholesky form of the inverse
 * ("GPTQ量化算法深度解析" §2.4, §3.1 steps 1-2, §3.3 desc_act and damp).
 *
 *   perm  = identity, or the stable order of descending diag(H) (act_order);
 *   Hp    = H[perm][perm];  H_d = Hp + lambda*I, lambda = damp * mean(diag H);
 *   U     = upper-triangular with positive diagonal, H_d^{-1} = U^T U.
 *
 * In place: on entry H holds the upper triangle of the undamped Hessian
 * (as left by gptq_hessian_accumulate); on OK return H holds U (row stride
 * d_in, sweep order) with its strict lower triangle set to zero.
 * perm: d_in int32, perm[k] = original index of the k-th swept column.
 * U is obtained as R^{-1} where H_d = R R^T, R upper (a Cholesky
 * factorisation of the index-reversed matrix), which equals the upper
 * Cholesky factor of H_d^{-1} (the factor is unique).
 * Synchronous: returns GPTQ_ERR_NONFINITE if H holds NaN/Inf and
 * GPTQ_ERR_NOT_PD if a pivot is <= 0 (e.g. all-zero H, or damp = 0 with a
 * singular H).  The library never raises damp by itself; retrying with a
 * larger damp (0.1 is the pages' remedy) is the caller's choice.  On error
 * the contents of H and perm are unspecified.
 * workspace: gptq_prepare_hinv_workspace(d_in) bytes.
 * ------------------------------------------------------------------------ */
size_t gptq_prepare_hinv_workspace(int64_t d_in);
gptq_status gptq_prepare_hinv(double* H, int64_t d_in, const gptq_config* cfg,
                              int32_t* perm, void* workspace, size_t ws_bytes,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * Step 3 -- blocked column sweep with error compensation and lazy updates
 * ("GPTQ量化算法深度解析" §2.2, §2.4, §3.1 step 3; grid per "通义千问...
 * GPTQ-Int4" §2.1-2.2).
 *
 * Columns are swept in the order perm (U is in that order).  For sweep
 * column c, with w the column's current values:
 *   at the first column of each group: per row, xmin = min(0, min w_group),
 *     xmax = max(0, max w_group) over the group's current values;
 *     asym: scale = (xmax - xmin)/maxq, zero = rint(-xmin/scale)
 *           (xmin = -1, xmax = 1 if both are 0);
 *     sym:  scale = 2*max(|xmin|, xmax)/maxq (amax 0 -> 1), zero = 2^(bits-1);
 *   code = clamp(rint(w/scale) + zero, 0, maxq), q = scale*(code - zero);
 *   err  = (w - q)/U[c][c]; later columns j of the block: w_j -= err*U[c][j];
 *   after each block [i1,i2): W[:, i2:] -= Err * U[i1:i2, i2:].
 *
 * W: d_out x d_in of w_dtype, row stride ld_w (>= d_in); not modified.
 * U, perm: as returned by gptq_prepare_hinv (U row stride d_in; the strict
 * lower triangle of U must be zero, as that call leaves it).
 * Outputs, all in ORIGINAL column order:
 *   codes   d_out x d_in uint8 (row stride d_in);
 *   scales, zeros   n_groups x d_out float32, [group][row], n_groups =
 *                   ceil(d_in/group_size) (1 when group_size <= 0);
 *   g_idx   d_in int32, the group of each original column (sweep position / g;
 *           with static_groups, original column / g);
 *   w_hat   (nullable) d_out x d_in float32, scale*(code - zero);
 *   row_loss (nullable) d_out float64, sum_c (w_c - q_c)^2 / (2 U_cc^2).
 * Synchronous at the end: returns GPTQ_ERR_INVALID_ARG if perm is not a
 * permutation of 0..d_in-1 and GPTQ_ERR_NONFINITE if W holds NaN/Inf
 * (outputs then unspecified).
 * workspace: gptq_quantize_layer_workspace(d_out, d_in, cfg) bytes.
 * ------------------------------------------------------------------------ */
size_t gptq_quantize_layer_workspace(int64_t d_out, int64_t d_in, const gptq_config* cfg);
gptq_status gptq_quantize_layer(const void* W, gptq_dtype w_dtype, int64_t d_out, int64_t d_in,
                                int64_t ld_w, const double* U, const int32_t* perm,
                                const gptq_config* cfg, uint8_t* codes, float* scales,
                                float* zeros, int32_t* g_idx, float* w_hat, double* row_loss,
                                void* workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Steps 2-3 in factored form: the same quantization without forming the
 * off-diagonal blocks of U ("GPTQ量化算法深度解析" §2.2 compensation, §2.4
 * lazy batch updates, §3.1 steps 2-3).
 *
 * With R = U^{-1} (upper; H_d = R R^T, the Cholesky factorisation of the
 * index-reversed matrix that gptq_prepare_hinv also computes), E the scaled
 * errors of the sweep and Q the quantized weights, the sweep satisfies
 * W0 - Q = E U (W0: the weights before the sweep, in sweep order).  For the
 * 128-column blocks K_k, the compensation that block l receives from the
 * earlier blocks, E[:, <l] U[<l, K_l], then equals
 *   -(W0 - Q)[:, <l] R[<l, K_l] U_ll,   U_ll = U[K_l, K_l] = R_ll^{-1},
 * so the lazy update after block k is W[:, K_l] += (W0 - Q)[:, K_k] F[K_k, K_l]
 * with F[K_k, K_l] = R[K_k, K_l] U_ll, and the sweep inside a block uses U_ll
 * as before.  Only the inverses of R's diagonal blocks are formed: the
 * factorisation skips the inverse products that nothing reads (the
 * off-diagonal blocks of U), about 40 % of its flops.
 *
 * gptq_prepare_hinv_factored: as gptq_prepare_hinv (same inputs, perm and
 * errors) but on OK H holds F (row stride d_in, sweep order): the diagonal
 * 128 x 128 blocks are those of U, the blocks above them R[K_k, K_l] U_ll,
 * the strict lower triangle zero.  d_in must be a multiple of 128
 * (GPTQ_ERR_UNSUPPORTED otherwise).  workspace:
 * gptq_prepare_hinv_factored_workspace(d_in) bytes (0 when unsupported).
 *
 * gptq_quantize_layer_factored: as gptq_quantize_layer (same arguments and
 * outputs, equal to those given U up to float64 rounding) with F in U's
 * place.  Needs cfg->block_size == 128 and every group inside one block:
 * static_groups, or group_size <= 0 or >= d_in (one group per row, a
 * multiple of 8), or a divisor of 128 that is a multiple of 8; otherwise
 * GPTQ_ERR_UNSUPPORTED.  workspace:
 * gptq_quantize_layer_factored_workspace(d_out, d_in, cfg) bytes (that of
 * gptq_quantize_layer plus a float64 copy of W; 0 when unsupported).
 * ------------------------------------------------------------------------ */
size_t gptq_prepare_hinv_factored_workspace(int64_t d_in);
gptq_status gptq_prepare_hinv_factored(double* H, int64_t d_in, const gptq_config* cfg,
                                       int32_t* perm, void* workspace, size_t ws_bytes,
                                       hipStream_t stream);
size_t gptq_quantize_layer_factored_workspace(int64_t d_out, int64_t d_in, const gptq_config* cfg);
gptq_status gptq_quantize_layer_factored(const void* W, gptq_dtype w_dtype, int64_t d_out,
                                         int64_t d_in, int64_t ld_w, const double* F,
                                         const int32_t* perm, const gptq_config* cfg,
                                         uint8_t* codes, float* scales, float* zeros,
                                         int32_t* g_idx, float* w_hat, double* row_loss,
                                         void* workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Step 4 -- packing ("gptq-for-llama" article, "工程细节").
 *
 * Per row, code k occupies bits [bits*k, bits*k + bits) of a little-endian
 * bit stream (bit 0 = least significant bit of word 0); a 3-bit code may
 * straddle two words; bits past the last code are zero.
 * codes: d_out x d_in uint8 (row stride d_in), values < 2^bits (higher bits
 * are masked off).  packed: d_out x gptq_packed_words_per_row(d_in, bits)
 * uint32.  bits: 2, 3, 4 or 8.
 * ------------------------------------------------------------------------ */
int64_t gptq_packed_words_per_row(int64_t d_in, int32_t bits);
gptq_status gptq_pack(const uint8_t* codes, int64_t d_out, int64_t d_in, int32_t bits,
                      uint32_t* packed, hipStream_t stream);

/* Packing in a given column order: stream position k of every row holds the
 * code of column perm[k] ("GPTQ量化算法深度解析" §3.3: with act-order the
 * columns of a group are scattered, and inference gathers them; packing in
 * the quantization order makes each group consecutive again, so that
 * gptq_dequant_matmul gathers activations instead of scales).
 * perm: device int32[d_in], a permutation of 0..d_in-1 (the perm that
 * gptq_prepare_hinv returns); an entry outside [0, d_in) packs code 0.
 * Otherwise as gptq_pack.  Asynchronous. */
gptq_status gptq_pack_permuted(const uint8_t* codes, int64_t d_out, int64_t d_in, int32_t bits,
                               const int32_t* perm, uint32_t* packed, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Product with the quantized weights ("通义千问1.5-1.8B-Chat-GPTQ-Int4模型
 * 压缩技术解析" §2.2: the integer codes with their per-group scale and zero
 * point are turned back into weights for the computation, activations stay
 * in 16-bit; "gptq-for-llama" article, "工程细节": matrix products run
 * directly on the packed words):
 *
 *   Y[t][r] = sum_{k < d_in} X[t][a(k)] * scale[g(k)][r] * (c_r(k) - zero[g(k)][r])
 *
 * with c_r(k) the code at stream position k of packed row r (the layout of
 * gptq_pack).  Three forms of the column order:
 *   perm == NULL, g_idx == NULL: a(k) = k,       g(k) = k / group_size;
 *   perm == NULL, g_idx != NULL: a(k) = k,       g(k) = g_idx[k]
 *                                (original order, as gptq_quantize_layer
 *                                 writes codes and g_idx);
 *   perm != NULL, g_idx == NULL: a(k) = perm[k], g(k) = k / group_size
 *                                (words from gptq_pack_permuted, same perm).
 * group_size <= 0 (or >= d_in): one group, g(k) = 0.
 *
 * X: device, n_tok x d_in, row stride ld_x elements, bf16 / f16 / f32.
 * packed: device uint32, d_out x gptq_packed_words_per_row(d_in, bits).
 * scales, zeros: device float32 [n_groups][d_out]; zeros hold the integer
 * zero points.  n_groups: ceil(d_in / group_size) (1 for one group), or with
 * g_idx the caller's group count (g_idx entries in [0, n_groups)).
 * Y: device float32, n_tok x d_out, row stride ld_y; overwritten.
 * Arithmetic: float32 throughout.  With bf16 / f16 activations, no g_idx and
 * a group size that is a multiple of 32 (or one group), the codes enter
 * half-precision dot products exactly as 2^bits + c and the offset is
 * removed per 32 columns in float32 (8-bit codes with bf16 activations take
 * the per-column route); from 2 tokens on, without perm, the same values
 * go through the matrix cores with float32 sums per group (16 rows x 16-64
 * tokens per workgroup below 128 tokens, 128 x 128 tiles from 128 on);
 * otherwise each weight is formed once in float32.
 * Errors (before any launch): GPTQ_ERR_INVALID_ARG for a bad dtype or bits,
 * sizes outside [0, 2^20] (d_in >= 1), ld_x < d_in, ld_y < d_out, both perm
 * and g_idx given, an n_groups that does not match, or a null pointer;
 * GPTQ_ERR_UNSUPPORTED when the per-column route would need more than
 * gptq_dequant_max_groups() groups.  perm or g_idx entries out of range are
 * not read through: they make the affected outputs NaN.  n_tok == 0 or
 * d_out == 0: nothing is launched.  Asynchronous on `stream`; no allocation.
 * ------------------------------------------------------------------------ */
/* Column gather Xg[t][k] = X[t][perm[k]] ("GPTQ量化算法深度解析" §3.3:
 * act-order puts a gather in front of inference).  With the words from
 * gptq_pack_permuted, gptq_dequant_matmul(Xg, ..., perm = NULL, g_idx =
 * NULL) computes the same product as with perm, and from 2 tokens on it
 * takes the matrix-core routes (with perm, gptq_dequant_matmul reads the
 * activations through perm token by token): for 2 or more tokens the gather
 * followed by the product without perm is the faster form (at 4096 x 11008,
 * 4-bit g128: 24 us against 99 us for 16 tokens).  X: device, n_tok x d_in,
 * row stride ld_x;
 * Xg: device, n_tok x d_in, row stride ld_g (caller-owned, not aliasing X);
 * both of x_dtype.  perm entries outside [0, d_in) give NaN.
 * Errors: GPTQ_ERR_INVALID_ARG for a bad dtype, sizes, strides or a null
 * pointer (n_tok == 0: nothing is launched).  Asynchronous. */
gptq_status gptq_gather_columns(const void* X, gptq_dtype x_dtype, int64_t n_tok, int64_t d_in,
                                int64_t ld_x, const int32_t* perm, void* Xg, int64_t ld_g,
                                hipStream_t stream);

int64_t gptq_dequant_max_groups(void);
gptq_status gptq_dequant_matmul(const void* X, gptq_dtype x_dtype, int64_t n_tok, int64_t d_in,
                                int64_t ld_x, const uint32_t* packed, int32_t bits,
                                const float* scales, const float* zeros, int64_t n_groups,
                                const int32_t* g_idx, const int32_t* perm, int32_t group_size,
                                int64_t d_out, float* Y, int64_t ld_y, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* gptq_status_string(gptq_status status);

/* Library version as "major.minor.patch" (static string). */
const char* gptq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
