// Internal launch wrappers shared by the C-ABI translation unit.
#pragma once

#include "common.hpp"

namespace gptq {

// Raises a kernel's dynamic LDS limit to at least `bytes` on the current
// device, calling the runtime only the first time for that (device, kernel,
// size): the attribute persists, and the call costs a runtime lookup.
hipError_t ensure_lds_limit(const void* kernel, int bytes);

// Triangular structure of one operand, used to skip the zero part of K
// (the operand's zero entries inside the tile's range must be stored zeros):
//   KEND_ROW: A is lower triangular (A[m][k] = 0 for k > m): K ends at the tile's last row;
//   KEND_COL: op(B) is upper triangular (zero for k > n): K ends at the tile's last column;
//   KBEG_COL: op(B) is lower triangular (zero for k < n): K starts at the tile's first column.
enum GemmTri : int { GEMM_TRI_NONE = 0, GEMM_TRI_KEND_ROW = 1, GEMM_TRI_KEND_COL = 2, GEMM_TRI_KBEG_COL = 3 };

// C = alpha * A * op(B) + beta * C in float64 on MFMA (128x128 or 64x64
// output tiles).  A: M x K row-major (lda); op(B) = B (K x N, ldb) or B^T
// (B is N x K, ldb).
// lower_tiles: only tiles with tile_row >= tile_col are computed
// (M == N required; entries above the diagonal inside diagonal tiles are
// written too).  beta == 0 never reads C.  C may alias an operand only where
// every tile reads nothing but its own rows (of A) or its own columns (of
// B): each tile reads all of K before it writes.
// one_per_cu: at most one workgroup of this launch per CU, which leaves
// registers and LDS on every CU to kernels of other streams.
// max_wg > 0 (products with M or N above 512): at most that many workgroups
// (rounded down to a multiple of 8), each looping over several tiles, so
// that the launch never holds workgroups waiting for a CU: work that other
// streams launch meanwhile is dispatched at once instead of queueing behind
// them.
gptq_status launch_gemm_f64(hipStream_t s, int64_t M, int64_t N, int64_t K, double alpha,
                            const double* A, int64_t lda, const double* B, int64_t ldb,
                            bool transB, double beta, double* C, int64_t ldc, bool lower_tiles,
                            GemmTri tri = GEMM_TRI_NONE, bool one_per_cu = false, int64_t max_wg = 0);

// Two independent small products (both with M, N <= 512) in one launch:
// x a symmetric update (lower_tiles, transB, no triangular range), y a plain
// product (no transB, no lower_tiles, any triangular range).  Anything else
// returns GPTQ_ERR_UNSUPPORTED.  K = 0 products write beta * C (not read when
// beta == 0).
struct GemmCall {
    int64_t M, N, K;
    double alpha;
    const double* A;
    int64_t lda;
    const double* B;
    int64_t ldb;
    bool transB;
    double beta;
    double* C;
    int64_t ldc;
    bool lower_tiles;
    GemmTri tri;
};
gptq_status launch_gemm_f64_pair(hipStream_t s, const GemmCall& x, const GemmCall& y);

// F (sweep order, row stride d, d a multiple of 128) from the lower factor L
// of the reversed damped matrix (row stride d; its off-diagonal 128-blocks
// are read) and Mrev (d/128 blocks of 128 x 128: the inverse of each of L's
// diagonal blocks, columns reversed): F[K_k, K_l] = R[K_k, K_l] U_ll for
// k < l, U_kk on the diagonal, zero below (R = J L J, U_ll = J M_ll J).
gptq_status launch_factor_blocks(hipStream_t s, const double* L, const double* Mrev, double* F, int64_t d);

// Hessian: H (upper) += 2 X^T X.  ws: hessian_workspace_bytes(n_tok, d)
// bytes (float64 partial tiles of narrow layers; an aligned copy of a token
// chunk for inputs whose rows are not 16-byte aligned); unused for fp32
// inputs.  ev: null, or 2 * hessian_syrk_launches(...) events recorded
// around each launch of the Hessian product kernel (start, end) on s.
size_t hessian_workspace_bytes(int64_t n_tok, int64_t d);
int64_t hessian_syrk_launches(int64_t n_tok, gptq_dtype dt, int64_t d, int64_t ld_x, const void* X);
gptq_status hessian_launch(double* H, const void* X, gptq_dtype dt, int64_t n_tok, int64_t d,
                           int64_t ld_x, void* ws, hipStream_t s, hipEvent_t* ev = nullptr);
// The same product with all scratch memory taken from `scratch` (scratch_bytes
// bytes): fewer partial tiles (longer windows, or one window of tiles per
// launch) and shorter copied chunks when they do not fit.  GPTQ_ERR_WORKSPACE
// if a misaligned input's 256-token chunk does not fit in a quarter of it.
gptq_status hessian_launch_scratch(double* H, const void* X, gptq_dtype dt, int64_t n_tok, int64_t d,
                                   int64_t ld_x, void* scratch, size_t scratch_bytes, hipStream_t s);

// Column order, damping, Cholesky of the reversed matrix, triangular inverse,
// rotation into U; factored: the factored form F instead of U (d a multiple
// of 128).  ws layout described in chol.hip.
size_t hinv_workspace_bytes(int64_t d, bool factored = false);
gptq_status hinv_launch(double* H, int64_t d, const gptq_config* cfg, int32_t* perm,
                        void* ws, hipStream_t s, int* host_flags, bool factored = false);

// Column sweep with lazy updates; ws layout described in sweep.hip.
// factored: U is the factored form F (and the lazy updates use it).
size_t sweep_workspace_bytes(int64_t d_out, int64_t d_in, const gptq_config* cfg, bool factored = false);
bool sweep_factored_supported(int64_t d_in, const gptq_config* cfg);
gptq_status sweep_launch(const void* W, gptq_dtype dt, int64_t d_out, int64_t d_in, int64_t ld_w,
                         const double* U, const int32_t* perm, const gptq_config* cfg,
                         uint8_t* codes, float* scales, float* zeros, int32_t* g_idx,
                         float* w_hat, double* row_loss, void* ws, hipStream_t s,
                         int* host_flags, bool factored = false);

// perm: null (stream order = column order) or stream position -> column.
gptq_status pack_launch(const uint8_t* codes, int64_t d_out, int64_t d_in, int32_t bits, const int32_t* perm,
                        uint32_t* packed, hipStream_t s);

// Y = X W_hat^T from packed words (dequant.hip).  perm and g_idx as in
// gptq_dequant_matmul; arguments already validated.
int64_t dequant_max_groups();
gptq_status gather_columns_launch(const void* X, gptq_dtype dt, int64_t n_tok, int64_t d_in, int64_t ld_x,
                                  const int32_t* perm, void* Xg, int64_t ld_g, hipStream_t s);
bool dequant_uses_block_path(gptq_dtype dt, int32_t bits, int64_t d_in, int64_t group_size, bool has_g_idx);
gptq_status dequant_matmul_launch(const void* X, gptq_dtype dt, int64_t n_tok, int64_t d_in, int64_t ld_x,
                                  const uint32_t* packed, int32_t bits, const float* scales, const float* zeros,
                                  int64_t n_groups, const int32_t* g_idx, const int32_t* perm, int64_t group_size,
                                  int64_t d_out, float* Y, int64_t ld_y, hipStream_t s);

}  // namespace gptq
