// Float64 GEMM on the gfx950 matrix cores (v_mfma_f64_16x16x4_f64).
//
// Serves the three dense contractions of the solver:
//   * the lazy block update of the weights, W[:, i2:] -= Err * U[i1:i2, i2:]
//     ("GPTQ量化算法深度解析" §2.4 lazy batch update, §3.1 step 3);
//   * the trailing rank-NB updates of the blocked Cholesky factorisation and
//     of the blocked triangular inverse (§2.4 / §3.1 step 2).
//
// One workgroup (4 wave64s) computes a 64x64 tile of C; each wave owns a
// 32x32 quarter as 2x2 MFMA 16x16 tiles.  K is staged through LDS in chunks
// of 32, transposed so that each MFMA operand fetch is 16 consecutive
// doubles per 16 lanes.
#include "internal.hpp"

namespace gptq {
namespace {

constexpr int TM = 64, TN = 64, KC = 32, PAD = 2, LDS_LD = TM + PAD;

__device__ __forceinline__ void tri_index(int64_t t, int64_t& r, int64_t& c) {
    // t -> (r, c) with r >= c, enumerating rows of the lower triangle.
    int64_t x = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while (x * (x + 1) / 2 > t) --x;
    while ((x + 1) * (x + 2) / 2 <= t) ++x;
    r = x;
    c = t - x * (x + 1) / 2;
}

// Load a 64(rows) x KC(k) panel of a row-major matrix P (row stride ld) whose
// rows are the tile's M or N index and whose columns are k, into
// lds[k][row].  Out-of-range entries are zero.
__device__ __forceinline__ void load_rows_by_k(double (*lds)[LDS_LD], const double* P, int64_t ld,
                                               int64_t row0, int64_t nrows, int64_t k0, int64_t K,
                                               bool vec) {
    const int t = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int r = it * 16 + (t >> 4);
        const int k = (t & 15) * 2;
        const int64_t gr = row0 + r, gk = k0 + k;
        double v0 = 0.0, v1 = 0.0;
        if (gr < nrows) {
            const double* p = P + gr * ld + gk;
            if (vec && gk + 1 < K) {
                double2 v = *(const double2*)p;
                v0 = v.x;
                v1 = v.y;
            } else {
                if (gk < K) v0 = p[0];
                if (gk + 1 < K) v1 = p[1];
            }
        }
        lds[k][r] = v0;
        lds[k + 1][r] = v1;
    }
}

// Load a KC(k) x 64(cols) panel of a row-major K x N matrix into lds[k][col].
__device__ __forceinline__ void load_k_by_cols(double (*lds)[LDS_LD], const double* P, int64_t ld,
                                               int64_t k0, int64_t K, int64_t col0, int64_t ncols,
                                               bool vec) {
    const int t = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int k = it * 8 + (t >> 5);
        const int c = (t & 31) * 2;
        const int64_t gk = k0 + k, gc = col0 + c;
        double v0 = 0.0, v1 = 0.0;
        if (gk < K) {
            const double* p = P + gk * ld + gc;
            if (vec && gc + 1 < ncols) {
                double2 v = *(const double2*)p;
                v0 = v.x;
                v1 = v.y;
            } else {
                if (gc < ncols) v0 = p[0];
                if (gc + 1 < ncols) v1 = p[1];
            }
        }
        lds[k][c] = v0;
        lds[k][c + 1] = v1;
    }
}

template <bool TRANS_B, bool LOWER>
__global__ __launch_bounds__(256) void gemm_f64_kernel(int64_t M, int64_t N, int64_t K, double alpha,
                                                       const double* __restrict__ A, int64_t lda,
                                                       const double* __restrict__ B, int64_t ldb,
                                                       double beta, double* C, int64_t ldc,
                                                       int64_t tiles_n, int vecA, int vecB) {
    __shared__ double sA[KC][LDS_LD];
    __shared__ double sB[KC][LDS_LD];

    int64_t tm, tn;
    if (LOWER) {
        tri_index(blockIdx.x, tm, tn);
    } else {
        tm = blockIdx.x / tiles_n;
        tn = blockIdx.x % tiles_n;
    }
    const int64_t m0 = tm * TM, n0 = tn * TN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = wave >> 1, wc = wave & 1;

    d4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = d4_t{0.0, 0.0, 0.0, 0.0};

    for (int64_t k0 = 0; k0 < K; k0 += KC) {
        load_rows_by_k(sA, A + k0, lda, m0, M, 0, K - k0, vecA);
        if (TRANS_B)
            load_rows_by_k(sB, B + k0, ldb, n0, N, 0, K - k0, vecB);
        else
            load_k_by_cols(sB, B + k0 * ldb, ldb, 0, K - k0, n0, N, vecB);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KC / 4; ++kk) {
            const int kr = kk * 4 + (lane >> 4);
            double a0 = sA[kr][wr * 32 + (lane & 15)];
            double a1 = sA[kr][wr * 32 + 16 + (lane & 15)];
            double b0 = sB[kr][wc * 32 + (lane & 15)];
            double b1 = sB[kr][wc * 32 + 16 + (lane & 15)];
            acc[0][0] = mfma_f64_16x16x4(a0, b0, acc[0][0]);
            acc[0][1] = mfma_f64_16x16x4(a0, b1, acc[0][1]);
            acc[1][0] = mfma_f64_16x16x4(a1, b0, acc[1][0]);
            acc[1][1] = mfma_f64_16x16x4(a1, b1, acc[1][1]);
        }
        __syncthreads();
    }

#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wr * 32 + mi * 16 + 4 * r + (lane >> 4);
                const int64_t n = n0 + wc * 32 + ni * 16 + (lane & 15);
                if (m < M && n < N) {
                    double* p = C + m * ldc + n;
                    double v = alpha * acc[mi][ni][r];
                    if (beta != 0.0) v += beta * (*p);
                    *p = v;
                }
            }
}

}  // namespace

gptq_status launch_gemm_f64(hipStream_t s, int64_t M, int64_t N, int64_t K, double alpha,
                            const double* A, int64_t lda, const double* B, int64_t ldb,
                            bool transB, double beta, double* C, int64_t ldc, bool lower_tiles) {
    if (M <= 0 || N <= 0) return GPTQ_OK;
    if (K <= 0) {
        if (beta == 1.0) return GPTQ_OK;
        return GPTQ_ERR_UNSUPPORTED;
    }
    const int64_t tiles_m = ceil_div(M, TM), tiles_n = ceil_div(N, TN);
    const int64_t n_tiles = lower_tiles ? tiles_m * (tiles_m + 1) / 2 : tiles_m * tiles_n;
    if (lower_tiles && M != N) return GPTQ_ERR_INVALID_ARG;
    const int vecA = ((uintptr_t)A % 16 == 0) && (lda % 2 == 0);
    const int vecB = ((uintptr_t)B % 16 == 0) && (ldb % 2 == 0);
    dim3 grid((unsigned)n_tiles), block(256);
    if (transB) {
        if (lower_tiles)
            hipLaunchKernelGGL((gemm_f64_kernel<true, true>), grid, block, 0, s, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tiles_n, vecA, vecB);
        else
            hipLaunchKernelGGL((gemm_f64_kernel<true, false>), grid, block, 0, s, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tiles_n, vecA, vecB);
    } else {
        if (lower_tiles)
            hipLaunchKernelGGL((gemm_f64_kernel<false, true>), grid, block, 0, s, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tiles_n, vecA, vecB);
        else
            hipLaunchKernelGGL((gemm_f64_kernel<false, false>), grid, block, 0, s, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tiles_n, vecA, vecB);
    }
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

}  // namespace gptq
