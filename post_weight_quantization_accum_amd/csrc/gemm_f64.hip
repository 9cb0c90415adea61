// Float64 GEMM on the gfx950 matrix cores (v_mfma_f64_16x16x4_f64).
//
// Serves the three dense contractions of the solver:
//   * the lazy block update of the weights, W[:, i2:] -= Err * U[i1:i2, i2:]
//     ("GPTQ量化算法深度解析" §2.4 lazy batch update, §3.1 step 3);
//   * the trailing updates of the blocked Cholesky factorisation and of the
//     blocked triangular inverse (§2.4 / §3.1 step 2).
//
// One workgroup (4 wave64s) computes a 128x128 tile of C; each wave owns a
// 64x64 quarter as 4x4 MFMA 16x16 tiles (64 float64 accumulators per lane).
// K is staged through double-buffered LDS in chunks of 16, laid out [k][m]
// with a row stride of 144 doubles, so that each MFMA operand fetch (16
// consecutive doubles per 16 lanes) is conflict-free; the next chunk's
// global loads are in flight while the current chunk is multiplied.
// Workgroups are mapped to tiles so that the ~32 workgroups resident on one
// XCD share rows of A (L2 reuse).
#include "internal.hpp"

namespace gptq {
namespace {

constexpr int TM = 128, TN = 128, KC = 16, LDS_LD = 144;

__device__ __forceinline__ void tri_index(int64_t t, int64_t& r, int64_t& c) {
    // t -> (r, c) with r >= c, enumerating rows of the lower triangle.
    int64_t x = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while (x * (x + 1) / 2 > t) --x;
    while ((x + 1) * (x + 2) / 2 <= t) ++x;
    r = x;
    c = t - x * (x + 1) / 2;
}

// Registers holding one K chunk of a 128-row operand whose K index runs
// along memory rows' columns (A, or B^T): thread t loads row t/2, k range
// (t%2)*8 .. +8.
struct RowsChunk {
    double v[8];
};

template <bool VEC>
__device__ __forceinline__ void load_rows(RowsChunk& c, const double* P, int64_t ld, int64_t row0, int64_t nrows,
                                          int64_t k0, int64_t K) {
    const int t = threadIdx.x;
    const int64_t r = row0 + (t >> 1);
    const int64_t k = k0 + (t & 1) * 8;
    const bool rok = r < nrows;
    const double* p = P + (rok ? r : 0) * ld + k;
    if (VEC && rok && k + 8 <= K) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double2 v = ((const double2*)p)[i];
            c.v[2 * i] = v.x;
            c.v[2 * i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) c.v[i] = (rok && k + i < K) ? p[i] : 0.0;
    }
}

__device__ __forceinline__ void store_rows(double (*lds)[LDS_LD], const RowsChunk& c) {
    const int t = threadIdx.x;
    const int m = t >> 1, kb = (t & 1) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) lds[kb + i][m] = c.v[i];
}

// One K chunk of a K x N row-major operand: thread t loads k = t/16, columns
// (t%16)*8 .. +8.
template <bool VEC>
__device__ __forceinline__ void load_kcols(RowsChunk& c, const double* P, int64_t ld, int64_t k0, int64_t K,
                                           int64_t col0, int64_t ncols) {
    const int t = threadIdx.x;
    const int64_t k = k0 + (t >> 4);
    const int64_t n = col0 + (t & 15) * 8;
    const bool kok = k < K;
    const double* p = P + (kok ? k : 0) * ld + n;
    if (VEC && kok && n + 8 <= ncols) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double2 v = ((const double2*)p)[i];
            c.v[2 * i] = v.x;
            c.v[2 * i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) c.v[i] = (kok && n + i < ncols) ? p[i] : 0.0;
    }
}

__device__ __forceinline__ void store_kcols(double (*lds)[LDS_LD], const RowsChunk& c) {
    const int t = threadIdx.x;
    const int k = t >> 4, n = (t & 15) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) lds[k][n + i] = c.v[i];
}

template <bool TRANS_B, bool LOWER, bool VEC>
__global__ __launch_bounds__(256, 2) void gemm_f64_kernel(int64_t M, int64_t N, int64_t K, double alpha,
                                                       const double* __restrict__ A, int64_t lda,
                                                       const double* __restrict__ B, int64_t ldb,
                                                       double beta, double* C, int64_t ldc,
                                                       int64_t tiles_n, int64_t n_tiles, int64_t per_xcd) {
    __shared__ double sA[2][KC][LDS_LD];
    __shared__ double sB[2][KC][LDS_LD];

    const int64_t b = blockIdx.x;
    const int64_t lin = (b % 8) * per_xcd + b / 8;
    if (lin >= n_tiles) return;
    int64_t tm, tn;
    if (LOWER) {
        tri_index(lin, tm, tn);
    } else {
        tm = lin / tiles_n;
        tn = lin % tiles_n;
    }
    const int64_t m0 = tm * TM, n0 = tn * TN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = wave >> 1, wc = wave & 1;

    d4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = d4_t{0.0, 0.0, 0.0, 0.0};

    const int64_t n_chunks = ceil_div(K, KC);
    RowsChunk ra, rb;
    load_rows<VEC>(ra, A, lda, m0, M, 0, K);
    if (TRANS_B) load_rows<VEC>(rb, B, ldb, n0, N, 0, K);
    else load_kcols<VEC>(rb, B, ldb, 0, K, n0, N);
    store_rows(sA[0], ra);
    if (TRANS_B) store_rows(sB[0], rb);
    else store_kcols(sB[0], rb);
    __syncthreads();

    for (int64_t c = 0; c < n_chunks; ++c) {
        const int cur = c & 1;
        if (c + 1 < n_chunks) {
            const int64_t k0 = (c + 1) * KC;
            load_rows<VEC>(ra, A, lda, m0, M, k0, K);
            if (TRANS_B) load_rows<VEC>(rb, B, ldb, n0, N, k0, K);
            else load_kcols<VEC>(rb, B, ldb, k0, K, n0, N);
        }
#pragma unroll
        for (int kk = 0; kk < KC / 4; ++kk) {
            const int kr = kk * 4 + (lane >> 4);
            double a[4], bb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = sA[cur][kr][wr * 64 + i * 16 + (lane & 15)];
                bb[i] = sB[cur][kr][wc * 64 + i * 16 + (lane & 15)];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f64_16x16x4(a[i], bb[j], acc[i][j]);
        }
        if (c + 1 < n_chunks) {
            store_rows(sA[cur ^ 1], ra);
            if (TRANS_B) store_rows(sB[cur ^ 1], rb);
            else store_kcols(sB[cur ^ 1], rb);
        }
        __syncthreads();
    }

#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + wr * 64 + mi * 16 + 4 * r + (lane >> 4);
            if (m >= M) continue;
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const int64_t n = n0 + wc * 64 + ni * 16 + (lane & 15);
                if (n < N) {
                    double* p = C + m * ldc + n;
                    double v = alpha * acc[mi][ni][r];
                    if (beta != 0.0) v += beta * (*p);
                    *p = v;
                }
            }
        }
}

template <bool TRANS_B, bool LOWER>
void launch_t(hipStream_t s, bool vec, dim3 grid, int64_t M, int64_t N, int64_t K, double alpha, const double* A,
              int64_t lda, const double* B, int64_t ldb, double beta, double* C, int64_t ldc, int64_t tiles_n,
              int64_t n_tiles, int64_t per_xcd) {
    if (vec)
        hipLaunchKernelGGL((gemm_f64_kernel<TRANS_B, LOWER, true>), grid, dim3(256), 0, s, M, N, K, alpha, A, lda, B,
                           ldb, beta, C, ldc, tiles_n, n_tiles, per_xcd);
    else
        hipLaunchKernelGGL((gemm_f64_kernel<TRANS_B, LOWER, false>), grid, dim3(256), 0, s, M, N, K, alpha, A, lda, B,
                           ldb, beta, C, ldc, tiles_n, n_tiles, per_xcd);
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
    if (lower_tiles && M != N) return GPTQ_ERR_INVALID_ARG;
    const int64_t tiles_m = ceil_div(M, TM), tiles_n = ceil_div(N, TN);
    const int64_t n_tiles = lower_tiles ? tiles_m * (tiles_m + 1) / 2 : tiles_m * tiles_n;
    const int64_t per_xcd = ceil_div(n_tiles, 8);
    const bool vec = ((uintptr_t)A % 16 == 0) && (lda % 2 == 0) && ((uintptr_t)B % 16 == 0) && (ldb % 2 == 0);
    const dim3 grid((unsigned)(per_xcd * 8));
    if (transB) {
        if (lower_tiles) launch_t<true, true>(s, vec, grid, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tiles_n, n_tiles, per_xcd);
        else launch_t<true, false>(s, vec, grid, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tiles_n, n_tiles, per_xcd);
    } else {
        if (lower_tiles) launch_t<false, true>(s, vec, grid, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tiles_n, n_tiles, per_xcd);
        else launch_t<false, false>(s, vec, grid, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tiles_n, n_tiles, per_xcd);
    }
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

}  // namespace gptq
