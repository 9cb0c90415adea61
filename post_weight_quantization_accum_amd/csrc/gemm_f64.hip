// Float64 GEMM on the gfx950 matrix cores (v_mfma_f64_16x16x4_f64).
//
// Serves the dense contractions of the solver:
//   * the lazy block update of the weights, W[:, i2:] -= Err * U[i1:i2, i2:]
//     ("GPTQ量化算法深度解析" §2.4 lazy batch update, §3.1 step 3);
//   * the off-diagonal products of the recursive Cholesky factorisation and
//     triangular inverse (§2.4 / §3.1 step 2), where one operand is a
//     triangular inverse: each tile then runs K only over the range where
//     that operand is non-zero (GemmTri), which halves those products.
//
// One workgroup (4 wave64s) computes a 128x128 tile of C (each wave a 64x64
// quarter as 4x4 MFMA 16x16 tiles), or a 64x64 tile when the problem has too
// few 128x128 tiles to fill the chip.  K is staged through double-buffered
// LDS in chunks of 16, laid out [k][m] with a row stride of TILE + 16
// doubles, so that each MFMA operand fetch (16 consecutive doubles per 16
// lanes) is conflict-free; the next chunk's global loads are in flight while
// the current chunk is multiplied.  Two workgroups per CU.
// Workgroups are mapped to tiles so that the ~32 workgroups resident on one
// XCD share rows of A (L2 reuse).
#include "internal.hpp"

namespace gptq {
namespace {

constexpr int KC = 16;

__device__ __forceinline__ void tri_index(int64_t t, int64_t& r, int64_t& c) {
    // t -> (r, c) with r >= c, enumerating rows of the lower triangle.
    int64_t x = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while (x * (x + 1) / 2 > t) --x;
    while ((x + 1) * (x + 2) / 2 <= t) ++x;
    r = x;
    c = t - x * (x + 1) / 2;
}

// TILE x TILE output tile (TILE = 64 or 128), 4 waves of (TILE/2)^2.
template <int TILE>
struct Cfg {
    static constexpr int EPT = TILE / 16;        // doubles per thread per operand chunk
    static constexpr int TPR = 16 / EPT;         // threads per row (rows-by-k loads)
    static constexpr int LD = TILE + 16;         // LDS row stride: 32 dwords mod 64 banks
    static constexpr int WT = TILE / 2;          // wave tile edge
    static constexpr int NT = WT / 16;           // MFMA tiles per wave edge
};

// One K chunk of a TILE-row operand whose K index runs along memory rows
// (A, or B^T): thread t loads row t/TPR, k range (t%TPR)*EPT .. +EPT.
template <int TILE, bool VEC>
__device__ __forceinline__ void load_rows(double (&v)[Cfg<TILE>::EPT], const double* P, int64_t ld, int64_t row0,
                                          int64_t nrows, int64_t k0, int64_t K) {
    constexpr int EPT = Cfg<TILE>::EPT, TPR = Cfg<TILE>::TPR;
    const int t = threadIdx.x;
    const int64_t r = row0 + t / TPR;
    const int64_t k = k0 + (t % TPR) * EPT;
    const bool rok = r < nrows;
    const double* p = P + (rok ? r : 0) * ld + k;
    if (VEC && rok && k + EPT <= K) {
#pragma unroll
        for (int i = 0; i < EPT / 2; ++i) {
            const double2 x = ((const double2*)p)[i];
            v[2 * i] = x.x;
            v[2 * i + 1] = x.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < EPT; ++i) v[i] = (rok && k + i < K) ? p[i] : 0.0;
    }
}

template <int TILE>
__device__ __forceinline__ void store_rows(double (*lds)[Cfg<TILE>::LD], const double (&v)[Cfg<TILE>::EPT]) {
    constexpr int EPT = Cfg<TILE>::EPT, TPR = Cfg<TILE>::TPR;
    const int t = threadIdx.x;
    const int m = t / TPR, kb = (t % TPR) * EPT;
#pragma unroll
    for (int i = 0; i < EPT; ++i) lds[kb + i][m] = v[i];
}

// One K chunk of a K x N row-major operand: thread t loads k = t/16,
// columns (t%16)*EPT .. +EPT.
template <int TILE, bool VEC>
__device__ __forceinline__ void load_kcols(double (&v)[Cfg<TILE>::EPT], const double* P, int64_t ld, int64_t k0,
                                           int64_t K, int64_t col0, int64_t ncols) {
    constexpr int EPT = Cfg<TILE>::EPT;
    const int t = threadIdx.x;
    const int64_t k = k0 + (t >> 4);
    const int64_t n = col0 + (t & 15) * EPT;
    const bool kok = k < K;
    const double* p = P + (kok ? k : 0) * ld + n;
    if (VEC && kok && n + EPT <= ncols) {
#pragma unroll
        for (int i = 0; i < EPT / 2; ++i) {
            const double2 x = ((const double2*)p)[i];
            v[2 * i] = x.x;
            v[2 * i + 1] = x.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < EPT; ++i) v[i] = (kok && n + i < ncols) ? p[i] : 0.0;
    }
}

template <int TILE>
__device__ __forceinline__ void store_kcols(double (*lds)[Cfg<TILE>::LD], const double (&v)[Cfg<TILE>::EPT]) {
    constexpr int EPT = Cfg<TILE>::EPT;
    const int t = threadIdx.x;
    const int k = t >> 4, n = (t & 15) * EPT;
#pragma unroll
    for (int i = 0; i < EPT; ++i) lds[k][n + i] = v[i];
}

// Tile of virtual workgroup b (the mapping below assumes that b % 8 is the
// XCD the workgroup runs on, which holds for any grid of a multiple of 8
// workgroups looping over b = blockIdx.x + i * gridDim.x).
template <int TILE, bool TRANS_B, bool LOWER, bool VEC>
__device__ __forceinline__ void gemm_tile(int64_t M, int64_t N, int64_t K, double alpha,
                                          const double* __restrict__ A, int64_t lda,
                                          const double* __restrict__ B, int64_t ldb, double beta, double* C,
                                          int64_t ldc, int64_t tiles_m, int64_t tiles_n, int64_t n_tiles,
                                          int64_t per_xcd, int tri, const int64_t b,
                                          double (&sA)[2][KC][Cfg<TILE>::LD], double (&sB)[2][KC][Cfg<TILE>::LD]) {
    using G = Cfg<TILE>;
    int64_t tm, tn;
    if (LOWER) {
        const int64_t lin = (b % 8) * per_xcd + b / 8;
        if (lin >= n_tiles) return;
        tri_index(lin, tm, tn);
    } else if (tri != GEMM_TRI_NONE && tiles_m >= 16) {
        // triangular operand: tile work varies with the row or the column.
        // Balanced over the XCDs: with f = tiles_m / 8, XCD x takes f whole
        // row bands (rows of A stay in its L2), and the tiles of the
        // remaining r = tiles_m % 8 bands are dealt out by column: tile
        // (leftover band j, column c) goes to XCD (c + 3j) mod 8.  Heaviest
        // tiles are dispatched first.
        const int64_t x = b % 8, q = b / 8;
        const int64_t f = tiles_m / 8, r = tiles_m % 8;
        // leftover band j whose tile in column c belongs to this XCD (3 * 3 = 1 mod 8)
        auto left_j = [&](int64_t c) { return (3 * (x - c % 8) % 8 + 8) % 8; };
        if (tri == GEMM_TRI_KEND_ROW) {
            // work grows with the row.  Whole bands by rank (0 = heaviest,
            // tm = tiles_m - 1 - rank), boustrophedon over the XCDs; the
            // leftover bands are the lightest rows, their tiles last.
            if (q < f * tiles_n) {
                const int64_t k = q / tiles_n;
                const int64_t rank = (k & 1) ? 8 * k + 7 - x : 8 * k + x;
                tm = tiles_m - 1 - rank;
                tn = q % tiles_n;
            } else {
                int64_t rest = q - f * tiles_n;
                tm = -1;
                for (int64_t c = 0; c < tiles_n; ++c) {
                    const int64_t j = left_j(c);
                    if (j >= r) continue;
                    if (rest == 0) {
                        tm = r - 1 - j;   // leftover ranks 8f + j, lightest rows
                        tn = c;
                        break;
                    }
                    --rest;
                }
                if (tm < 0) return;
            }
        } else {
            // work varies along the columns: column-major, heaviest column
            // first; per column the XCD's f whole bands, then its leftover
            // tile of that column if it has one
            int64_t rest = q;
            tm = -1;
            for (int64_t ci = 0; ci < tiles_n; ++ci) {
                const int64_t c = (tri == GEMM_TRI_KEND_COL) ? tiles_n - 1 - ci : ci;
                const int64_t j = left_j(c);
                const int64_t cnt = f + (j < r ? 1 : 0);
                if (rest < cnt) {
                    tm = (rest < f) ? x + 8 * rest : 8 * f + j;
                    tn = c;
                    break;
                }
                rest -= cnt;
            }
            if (tm < 0) return;
        }
    } else {
        const int64_t lin = (b % 8) * per_xcd + b / 8;
        if (lin >= n_tiles) return;
        tm = lin / tiles_n;
        tn = lin % tiles_n;
    }
    const int64_t m0 = tm * TILE, n0 = tn * TILE;
    // K range of this tile: the triangular operand is zero outside it
    int64_t kbeg = 0, kend = K;
    if (tri == GEMM_TRI_KEND_ROW) kend = (m0 + TILE < K) ? m0 + TILE : K;
    else if (tri == GEMM_TRI_KEND_COL) kend = (n0 + TILE < K) ? n0 + TILE : K;
    else if (tri == GEMM_TRI_KBEG_COL) kbeg = (n0 < K) ? n0 : K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = wave >> 1, wc = wave & 1;

    d4_t acc[G::NT][G::NT];
#pragma unroll
    for (int i = 0; i < G::NT; ++i)
#pragma unroll
        for (int j = 0; j < G::NT; ++j) acc[i][j] = d4_t{0.0, 0.0, 0.0, 0.0};

    const int64_t n_chunks = ceil_div(kend - kbeg, KC);
    double ra[G::EPT], rb[G::EPT];
    load_rows<TILE, VEC>(ra, A, lda, m0, M, kbeg, kend);
    if (TRANS_B) load_rows<TILE, VEC>(rb, B, ldb, n0, N, kbeg, kend);
    else load_kcols<TILE, VEC>(rb, B, ldb, kbeg, kend, n0, N);
    store_rows<TILE>(sA[0], ra);
    if (TRANS_B) store_rows<TILE>(sB[0], rb);
    else store_kcols<TILE>(sB[0], rb);
    __syncthreads();

    for (int64_t c = 0; c < n_chunks; ++c) {
        const int cur = c & 1;
        if (c + 1 < n_chunks) {
            const int64_t k0 = kbeg + (c + 1) * KC;
            load_rows<TILE, VEC>(ra, A, lda, m0, M, k0, kend);
            if (TRANS_B) load_rows<TILE, VEC>(rb, B, ldb, n0, N, k0, kend);
            else load_kcols<TILE, VEC>(rb, B, ldb, k0, kend, n0, N);
        }
#pragma unroll
        for (int kk = 0; kk < KC / 4; ++kk) {
            const int kr = kk * 4 + (lane >> 4);
            double a[G::NT], bb[G::NT];
#pragma unroll
            for (int i = 0; i < G::NT; ++i) {
                a[i] = sA[cur][kr][wr * G::WT + i * 16 + (lane & 15)];
                bb[i] = sB[cur][kr][wc * G::WT + i * 16 + (lane & 15)];
            }
#pragma unroll
            for (int i = 0; i < G::NT; ++i)
#pragma unroll
                for (int j = 0; j < G::NT; ++j) acc[i][j] = mfma_f64_16x16x4(a[i], bb[j], acc[i][j]);
        }
        if (c + 1 < n_chunks) {
            store_rows<TILE>(sA[cur ^ 1], ra);
            if (TRANS_B) store_rows<TILE>(sB[cur ^ 1], rb);
            else store_kcols<TILE>(sB[cur ^ 1], rb);
        }
        __syncthreads();
    }

    // C = alpha * acc + beta * C.  The C values of MFMA row group mi + 1 are
    // loaded before group mi is stored, so the reads of the read-modify-write
    // overlap instead of waiting one by one (the compiler cannot reorder a
    // load of C after a store to C).
    const int64_t mrow = m0 + wr * G::WT + (lane >> 4), ncol = n0 + wc * G::WT + (lane & 15);
    double cv[2][4][G::NT];
    auto load_c = [&](double (&dst)[4][G::NT], int mi) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int ni = 0; ni < G::NT; ++ni) {
                const int64_t m = mrow + mi * 16 + 4 * r, n = ncol + ni * 16;
                dst[r][ni] = (beta != 0.0 && m < M && n < N) ? C[m * ldc + n] : 0.0;
            }
    };
    load_c(cv[0], 0);
#pragma unroll
    for (int mi = 0; mi < G::NT; ++mi) {
        if (mi + 1 < G::NT) load_c(cv[(mi + 1) & 1], mi + 1);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int ni = 0; ni < G::NT; ++ni) {
                const int64_t m = mrow + mi * 16 + 4 * r, n = ncol + ni * 16;
                if (m < M && n < N) C[m * ldc + n] = alpha * acc[mi][ni][r] + beta * cv[mi & 1][r][ni];
            }
    }
}

// n_virtual: the tile enumeration's workgroup count; a smaller grid (a
// multiple of 8) loops over it, so that the launch holds at most that many
// workgroups at any time.  The last LDS access of a tile is followed by a
// barrier, and the epilogue uses no LDS, so the next tile may refill it.
template <int TILE, bool TRANS_B, bool LOWER, bool VEC>
__global__ __launch_bounds__(256, 2) void gemm_f64_kernel(int64_t M, int64_t N, int64_t K, double alpha,
                                                          const double* __restrict__ A, int64_t lda,
                                                          const double* __restrict__ B, int64_t ldb,
                                                          double beta, double* C, int64_t ldc,
                                                          int64_t tiles_m, int64_t tiles_n, int64_t n_tiles,
                                                          int64_t per_xcd, int tri, int prio, int64_t n_virtual) {
    using G = Cfg<TILE>;
    __shared__ double sA[2][KC][G::LD];
    __shared__ double sB[2][KC][G::LD];
    // prio: issue priority over the waves of a one-per-CU launch (the far
    // lazy update on a second stream, which shares every CU with this one)
    if (prio) __builtin_amdgcn_s_setprio(2);
    for (int64_t b = blockIdx.x; b < n_virtual; b += gridDim.x)
        gemm_tile<TILE, TRANS_B, LOWER, VEC>(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tiles_m, tiles_n, n_tiles,
                                             per_xcd, tri, b, sA, sB);
}

// Small products (M, N <= SMALL_MN: the lower levels of the recursive
// factorisation): one wave per 16x16 tile of C, operands straight from
// memory (L2) into MFMA registers, 64 values of K per group with the next
// group's loads in flight while the current one multiplies; no LDS and no
// barriers, so a launch costs about one memory round trip plus its MFMAs.
// Per-tile K ranges for triangular operands at 16-column granularity.
constexpr int64_t SMALL_MN = 512;

struct SmallArgs {
    int64_t M, N, K;
    double alpha;
    const double* A;
    int64_t lda;
    const double* B;
    int64_t ldb;
    double beta;
    double* C;
    int64_t ldc, tiles_m, tiles_n, n_tiles;
    int tri;
};

SmallArgs small_args(int64_t M, int64_t N, int64_t K, double alpha, const double* A, int64_t lda, const double* B,
                     int64_t ldb, double beta, double* C, int64_t ldc, bool lower, int tri) {
    const int64_t tm = ceil_div(M, 16), tn = ceil_div(N, 16);
    return SmallArgs{M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tm, tn, lower ? tm * (tm + 1) / 2 : tm * tn, tri};
}

// Tile t of one small product, computed by the calling wave.
template <bool TRANS_B, bool LOWER>
__device__ __forceinline__ void small_tile(const SmallArgs& p, int64_t t, int lane) {
    if (t >= p.n_tiles) return;
    int64_t tm, tn;
    if (LOWER) {
        tri_index(t, tm, tn);
    } else {
        tm = t / p.tiles_n;
        tn = t % p.tiles_n;
    }
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t m0 = tm * 16, n0 = tn * 16;
    int64_t kbeg = 0, kend = K;
    if (p.tri == GEMM_TRI_KEND_ROW) kend = (m0 + 16 < K) ? m0 + 16 : K;
    else if (p.tri == GEMM_TRI_KEND_COL) kend = (n0 + 16 < K) ? n0 + 16 : K;
    else if (p.tri == GEMM_TRI_KBEG_COL) kbeg = (n0 < K) ? n0 : K;
    const int r = lane & 15, kq = lane >> 4;
    const int64_t m = m0 + r, n = n0 + r;
    const double* pa = p.A + (m < M ? m : 0) * p.lda;
    const double* pb = TRANS_B ? p.B + (n < N ? n : 0) * p.ldb : p.B + (n < N ? n : 0);
    const int64_t ldb = p.ldb;
    // operand k of this lane: A[m][k] and op(B)[k][n]; zero outside the ranges
    constexpr int G = 4;   // MFMA K-steps of 16 per group
    auto load_group = [&](double (&a)[G][4], double (&b)[G][4], int64_t k0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t k = k0 + 16 * g + 4 * q + kq;
                const bool kok = k < kend;
                a[g][q] = (kok && m < M) ? pa[k] : 0.0;
                b[g][q] = (kok && n < N) ? (TRANS_B ? pb[k] : pb[k * ldb]) : 0.0;
            }
    };
    double a0[G][4], b0[G][4], a1[G][4], b1[G][4];
    d4_t acc = {0.0, 0.0, 0.0, 0.0};
    const int64_t ngroups = (kend > kbeg) ? ceil_div(kend - kbeg, 16 * G) : 0;
    if (ngroups > 0) load_group(a0, b0, kbeg);
    for (int64_t gi = 0; gi < ngroups; gi += 2) {
        if (gi + 1 < ngroups) load_group(a1, b1, kbeg + (gi + 1) * 16 * G);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = mfma_f64_16x16x4(a0[g][q], b0[g][q], acc);
        if (gi + 1 >= ngroups) break;
        if (gi + 2 < ngroups) load_group(a0, b0, kbeg + (gi + 2) * 16 * G);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = mfma_f64_16x16x4(a1[g][q], b1[g][q], acc);
    }
    // result element i of this lane: C[m0 + 4i + kq][n0 + r]; C read before any store
    double cv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t mi = m0 + 4 * i + kq;
        cv[i] = (p.beta != 0.0 && mi < M && n < N) ? p.C[mi * p.ldc + n] : 0.0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t mi = m0 + 4 * i + kq;
        if (mi < M && n < N) p.C[mi * p.ldc + n] = p.alpha * acc[i] + p.beta * cv[i];
    }
}

template <bool TRANS_B, bool LOWER>
__global__ __launch_bounds__(256) void gemm_f64_small_kernel(SmallArgs p) {
    small_tile<TRANS_B, LOWER>(p, (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6), threadIdx.x & 63);
}

// Two independent small products in one launch: a symmetric update
// (lower tiles, op(B) = B^T) and a plain product; the workgroups of the
// second follow those of the first.
__global__ __launch_bounds__(256) void gemm_f64_small_pair_kernel(SmallArgs p1, SmallArgs p2, int64_t nb1) {
    const int64_t b = blockIdx.x;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (b < nb1) small_tile<true, true>(p1, b * 4 + w, lane);
    else small_tile<false, false>(p2, (b - nb1) * 4 + w, lane);
}

// The factored form of the inverse's Cholesky factor (sweep order): for
// 128-column blocks k < l, F[K_k, K_l] = R[K_k, K_l] U_ll with R = J L J
// (L the lower factor of the reversed matrix, in Lf) and U_ll = J M_ll J
// (M_ll the inverse of L's diagonal block); F's diagonal blocks are U_ll,
// its strict lower triangle zero.  Mrev holds each M_ll with its columns
// reversed ([block][k][127 - n] = M_ll[k][n]), so that one product per
// block pair writes F rotated: row r' of L goes to row d - 1 - r' of F and
// column n of the product to column d - 128 - 128 l + n.  One workgroup per
// block pair (j >= l, reversed order): j > l computes its block and zeroes
// the mirrored block below F's diagonal; j == l writes U_ll.
__global__ __launch_bounds__(256, 2) void factor_blocks_kernel(const double* __restrict__ Lf,
                                                               const double* __restrict__ Mrev, double* F,
                                                               int64_t d) {
    constexpr int T = 128;
    __shared__ double sA[2][KC][Cfg<T>::LD];
    __shared__ double sB[2][KC][Cfg<T>::LD];
    int64_t j, l;
    tri_index(blockIdx.x, j, l);
    const int64_t nb = d / T;
    const double* Ml = Mrev + l * T * T;
    if (j == l) {
        const int64_t k = nb - 1 - l;   // F's block
        for (int e = threadIdx.x; e < T * T; e += 256) {
            const int i = e / T, jj = e % T;
            F[(k * T + i) * d + k * T + jj] = (i <= jj) ? Ml[(T - 1 - i) * T + jj] : 0.0;
        }
        return;
    }
    // the mirrored block under F's diagonal: rows of F's block nb-1-l, columns of nb-1-j
    {
        const int64_t br = nb - 1 - l, bc = nb - 1 - j;
        for (int e = threadIdx.x; e < T * T; e += 256) F[(br * T + e / T) * d + bc * T + e % T] = 0.0;
    }
    double* C = F + (d - 1 - j * T) * d + (d - T - l * T);
    gemm_tile<T, false, false, true>(T, T, T, 1.0, Lf + (j * T) * d + l * T, d, Ml, T, 0.0, C, -d, 1, 1, 1, 1,
                                     GEMM_TRI_NONE, 0, sA, sB);
}

template <bool TRANS_B, bool LOWER>
void launch_small(hipStream_t s, int64_t M, int64_t N, int64_t K, double alpha, const double* A, int64_t lda,
                  const double* B, int64_t ldb, double beta, double* C, int64_t ldc, int tri) {
    const SmallArgs p = small_args(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, LOWER, tri);
    hipLaunchKernelGGL((gemm_f64_small_kernel<TRANS_B, LOWER>), dim3((unsigned)ceil_div(p.n_tiles, 4)), dim3(256),
                       0, s, p);
}

// LDS a workgroup must hold so that only one fits on a CU (160 KiB each).
constexpr size_t CU_LDS = 160 * 1024;

template <int TILE, bool TRANS_B, bool LOWER>
void launch_t(hipStream_t s, bool vec, int64_t M, int64_t N, int64_t K, double alpha, const double* A, int64_t lda,
              const double* B, int64_t ldb, double beta, double* C, int64_t ldc, int tri, bool one_per_cu,
              int64_t max_wg) {
    const int64_t tiles_m = ceil_div(M, TILE), tiles_n = ceil_div(N, TILE);
    const int64_t n_tiles = LOWER ? tiles_m * (tiles_m + 1) / 2 : tiles_m * tiles_n;
    // per XCD: whole bands plus at most one leftover tile per column (triangular case)
    const int64_t per_xcd = (!LOWER && tri != GEMM_TRI_NONE && tiles_m >= 16) ? (tiles_m / 8 + 1) * tiles_n
                                                                              : ceil_div(n_tiles, 8);
    const int64_t n_virtual = per_xcd * 8;
    const int64_t bounded = (max_wg / 8) * 8;
    const dim3 grid((unsigned)((bounded > 0 && bounded < n_virtual) ? bounded : n_virtual));
    // one_per_cu: unused dynamic LDS beyond half a CU's, so that a second
    // workgroup of this launch never shares the CU (room for other streams)
    constexpr size_t static_lds = 2 * 2 * KC * Cfg<TILE>::LD * sizeof(double);
    const size_t pad = one_per_cu ? CU_LDS / 2 + 1024 - static_lds : 0;
    if (vec)
        hipLaunchKernelGGL((gemm_f64_kernel<TILE, TRANS_B, LOWER, true>), grid, dim3(256), pad, s, M, N, K, alpha,
                           A, lda, B, ldb, beta, C, ldc, tiles_m, tiles_n, n_tiles, per_xcd, tri, one_per_cu ? 0 : 1,
                           n_virtual);
    else
        hipLaunchKernelGGL((gemm_f64_kernel<TILE, TRANS_B, LOWER, false>), grid, dim3(256), pad, s, M, N, K, alpha,
                           A, lda, B, ldb, beta, C, ldc, tiles_m, tiles_n, n_tiles, per_xcd, tri, one_per_cu ? 0 : 1,
                           n_virtual);
}

template <bool TRANS_B, bool LOWER>
void launch_sel(hipStream_t s, bool vec, int64_t M, int64_t N, int64_t K, double alpha, const double* A, int64_t lda,
                const double* B, int64_t ldb, double beta, double* C, int64_t ldc, int tri, bool one_per_cu,
                int64_t max_wg) {
    // 128x128 tiles when there are enough of them to fill the chip twice,
    // else 64x64 tiles (4x the workgroups)
    const int64_t tm = ceil_div(M, 128), tn = ceil_div(N, 128);
    const int64_t t128 = LOWER ? tm * (tm + 1) / 2 : tm * tn;
    if (t128 >= 512)
        launch_t<128, TRANS_B, LOWER>(s, vec, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tri, one_per_cu, max_wg);
    else
        launch_t<64, TRANS_B, LOWER>(s, vec, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, tri, one_per_cu, max_wg);
}

}  // namespace

gptq_status launch_gemm_f64(hipStream_t s, int64_t M, int64_t N, int64_t K, double alpha,
                            const double* A, int64_t lda, const double* B, int64_t ldb,
                            bool transB, double beta, double* C, int64_t ldc, bool lower_tiles, GemmTri tri,
                            bool one_per_cu, int64_t max_wg) {
    if (M <= 0 || N <= 0) return GPTQ_OK;
    if (lower_tiles && tri != GEMM_TRI_NONE) return GPTQ_ERR_INVALID_ARG;
    if (K <= 0) {
        if (beta == 1.0) return GPTQ_OK;
        return GPTQ_ERR_UNSUPPORTED;
    }
    if (lower_tiles && M != N) return GPTQ_ERR_INVALID_ARG;
    if (M <= SMALL_MN && N <= SMALL_MN) {
        if (transB) {
            if (lower_tiles) launch_small<true, true>(s, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, (int)tri);
            else launch_small<true, false>(s, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, (int)tri);
        } else {
            if (lower_tiles) launch_small<false, true>(s, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, (int)tri);
            else launch_small<false, false>(s, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, (int)tri);
        }
        GPTQ_LAUNCH_CHECK();
        return GPTQ_OK;
    }
    const bool vec = ((uintptr_t)A % 16 == 0) && (lda % 2 == 0) && ((uintptr_t)B % 16 == 0) && (ldb % 2 == 0);
    if (transB) {
        if (lower_tiles)
            launch_sel<true, true>(s, vec, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, (int)tri, one_per_cu, max_wg);
        else
            launch_sel<true, false>(s, vec, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, (int)tri, one_per_cu, max_wg);
    } else {
        if (lower_tiles)
            launch_sel<false, true>(s, vec, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, (int)tri, one_per_cu, max_wg);
        else
            launch_sel<false, false>(s, vec, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, (int)tri, one_per_cu, max_wg);
    }
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

gptq_status launch_factor_blocks(hipStream_t s, const double* L, const double* Mrev, double* F, int64_t d) {
    if (d <= 0 || d % 128 != 0) return GPTQ_ERR_UNSUPPORTED;
    const int64_t nb = d / 128;
    if (nb * (nb + 1) / 2 > INT32_MAX) return GPTQ_ERR_UNSUPPORTED;
    if ((uintptr_t)L % 16 != 0 || (uintptr_t)Mrev % 16 != 0) return GPTQ_ERR_INVALID_ARG;
    hipLaunchKernelGGL(factor_blocks_kernel, dim3((unsigned)(nb * (nb + 1) / 2)), dim3(256), 0, s, L, Mrev, F, d);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

gptq_status launch_gemm_f64_pair(hipStream_t s, const GemmCall& x, const GemmCall& y) {
    const bool small = x.M <= SMALL_MN && x.N <= SMALL_MN && y.M <= SMALL_MN && y.N <= SMALL_MN;
    if (!small || !x.transB || !x.lower_tiles || x.tri != GEMM_TRI_NONE || y.transB || y.lower_tiles ||
        x.M != x.N || x.M <= 0 || y.M <= 0 || y.N <= 0 || x.K < 0 || y.K < 0)
        return GPTQ_ERR_UNSUPPORTED;
    const SmallArgs p1 = small_args(x.M, x.N, x.K, x.alpha, x.A, x.lda, x.B, x.ldb, x.beta, x.C, x.ldc, true, x.tri);
    const SmallArgs p2 = small_args(y.M, y.N, y.K, y.alpha, y.A, y.lda, y.B, y.ldb, y.beta, y.C, y.ldc, false, y.tri);
    const int64_t nb1 = ceil_div(p1.n_tiles, 4), nb2 = ceil_div(p2.n_tiles, 4);
    hipLaunchKernelGGL(gemm_f64_small_pair_kernel, dim3((unsigned)(nb1 + nb2)), dim3(256), 0, s, p1, p2, nb1);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

}  // namespace gptq
