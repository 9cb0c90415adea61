// Column order, damping and the Cholesky form of the inverse Hessian
// ("GPTQ量化算法深度解析" §2.4: a Cholesky factorisation replaces repeated,
// unstable inversion; §3.1 steps 1-2: H_d = H + lambda*I is factored once;
// §3.3: desc_act order and damp_percent).
//
// The sweep needs U, upper triangular with H_d^{-1} = U^T U.  Instead of
// factoring H_d, inverting, forming H_d^{-1} and factoring again, this file
// factors the index-reversed matrix Hr = J H_d J = L L^T (lower), inverts L
// (M = L^{-1}) and reads U off as U = J M J: with R = J L J upper,
// H_d = R R^T, so H_d^{-1} = (R^{-1})^T R^{-1} and R^{-1} = J M J is the
// unique upper factor with positive diagonal.  That is 2/3 d^3 flops instead
// of 4/3 d^3, all in float64.
//
// Blocked right-looking Cholesky and blocked forward-substitution inverse
// with NB = 64 (blocks handled in pairs, so the large trailing updates run
// with K = 128): a one-workgroup kernel factors and inverts each 64x64
// diagonal block in LDS; the panel solves and the trailing updates are
// float64 MFMA GEMMs (gemm_f64.hip).
//
// Workspace layout (byte offsets):
//   [0, 256)             int flags[N_FLAGS]; double lambda at 64; double diag sum at 72
//   [256, 256+P)         diagonal-block inverses, nblk x NB x NB doubles
//   [.., + d*d*8)        Hr / L (lower triangle), later U before the copy-back
#include "internal.hpp"

namespace gptq {
namespace {

constexpr int NB = 64;

struct Ws {
    int* flags;
    double* lambda;
    double* dinv;
    double* L;
};

Ws carve(void* ws, int64_t d) {
    char* p = (char*)ws;
    Ws w;
    w.flags = (int*)p;
    w.lambda = (double*)(p + 64);
    const int64_t nblk = ceil_div(d, NB);
    w.dinv = (double*)(p + 256);
    size_t off = align_up(256 + (size_t)nblk * NB * NB * sizeof(double), 256);
    w.L = (double*)(p + off);
    return w;
}

// lambda = damp * mean(diag H); flags non-finite diagonal entries.
__global__ __launch_bounds__(1024) void diag_stats_kernel(const double* __restrict__ H, int64_t d, double damp,
                                                          double* lambda, int* flags) {
    __shared__ double part[1024];
    const int t = threadIdx.x;
    double s = 0.0;
    for (int64_t i = t; i < d; i += 1024) {
        const double v = H[i * d + i];
        if (!isfinite(v)) raise_flag(flags, FLAG_NONFINITE);
        s += v;
    }
    part[t] = s;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if (t < w) part[t] += part[t + w];
        __syncthreads();
    }
    if (t == 0) *lambda = damp * (part[0] / (double)d);
}

// act-order: perm[rank(j)] = j, rank by (descending diag, ascending index).
// NaN keys sort last; the ranks always form a permutation.
__device__ __forceinline__ bool before(double ki, int64_t i, double kj, int64_t j) {
    const bool ni = isnan(ki), nj = isnan(kj);
    if (ni || nj) return (ni == nj) ? (i < j) : nj;
    return (ki > kj) || (ki == kj && i < j);
}

__global__ __launch_bounds__(256) void rank_kernel(const double* __restrict__ H, int64_t d, int32_t* perm) {
    __shared__ double keys[1024];
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const double kj = (j < d) ? H[j * d + j] : 0.0;
    int64_t rank = 0;
    for (int64_t base = 0; base < d; base += 1024) {
        __syncthreads();
        for (int e = threadIdx.x; e < 1024; e += 256) {
            const int64_t i = base + e;
            keys[e] = (i < d) ? H[i * d + i] : 0.0;
        }
        __syncthreads();
        const int64_t lim = (d - base < 1024) ? d - base : 1024;
        for (int64_t e = 0; e < lim; ++e) rank += before(keys[e], base + e, kj, j) ? 1 : 0;
    }
    if (j < d) perm[rank] = (int32_t)j;
}

__global__ void iota_kernel(int32_t* perm, int64_t d) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k < d) perm[k] = (int32_t)k;
}

// Mirror the upper triangle into the lower one (32x32 tiles through LDS) and
// flag non-finite entries.
__global__ __launch_bounds__(256) void symmetrize_kernel(double* H, int64_t d, int* flags) {
    __shared__ double tile[32][33];
    // lower-triangle tile (bi >= bj) receives the transpose of upper tile (bj, bi)
    int64_t t = blockIdx.x;
    int64_t x = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while (x * (x + 1) / 2 > t) --x;
    while ((x + 1) * (x + 2) / 2 <= t) ++x;
    const int64_t bi = x, bj = t - x * (x + 1) / 2;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    bool bad = false;
    for (int r = ty; r < 32; r += 8) {
        const int64_t i = bj * 32 + r, j = bi * 32 + tx;  // upper source (i <= j)
        double v = 0.0;
        if (i < d && j < d && i <= j) {
            v = H[i * d + j];
            bad |= !isfinite(v);
        }
        tile[r][tx] = v;
    }
    __syncthreads();
    for (int r = ty; r < 32; r += 8) {
        const int64_t i = bi * 32 + r, j = bj * 32 + tx;  // lower destination (i > j)
        if (i < d && j < d && i > j) H[i * d + j] = tile[tx][r];
    }
    if (bad) raise_flag(flags, FLAG_NONFINITE);
}

// Hr[a][b] = H[p[d-1-a]][p[d-1-b]] (+ lambda on the diagonal), b <= a.
__global__ __launch_bounds__(256) void gather_reverse_kernel(const double* __restrict__ H, int64_t d,
                                                             const int32_t* __restrict__ perm,
                                                             const double* __restrict__ lambda, double* Hr) {
    const int64_t a = blockIdx.x;
    const int64_t pa = perm[d - 1 - a];
    const double lam = *lambda;
    const double* row = H + pa * d;
    for (int64_t b = threadIdx.x; b <= a; b += 256) {
        const int64_t pb = perm[d - 1 - b];
        double v = row[pb];
        if (b == a) v += lam;
        Hr[a * d + b] = v;
    }
}

// Factor the k-th 64x64 diagonal block of L in place (lower), store its
// inverse into dinv[k] and into the diagonal block of Minv.
__global__ __launch_bounds__(256) void diag_block_kernel(double* L, int64_t d, int64_t k, double* dinv,
                                                         double* Minv, int* flags) {
    __shared__ double A[NB][NB + 1];
    __shared__ double D[NB][NB + 1];
    __shared__ double red[4][NB];
    const int t = threadIdx.x;
    const int64_t o = k * NB;
    const int nb = (int)((d - o < NB) ? d - o : NB);
    for (int e = t; e < NB * NB; e += 256) {
        const int i = e / NB, j = e % NB;
        double v;
        if (i < nb && j < nb) v = (j <= i) ? L[(o + i) * d + o + j] : 0.0;
        else v = (i == j) ? 1.0 : 0.0;
        A[i][j] = v;
    }
    __syncthreads();
    // unblocked right-looking Cholesky
    for (int j = 0; j < NB; ++j) {
        double piv = A[j][j];
        if (!(piv > 0.0)) {
            if (t == 0) raise_flag(flags, isnan(piv) ? FLAG_NONFINITE : FLAG_NOT_PD);
            piv = 1.0;
        }
        const double ljj = sqrt(piv);
        __syncthreads();
        if (t < NB) {
            if (t == j) A[j][j] = ljj;
            else if (t > j) A[t][j] = A[t][j] / ljj;
        }
        __syncthreads();
        {
            const int i = t & 63, cg = t >> 6;
            if (i > j) {
                const double lij = A[i][j];
                for (int c = j + 1 + cg; c <= i; c += 4) A[i][c] = fma(-lij, A[c][j], A[i][c]);
            }
        }
        __syncthreads();
    }
    // inverse by rows: D[i][c] = (delta_ic - sum_{c<=m<i} A[i][m] D[m][c]) / A[i][i]
    for (int i = 0; i < NB; ++i) {
        const int c = t & 63, part = t >> 6;
        double s = 0.0;
        if (c < i)
            for (int m = c + part; m < i; m += 4) s = fma(A[i][m], D[m][c], s);
        red[part][c] = s;
        __syncthreads();
        if (t < NB) {
            double v = 0.0;
            if (t < i) v = -(((red[0][t] + red[1][t]) + red[2][t]) + red[3][t]) / A[i][i];
            else if (t == i) v = 1.0 / A[i][i];
            D[i][t] = v;
        }
        __syncthreads();
    }
    double* dk = dinv + k * NB * NB;
    for (int e = t; e < NB * NB; e += 256) {
        const int i = e / NB, j = e % NB;
        dk[e] = (i < nb && j < nb) ? D[i][j] : 0.0;
        if (i < nb && j <= i) {
            L[(o + i) * d + o + j] = A[i][j];
            Minv[(o + i) * d + o + j] = D[i][j];
        }
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(double* p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) p[i] = 0.0;
}

// U[c][j] = M[d-1-c][d-1-j] for j >= c, 0 below the diagonal.
__global__ __launch_bounds__(256) void rotate_kernel(const double* __restrict__ M, int64_t d, double* U) {
    const int64_t c = blockIdx.x;
    for (int64_t j = threadIdx.x; j < d; j += 256)
        U[c * d + j] = (j >= c) ? M[(d - 1 - c) * d + (d - 1 - j)] : 0.0;
}

}  // namespace

size_t hinv_workspace_bytes(int64_t d) {
    const int64_t nblk = ceil_div(d, NB);
    return align_up(256 + (size_t)nblk * NB * NB * sizeof(double), 256) + (size_t)d * d * sizeof(double);
}

gptq_status hinv_launch(double* H, int64_t d, const gptq_config* cfg, int32_t* perm, void* ws,
                        hipStream_t s, int* host_flags) {
    Ws w = carve(ws, d);
    double* L = w.L;
    GPTQ_HIP(hipMemsetAsync(w.flags, 0, 256, s));

    hipLaunchKernelGGL(diag_stats_kernel, dim3(1), dim3(1024), 0, s, H, d, cfg->damp, w.lambda, w.flags);
    GPTQ_LAUNCH_CHECK();
    const unsigned gd = (unsigned)ceil_div(d, 256);
    if (cfg->act_order)
        hipLaunchKernelGGL(rank_kernel, dim3(gd), dim3(256), 0, s, H, d, perm);
    else
        hipLaunchKernelGGL(iota_kernel, dim3(gd), dim3(256), 0, s, perm, d);
    GPTQ_LAUNCH_CHECK();
    const int64_t T32 = ceil_div(d, 32);
    hipLaunchKernelGGL(symmetrize_kernel, dim3((unsigned)(T32 * (T32 + 1) / 2)), dim3(256), 0, s, H, d, w.flags);
    GPTQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(gather_reverse_kernel, dim3((unsigned)d), dim3(256), 0, s, H, d, perm, w.lambda, L);
    GPTQ_LAUNCH_CHECK();
    // H's buffer now becomes the inverse M (lower block triangle), zero first.
    hipLaunchKernelGGL(fill_zero_kernel, dim3(2048), dim3(256), 0, s, H, d * d);
    GPTQ_LAUNCH_CHECK();

    // Blocked right-looking Cholesky, 64-column blocks taken in pairs: the
    // second block of a pair is brought up to date with a thin update, so
    // the big trailing update of the rest has K = 128.
    const int64_t nblk = ceil_div(d, NB);
    gptq_status st;
    for (int64_t k = 0; k < nblk; k += 2) {
        const int64_t o = k * NB;
        hipLaunchKernelGGL(diag_block_kernel, dim3(1), dim3(256), 0, s, L, d, k, w.dinv, H, w.flags);
        GPTQ_LAUNCH_CHECK();
        const int64_t r1 = d - o - NB;  // rows below block k
        if (r1 <= 0) break;
        // panel k: L[o+NB:, o:o+NB] <- L[o+NB:, o:o+NB] * Dinv_k^T
        st = launch_gemm_f64(s, r1, NB, NB, 1.0, L + (o + NB) * d + o, d, w.dinv + k * NB * NB, NB, true, 0.0,
                             L + (o + NB) * d + o, d, false);
        if (st != GPTQ_OK) return st;
        // block column k+1 -= panel k * (its rows of panel k)^T
        const int64_t nb1 = (r1 < NB) ? r1 : NB;
        st = launch_gemm_f64(s, r1, nb1, NB, -1.0, L + (o + NB) * d + o, d, L + (o + NB) * d + o, d, true, 1.0,
                             L + (o + NB) * d + o + NB, d, false);
        if (st != GPTQ_OK) return st;
        hipLaunchKernelGGL(diag_block_kernel, dim3(1), dim3(256), 0, s, L, d, k + 1, w.dinv, H, w.flags);
        GPTQ_LAUNCH_CHECK();
        const int64_t r2 = d - o - 2 * NB;  // rows below block k+1
        if (r2 <= 0) break;
        st = launch_gemm_f64(s, r2, NB, NB, 1.0, L + (o + 2 * NB) * d + o + NB, d, w.dinv + (k + 1) * NB * NB, NB,
                             true, 0.0, L + (o + 2 * NB) * d + o + NB, d, false);
        if (st != GPTQ_OK) return st;
        // trailing: L[o+2NB:, o+2NB:] -= P P^T, P = L[o+2NB:, o:o+2NB] (lower tiles)
        st = launch_gemm_f64(s, r2, r2, 2 * NB, -1.0, L + (o + 2 * NB) * d + o, d, L + (o + 2 * NB) * d + o, d, true,
                             1.0, L + (o + 2 * NB) * d + o + 2 * NB, d, true);
        if (st != GPTQ_OK) return st;
    }
    // Blocked forward substitution M = L^{-1} (in H's buffer, whose diagonal
    // blocks already hold Dinv_i): block row i becomes M[i, :i] = Dinv_i B[i, :i];
    // rows below then lose L[r, i] M[i, :].  Block rows are taken in pairs so
    // that the update of the rows below has K = 128.
    for (int64_t i = 0; i < nblk; i += 2) {
        const int64_t o = i * NB;
        const int64_t nb0 = (d - o < NB) ? d - o : NB;
        if (i > 0) {
            st = launch_gemm_f64(s, nb0, o, nb0, 1.0, w.dinv + i * NB * NB, NB, H + o * d, d, false, 0.0, H + o * d, d,
                                 false);
            if (st != GPTQ_OK) return st;
        }
        const int64_t r1 = d - o - nb0;
        if (r1 <= 0) break;
        const int64_t nb1 = (r1 < NB) ? r1 : NB;
        // block row i+1: B[i+1, :i+1] -= L[i+1, i] M[i, :i+1]; then M[i+1, :i+1] = Dinv_{i+1} B[i+1, :i+1]
        st = launch_gemm_f64(s, nb1, o + nb0, nb0, -1.0, L + (o + nb0) * d + o, d, H + o * d, d, false, 1.0,
                             H + (o + nb0) * d, d, false);
        if (st != GPTQ_OK) return st;
        st = launch_gemm_f64(s, nb1, o + nb0, nb1, 1.0, w.dinv + (i + 1) * NB * NB, NB, H + (o + nb0) * d, d, false,
                             0.0, H + (o + nb0) * d, d, false);
        if (st != GPTQ_OK) return st;
        const int64_t r2 = r1 - nb1;
        if (r2 <= 0) break;
        const int64_t kk = nb0 + nb1;
        st = launch_gemm_f64(s, r2, o + kk, kk, -1.0, L + (o + kk) * d + o, d, H + o * d, d, false, 1.0,
                             H + (o + kk) * d, d, false);
        if (st != GPTQ_OK) return st;
    }
    hipLaunchKernelGGL(rotate_kernel, dim3((unsigned)d), dim3(256), 0, s, H, d, L);
    GPTQ_LAUNCH_CHECK();
    GPTQ_HIP(hipMemcpyAsync(H, L, (size_t)d * d * sizeof(double), hipMemcpyDeviceToDevice, s));
    GPTQ_HIP(hipMemcpyAsync(host_flags, w.flags, N_FLAGS * sizeof(int), hipMemcpyDeviceToHost, s));
    GPTQ_HIP(hipStreamSynchronize(s));
    return GPTQ_OK;
}

}  // namespace gptq
