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
// L and M come out of one recursion over halves (split at a multiple of
// 128).  For Hr = [A11 .; A21 A22]:
//   (L11, M11) = chol_inv(A11)
//   L21 = A21 M11^T                   (M11^T upper: K ends at the tile's column)
//   A22 <- A22 - L21 L21^T            (lower tiles)
//   T   = L21 M11                     (M11 lower: K starts at the tile's column)
//   (L22, M22) = chol_inv(A22)
//   M21 = -M22 T                      (M22 lower: K ends at the tile's row)
// so the big products have K up to d/2 and run near the float64 MFMA peak,
// where a right-looking blocked factorisation would be stuck at K = 64..128.
// The leaves are 128x128 blocks factored and inverted by one workgroup in
// LDS (16x16 inner blocks; see leaf_blocked_kernel).  L itself is never
// stored outside the leaves: only M (written into H's buffer) is needed.
//
// Workspace layout (byte offsets):
//   [0, 256)             int flags[N_FLAGS]; double lambda at 64
//   [256, +8d)           diag(H), contiguous (act-order keys)
//   [.., +4d)            inverse permutation
//   [.., + d*d*8)        Hr (lower triangle); T blocks replace the A21 blocks
//   per depth k          L21 scratch, max n1*n2 doubles over the nodes at depth k
#include "internal.hpp"

namespace gptq {
namespace {

constexpr int LEAF = 128;         // leaf block edge

void split(int64_t n, int64_t& n1, int64_t& n2) {
    const int64_t nb = ceil_div(n, LEAF);
    n1 = LEAF * ((nb + 1) / 2);
    n2 = n - n1;
}

constexpr int MAX_DEPTH = 16;  // d <= 2^20 gives at most 13 levels above the leaves

// Per recursion depth, the largest n1 x n2 of a node there (L21 scratch).
void depth_sizes(int64_t n, int depth, size_t* sz) {
    if (n <= LEAF) return;
    int64_t n1, n2;
    split(n, n1, n2);
    const size_t m = (size_t)n1 * (size_t)n2;
    if (m > sz[depth]) sz[depth] = m;
    depth_sizes(n1, depth + 1, sz);
    depth_sizes(n2, depth + 1, sz);
}

struct Ws {
    int* flags;
    double* lambda;
    double* diag;
    int32_t* pinv;
    double* L;
    double* tmp[MAX_DEPTH];
};

// Layout: flags/lambda | diag (d doubles) | pinv (d ints) | Hr (d*d) | one L21
// scratch per depth; returns the total size.
size_t layout(int64_t d, Ws* w, char* p) {
    size_t off = 256;
    if (w) w->diag = (double*)(p + off);
    off = align_up(off + (size_t)d * sizeof(double), 256);
    if (w) w->pinv = (int32_t*)(p + off);
    off = align_up(off + (size_t)d * sizeof(int32_t), 256);
    if (w) w->L = (double*)(p + off);
    off = align_up(off + (size_t)d * (size_t)d * sizeof(double), 256);
    size_t sz[MAX_DEPTH] = {};
    depth_sizes(d, 0, sz);
    for (int k = 0; k < MAX_DEPTH; ++k) {
        if (w) w->tmp[k] = (double*)(p + off);
        off = align_up(off + sz[k] * sizeof(double), 256);
    }
    if (w) {
        w->flags = (int*)p;
        w->lambda = (double*)(p + 64);
    }
    return off;
}

// lambda = damp * mean(diag H); copies the diagonal out and flags
// non-finite entries.
__global__ __launch_bounds__(1024) void diag_stats_kernel(const double* __restrict__ H, int64_t d, double damp,
                                                          double* lambda, double* diag, int* flags) {
    __shared__ double part[1024];
    const int t = threadIdx.x;
    double s = 0.0;
    for (int64_t i = t; i < d; i += 1024) {
        const double v = H[i * d + i];
        if (!isfinite(v)) raise_flag(flags, FLAG_NONFINITE);
        diag[i] = v;
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

// act-order: perm[rank(j)] = j and pinv[j] = rank(j), rank by (descending
// diag, ascending index).  NaN keys are counted as -inf (H with a non-finite
// entry is rejected anyway); the ranks always form a permutation.
// 64 columns j per block, each scanned by 4 threads over a quarter of every
// 2048-key tile; the partial counts are summed in LDS.
__global__ __launch_bounds__(256) void rank_kernel(const double* __restrict__ diag, int64_t d, int32_t* perm,
                                                   int32_t* pinv) {
    __shared__ double keys[2048];
    __shared__ int part_rank[4][64];
    const int jl = threadIdx.x & 63, part = threadIdx.x >> 6;
    const int64_t j = (int64_t)blockIdx.x * 64 + jl;
    double kj = (j < d) ? diag[j] : 0.0;
    if (isnan(kj)) kj = -INFINITY;
    int rank = 0;
    for (int64_t base = 0; base < d; base += 2048) {
        __syncthreads();
        for (int e = threadIdx.x; e < 2048; e += 256) {
            const int64_t i = base + e;
            double v = (i < d) ? diag[i] : -INFINITY;
            keys[e] = isnan(v) ? -INFINITY : v;
        }
        __syncthreads();
        const int64_t lim = (d - base < 2048) ? d - base : 2048;
        const int e0 = part * 512;
        const int e1 = (e0 + 512 < lim) ? e0 + 512 : (int)lim;
        // keys before j in the order: larger, or equal with a smaller index
        const int64_t jrel = j - base;
#pragma unroll 8
        for (int e = e0; e < e1; ++e) {
            const double ki = keys[e];
            rank += (ki > kj || (ki == kj && e < jrel)) ? 1 : 0;
        }
    }
    part_rank[part][jl] = rank;
    __syncthreads();
    if (part == 0 && j < d) {
        const int r = part_rank[0][jl] + part_rank[1][jl] + part_rank[2][jl] + part_rank[3][jl];
        perm[r] = (int32_t)j;
        pinv[j] = r;
    }
}

__global__ void iota_kernel(int32_t* perm, int32_t* pinv, int64_t d) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k < d) {
        perm[k] = (int32_t)k;
        pinv[k] = (int32_t)k;
    }
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
// One block per row a reads row p[d-1-a] of the (symmetrised) H in order,
// coalesced, and scatters entry c to b = d-1-pinv[c]; the scattered stores
// of one row merge in L2.
__global__ __launch_bounds__(256) void gather_reverse_kernel(const double* __restrict__ H, int64_t d,
                                                             const int32_t* __restrict__ perm,
                                                             const int32_t* __restrict__ pinv,
                                                             const double* __restrict__ lambda, double* Hr) {
    const int64_t a = blockIdx.x;
    const int64_t pa = perm[d - 1 - a];
    const double lam = *lambda;
    const double* row = H + pa * d;
    double* out = Hr + a * d;
    for (int64_t c = threadIdx.x; c < d; c += 256) {
        const int64_t b = d - 1 - pinv[c];
        if (b <= a) {
            double v = row[c];
            if (b == a) v += lam;
            out[b] = v;
        }
    }
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// 1/sqrt(p) for a positive normal p: hardware estimate and two Newton steps
// (each squares the relative error), good to about one ulp.
__device__ __forceinline__ double rsqrt_nr(double p) {
    double y = __builtin_amdgcn_rsq(p);
    const double h = 0.5 * p;
    double e = fma(-h * y, y, 0.5);
    y = fma(y, e, y);
    e = fma(-h * y, y, 0.5);
    return fma(y, e, y);
}

// Leaf of the recursion: the n x n (n <= 128) diagonal block of Hr at
// offset o is factored, A = L L^T, and M = L^{-1} is written to the same
// block of Mi (lower, zeros above the diagonal; the padding up to 128 acts
// as an identity block), with the 128x128 block in LDS and 16x16 inner
// blocks.  L is formed in place (lower triangle); M is formed along
// by forward elimination: R starts as the identity, and at block step k
// block row k of M is Dinv_k R_k (Dinv_k the inverse of the diagonal
// factor) while the rows below lose L[r][k-block] M_k.  The off-diagonal
// blocks of R / M live transposed in the free upper triangle of the LDS
// block; M's diagonal blocks are the Dinv_k.
//   setup: wave 0 factors diagonal block 0;
//   block step k: (A) rows below get L[r][k-block] = A[r][k-block] Dinv_k^T,
//                     and block row k of M = Dinv_k R_k;
//                 (B) wave 0 updates diagonal block k+1 and factors it while
//                     the other waves update the rest of the trailing lower
//                     part and the rows of R below block k.
// The 16x16 factor: one wave, lane = (row r, 4 columns), column j of L and
// row j of its inverse exchanged through LDS inside the wave.
constexpr int LB = 16;               // inner block edge
constexpr int NIB = LEAF / LB;       // inner blocks per edge
constexpr int LDA = LEAF + 1;        // LDS row stride (doubles)
constexpr size_t LEAF_LDS = (size_t)(LEAF * LDA + NIB * LB * LB + 2 * LB) * sizeof(double);

// Factor the 16x16 diagonal block at (k0, k0) of As in place (lower) and
// write the inverse of the factor to dinv (16x16, zeros above).  Wave 0.
__device__ __forceinline__ void diag16(double* As, int k0, double* dinv, double* colb, double* rowb, int lane,
                                       bool& bad_pd, bool& bad_nan) {
    // A wave executes its LDS operations in order; compiler memory barriers
    // between the stores and the loads of a step (and before the next
    // step's stores) keep the compiler from reusing earlier loaded values.
    const int r = lane >> 2, cg = lane & 3;
    double a[4], x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = 4 * cg + q;
        const double v = As[(k0 + r) * LDA + k0 + c];
        a[q] = (c <= r) ? v : 0.0;
        x[q] = (c == r) ? 1.0 : 0.0;
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
        double piv = readlane_f64(a[j & 3], 4 * j + (j >> 2));
        if (!(piv > 0.0)) {
            bad_nan |= isnan(piv);
            bad_pd |= !isnan(piv);
            piv = 1.0;
        }
        const double rs = rsqrt_nr(piv);
        const bool owner = cg == (j >> 2);
        const double lv = (r > j) ? a[j & 3] * rs : ((r == j) ? piv * rs : 0.0);
        a[j & 3] = owner ? lv : a[j & 3];
        if (owner) colb[r] = lv;
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = (r == j) ? x[q] * rs : x[q];
        if (r == j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) rowb[4 * cg + q] = x[q];
        }
        asm volatile("" ::: "memory");
        const double lr = colb[r];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 4 * cg + q;
            const double lcv = colb[c];
            const double xsv = rowb[c];
            a[q] = fma(-lr, (c > j) ? lcv : 0.0, a[q]);
            x[q] = fma(-lr, (r > j) ? xsv : 0.0, x[q]);
        }
        asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = 4 * cg + q;
        if (c <= r) As[(k0 + r) * LDA + k0 + c] = a[q];
        dinv[r * LB + c] = x[q];
    }
}

__global__ __launch_bounds__(512) void leaf_blocked_kernel(const double* __restrict__ A, double* Mi, int64_t d,
                                                           int64_t o, int n, int* flags) {
    extern __shared__ double sm[];
    double* As = sm;                        // [LEAF][LDA]: L (lower); R / M transposed (upper)
    double* Dv = sm + LEAF * LDA;           // [NIB][LB][LB]: inverses of the diagonal factors
    double* colb = Dv + NIB * LB * LB;      // [LB] column exchange of the 16x16 factor
    double* rowb = colb + LB;               // [LB] row exchange of its inverse
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

    // Hr block (lower; identity padding); R = I: zeros above the diagonal
    for (int e = t; e < LEAF * LEAF; e += 512) {
        const int r = e >> 7, c = e & (LEAF - 1);
        double v = 0.0;
        if (c <= r) {
            if (r < n && c < n) v = A[(o + r) * d + o + c];
            else v = (r == c) ? 1.0 : 0.0;
        }
        As[r * LDA + c] = v;
    }
    __syncthreads();
    bool bad_pd = false, bad_nan = false;
    if (wave == 0) diag16(As, 0, Dv, colb, rowb, lane, bad_pd, bad_nan);
    __syncthreads();

    for (int kb = 0; kb < NIB; ++kb) {
        const int k0 = kb * LB;
        const int rows = LEAF - k0 - LB;   // rows below the block
        const double* dk = Dv + kb * LB * LB;
        // (A) panel of L: one thread per row below; block row kb of M:
        //     M[k0+r][c] = sum_{q<=r} Dinv_k[r][q] R[k0+q][c], one thread per column c < k0
        if (t < rows) {
            const int r = k0 + LB + t;
            double a[LB];
#pragma unroll
            for (int k = 0; k < LB; ++k) a[k] = As[r * LDA + k0 + k];
#pragma unroll
            for (int c = 0; c < LB; ++c) {
                double s = 0.0;
#pragma unroll
                for (int k = 0; k <= c; ++k) s = fma(a[k], dk[c * LB + k], s);
                As[r * LDA + k0 + c] = s;
            }
        } else if (t >= 128 && t - 128 < k0) {
            const int c = t - 128;   // R[k0+q][c] stored at As[c][k0+q]
            double rv[LB];
#pragma unroll
            for (int q = 0; q < LB; ++q) rv[q] = As[c * LDA + k0 + q];
#pragma unroll
            for (int rr = 0; rr < LB; ++rr) {
                double s = 0.0;
#pragma unroll
                for (int q = 0; q <= rr; ++q) s = fma(dk[rr * LB + q], rv[q], s);
                As[c * LDA + k0 + rr] = s;
            }
        }
        __syncthreads();
        if (rows == 0) break;
        // (B)
        if (wave == 0) {
            // diagonal block kb+1 loses L[.][k-block] L[.][k-block]^T, then is factored
            const int b0 = k0 + LB;
            for (int e = lane; e < LB * LB; e += 64) {
                const int r = e >> 4, c = e & (LB - 1);
                if (c > r) continue;
                double s = 0.0;
#pragma unroll
                for (int k = 0; k < LB; ++k) s = fma(As[(b0 + r) * LDA + k0 + k], As[(b0 + c) * LDA + k0 + k], s);
                As[(b0 + r) * LDA + b0 + c] -= s;
            }
            asm volatile("" ::: "memory");
            diag16(As, b0, Dv + (kb + 1) * LB * LB, colb, rowb, lane, bad_pd, bad_nan);
        } else {
            const int tt = t - 64;   // 448 threads
            // trailing lower part below/right of block kb+1's diagonal block:
            // rows and columns >= k0+16, 4x4 tiles, except the 10 tiles of the
            // diagonal block kb+1 (handled by wave 0)
            const int T4 = rows / 4;
            const int ntl = T4 * (T4 + 1) / 2;
            // rows of R below block kb: R[r][c] -= sum_q L[r][k0+q] M[k0+q][c], c < k0+16,
            // R[r][c] at As[c][r]; M[k0+q][c] = Dinv_k[q][c-k0] for c >= k0, else As[c][k0+q]
            const int C4 = (k0 + LB) / 4;
            const int nx = T4 * C4;
            for (int w = tt; w < ntl + nx; w += 448) {
                if (w < ntl) {
                    int ti = 0;
                    while ((ti + 1) * (ti + 2) / 2 <= w) ++ti;
                    const int tj = w - ti * (ti + 1) / 2;
                    if (ti < 4) continue;  // the diagonal block kb+1 (tiles 0..9)
                    const int r0 = k0 + LB + 4 * ti, c0 = k0 + LB + 4 * tj;
                    double acc[4][4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
#pragma unroll 4
                    for (int k = 0; k < LB; ++k) {
                        double lr[4], lc[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            lr[i] = As[(r0 + i) * LDA + k0 + k];
                            lc[i] = As[(c0 + i) * LDA + k0 + k];
                        }
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int j = 0; j < 4; ++j) acc[i][j] = fma(lr[i], lc[j], acc[i][j]);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) As[(r0 + i) * LDA + c0 + j] -= acc[i][j];
                } else {
                    const int x = w - ntl;
                    const int r0 = k0 + LB + 4 * (x / C4), c0 = 4 * (x % C4);
                    const bool diagc = c0 >= k0;   // columns inside block kb: M = Dinv_k
                    double acc[4][4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
#pragma unroll 4
                    for (int q = 0; q < LB; ++q) {
                        double lr[4], mq[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) lr[i] = As[(r0 + i) * LDA + k0 + q];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            mq[j] = diagc ? dk[q * LB + (c0 - k0) + j] : As[(c0 + j) * LDA + k0 + q];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int j = 0; j < 4; ++j) acc[i][j] = fma(lr[i], mq[j], acc[i][j]);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) As[(c0 + j) * LDA + r0 + i] -= acc[i][j];
                }
            }
        }
        __syncthreads();
    }
    if (bad_nan) raise_flag(flags, FLAG_NONFINITE);
    if (bad_pd) raise_flag(flags, FLAG_NOT_PD);

    // write M (lower, zeros above the diagonal) for the n x n part
    for (int e = t; e < LEAF * LEAF; e += 512) {
        const int r = e >> 7, c = e & (LEAF - 1);
        if (r >= n || c >= n) continue;
        double v = 0.0;
        if (r / LB == c / LB) v = Dv[((r / LB) * LB + (r % LB)) * LB + (c % LB)];
        else if (r > c) v = As[c * LDA + r];
        Mi[(o + r) * d + o + c] = v;
    }
}

// U = J M J in place: the lower triangle of M (with its diagonal) moves to
// the mirrored upper position, the strict lower triangle becomes zero.
__global__ __launch_bounds__(256) void rotate_inplace_kernel(double* M, int64_t d) {
    const int64_t i = blockIdx.x;
    for (int64_t j = threadIdx.x; j <= i; j += 256) {
        if (j < i) {
            const double v = M[i * d + j];
            M[(d - 1 - i) * d + (d - 1 - j)] = v;
            M[i * d + j] = 0.0;
        } else if (i < d - 1 - i) {
            const int64_t k = d - 1 - i;
            const double v = M[i * d + i];
            M[i * d + i] = M[k * d + k];
            M[k * d + k] = v;
        }
    }
}

// T = L21 M11 of a node does not feed the recursion into A22, only the
// final M21 = -M22 T: it runs on a second stream, overlapping the
// latency-bound leaves and small products of that recursion.  Each depth
// has its own L21 scratch, so the recursion below cannot overwrite the
// operand of a T still in flight; the events of a depth are reused only
// after the main stream has waited for that depth's previous T.
struct Rec {
    hipStream_t s = nullptr, side = nullptr;
    double* L = nullptr;    // Hr, lower; T blocks replace A21 blocks
    double* M = nullptr;    // inverse factor (lower)
    double* tmp[MAX_DEPTH] = {};
    int64_t d = 0;
    int* flags = nullptr;
    hipEvent_t l21_ready[MAX_DEPTH] = {}, t_done[MAX_DEPTH] = {};
    hipError_t init() {
        hipError_t e = hipStreamCreateWithFlags(&side, hipStreamNonBlocking);
        for (int k = 0; k < MAX_DEPTH && e == hipSuccess; ++k) {
            e = hipEventCreateWithFlags(&l21_ready[k], hipEventDisableTiming);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&t_done[k], hipEventDisableTiming);
        }
        return e;
    }
    ~Rec() {
        if (side) {
            (void)hipStreamSynchronize(side);
            (void)hipStreamDestroy(side);
        }
        for (int k = 0; k < MAX_DEPTH; ++k) {
            if (l21_ready[k]) (void)hipEventDestroy(l21_ready[k]);
            if (t_done[k]) (void)hipEventDestroy(t_done[k]);
        }
    }
};

gptq_status chol_inv(const Rec& c, int64_t o, int64_t n, int depth) {
    const int64_t d = c.d;
    if (n <= LEAF) {
        hipLaunchKernelGGL(leaf_blocked_kernel, dim3(1), dim3(512), LEAF_LDS, c.s, c.L, c.M, d, o, (int)n, c.flags);
        GPTQ_LAUNCH_CHECK();
        return GPTQ_OK;
    }
    if (depth >= MAX_DEPTH) return GPTQ_ERR_UNSUPPORTED;
    int64_t n1, n2;
    split(n, n1, n2);
    double* A21 = c.L + (o + n1) * d + o;   // becomes T
    double* A22 = c.L + (o + n1) * d + o + n1;
    const double* M11 = c.M + o * d + o;
    const double* M22 = c.M + (o + n1) * d + o + n1;
    double* M21 = c.M + (o + n1) * d + o;
    double* L21 = c.tmp[depth];
    gptq_status st = chol_inv(c, o, n1, depth + 1);
    if (st != GPTQ_OK) return st;
    // L21 = A21 M11^T
    st = launch_gemm_f64(c.s, n2, n1, n1, 1.0, A21, d, M11, d, true, 0.0, L21, n1, false, GEMM_TRI_KEND_COL);
    if (st != GPTQ_OK) return st;
    // A22 -= L21 L21^T
    st = launch_gemm_f64(c.s, n2, n2, n1, -1.0, L21, n1, L21, n1, true, 1.0, A22, d, true);
    if (st != GPTQ_OK) return st;
    // T = L21 M11 (into A21's place), on the side stream
    GPTQ_HIP(hipEventRecord(c.l21_ready[depth], c.s));
    GPTQ_HIP(hipStreamWaitEvent(c.side, c.l21_ready[depth], 0));
    st = launch_gemm_f64(c.side, n2, n1, n1, 1.0, L21, n1, M11, d, false, 0.0, A21, d, false, GEMM_TRI_KBEG_COL);
    if (st != GPTQ_OK) return st;
    GPTQ_HIP(hipEventRecord(c.t_done[depth], c.side));
    st = chol_inv(c, o + n1, n2, depth + 1);
    if (st != GPTQ_OK) return st;
    // M21 = -M22 T
    GPTQ_HIP(hipStreamWaitEvent(c.s, c.t_done[depth], 0));
    return launch_gemm_f64(c.s, n2, n1, n2, -1.0, M22, d, A21, d, false, 0.0, M21, d, false, GEMM_TRI_KEND_ROW);
}

}  // namespace

size_t hinv_workspace_bytes(int64_t d) { return layout(d, nullptr, nullptr); }

gptq_status hinv_launch(double* H, int64_t d, const gptq_config* cfg, int32_t* perm, void* ws,
                        hipStream_t s, int* host_flags) {
    Ws w;
    layout(d, &w, (char*)ws);
    GPTQ_HIP(hipFuncSetAttribute((const void*)leaf_blocked_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)LEAF_LDS));
    GPTQ_HIP(hipMemsetAsync(w.flags, 0, 256, s));

    hipLaunchKernelGGL(diag_stats_kernel, dim3(1), dim3(1024), 0, s, H, d, cfg->damp, w.lambda, w.diag, w.flags);
    GPTQ_LAUNCH_CHECK();
    if (cfg->act_order)
        hipLaunchKernelGGL(rank_kernel, dim3((unsigned)ceil_div(d, 64)), dim3(256), 0, s, w.diag, d, perm, w.pinv);
    else
        hipLaunchKernelGGL(iota_kernel, dim3((unsigned)ceil_div(d, 256)), dim3(256), 0, s, perm, w.pinv, d);
    GPTQ_LAUNCH_CHECK();
    const int64_t T32 = ceil_div(d, 32);
    hipLaunchKernelGGL(symmetrize_kernel, dim3((unsigned)(T32 * (T32 + 1) / 2)), dim3(256), 0, s, H, d, w.flags);
    GPTQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(gather_reverse_kernel, dim3((unsigned)d), dim3(256), 0, s, H, d, perm, w.pinv, w.lambda,
                       w.L);
    GPTQ_LAUNCH_CHECK();

    // H's buffer now receives M = L^{-1} (lower), then U = J M J in place.
    Rec c;
    GPTQ_HIP(c.init());
    c.s = s;
    c.L = w.L;
    c.M = H;
    for (int k = 0; k < MAX_DEPTH; ++k) c.tmp[k] = w.tmp[k];
    c.d = d;
    c.flags = w.flags;
    gptq_status st = chol_inv(c, 0, d, 0);
    if (st != GPTQ_OK) return st;
    hipLaunchKernelGGL(rotate_inplace_kernel, dim3((unsigned)d), dim3(256), 0, s, H, d);
    GPTQ_LAUNCH_CHECK();
    GPTQ_HIP(hipMemcpyAsync(host_flags, w.flags, N_FLAGS * sizeof(int), hipMemcpyDeviceToHost, s));
    GPTQ_HIP(hipStreamSynchronize(s));
    return GPTQ_OK;
}

}  // namespace gptq
