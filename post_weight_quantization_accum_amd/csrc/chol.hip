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
    double* mrev;   // factored form: the diagonal blocks of M, columns reversed
    double* lst;    // factored form: the off-diagonal blocks of L (row stride d)
};

// Layout: flags/lambda | diag (d doubles) | pinv (d ints) | Hr (d*d) | one L21
// scratch per depth | factored form: the diagonal blocks of M, the factor's
// off-diagonal blocks (d*d); returns the total size.
size_t layout(int64_t d, Ws* w, char* p, bool factored) {
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
    if (w) w->mrev = factored ? (double*)(p + off) : nullptr;
    if (factored) off = align_up(off + (size_t)ceil_div(d, LEAF) * LEAF * LEAF * sizeof(double), 256);
    if (w) w->lst = factored ? (double*)(p + off) : nullptr;
    if (factored) off = align_up(off + (size_t)d * (size_t)d * sizeof(double), 256);
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

// The same gather with the source row staged in LDS (d doubles, up to
// GATHER_LDS_MAX): row p[d-1-a] is read in order, then row a of Hr is
// written in order, b = 0..a, each value picked from LDS at p[d-1-b].
constexpr int64_t GATHER_LDS_MAX = 19456;   // 152 KiB of LDS
__global__ __launch_bounds__(512) void gather_rows_lds_kernel(const double* __restrict__ H, int64_t d,
                                                              const int32_t* __restrict__ perm,
                                                              const double* __restrict__ lambda, double* Hr) {
    extern __shared__ double srow[];
    const int64_t a = blockIdx.x;
    const double* row = H + (int64_t)perm[d - 1 - a] * d;
#pragma unroll 8
    for (int64_t c = threadIdx.x; c < d; c += 512) srow[c] = row[c];
    __syncthreads();
    const double lam = *lambda;
    double* out = Hr + a * d;
#pragma unroll 4
    for (int64_t b = threadIdx.x; b <= a; b += 512) {
        double v = srow[perm[d - 1 - b]];
        if (b == a) v += lam;
        out[b] = v;
    }
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Value of v in lane src (ds_bpermute, no LDS memory involved).
__device__ __forceinline__ double bperm_f64(double v, int src) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int a = src << 2;
    const int lo = __builtin_amdgcn_ds_bpermute(a, (int)(uint32_t)b);
    const int hi = __builtin_amdgcn_ds_bpermute(a, (int)(uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// 1/sqrt(p) and 1/p for a positive normal p: hardware estimate and two
// Newton steps (each squares the relative error), good to about one ulp.
__device__ __forceinline__ double rsqrt_nr(double p) {
    double y = __builtin_amdgcn_rsq(p);
    const double h = 0.5 * p;
    double e = fma(-h * y, y, 0.5);
    y = fma(y, e, y);
    e = fma(-h * y, y, 0.5);
    return fma(y, e, y);
}
__device__ __forceinline__ double rcp_nr(double p) {
    double y = __builtin_amdgcn_rcp(p);
    double e = fma(-p, y, 1.0);
    y = fma(y, e, y);
    e = fma(-p, y, 1.0);
    return fma(y, e, y);
}

// Leaf of the recursion: the n x n (n <= 128) diagonal block of Hr at
// offset o is factored, A = L L^T, and M = L^{-1} is written to the same
// block of Mi (lower, zeros above the diagonal; the padding up to 128 acts
// as an identity block), with the 128x128 block in LDS and 16x16 inner
// blocks.  L is formed in place (lower triangle); M is formed along by
// forward elimination: R starts as the identity, and at block step k block
// row k of M is Dinv_k R_k (Dinv_k the inverse of the diagonal factor)
// while the rows below lose L[r][k-block] M_k.  The off-diagonal blocks of
// R / M live transposed in the free upper triangle of the LDS block; M's
// diagonal blocks are the Dinv_k.
//   setup: wave 0 factors diagonal block 0;
//   block step k: (A) seven 16x16 tiles, one per wave: the row tiles of L
//                     below block k (L = A Dinv_k^T) and the column tiles
//                     of block row k of M (Dinv_k R_k);
//                 (B) wave 0 updates diagonal block k+1 and factors it while
//                     the other waves update the rest of the trailing lower
//                     part and the rows of R below block k.
// Every 16x16 product runs on the float64 matrix cores (four
// v_mfma_f64_16x16x4 for K = 16); the row stride of 130 doubles makes the
// operand fetches (16 rows x 2 k per 32 lanes) hit distinct LDS banks.
// The 16x16 diagonal factor is split into 8x8 halves with one element per
// lane (see diag8).
constexpr int LB = 16;               // inner block edge
constexpr int NIB = LEAF / LB;       // inner blocks per edge
constexpr int LDA = LEAF + 2;        // LDS row stride (doubles)
constexpr int DLD = LB + 1;          // row stride of the stored diagonal inverses
constexpr int DSZ = LB * DLD;
constexpr int SC8 = 8 * 9;           // one 8x8 scratch matrix, row stride 9
constexpr size_t LEAF_LDS = (size_t)(LEAF * LDA + NIB * DSZ + 4 * SC8) * sizeof(double);

__device__ __forceinline__ d4_t mfma4(double a, double b, d4_t c) { return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0); }

// 16x16 tile of a product with K = 16 on the matrix cores: element (i, k) of
// the left operand at pa[i * sa_r + k * sa_k], element (k, j) of the right
// operand at pb[j * sb_c + k * sb_k]; acc[r] = C[4r + lane/16][lane%16].
__device__ __forceinline__ d4_t tile16(const double* pa, int sa_r, int sa_k, const double* pb, int sb_c, int sb_k,
                                       int lane) {
    const int r = lane & 15, kq = lane >> 4;
    double av[4], bv[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        av[s] = pa[r * sa_r + (4 * s + kq) * sa_k];
        bv[s] = pb[r * sb_c + (4 * s + kq) * sb_k];
    }
    d4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma4(av[s], bv[s], acc);
    return acc;
}

// 8x8 factor in one wave, lane = 8i + j holding the symmetric A[i][j]:
// a = L[i][j] on return (meaningful for j <= i), x = L^{-1}[i][j] (zero for
// j > i).  Step J eliminates with the unscaled column, a[i][j] -=
// a[i][J] a[J][j] / p_J (the same update as with the scaled column of L),
// and x[i] -= (a[i][J] / p_J) x[J]; the scale 1/sqrt(p_J) of column J of L
// and of row J of the inverse is applied at the end, where the pivots are
// also checked.  Row J and column J arrive through ds_bpermute, the pivot
// through readlane.
__device__ __forceinline__ void diag8(double& a, double& x, int lane, bool& bad_pd, bool& bad_nan) {
    const int i = lane >> 3, j = lane & 7;
    x = (i == j) ? 1.0 : 0.0;
    double pv[8], pu[8];   // pivots as found, and as used (1 in place of a bad one)
#pragma unroll
    for (int J = 0; J < 8; ++J) {
        const double colr = bperm_f64(a, (lane & ~7) + J);   // a[i][J]
        const double colc = bperm_f64(a, 8 * J + j);         // a[J][j]
        const double xrow = bperm_f64(x, 8 * J + j);         // x[J][j]
        pv[J] = readlane_f64(a, 9 * J);
        pu[J] = (pv[J] > 0.0) ? pv[J] : 1.0;
        const double cr = (i > J) ? colr * rcp_nr(pu[J]) : 0.0;
        a = fma(-cr, (j > J) ? colc : 0.0, a);
        x = fma(-cr, xrow, x);
    }
    double pi = pu[0], pj = pu[0];
#pragma unroll
    for (int J = 0; J < 8; ++J) {
        pi = (i == J) ? pu[J] : pi;
        pj = (j == J) ? pu[J] : pj;
        bad_nan |= isnan(pv[J]);
        bad_pd |= !(pv[J] > 0.0) && !isnan(pv[J]);
    }
    a *= rsqrt_nr(pj);
    x *= rsqrt_nr(pi);
}

// Factor the 16x16 diagonal block at (b0, b0) of As in place (lower) and
// write the inverse of the factor to D (row stride DLD, zeros above the
// diagonal).  Wave 0.  With A = [A11 .; A21 A22]: L11, X11 = L11^{-1};
// L21 = A21 X11^T; L22, X22 from A22 - L21 L21^T; X21 = -X22 (L21 X11).
// The 8x8 intermediates go through LDS scratch; a wave executes its LDS
// operations in order, and compiler memory barriers keep the compiler from
// reusing values loaded before a store.
__device__ __forceinline__ void diag16(double* As, int b0, double* D, double* sc, int lane, bool& bad_pd,
                                       bool& bad_nan) {
    const int i = lane >> 3, j = lane & 7;
    double* SX11 = sc;
    double* SL21 = sc + SC8;
    double* ST = sc + 2 * SC8;
    double* SX22 = sc + 3 * SC8;
    double a11 = (j <= i) ? As[(b0 + i) * LDA + b0 + j] : As[(b0 + j) * LDA + b0 + i];
    double a22 = (j <= i) ? As[(b0 + 8 + i) * LDA + b0 + 8 + j] : As[(b0 + 8 + j) * LDA + b0 + 8 + i];
    double a21[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) a21[k] = As[(b0 + 8 + i) * LDA + b0 + k];
    double x11;
    diag8(a11, x11, lane, bad_pd, bad_nan);
    SX11[i * 9 + j] = x11;
    asm volatile("" ::: "memory");
    double l21 = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) l21 = fma(a21[k], SX11[j * 9 + k], l21);
    SL21[i * 9 + j] = l21;
    asm volatile("" ::: "memory");
    double s22 = 0.0, tt = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const double li = SL21[i * 9 + k];
        s22 = fma(li, SL21[j * 9 + k], s22);
        tt = fma(li, SX11[k * 9 + j], tt);
    }
    a22 -= s22;
    ST[i * 9 + j] = tt;
    double x22;
    diag8(a22, x22, lane, bad_pd, bad_nan);
    SX22[i * 9 + j] = x22;
    asm volatile("" ::: "memory");
    double x21 = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) x21 = fma(SX22[i * 9 + k], ST[k * 9 + j], x21);
    if (j <= i) {
        As[(b0 + i) * LDA + b0 + j] = a11;
        As[(b0 + 8 + i) * LDA + b0 + 8 + j] = a22;
    }
    As[(b0 + 8 + i) * LDA + b0 + j] = l21;
    D[i * DLD + j] = x11;
    D[i * DLD + 8 + j] = 0.0;
    D[(8 + i) * DLD + j] = -x21;
    D[(8 + i) * DLD + 8 + j] = x22;
    asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(512) void leaf_blocked_kernel(const double* __restrict__ A, double* Mi, int64_t d,
                                                           int64_t o, int n, int* flags) {
    extern __shared__ double sm[];
    double* As = sm;                 // [LEAF][LDA]: L (lower); R / M transposed (upper, off-diagonal blocks)
    double* Dv = sm + LEAF * LDA;    // [NIB][LB][DLD]: inverses of the diagonal factors
    double* sc = Dv + NIB * DSZ;     // 8x8 scratch of the diagonal factor
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    constexpr int PER = LEAF * LEAF / 512;   // elements per thread when the block moves

    // Hr block (lower; identity padding), zeros above the diagonal; all
    // loads of a thread issued before its stores
    {
        // r < 128 and d <= 2^20: offsets from the block's corner fit 32 bits
        const double* Ab = A + o * d + o;
        double v[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = t + 512 * q;
            const int r = e >> 7, c = e & (LEAF - 1);
            const bool in = c <= r && r < n && c < n;
            const double x = Ab[(uint32_t)(in ? r : 0) * (uint32_t)d + (uint32_t)(in ? c : 0)];
            v[q] = in ? x : ((c == r) ? 1.0 : 0.0);
        }
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = t + 512 * q;
            As[(e >> 7) * LDA + (e & (LEAF - 1))] = v[q];
        }
    }
    __syncthreads();
    bool bad_pd = false, bad_nan = false;
    if (wave == 0) diag16(As, 0, Dv, sc, lane, bad_pd, bad_nan);
    __syncthreads();

    for (int kb = 0; kb < NIB; ++kb) {
        const int k0 = kb * LB;
        const double* dk = Dv + kb * DSZ;
        // (A) wave w < 7: row tile w of L below block kb, or column tile of
        //     block row kb of M (M[k0+r][c] = sum_q Dinv_k[r][q] R[k0+q][c],
        //     R[k0+q][c] stored at As[c][k0+q])
        if (wave < NIB - 1) {
            const int nbelow = NIB - 1 - kb;
            if (wave < nbelow) {
                const int r0 = k0 + LB + LB * wave;
                const d4_t acc = tile16(As + r0 * LDA + k0, LDA, 1, dk, DLD, 1, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) As[(r0 + 4 * r + (lane >> 4)) * LDA + k0 + (lane & 15)] = acc[r];
            } else {
                const int c0 = LB * (wave - nbelow);
                const d4_t acc = tile16(dk, DLD, 1, As + c0 * LDA + k0, LDA, 1, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) As[(c0 + (lane & 15)) * LDA + k0 + 4 * r + (lane >> 4)] = acc[r];
            }
        }
        __syncthreads();
        if (kb == NIB - 1) break;
        // (B)
        const int b0 = k0 + LB;
        if (wave == 0) {
            // diagonal block kb+1 loses L[.][k-block] L[.][k-block]^T, then is factored
            const d4_t acc = tile16(As + b0 * LDA + k0, LDA, 1, As + b0 * LDA + k0, LDA, 1, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) As[(b0 + 4 * r + (lane >> 4)) * LDA + b0 + (lane & 15)] -= acc[r];
            asm volatile("" ::: "memory");
            diag16(As, b0, Dv + (kb + 1) * DSZ, sc, lane, bad_pd, bad_nan);
        } else {
            // waves 1..7: tiles (ti, tj) of the trailing lower part below
            // block kb (ti >= tj, except the diagonal tile of block kb+1),
            // then tiles of R below block kb: R[r][c] -= sum_q L[r][k0+q]
            // M[k0+q][c] for c < k0+16 (M = Dinv_k inside block kb)
            const int T = NIB - 1 - kb;
            const int ntr = T * (T + 1) / 2 - 1;
            const int nr = T * (kb + 1);
            for (int w = wave - 1; w < ntr + nr; w += NIB - 1) {
                if (w < ntr) {
                    const int x = w + 1;
                    int ti = 0;
                    while ((ti + 1) * (ti + 2) / 2 <= x) ++ti;
                    const int tj = x - ti * (ti + 1) / 2;
                    const int i0 = b0 + LB * ti, j0 = b0 + LB * tj;
                    const d4_t acc = tile16(As + i0 * LDA + k0, LDA, 1, As + j0 * LDA + k0, LDA, 1, lane);
#pragma unroll
                    for (int r = 0; r < 4; ++r) As[(i0 + 4 * r + (lane >> 4)) * LDA + j0 + (lane & 15)] -= acc[r];
                } else {
                    const int x = w - ntr;
                    const int ti = x / (kb + 1), tc = x % (kb + 1);
                    const int r0 = b0 + LB * ti, c0 = LB * tc;
                    d4_t acc;
                    if (tc == kb) acc = tile16(As + r0 * LDA + k0, LDA, 1, dk, 1, DLD, lane);
                    else acc = tile16(As + r0 * LDA + k0, LDA, 1, As + c0 * LDA + k0, LDA, 1, lane);
#pragma unroll
                    for (int r = 0; r < 4; ++r) As[(c0 + (lane & 15)) * LDA + r0 + 4 * r + (lane >> 4)] -= acc[r];
                }
            }
        }
        __syncthreads();
    }
    if (bad_nan) raise_flag(flags, FLAG_NONFINITE);
    if (bad_pd) raise_flag(flags, FLAG_NOT_PD);

    // write M (lower, zeros above the diagonal) for the n x n part; both
    // candidate LDS values are read unconditionally (in range for any r, c)
    // so that the reads are in flight together
    {
        double* Mb = Mi + o * d + o;
        double v[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = t + 512 * q;
            const int r = e >> 7, c = e & (LEAF - 1);
            const double xd = Dv[(r / LB) * DSZ + (r % LB) * DLD + (c % LB)];
            const double xa = As[c * LDA + r];
            v[q] = (r / LB == c / LB) ? xd : ((r > c) ? xa : 0.0);
        }
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = t + 512 * q;
            const int r = e >> 7, c = e & (LEAF - 1);
            if (r < n && c < n) Mb[(uint32_t)r * (uint32_t)d + (uint32_t)c] = v[q];
        }
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
//
// A T product launched with one workgroup per tile would fill every CU and
// keep workgroups queued until it drains; the leaves and small products
// that the main stream launches meanwhile then wait behind them (a leaf
// needs most of a CU's LDS).  T therefore runs with fewer workgroups than
// CUs, each looping over tiles, and CUs stay free for the main stream.
#ifndef GPTQ_T_FREE
#define GPTQ_T_FREE 8
#endif
constexpr int T_FREE = GPTQ_T_FREE;   // CUs left to the main stream

struct Rec {
    hipStream_t s = nullptr, side = nullptr;
    double* L = nullptr;    // Hr, lower; T blocks replace A21 blocks
    double* M = nullptr;    // inverse factor (lower)
    double* tmp[MAX_DEPTH] = {};
    int64_t d = 0;
    int* flags = nullptr;
    hipEvent_t l21_ready[MAX_DEPTH] = {}, t_done[MAX_DEPTH] = {};
    int64_t t_wg = 0;   // workgroups of a T product
    double* lst = nullptr;   // factored form: the factor's off-diagonal blocks (row stride d)
    // created on first use: factors of at most 1024 columns never need them
    hipError_t init() {
        if (side) return hipSuccess;
        int dev = 0, n_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        t_wg = n_cu - T_FREE >= 64 ? n_cu - T_FREE : 0;
        e = hipStreamCreateWithFlags(&side, hipStreamNonBlocking);
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

// need_m: the caller reads this node's whole inverse M (a left child: its
// M11 feeds the parent's L21).  Without it (the root and the right children
// below it, in the factored form) T and M21 are skipped: only the diagonal
// blocks of M, which the leaves form, are read afterwards.
// c.lst (factored form): each node's L21 goes to its place in a d x d store
// of the factor's off-diagonal blocks (read at the end) instead of the
// depth's scratch.
gptq_status chol_inv(Rec& c, int64_t o, int64_t n, int depth, bool need_m = true) {
    const int64_t d = c.d;
    if (n <= LEAF) {
        hipLaunchKernelGGL(leaf_blocked_kernel, dim3(1), dim3(512), LEAF_LDS, c.s, c.L, c.M, d, o, (int)n, c.flags);
        GPTQ_LAUNCH_CHECK();
        return GPTQ_OK;
    }
    if (depth >= MAX_DEPTH) return GPTQ_ERR_UNSUPPORTED;
    int64_t n1, n2;
    split(n, n1, n2);
    double* A21 = c.L + (o + n1) * d + o;
    double* A22 = c.L + (o + n1) * d + o + n1;
    const double* M11 = c.M + o * d + o;
    const double* M22 = c.M + (o + n1) * d + o + n1;
    double* M21 = c.M + (o + n1) * d + o;
    double* const L21 = c.lst ? c.lst + (o + n1) * d + o : c.tmp[depth];
    const int64_t ld_l = c.lst ? d : n1;
    double* const T = A21;   // T replaces A21
    const int64_t ld_t = d;
    gptq_status st = chol_inv(c, o, n1, depth + 1, true);
    if (st != GPTQ_OK) return st;
    // L21 = A21 M11^T
    st = launch_gemm_f64(c.s, n2, n1, n1, 1.0, A21, d, M11, d, true, 0.0, L21, ld_l, false, GEMM_TRI_KEND_COL);
    if (st != GPTQ_OK) return st;
    if (n1 <= 512 && n2 <= 512) {
        // small node: A22 -= L21 L21^T and T = L21 M11 in one launch, all on
        // the main stream (no cross-stream events on the short chain)
        const GemmCall syrk{n2, n2, n1, -1.0, L21, ld_l, L21, ld_l, true, 1.0, A22, d, true, GEMM_TRI_NONE};
        if (need_m) {
            const GemmCall tprod{n2, n1, n1, 1.0, L21, ld_l, M11, d, false, 0.0, T, ld_t, false, GEMM_TRI_KBEG_COL};
            st = launch_gemm_f64_pair(c.s, syrk, tprod);
        } else {
            st = launch_gemm_f64(c.s, n2, n2, n1, -1.0, L21, ld_l, L21, ld_l, true, 1.0, A22, d, true);
        }
        if (st != GPTQ_OK) return st;
        st = chol_inv(c, o + n1, n2, depth + 1, need_m);
        if (st != GPTQ_OK) return st;
        if (!need_m) return GPTQ_OK;
        return launch_gemm_f64(c.s, n2, n1, n2, -1.0, M22, d, T, ld_t, false, 0.0, M21, d, false, GEMM_TRI_KEND_ROW);
    }
    // A22 -= L21 L21^T
    st = launch_gemm_f64(c.s, n2, n2, n1, -1.0, L21, ld_l, L21, ld_l, true, 1.0, A22, d, true);
    if (st != GPTQ_OK) return st;
    if (!need_m) return chol_inv(c, o + n1, n2, depth + 1, false);
    // T = L21 M11, on the side stream
    GPTQ_HIP(c.init());
    GPTQ_HIP(hipEventRecord(c.l21_ready[depth], c.s));
    GPTQ_HIP(hipStreamWaitEvent(c.side, c.l21_ready[depth], 0));
    st = launch_gemm_f64(c.side, n2, n1, n1, 1.0, L21, ld_l, M11, d, false, 0.0, T, ld_t, false, GEMM_TRI_KBEG_COL,
                         false, c.t_wg);
    if (st != GPTQ_OK) return st;
    GPTQ_HIP(hipEventRecord(c.t_done[depth], c.side));
    st = chol_inv(c, o + n1, n2, depth + 1, true);
    if (st != GPTQ_OK) return st;
    // M21 = -M22 T
    GPTQ_HIP(hipStreamWaitEvent(c.s, c.t_done[depth], 0));
    return launch_gemm_f64(c.s, n2, n1, n2, -1.0, M22, d, T, ld_t, false, 0.0, M21, d, false, GEMM_TRI_KEND_ROW);
}

// Each 128 x 128 diagonal block of M (lower) with its columns reversed:
// Mrev[l][k][n] = M_ll[k][127 - n], zero above the diagonal.
__global__ __launch_bounds__(256) void diag_blocks_rev_kernel(const double* __restrict__ M, int64_t d,
                                                              double* __restrict__ Mrev) {
    const int64_t l = blockIdx.x;
    const double* src = M + (l * LEAF) * d + l * LEAF;
    double* dst = Mrev + l * LEAF * LEAF;
    for (int e = threadIdx.x; e < LEAF * LEAF; e += 256) {
        const int k = e / LEAF, n = e % LEAF, col = LEAF - 1 - n;
        dst[e] = (col <= k) ? src[(int64_t)k * d + col] : 0.0;
    }
}

}  // namespace

size_t hinv_workspace_bytes(int64_t d, bool factored) { return layout(d, nullptr, nullptr, factored); }

gptq_status hinv_launch(double* H, int64_t d, const gptq_config* cfg, int32_t* perm, void* ws,
                        hipStream_t s, int* host_flags, bool factored) {
    if (factored && (d % LEAF) != 0) return GPTQ_ERR_UNSUPPORTED;
    Ws w;
    layout(d, &w, (char*)ws, factored);
    GPTQ_HIP(ensure_lds_limit((const void*)leaf_blocked_kernel, (int)LEAF_LDS));
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
    if (d <= GATHER_LDS_MAX) {
        const size_t lds = (size_t)d * sizeof(double);
        GPTQ_HIP(ensure_lds_limit((const void*)gather_rows_lds_kernel, (int)lds));
        hipLaunchKernelGGL(gather_rows_lds_kernel, dim3((unsigned)d), dim3(512), lds, s, H, d, perm, w.lambda, w.L);
    } else {
        hipLaunchKernelGGL(gather_reverse_kernel, dim3((unsigned)d), dim3(256), 0, s, H, d, perm, w.pinv, w.lambda,
                           w.L);
    }
    GPTQ_LAUNCH_CHECK();

    // H's buffer now receives M = L^{-1} (lower), then U = J M J in place.
    Rec c;
    c.s = s;
    c.L = w.L;
    c.M = H;
    for (int k = 0; k < MAX_DEPTH; ++k) c.tmp[k] = w.tmp[k];
    c.d = d;
    c.flags = w.flags;
    c.lst = w.lst;
    gptq_status st = chol_inv(c, 0, d, 0, !factored);
    if (st != GPTQ_OK) return st;
    if (factored) {
        hipLaunchKernelGGL(diag_blocks_rev_kernel, dim3((unsigned)(d / LEAF)), dim3(256), 0, s, H, d, w.mrev);
        GPTQ_LAUNCH_CHECK();
        st = launch_factor_blocks(s, w.lst, w.mrev, H, d);
        if (st != GPTQ_OK) return st;
    } else {
        hipLaunchKernelGGL(rotate_inplace_kernel, dim3((unsigned)d), dim3(256), 0, s, H, d);
        GPTQ_LAUNCH_CHECK();
    }
    GPTQ_HIP(hipMemcpyAsync(host_flags, w.flags, N_FLAGS * sizeof(int), hipMemcpyDeviceToHost, s));
    GPTQ_HIP(hipStreamSynchronize(s));
    return GPTQ_OK;
}

}  // namespace gptq
