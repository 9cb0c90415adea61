// Hessian accumulation H += 2 X^T X ("GPTQ量化算法深度解析" §3.1 step 1),
// upper triangle, on the gfx950 matrix cores.
//
// bf16 / fp16 activations: products are exact in float32, so the MFMA
// v_mfma_f32_32x32x16_{bf16,f16} accumulates chunks of CHUNK tokens in
// float32 registers; each chunk is then added to float64 registers, and the
// tile is added to H (float64) once at the end.  One workgroup owns one
// 128x128 tile of the upper triangle for the whole token range, so the
// summation order is fixed and the result bit-reproducible.
//
// The diagonal is recomputed in float64 from the same staged values (squares
// of bf16/fp16 values are exact in float64): the act-order key diag(H) then
// agrees with a float64 reference to rounding order, so the column order
// does not depend on float32 accumulation error.
//
// X is token-major (row = token).  The MFMA operands need 8 consecutive
// tokens of one column per lane, so each thread loads 2 adjacent columns of
// 8 tokens (coalesced 4-byte loads along a token row), transposes them in
// registers, and writes column-major runs of 8 tokens into LDS.
//
// fp32 activations take a float64 path (products of fp32 values are exact
// in float64): a plain tiled float64 kernel.
#include "internal.hpp"

namespace gptq {
namespace {

constexpr int BT = 128;          // tile edge
constexpr int KT = 32;           // tokens per LDS stage
constexpr int SK = KT + 8;       // LDS row stride in 16-bit elements (80 B)
constexpr int CHUNK = 4096;      // tokens accumulated in float32 before the float64 add

__device__ __forceinline__ void upper_tile(int64_t t, int64_t& ti, int64_t& tj) {
    int64_t x = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while (x * (x + 1) / 2 > t) --x;
    while ((x + 1) * (x + 2) / 2 <= t) ++x;
    tj = x;                       // row of the lower-triangle enumeration
    ti = t - x * (x + 1) / 2;     // ti <= tj
}

template <typename Tag>
__device__ __forceinline__ double elem_f64(uint16_t b);
template <>
__device__ __forceinline__ double elem_f64<bf16x8_t>(uint16_t b) { return bf16_bits_to_f64(b); }
template <>
__device__ __forceinline__ double elem_f64<h16x8_t>(uint16_t b) { return f16_bits_to_f64(b); }

// Load 8 tokens x 2 columns (col, col+1) as 8 packed 32-bit words.
template <bool VEC>
__device__ __forceinline__ void load_pairs(uint32_t v[8], const uint16_t* X, int64_t ld, int64_t n_tok,
                                           int64_t d, int64_t tok0, int64_t col) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int64_t t = tok0 + r;
        uint32_t w = 0;
        if (t < n_tok) {
            const uint16_t* p = X + t * ld + col;
            if (VEC && col + 1 < d) {
                w = *(const uint32_t*)p;
            } else {
                if (col < d) w = p[0];
                if (col + 1 < d) w |= ((uint32_t)p[1]) << 16;
            }
        }
        v[r] = w;
    }
}

template <typename Tag, bool VEC>
__global__ __launch_bounds__(256) void hess_syrk_kernel(double* __restrict__ H, const uint16_t* __restrict__ X,
                                                        int64_t n_tok, int64_t d, int64_t ld) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[BT * SK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[BT * SK];
    __shared__ double red[4][BT];

    int64_t ti, tj;
    upper_tile(blockIdx.x, ti, tj);
    const bool diag = (ti == tj);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int cp = t & 63, tg = t >> 6;
    const int64_t colA = ti * BT + 2 * cp, colB = tj * BT + 2 * cp;

    f16_t acc[2][2];
    double acc64[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[i][j][r] = 0.0f;
                acc64[i][j][r] = 0.0;
            }
        }
    double dsq0 = 0.0, dsq1 = 0.0;

    uint32_t va[8], vb[8];
    load_pairs<VEC>(va, X, ld, n_tok, d, tg * 8, colA);
    if (!diag) load_pairs<VEC>(vb, X, ld, n_tok, d, tg * 8, colB);

    const int64_t n_stages = ceil_div(n_tok, KT);
    const int stages_per_chunk = CHUNK / KT;
    for (int64_t s = 0; s < n_stages; ++s) {
        // registers -> LDS, transposed to [column][token]
        {
            u32x4_t c0, c1;
            c0.x = (va[0] & 0xFFFFu) | (va[1] << 16);
            c0.y = (va[2] & 0xFFFFu) | (va[3] << 16);
            c0.z = (va[4] & 0xFFFFu) | (va[5] << 16);
            c0.w = (va[6] & 0xFFFFu) | (va[7] << 16);
            c1.x = (va[0] >> 16) | (va[1] & 0xFFFF0000u);
            c1.y = (va[2] >> 16) | (va[3] & 0xFFFF0000u);
            c1.z = (va[4] >> 16) | (va[5] & 0xFFFF0000u);
            c1.w = (va[6] >> 16) | (va[7] & 0xFFFF0000u);
            *(u32x4_t*)&sA[(2 * cp) * SK + tg * 8] = c0;
            *(u32x4_t*)&sA[(2 * cp + 1) * SK + tg * 8] = c1;
            if (diag) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const double x0 = elem_f64<Tag>((uint16_t)(va[r] & 0xFFFFu));
                    const double x1 = elem_f64<Tag>((uint16_t)(va[r] >> 16));
                    dsq0 = fma(x0, x0, dsq0);
                    dsq1 = fma(x1, x1, dsq1);
                }
            } else {
                c0.x = (vb[0] & 0xFFFFu) | (vb[1] << 16);
                c0.y = (vb[2] & 0xFFFFu) | (vb[3] << 16);
                c0.z = (vb[4] & 0xFFFFu) | (vb[5] << 16);
                c0.w = (vb[6] & 0xFFFFu) | (vb[7] << 16);
                c1.x = (vb[0] >> 16) | (vb[1] & 0xFFFF0000u);
                c1.y = (vb[2] >> 16) | (vb[3] & 0xFFFF0000u);
                c1.z = (vb[4] >> 16) | (vb[5] & 0xFFFF0000u);
                c1.w = (vb[6] >> 16) | (vb[7] & 0xFFFF0000u);
                *(u32x4_t*)&sB[(2 * cp) * SK + tg * 8] = c0;
                *(u32x4_t*)&sB[(2 * cp + 1) * SK + tg * 8] = c1;
            }
        }
        __syncthreads();
        // prefetch the next stage while this one is multiplied
        if (s + 1 < n_stages) {
            const int64_t tok = (s + 1) * KT + tg * 8;
            load_pairs<VEC>(va, X, ld, n_tok, d, tok, colA);
            if (!diag) load_pairs<VEC>(vb, X, ld, n_tok, d, tok, colB);
        }
        const uint16_t* sBB = diag ? sA : sB;
#pragma unroll
        for (int ks = 0; ks < KT / 16; ++ks) {
            const int ko = ks * 16 + 8 * (lane >> 5);
            u32x4_t a0 = *(const u32x4_t*)&sA[(wr * 64 + (lane & 31)) * SK + ko];
            u32x4_t a1 = *(const u32x4_t*)&sA[(wr * 64 + 32 + (lane & 31)) * SK + ko];
            u32x4_t b0 = *(const u32x4_t*)&sBB[(wc * 64 + (lane & 31)) * SK + ko];
            u32x4_t b1 = *(const u32x4_t*)&sBB[(wc * 64 + 32 + (lane & 31)) * SK + ko];
            acc[0][0] = mfma_32x32x16(a0, b0, acc[0][0], (Tag*)nullptr);
            acc[0][1] = mfma_32x32x16(a0, b1, acc[0][1], (Tag*)nullptr);
            acc[1][0] = mfma_32x32x16(a1, b0, acc[1][0], (Tag*)nullptr);
            acc[1][1] = mfma_32x32x16(a1, b1, acc[1][1], (Tag*)nullptr);
        }
        if ((s + 1) % stages_per_chunk == 0 || s + 1 == n_stages) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        acc64[i][j][r] += (double)acc[i][j][r];
                        acc[i][j][r] = 0.0f;
                    }
        }
        __syncthreads();
    }

    // strict upper part of the tile (the diagonal comes from the float64 sums)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t i = ti * BT + wr * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int64_t j = tj * BT + wc * 64 + ni * 32 + (lane & 31);
                if (i < j && j < d) H[i * d + j] += 2.0 * acc64[mi][ni][r];
            }

    if (diag) {
        red[tg][2 * cp] = dsq0;
        red[tg][2 * cp + 1] = dsq1;
        __syncthreads();
        if (t < BT) {
            const int64_t c = ti * BT + t;
            if (c < d) {
                const double sum = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
                H[c * d + c] += 2.0 * sum;
            }
        }
    }
}

// fp32 activations: float64 products and sums.  64x64 tiles of the upper
// triangle, 256 threads, each thread a 4x4 block, 16 tokens per stage.
constexpr int FT = 64, FK = 16;

__global__ __launch_bounds__(256) void hess_f32_kernel(double* __restrict__ H, const float* __restrict__ X,
                                                       int64_t n_tok, int64_t d, int64_t ld) {
    __shared__ double sA[FK][FT];
    __shared__ double sB[FK][FT];
    int64_t ti, tj;
    upper_tile(blockIdx.x, ti, tj);
    const int t = threadIdx.x;
    const int ty = t >> 4, tx = t & 15;
    double acc[4][4] = {};
    for (int64_t t0 = 0; t0 < n_tok; t0 += FK) {
        for (int e = t; e < FK * FT; e += 256) {
            const int k = e / FT, c = e % FT;
            const int64_t tok = t0 + k;
            const int64_t ca = ti * FT + c, cb = tj * FT + c;
            sA[k][c] = (tok < n_tok && ca < d) ? (double)X[tok * ld + ca] : 0.0;
            sB[k][c] = (tok < n_tok && cb < d) ? (double)X[tok * ld + cb] : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < FK; ++k) {
            double a[4], b[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                a[u] = sA[k][ty * 4 + u];
                b[u] = sB[k][tx * 4 + u];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[u][v] = fma(a[u], b[v], acc[u][v]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t i = ti * FT + ty * 4 + u, j = tj * FT + tx * 4 + v;
            if (i <= j && j < d) H[i * d + j] += 2.0 * acc[u][v];
        }
}

}  // namespace

gptq_status hessian_launch(double* H, const void* X, gptq_dtype dt, int64_t n_tok, int64_t d,
                           int64_t ld_x, hipStream_t s) {
    if (n_tok == 0) return GPTQ_OK;
    if (dt == GPTQ_F32) {
        const int64_t T = ceil_div(d, FT);
        hipLaunchKernelGGL(hess_f32_kernel, dim3((unsigned)(T * (T + 1) / 2)), dim3(256), 0, s, H,
                           (const float*)X, n_tok, d, ld_x);
        GPTQ_LAUNCH_CHECK();
        return GPTQ_OK;
    }
    const int64_t T = ceil_div(d, BT);
    const dim3 grid((unsigned)(T * (T + 1) / 2)), block(256);
    const bool vec = (ld_x % 2 == 0) && ((uintptr_t)X % 4 == 0);
    const uint16_t* x = (const uint16_t*)X;
    if (dt == GPTQ_BF16) {
        if (vec) hipLaunchKernelGGL((hess_syrk_kernel<bf16x8_t, true>), grid, block, 0, s, H, x, n_tok, d, ld_x);
        else hipLaunchKernelGGL((hess_syrk_kernel<bf16x8_t, false>), grid, block, 0, s, H, x, n_tok, d, ld_x);
    } else {
        if (vec) hipLaunchKernelGGL((hess_syrk_kernel<h16x8_t, true>), grid, block, 0, s, H, x, n_tok, d, ld_x);
        else hipLaunchKernelGGL((hess_syrk_kernel<h16x8_t, false>), grid, block, 0, s, H, x, n_tok, d, ld_x);
    }
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

}  // namespace gptq
