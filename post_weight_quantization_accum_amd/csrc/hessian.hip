// Hessian accumulation H += 2 X^T X ("GPTQ量化算法深度解析" §3.1 step 1),
// upper triangle, on the gfx950 matrix cores.
//
// bf16 / fp16 activations: products are exact in float32, so the MFMA
// v_mfma_f32_32x32x16_{bf16,f16} accumulates chunks of CHUNK tokens in
// float32 registers (one launch per chunk); at the end of a launch the
// partial tile is added to H in float64 (a read-modify-write of the tile
// that the workgroup owns alone, staged through LDS one wave-quarter at a
// time); launches run in token order.
// One workgroup owns one 256x256 tile of the upper triangle for a chunk,
// chunks are added in token order, so the summation order is fixed and the
// result bit-reproducible.
//
// The diagonal is recomputed in float64 from the same staged values (squares
// of bf16/fp16 values are exact in float64): the act-order key diag(H) then
// agrees with a float64 reference to rounding order, so the column order
// does not depend on float32 accumulation error.
//
// Tiling: 8 wave64s per workgroup (two per SIMD), each owning a 128x64
// part as 4x2 MFMA 32x32 tiles (128 float32 accumulators per lane).  X is token-major,
// while each MFMA operand is 8 consecutive tokens of one column, so every
// thread loads an 8-token x 8-column block with 16-byte loads, transposes it
// in registers (v_perm_b32) and writes eight 16-byte column runs into LDS
// laid out [column][token] (row stride 72 elements: conflict-free for both
// the writes and the operand reads).  LDS is double-buffered and the next
// stage's global loads are in flight while the current stage is multiplied.
// Workgroups are mapped to tiles so that the ~32 workgroups resident on one
// XCD work on a compact block of about 6x6 tiles (about 12 column panels of
// X shared through that XCD's L2).
//
// fp32 activations take a float64 path (products of fp32 values are exact
// in float64): a plain tiled float64 kernel.
#include "internal.hpp"

namespace gptq {
namespace {

constexpr int BT = 256;          // tile edge
constexpr int KT = 64;           // tokens per LDS stage
constexpr int SK = KT + 8;       // LDS row stride in 16-bit elements (144 B)
constexpr int CHUNK = 32768;     // tokens accumulated in float32 before the float64 add
constexpr int SP = 132;          // row stride (floats) of the staged 128x128 quarter
constexpr int PANEL = BT * SK;   // 16-bit elements per panel buffer

constexpr int BAND = 6;  // tile rows per band of the tile enumeration

// Enumeration of the upper-triangle tiles in bands of BAND tile rows, column
// by column inside a band (rows ascending within a column): a run of ~32
// consecutive tiles covers about 6 rows x 6 columns of tiles, i.e. needs
// about 12 column panels of X instead of ~33 for a row-major run.
__device__ __forceinline__ void upper_tile(int64_t t, int64_t& ti, int64_t& tj, int64_t T) {
    int64_t r0 = 0;
    for (;;) {
        const int64_t r1 = (r0 + BAND < T) ? r0 + BAND : T;
        // tiles of this band: sum over columns c >= r0 of (min(r1-1, c) - r0 + 1)
        const int64_t h = r1 - r0;
        const int64_t band_tiles = h * (h + 1) / 2 + h * (T - r1);
        if (t < band_tiles) {
            int64_t c = r0;
            for (;;) {
                const int64_t cnt = ((c < r1 - 1) ? c : r1 - 1) - r0 + 1;
                if (t < cnt) {
                    ti = r0 + t;
                    tj = c;
                    return;
                }
                t -= cnt;
                ++c;
            }
        }
        t -= band_tiles;
        r0 = r1;
    }
}

template <typename Tag>
__device__ __forceinline__ double elem_f64(uint16_t b);
template <>
__device__ __forceinline__ double elem_f64<bf16x8_t>(uint16_t b) { return bf16_bits_to_f64(b); }
template <>
__device__ __forceinline__ double elem_f64<h16x8_t>(uint16_t b) { return f16_bits_to_f64(b); }

// Buffer resources for one stage: resource r starts at token row
// s*KT + r and covers the stage's valid rows from there on, so a lane's
// offset (token group tg*8, column col) is in range exactly when token
// s*KT + r + tg*8 exists.  Out-of-range loads return 0 without touching
// memory.  The row offset lives in the (uniform) resource, not in soffset,
// because the range check applies to the vector offset only.
struct StageRsrc {
    __amdgpu_buffer_rsrc_t r[8];
};

__device__ __forceinline__ StageRsrc stage_rsrc(const uint16_t* X, int64_t s, int64_t ld, int64_t n_tok) {
    StageRsrc o;
    const int64_t t0 = s * KT;
    int64_t rows = n_tok - t0;
    rows = rows > KT ? KT : rows;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int64_t left = rows - r;
        const int nrec = left > 0 ? (int)(left * ld * 2) : 0;
        o.r[r] = __builtin_amdgcn_make_buffer_rsrc((void*)(X + (t0 + r) * ld), (short)0, nrec, 0x00020000);
    }
    return o;
}

constexpr uint32_t OOB = 0x80000000u;  // a byte offset beyond every resource's range

// 8 tokens x 8 columns, one u32x4 (8 columns) per token.  off is the byte
// offset of (token tg*8, column col) from a resource's first row, or OOB.
template <bool VEC>
__device__ __forceinline__ void load_block(u32x4_t v[8], const StageRsrc& rs, uint32_t off, int64_t col,
                                           int64_t d) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        if (VEC) {
            v[r] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs.r[r], (int)off, 0, 0));
        } else {
            uint32_t e[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t o = (col + c < d) ? off + 2u * c : OOB;
                e[c] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs.r[r], (int)o, 0, 0);
            }
            v[r].x = e[0] | (e[1] << 16);
            v[r].y = e[2] | (e[3] << 16);
            v[r].z = e[4] | (e[5] << 16);
            v[r].w = e[6] | (e[7] << 16);
        }
    }
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

__device__ __forceinline__ uint32_t word(const u32x4_t& v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Transpose the 8x8 block and store column runs of 8 tokens into LDS.
__device__ __forceinline__ void store_block(uint16_t* buf, const u32x4_t v[8], int cg, int tg) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t w0 = word(v[0], p), w1 = word(v[1], p), w2 = word(v[2], p), w3 = word(v[3], p);
        const uint32_t w4 = word(v[4], p), w5 = word(v[5], p), w6 = word(v[6], p), w7 = word(v[7], p);
        u32x4_t lo, hi;
        lo.x = lo_pair(w0, w1); lo.y = lo_pair(w2, w3); lo.z = lo_pair(w4, w5); lo.w = lo_pair(w6, w7);
        hi.x = hi_pair(w0, w1); hi.y = hi_pair(w2, w3); hi.z = hi_pair(w4, w5); hi.w = hi_pair(w6, w7);
        *(u32x4_t*)&buf[(cg * 8 + 2 * p) * SK + tg * 8] = lo;
        *(u32x4_t*)&buf[(cg * 8 + 2 * p + 1) * SK + tg * 8] = hi;
    }
}

template <typename Tag>
__device__ __forceinline__ void diag_accumulate(double dsq[8], const u32x4_t v[8]) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t w = word(v[r], p);
            const double x0 = elem_f64<Tag>((uint16_t)(w & 0xFFFFu));
            const double x1 = elem_f64<Tag>((uint16_t)(w >> 16));
            dsq[2 * p] = fma(x0, x0, dsq[2 * p]);
            dsq[2 * p + 1] = fma(x1, x1, dsq[2 * p + 1]);
        }
}

template <typename Tag, bool VEC>
__global__ __launch_bounds__(512) void hess_syrk_kernel(double* __restrict__ H, const uint16_t* __restrict__ X,
                                                        int64_t n_tok, int64_t d, int64_t ld, int64_t T,
                                                        int64_t n_tiles, int64_t per_xcd) {
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // [2 stages][2 panels][PANEL]
    // XCD-grouped tile order: workgroup b runs on XCD b % 8; each XCD takes a
    // contiguous range of the banded upper-triangle enumeration.
    const int64_t b = blockIdx.x;
    const int64_t lin = (b % 8) * per_xcd + b / 8;
    if (lin >= n_tiles) return;
    int64_t ti, tj;
    upper_tile(lin, ti, tj, T);
    const bool diag = (ti == tj);

    // 8 waves: wave (wr, wc) owns rows wr*128..+128 and columns wc*64..+64
    // of the tile as 4x2 MFMA 32x32 tiles.  For staging, threads 0..255 load
    // the row panel and threads 256..511 the column panel (idle on diagonal
    // tiles, where the two panels coincide).
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wr = wave >> 2, wc = wave & 3;
    const int pt = t & 255, panel = t >> 8;
    const int tg = lane & 7, cg = (pt >> 6) * 8 + (lane >> 3);
    const bool loader = !(diag && panel == 1);
    const int64_t col = (panel ? tj : ti) * BT + cg * 8;

    f16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // this launch covers tokens [0, n_tok) of X (the caller offsets X per chunk)
    const int64_t n_stages = ceil_div(n_tok, KT);
    const uint32_t row_bytes = (uint32_t)(ld * 2);
    const uint32_t off = (col < d && loader) ? (uint32_t)(tg * 8) * row_bytes + (uint32_t)(col * 2) : OOB;
    u32x4_t va[8];
    load_block<VEC>(va, stage_rsrc(X, 0, ld, n_tok), off, col, d);
    if (loader) store_block(lds + panel * PANEL, va, cg, tg);
    __syncthreads();
    if (n_stages > 1) load_block<VEC>(va, stage_rsrc(X, 1, ld, n_tok), off, col, d);

    for (int64_t s = 0; s < n_stages; ++s) {
        const uint16_t* bufA = lds + (s & 1) * 2 * PANEL;
        const uint16_t* bufB = diag ? bufA : bufA + PANEL;
#pragma unroll
        for (int ks = 0; ks < KT / 16; ++ks) {
            const int ko = ks * 16 + 8 * (lane >> 5);
            u32x4_t a[4], bb[2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *(const u32x4_t*)&bufA[(wr * 128 + i * 32 + (lane & 31)) * SK + ko];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bb[j] = *(const u32x4_t*)&bufB[(wc * 64 + j * 32 + (lane & 31)) * SK + ko];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma_32x32x16(a[i], bb[j], acc[i][j], (Tag*)nullptr);
        }
        if (s + 1 < n_stages) {
            if (loader) store_block(lds + ((s + 1) & 1) * 2 * PANEL + panel * PANEL, va, cg, tg);
            if (s + 2 < n_stages) load_block<VEC>(va, stage_rsrc(X, s + 2, ld, n_tok), off, col, d);
        }
        __syncthreads();
    }

    // float32 tile -> float64 H (strict upper part; the diagonal comes from a
    // float64 pass).  Waves stage their 128x64 parts in LDS two at a time
    // (one 128x128 quarter), then all threads add it to H with
    // row-contiguous accesses.
    float* stg = (float*)lds;
#pragma unroll 1
    for (int q = 0; q < 4; ++q) {
        // quarter q: rows (q>>1)*128, cols (q&1)*128 -> waves wr = q>>1, wc in {2(q&1), 2(q&1)+1}
        if (wr == (q >> 1) && (wc >> 1) == (q & 1)) {
            float* sl = stg + (4 * (lane >> 5)) * SP + (wc & 1) * 64 + (lane & 31);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        sl[(mi * 32 + 8 * (r >> 2) + (r & 3)) * SP + ni * 32] = acc[mi][ni][r];
        }
        __syncthreads();
        const int64_t ib = ti * BT + (q >> 1) * 128, jb = tj * BT + (q & 1) * 128;
        const int cl = t & 127;
        const int64_t j = jb + cl;
#pragma unroll 8
        for (int row = t >> 7; row < 128; row += 4) {
            const int64_t i = ib + row;
            if (i < j && j < d) H[i * d + j] += 2.0 * (double)stg[row * SP + cl];
        }
        __syncthreads();
    }
}

// diag(H) in float64: H[c][c] += 2 * sum_t x_tc^2.  Squares of bf16/fp16
// values are exact in float64.  Grid (column blocks of 256, token splits);
// each thread sums every 8th token of its split for 8 adjacent columns,
// the 8 token lanes are reduced in LDS in a fixed order, and a second
// kernel adds the splits in order: deterministic.
constexpr int DSPLIT = 32;

template <typename Tag, bool VEC>
__global__ __launch_bounds__(256) void colsq_kernel(const uint16_t* __restrict__ X, int64_t n_tok, int64_t d,
                                                    int64_t ld, double* __restrict__ part) {
    __shared__ double red[8][256];
    const int t = threadIdx.x, tl = t & 7, cc = t >> 3;
    const int64_t col = (int64_t)blockIdx.x * 256 + cc * 8;
    const int64_t per = ceil_div(n_tok, DSPLIT);
    const int64_t t0 = (int64_t)blockIdx.y * per;
    const int64_t t1 = (t0 + per < n_tok) ? t0 + per : n_tok;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (col < d) {
        for (int64_t tk = t0 + tl; tk < t1; tk += 8) {
            const uint16_t* p = X + tk * ld + col;
            uint16_t e[8];
            if (VEC) {
                const u32x4_t w = *(const u32x4_t*)p;
                e[0] = w.x & 0xFFFFu; e[1] = w.x >> 16; e[2] = w.y & 0xFFFFu; e[3] = w.y >> 16;
                e[4] = w.z & 0xFFFFu; e[5] = w.z >> 16; e[6] = w.w & 0xFFFFu; e[7] = w.w >> 16;
            } else {
#pragma unroll
                for (int c = 0; c < 8; ++c) e[c] = (col + c < d) ? p[c] : (uint16_t)0;
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const double x = elem_f64<Tag>(e[c]);
                acc[c] = fma(x, x, acc[c]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) red[tl][cc * 8 + c] = acc[c];
    __syncthreads();
    const int64_t c = (int64_t)blockIdx.x * 256 + t;
    if (c < d) {
        double sum = 0.0;
#pragma unroll
        for (int g = 0; g < 8; ++g) sum += red[g][t];
        part[(int64_t)blockIdx.y * d + c] = sum;
    }
}

__global__ __launch_bounds__(256) void colsq_finish_kernel(const double* __restrict__ part, int64_t d,
                                                           double* __restrict__ H) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= d) return;
    double sum = 0.0;
    for (int s = 0; s < DSPLIT; ++s) sum += part[(int64_t)s * d + c];
    H[c * d + c] += 2.0 * sum;
}

// fp32 activations: float64 products and sums.  64x64 tiles of the upper
// triangle, 256 threads, each thread a 4x4 block, 16 tokens per stage.
constexpr int FT = 64, FK = 16;

__global__ __launch_bounds__(256) void hess_f32_kernel(double* __restrict__ H, const float* __restrict__ X,
                                                       int64_t n_tok, int64_t d, int64_t ld) {
    __shared__ double sA[FK][FT];
    __shared__ double sB[FK][FT];
    int64_t ti, tj;
    {
        const int64_t tt = blockIdx.x;
        int64_t x = (int64_t)((sqrt(8.0 * (double)tt + 1.0) - 1.0) * 0.5);
        while (x * (x + 1) / 2 > tt) --x;
        while ((x + 1) * (x + 2) / 2 <= tt) ++x;
        tj = x;
        ti = tt - x * (x + 1) / 2;
    }
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

size_t hessian_workspace_bytes(int64_t d) { return (size_t)DSPLIT * d * sizeof(double); }

gptq_status hessian_launch(double* H, const void* X, gptq_dtype dt, int64_t n_tok, int64_t d,
                           int64_t ld_x, double* part, hipStream_t s) {
    if (n_tok == 0) return GPTQ_OK;
    if (dt == GPTQ_F32) {
        const int64_t T = ceil_div(d, FT);
        hipLaunchKernelGGL(hess_f32_kernel, dim3((unsigned)(T * (T + 1) / 2)), dim3(256), 0, s, H,
                           (const float*)X, n_tok, d, ld_x);
        GPTQ_LAUNCH_CHECK();
        return GPTQ_OK;
    }
    const int64_t T = ceil_div(d, BT);
    const int64_t n_tiles = T * (T + 1) / 2;
    const int64_t per_xcd = ceil_div(n_tiles, 8);
    const dim3 grid((unsigned)(per_xcd * 8)), block(512);
    const size_t shmem = 4 * PANEL * sizeof(uint16_t);
    const bool vec = (ld_x % 8 == 0) && (d % 8 == 0) && ((uintptr_t)X % 16 == 0);
    const uint16_t* x = (const uint16_t*)X;
    static bool attr_set = false;
    if (!attr_set) {
        GPTQ_HIP(hipFuncSetAttribute((const void*)hess_syrk_kernel<bf16x8_t, true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem));
        GPTQ_HIP(hipFuncSetAttribute((const void*)hess_syrk_kernel<bf16x8_t, false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem));
        GPTQ_HIP(hipFuncSetAttribute((const void*)hess_syrk_kernel<h16x8_t, true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem));
        GPTQ_HIP(hipFuncSetAttribute((const void*)hess_syrk_kernel<h16x8_t, false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem));
        attr_set = true;
    }
    const dim3 dgrid((unsigned)ceil_div(d, 256), DSPLIT), b256(256);
    if (dt == GPTQ_BF16) {
        if (vec) hipLaunchKernelGGL((colsq_kernel<bf16x8_t, true>), dgrid, b256, 0, s, x, n_tok, d, ld_x, part);
        else hipLaunchKernelGGL((colsq_kernel<bf16x8_t, false>), dgrid, b256, 0, s, x, n_tok, d, ld_x, part);
    } else {
        if (vec) hipLaunchKernelGGL((colsq_kernel<h16x8_t, true>), dgrid, b256, 0, s, x, n_tok, d, ld_x, part);
        else hipLaunchKernelGGL((colsq_kernel<h16x8_t, false>), dgrid, b256, 0, s, x, n_tok, d, ld_x, part);
    }
    GPTQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(colsq_finish_kernel, dim3((unsigned)ceil_div(d, 256)), b256, 0, s, part, d, H);
    GPTQ_LAUNCH_CHECK();
    // one launch per chunk of CHUNK tokens: each adds its float32 partial
    // tiles to H in float64, in token order
    for (int64_t c0 = 0; c0 < n_tok; c0 += CHUNK) {
        const int64_t nt = (n_tok - c0 < CHUNK) ? n_tok - c0 : CHUNK;
        const uint16_t* xc = x + c0 * ld_x;
        if (dt == GPTQ_BF16) {
            if (vec) hipLaunchKernelGGL((hess_syrk_kernel<bf16x8_t, true>), grid, block, shmem, s, H, xc, nt, d, ld_x, T, n_tiles, per_xcd);
            else hipLaunchKernelGGL((hess_syrk_kernel<bf16x8_t, false>), grid, block, shmem, s, H, xc, nt, d, ld_x, T, n_tiles, per_xcd);
        } else {
            if (vec) hipLaunchKernelGGL((hess_syrk_kernel<h16x8_t, true>), grid, block, shmem, s, H, xc, nt, d, ld_x, T, n_tiles, per_xcd);
            else hipLaunchKernelGGL((hess_syrk_kernel<h16x8_t, false>), grid, block, shmem, s, H, xc, nt, d, ld_x, T, n_tiles, per_xcd);
        }
        GPTQ_LAUNCH_CHECK();
    }
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

}  // namespace gptq
