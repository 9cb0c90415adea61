// Hessian accumulation H += 2 X^T X ("GPTQ量化算法深度解析" §3.1 step 1),
// upper triangle, on the gfx950 matrix cores.
//
// bf16 / fp16 activations: products are exact in float32, so the MFMA
// v_mfma_f32_32x32x16_{bf16,f16} accumulates chunks of up to 32768 tokens
// in float32 registers (one launch per chunk); at the end of a launch the
// partial tile is added to H in float64 (a read-modify-write of the tile
// that the workgroup owns alone, staged through LDS one quarter at a time);
// launches run in token order, so the summation order is fixed and the
// result bit-reproducible.
//
// The diagonal is recomputed in float64 from the same inputs (squares of
// bf16/fp16 values are exact in float64): the act-order key diag(H) then
// agrees with a float64 reference to rounding order, so the column order
// does not depend on float32 accumulation error.
//
// Each MFMA operand is 8 consecutive tokens of one column, while X is
// token-major.  A chunk is therefore first transposed (8x8 blocks in
// registers, v_perm_b32) into a feature-major copy Xt, zero-padded to a
// multiple of 256 features and of 64 tokens, stored stage-major: the 64
// tokens of all features for one stage form one contiguous block, so the
// stage of one 256-feature panel is 32 KiB of consecutive memory (few pages
// and DRAM rows per stage, instead of 256 rows a chunk-length apart).  The
// SYRK kernel then streams
// Xt straight from memory into LDS with buffer_load ... lds (no VGPR
// staging) through a ring of two 64-token stages (64 KiB each), one stage
// ahead of the MFMAs, one barrier per stage; the MFMA operands are
// software-pipelined in registers one k-step ahead, across the barrier.
// Within a stage a feature row is 128 bytes (eight 16-byte granules);
// granule g of row r is stored at slot g ^ ((r >> 1) & 7), so the rows read
// by one MFMA operand fetch hit distinct banks.
//
// Tiling: one workgroup per 256x256 tile of the upper triangle, 8 wave64s
// (two per SIMD), each owning a 128x64 part as 4x2 MFMA 32x32 tiles.
// Workgroups are mapped to tiles so that the ~32 workgroups resident on one
// XCD work on a compact block of about 6x6 tiles (about 12 column panels of
// Xt shared through that XCD's L2).
//
// fp32 activations take a float64 path (products of fp32 values are exact
// in float64): a plain tiled float64 kernel.
#include "internal.hpp"

namespace gptq {
namespace {

constexpr int BT = 256;          // tile edge
#ifndef GPTQ_KT
#define GPTQ_KT 64
#endif
#ifndef GPTQ_NSTAGE
#define GPTQ_NSTAGE 2
#endif
constexpr int KT = GPTQ_KT;           // tokens per LDS stage
constexpr int NSTAGE = GPTQ_NSTAGE;   // LDS ring depth
constexpr int GR = KT / 8;            // 16-byte token granules per feature row of a stage
constexpr int RPB = 128 / KT;         // feature rows per 256-byte bank window
constexpr int DMA_ROWS = 512 / KT;    // feature rows per 1 KiB wave-wide DMA load
constexpr int CHUNK = 32768;     // tokens accumulated in float32 before the float64 add
constexpr int SP = 132;          // row stride (floats) of the staged 128x128 quarter
constexpr int PANEL_BYTES = BT * KT * 2;           // one 256-feature x 32-token panel
constexpr int STAGE_BYTES = 2 * PANEL_BYTES;       // row panel + column panel
constexpr int RING_BYTES = NSTAGE * STAGE_BYTES;   // 128 KiB
constexpr size_t XT_MAX_BYTES = (size_t)1 << 30;   // transposed-chunk scratch cap

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

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

__device__ __forceinline__ uint32_t word(const u32x4_t& v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Xt[t / KT][f][t % KT] = X[t][f] for one chunk (stage-major: the KT tokens
// of all d_pad features for one stage are one contiguous block), n_tok
// tokens, zeros for t >= n_tok (up to ch) and for d <= f < d_pad; also the float64
// sums of squares of the block's 512 tokens per feature (diagonal of H).
// A block covers 512 tokens x 256 features in tiles of 64 tokens: a thread
// loads 8 tokens x 8 features (16-byte loads, 32 lanes along the features:
// 512 contiguous bytes per token row), transposes them in registers
// (v_perm_b32), and the tile goes through LDS so that every store writes
// whole 128-byte runs of one feature row.
constexpr int TSPAN = 512;      // tokens per transpose block
constexpr int TT = 64;          // tokens per tile
constexpr int TLD = TT + 8;     // LDS row stride (16-bit elements)

constexpr size_t TILE_BYTES = 256 * TLD * sizeof(uint16_t);
constexpr size_t TRANSPOSE_LDS = TILE_BYTES + 8 * 256 * sizeof(double);

// One transpose block (token block bx, feature block by) by 256 threads
// (t = 0..255) with LDS tile / red; barriers are those of the whole
// workgroup, so every thread of it calls this with the same bx.  active =
// false: the threads take part in the barriers only.
template <typename Tag, bool VEC>
__device__ __forceinline__ void transpose_block(const uint16_t* __restrict__ X, int64_t n_tok, int64_t d, int64_t ld,
                                                uint16_t* __restrict__ Xt, int64_t ch, int64_t d_pad,
                                                double* __restrict__ colsq, int64_t bx, int64_t by, bool active, int t,
                                                uint16_t* tile, double (*red)[256]) {
    static_assert(TT == KT, "a transpose tile is one stage");
    const int tg = t >> 5, fg = t & 31;
    const int64_t fblk = by * 256;
    const int64_t f = fblk + fg * 8;
    double sq[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int tt = 0; tt < TSPAN / TT; ++tt) {
        const int64_t tbase = bx * TSPAN + tt * TT;
        if (tbase >= ch) break;
        const int64_t t0 = tbase + tg * 8;
        u32x4_t v[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t tok = t0 + r;
            u32x4_t x = {0u, 0u, 0u, 0u};
            if (active && tok < n_tok) {
                const uint16_t* p = X + tok * ld + f;
                if (VEC) {
                    if (f < d) x = *(const u32x4_t*)p;
                } else {
                    uint32_t e[8];
#pragma unroll
                    for (int c = 0; c < 8; ++c) e[c] = (f + c < d) ? (uint32_t)p[c] : 0u;
                    x.x = e[0] | (e[1] << 16);
                    x.y = e[2] | (e[3] << 16);
                    x.z = e[4] | (e[5] << 16);
                    x.w = e[6] | (e[7] << 16);
                }
            }
            v[r] = x;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t w = word(v[r], p);
                const double x0 = elem_f64<Tag>((uint16_t)(w & 0xFFFFu));
                const double x1 = elem_f64<Tag>((uint16_t)(w >> 16));
                sq[2 * p] = fma(x0, x0, sq[2 * p]);
                sq[2 * p + 1] = fma(x1, x1, sq[2 * p + 1]);
            }
        __syncthreads();  // the previous tile has been written out
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t w0 = word(v[0], p), w1 = word(v[1], p), w2 = word(v[2], p), w3 = word(v[3], p);
            const uint32_t w4 = word(v[4], p), w5 = word(v[5], p), w6 = word(v[6], p), w7 = word(v[7], p);
            u32x4_t lo, hi;
            lo.x = lo_pair(w0, w1); lo.y = lo_pair(w2, w3); lo.z = lo_pair(w4, w5); lo.w = lo_pair(w6, w7);
            hi.x = hi_pair(w0, w1); hi.y = hi_pair(w2, w3); hi.z = hi_pair(w4, w5); hi.w = hi_pair(w6, w7);
            *(u32x4_t*)&tile[(fg * 8 + 2 * p) * TLD + tg * 8] = lo;
            *(u32x4_t*)&tile[(fg * 8 + 2 * p + 1) * TLD + tg * 8] = hi;
        }
        __syncthreads();
        // 256 feature rows x 8 granules of 8 tokens; 8 lanes per row
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int e = k * 256 + t;
            const int fr = e >> 3, gq = e & 7;
            const int64_t tok = tbase + gq * 8;
            if (active && tok < ch)
                *(u32x4_t*)&Xt[((tbase / KT) * d_pad + fblk + fr) * KT + gq * 8] =
                    *(const u32x4_t*)&tile[fr * TLD + gq * 8];
        }
    }
    // column sums of squares: the 8 token groups in a fixed order
#pragma unroll
    for (int c = 0; c < 8; ++c) red[tg][fg * 8 + c] = sq[c];
    __syncthreads();
    const int64_t fc = fblk + t;
    if (active && fc < d) {
        double sum = 0.0;
#pragma unroll
        for (int g = 0; g < 8; ++g) sum += red[g][t];
        colsq[bx * d + fc] = sum;
    }
}

template <typename Tag, bool VEC>
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ X, int64_t n_tok, int64_t d,
                                                        int64_t ld, uint16_t* __restrict__ Xt, int64_t ch,
                                                        int64_t d_pad, double* __restrict__ colsq) {
    __shared__ __attribute__((aligned(16))) char tl[TRANSPOSE_LDS];
    transpose_block<Tag, VEC>(X, n_tok, d, ld, Xt, ch, d_pad, colsq, blockIdx.x, blockIdx.y, true, threadIdx.x,
                              (uint16_t*)tl, (double(*)[256])(tl + TILE_BYTES));
}

// diag(H) += 2 * sum of the chunk's per-block column sums, blocks in order.
__global__ __launch_bounds__(256) void diag_add_kernel(const double* __restrict__ colsq, int64_t nblk, int64_t d,
                                                       double* __restrict__ H) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= d) return;
    double sum = 0.0;
    for (int64_t b = 0; b < nblk; ++b) sum += colsq[b * d + c];
    H[c * d + c] += 2.0 * sum;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt at
// their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) only (vmcnt and expcnt at their maxima).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// One stage of one panel: 256 feature rows x KT tokens, moved by wave-wide
// 1 KiB DMA loads of DMA_ROWS rows each; a call covers 32 rows.  Lane l of a
// load fills LDS granule l of its 1 KiB block: row r = block_row + l/GR,
// slot l%GR, which holds token granule g = slot ^ swz(r) of that row.
__device__ __forceinline__ int swz(int r) { return (r / RPB) % GR; }

__device__ __forceinline__ void dma_panel_rows(__amdgpu_buffer_rsrc_t rs, char* lds_panel, int row0, int lane,
                                               uint32_t prow, uint32_t soff) {
#pragma unroll
    for (int q = 0; q < 32 / DMA_ROWS; ++q) {
        const int rblk = row0 + DMA_ROWS * q;
        const int r = rblk + lane / GR;
        const int g = (lane % GR) ^ swz(r);
        const uint32_t voff = ((prow + (uint32_t)r) * KT + 8 * g) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(lds_panel + rblk * (KT * 2)), 16, (int)voff,
                                                 (int)soff, 0, 0);
    }
}

// MFMA operand fetch: row r of a staged panel, token granule g (8 tokens).
__device__ __forceinline__ u32x4_t lds_operand(const char* lds_panel, int r, int g) {
    return *(const u32x4_t*)(lds_panel + r * (KT * 2) + ((g ^ swz(r)) << 4));
}

// Stages [st0, st1) of the chunk.  part == null: the tile's float32 sums are
// added to H; otherwise they are written to part (256x256 floats, row-major)
// for a fixed-order reduction over the token slices of a tile.
template <typename Tag, bool DIAG, int NW>
__device__ __forceinline__ void syrk_tile(double* __restrict__ H, const uint16_t* __restrict__ Xt, int64_t ch, int64_t d_pad,
                                          int64_t d, int64_t ti, int64_t tj, char* lds, int64_t st0, int64_t st1,
                                          float* __restrict__ part) {
    constexpr int WCOLS = 512 / NW, NTL = WCOLS / 32, NCW = BT / WCOLS;
    constexpr int RPW = BT / NW;  // panel rows loaded per wave (multiple of 32)
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wr = wave / NCW, wc = wave % NCW;
    const int64_t n_st = st1 - st0;     // stages of this workgroup (local index st = 0 .. n_st-1)
    // one resource over the chunk; a stage of one panel is 256 consecutive
    // rows of KT tokens, at byte offset (st * d_pad + panel row) * KT * 2
    const uint32_t stage_bytes = (uint32_t)(d_pad * KT * 2);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)Xt, (short)0, (int)(stage_bytes * (uint32_t)(ch / KT)), 0x00020000);
    const uint32_t pa_row = (uint32_t)(ti * BT), pb_row = (uint32_t)(tj * BT);
    const int row0 = wave * RPW;
    // loads issued per wave per stage
    constexpr int NLD = (DIAG ? 1 : 2) * (RPW / DMA_ROWS);

    f16_t acc[4][NTL];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NTL; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto issue = [&](int64_t st) {
        char* sb = lds + (st % NSTAGE) * STAGE_BYTES;
#pragma unroll
        for (int rr = 0; rr < RPW; rr += 32) {
            dma_panel_rows(rs, sb, row0 + rr, lane, pa_row, (uint32_t)(st0 + st) * stage_bytes);
            if (!DIAG) dma_panel_rows(rs, sb + PANEL_BYTES, row0 + rr, lane, pb_row, (uint32_t)(st0 + st) * stage_bytes);
        }
    };
    auto read_ops = [&](u32x4_t (&a)[4], u32x4_t (&bb)[NTL], int64_t st, int ks) {
        const char* pa = lds + (st % NSTAGE) * STAGE_BYTES;
        const char* pb = DIAG ? pa : pa + PANEL_BYTES;
        const int g = 2 * ks + (lane >> 5);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = lds_operand(pa, wr * 128 + i * 32 + (lane & 31), g);
#pragma unroll
        for (int j = 0; j < NTL; ++j) bb[j] = lds_operand(pb, wc * WCOLS + j * 32 + (lane & 31), g);
    };
    // all NSTAGE ring slots in flight; stage 0 visible to every wave
#pragma unroll
    for (int k = 0; k < NSTAGE; ++k)
        if (k < n_st) issue(k);
    if (n_st >= NSTAGE) wait_vmcnt<NLD * (NSTAGE - 1)>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();

    // Software pipeline over k-steps: the operands of the next k-step are
    // read while the current one's MFMAs run.  At a stage boundary this
    // wave's reads of the finished stage are complete before the barrier,
    // so the slot is refilled right after it, and the last k-step's MFMAs
    // cover the first reads of the new stage.
    constexpr int KPS = KT / 16;
    static_assert(KPS % 2 == 0, "operand double buffer alternates per k-step");
    u32x4_t a0[4], b0[NTL], a1[4], b1[NTL];
    read_ops(a0, b0, 0, 0);
    for (int64_t st = 0; st < n_st; ++st) {
#pragma unroll
        for (int ks = 0; ks < KPS; ++ks) {
            u32x4_t (&ac)[4] = (ks & 1) ? a1 : a0;
            u32x4_t (&bc)[NTL] = (ks & 1) ? b1 : b0;
            u32x4_t (&an)[4] = (ks & 1) ? a0 : a1;
            u32x4_t (&bn)[NTL] = (ks & 1) ? b0 : b1;
            if (ks + 1 < KPS) {
                read_ops(an, bn, st, ks + 1);
            } else if (st + 1 < n_st) {
                wait_lgkm0();
                if (st + NSTAGE - 1 < n_st) wait_vmcnt<NLD * (NSTAGE - 2)>();
                else wait_vmcnt<0>();
                __builtin_amdgcn_s_barrier();
                if (st + NSTAGE < n_st) issue(st + NSTAGE);
                read_ops(an, bn, st + 1, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NTL; ++j) acc[i][j] = mfma_32x32x16(ac[i], bc[j], acc[i][j], (Tag*)nullptr);
        }
    }
    __syncthreads();

    if (part) {
        // lane l holds C[8*(r/4) + 4*(l/32) + r%4][l%32] of each 32x32 block
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < NTL; ++ni)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wr * 128 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const int col = wc * WCOLS + ni * 32 + (lane & 31);
                    part[row * BT + col] = acc[mi][ni][r];
                }
        return;
    }

    // float32 tile -> float64 H (strict upper part; the diagonal comes from a
    // float64 pass).  The 128x128 quarters are staged in LDS one at a time
    // by the waves that own them, then all threads add the quarter to H with
    // row-contiguous accesses.
    float* stg = (float*)lds;
#pragma unroll 1
    for (int q = 0; q < 4; ++q) {
        if (wr == (q >> 1) && (wc * WCOLS) / 128 == (q & 1)) {
            float* sl = stg + (4 * (lane >> 5)) * SP + (wc * WCOLS) % 128 + (lane & 31);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < NTL; ++ni)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        sl[(mi * 32 + 8 * (r >> 2) + (r & 3)) * SP + ni * 32] = acc[mi][ni][r];
        }
        __syncthreads();
        const int64_t ib = ti * BT + (q >> 1) * 128, jb = tj * BT + (q & 1) * 128;
        const int cl = t & 127;
        const int64_t j = jb + cl;
#pragma unroll 8
        for (int row = t >> 7; row < 128; row += NW / 2) {
            const int64_t i = ib + row;
            if (i < j && j < d) H[i * d + j] += 2.0 * (double)stg[row * SP + cl];
        }
        __syncthreads();
    }
}

// The next chunk, transposed by the workgroups past the tiles of a launch.
struct NextChunk {
    const uint16_t* X;   // its first token row
    int64_t n_tok, ld, ch;
    uint16_t* Xt;
    double* colsq;
};

// S > 1 (few tiles): each tile's stages are split into S consecutive token
// slices, one workgroup each, writing float32 partial tiles to part (slice s
// of tile t at part + (t * S + s) * 256 * 256); syrk_slices_add_kernel then
// adds them to H in slice order.
template <typename Tag, int NW, bool VEC>
__global__ __launch_bounds__(NW * 64) void hess_syrk_kernel(double* __restrict__ H, const uint16_t* __restrict__ Xt,
                                                            int64_t ch, int64_t d_pad, int64_t d, int64_t T,
                                                            int64_t n_tiles, int64_t per_xcd, NextChunk nx,
                                                            int64_t S, float* __restrict__ part) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int64_t b = blockIdx.x;
    if (b >= per_xcd * 8) {
        // Past the tiles: the next chunk's transpose, two 256-feature blocks
        // of one token block per workgroup.  These workgroups are dispatched
        // last and fill the CUs that the last round of tiles leaves idle.
        static_assert(NW * 64 == 512, "two transpose halves of 256 threads");
        const int64_t nby = d_pad / 256, npair = (nby + 1) / 2;
        const int64_t q = b - per_xcd * 8;
        const int half = (int)(threadIdx.x >> 8);
        const int64_t by = 2 * (q % npair) + half;
        char* h = lds + half * (RING_BYTES / 2);
        transpose_block<Tag, VEC>(nx.X, nx.n_tok, d, nx.ld, nx.Xt, nx.ch, d_pad, nx.colsq, q / npair, by, by < nby,
                                  (int)(threadIdx.x & 255), (uint16_t*)h, (double(*)[256])(h + TILE_BYTES));
        return;
    }
    // XCD-grouped tile order: workgroup b runs on XCD b % 8; each XCD takes a
    // contiguous range of the banded upper-triangle enumeration.
    const int64_t lin = (b % 8) * per_xcd + b / 8;
    if (lin >= n_tiles * S) return;
    const int64_t tile = lin / S, sl = lin % S, n_st = ch / KT;
    const int64_t st0 = sl * n_st / S, st1 = (sl + 1) * n_st / S;
    float* pt = (S > 1) ? part + lin * (int64_t)(BT * BT) : nullptr;
    int64_t ti, tj;
    upper_tile(tile, ti, tj, T);
    if (ti == tj) syrk_tile<Tag, true, NW>(H, Xt, ch, d_pad, d, ti, tj, lds, st0, st1, pt);
    else syrk_tile<Tag, false, NW>(H, Xt, ch, d_pad, d, ti, tj, lds, st0, st1, pt);
}

// H (strict upper) += 2 * sum over the S slices of each tile, in slice order,
// in float64.  One workgroup per 4 rows of a tile, one thread per column.
__global__ __launch_bounds__(256) void syrk_slices_add_kernel(double* __restrict__ H, const float* __restrict__ part,
                                                              int64_t T, int64_t S, int64_t d) {
    const int64_t tile = blockIdx.x / (BT / 4), rq = blockIdx.x % (BT / 4);
    int64_t ti, tj;
    upper_tile(tile, ti, tj, T);
    const int c = threadIdx.x;
    const int64_t j = tj * BT + c;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int row = (int)rq * 4 + k;
        const int64_t i = ti * BT + row;
        if (i < j && j < d) {
            const float* p = part + tile * S * (int64_t)(BT * BT) + row * BT + c;
            double sum = 0.0;
            for (int64_t s = 0; s < S; ++s) sum += (double)p[s * (int64_t)(BT * BT)];
            H[i * d + j] += 2.0 * sum;
        }
    }
}

#ifndef GPTQ_SYRK_WAVES
#define GPTQ_SYRK_WAVES 8
#endif
constexpr int SYRK_WAVES = GPTQ_SYRK_WAVES;

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

// Fewer upper tiles than this: each tile's tokens are split over several
// workgroups (token slices), ceil(512 / tiles) of them.
constexpr int64_t SLICE_TILES = 128;

int64_t tile_count(int64_t d) {
    const int64_t T = align_up((size_t)d, BT) / BT;
    return T * (T + 1) / 2;
}

// Tokens per chunk: every float32 sum covers at most CHUNK tokens (one tile,
// or one token slice of a sliced tile), and the transposed chunk (d_pad x ch
// 16-bit values) stays under XT_MAX_BYTES.
int64_t chunk_tokens(int64_t d) {
    const int64_t d_pad = align_up((size_t)d, BT);
    const int64_t n_tiles = tile_count(d);
    int64_t c = (int64_t)(XT_MAX_BYTES / (2 * (size_t)d_pad)) / KT * KT;
    const int64_t lim = n_tiles < SLICE_TILES ? CHUNK * ceil_div(512, n_tiles) : CHUNK;
    if (c > lim) c = lim;
    if (c < KT) c = KT;
    return c;
}

size_t part_bytes(int64_t d) {
    return align_up((size_t)ceil_div(chunk_tokens(d), TSPAN) * d * sizeof(double), 256);
}

}  // namespace

namespace {
// One chunk's slot of the workspace: column sums, then the transposed chunk.
size_t slot_bytes(int64_t n_tok, int64_t d) {
    const int64_t d_pad = align_up((size_t)d, BT);
    int64_t ch = align_up((size_t)(n_tok > 0 ? n_tok : 1), KT);
    const int64_t cmax = chunk_tokens(d);
    if (ch > cmax) ch = cmax;
    return part_bytes(d) + (size_t)d_pad * ch * sizeof(uint16_t);
}

// Token slices per tile: few tiles (small d) would leave most CUs idle, so
// each tile's chunk is split over S workgroups.
int64_t syrk_slices(int64_t n_tiles, int64_t n_st) {
    if (n_tiles >= SLICE_TILES) return 1;
    int64_t S = ceil_div(512, n_tiles);
    if (S > n_st) S = n_st;
    return S < 1 ? 1 : S;
}

// float32 partial tiles for the largest chunk of this call (zero if unsliced)
size_t slices_bytes(int64_t n_tok, int64_t d) {
    const int64_t T = align_up((size_t)d, BT) / BT, n_tiles = T * (T + 1) / 2;
    int64_t ch = align_up((size_t)(n_tok > 0 ? n_tok : 1), KT);
    if (ch > chunk_tokens(d)) ch = chunk_tokens(d);
    const int64_t S = syrk_slices(n_tiles, ch / KT);
    return S > 1 ? (size_t)n_tiles * S * BT * BT * sizeof(float) : 0;
}
}  // namespace

size_t hessian_workspace_bytes(int64_t n_tok, int64_t d) {
    const int nslots = (n_tok > chunk_tokens(d)) ? 2 : 1;
    return nslots * slot_bytes(n_tok, d) + slices_bytes(n_tok, d);
}

int64_t hessian_syrk_launches(int64_t n_tok, gptq_dtype dt, int64_t d) {
    if (n_tok <= 0) return 0;
    return dt == GPTQ_F32 ? 1 : ceil_div(n_tok, chunk_tokens(d));
}

gptq_status hessian_launch(double* H, const void* X, gptq_dtype dt, int64_t n_tok, int64_t d,
                           int64_t ld_x, void* ws, hipStream_t s, hipEvent_t* ev) {
    if (n_tok == 0) return GPTQ_OK;
    if (dt == GPTQ_F32) {
        const int64_t T = ceil_div(d, FT);
        if (ev) GPTQ_HIP(hipEventRecord(ev[0], s));
        hipLaunchKernelGGL(hess_f32_kernel, dim3((unsigned)(T * (T + 1) / 2)), dim3(256), 0, s, H,
                           (const float*)X, n_tok, d, ld_x);
        GPTQ_LAUNCH_CHECK();
        if (ev) GPTQ_HIP(hipEventRecord(ev[1], s));
        return GPTQ_OK;
    }
    const size_t slot = slot_bytes(n_tok, d);
    float* part = (float*)((char*)ws + ((n_tok > chunk_tokens(d)) ? 2 : 1) * slot);
    const int64_t d_pad = align_up((size_t)d, BT);
    const int64_t T = d_pad / BT;
    const int64_t n_tiles = T * (T + 1) / 2;
    const bool vec = (ld_x % 8 == 0) && (d % 8 == 0) && ((uintptr_t)X % 16 == 0);
    const bool bf = dt == GPTQ_BF16;
    const uint16_t* x = (const uint16_t*)X;
    const void* syrk = bf ? (vec ? (const void*)hess_syrk_kernel<bf16x8_t, SYRK_WAVES, true>
                                 : (const void*)hess_syrk_kernel<bf16x8_t, SYRK_WAVES, false>)
                          : (vec ? (const void*)hess_syrk_kernel<h16x8_t, SYRK_WAVES, true>
                                 : (const void*)hess_syrk_kernel<h16x8_t, SYRK_WAVES, false>);
    GPTQ_HIP(hipFuncSetAttribute(syrk, hipFuncAttributeMaxDynamicSharedMemorySize, RING_BYTES));
    const dim3 b256(256), dgrid((unsigned)ceil_div(d, 256));
    const int64_t cmax = chunk_tokens(d);
    const int64_t npair = (d_pad / 256 + 1) / 2;
    auto slot_part = [&](int64_t ci) { return (double*)((char*)ws + (ci & 1) * slot); };
    auto slot_xt = [&](int64_t ci) { return (uint16_t*)((char*)ws + (ci & 1) * slot + part_bytes(d)); };
    auto chunk_nt = [&](int64_t c0) { return (n_tok - c0 < cmax) ? n_tok - c0 : cmax; };
    // Chunk 0 is transposed on its own; chunk ci+1 by the workgroups past
    // the tiles of chunk ci's product launch, into the other workspace
    // slot.  Each chunk's diagonal sums are added after its transpose, in
    // token order.
    {
        const int64_t nt = chunk_nt(0), ch = align_up((size_t)nt, KT), nblk = ceil_div(ch, TSPAN);
        const dim3 tgrid((unsigned)nblk, (unsigned)(d_pad / 256));
        uint16_t* xt = slot_xt(0);
        double* part = slot_part(0);
        if (bf) {
            if (vec) hipLaunchKernelGGL((transpose_kernel<bf16x8_t, true>), tgrid, b256, 0, s, x, nt, d, ld_x, xt, ch, d_pad, part);
            else hipLaunchKernelGGL((transpose_kernel<bf16x8_t, false>), tgrid, b256, 0, s, x, nt, d, ld_x, xt, ch, d_pad, part);
        } else {
            if (vec) hipLaunchKernelGGL((transpose_kernel<h16x8_t, true>), tgrid, b256, 0, s, x, nt, d, ld_x, xt, ch, d_pad, part);
            else hipLaunchKernelGGL((transpose_kernel<h16x8_t, false>), tgrid, b256, 0, s, x, nt, d, ld_x, xt, ch, d_pad, part);
        }
        GPTQ_LAUNCH_CHECK();
        hipLaunchKernelGGL(diag_add_kernel, dgrid, b256, 0, s, part, nblk, d, H);
        GPTQ_LAUNCH_CHECK();
    }
    for (int64_t c0 = 0, ci = 0; c0 < n_tok; c0 += cmax, ++ci) {
        const int64_t ch = align_up((size_t)chunk_nt(c0), KT);
        NextChunk nx{nullptr, 0, ld_x, 0, nullptr, nullptr};
        int64_t n_tr = 0, nblk_next = 0;
        if (c0 + cmax < n_tok) {
            nx.X = x + (c0 + cmax) * ld_x;
            nx.n_tok = chunk_nt(c0 + cmax);
            nx.ch = align_up((size_t)nx.n_tok, KT);
            nx.Xt = slot_xt(ci + 1);
            nx.colsq = slot_part(ci + 1);
            nblk_next = ceil_div(nx.ch, TSPAN);
            n_tr = nblk_next * npair;
        }
        const int64_t S = syrk_slices(n_tiles, ch / KT);
        const int64_t per_xcd = ceil_div(n_tiles * S, 8);
        const dim3 grid((unsigned)(per_xcd * 8 + n_tr)), block(SYRK_WAVES * 64);
        uint16_t* xt = slot_xt(ci);
        if (ev) GPTQ_HIP(hipEventRecord(ev[2 * ci], s));
        if (bf) {
            if (vec) hipLaunchKernelGGL((hess_syrk_kernel<bf16x8_t, SYRK_WAVES, true>), grid, block, RING_BYTES, s, H, xt, ch, d_pad, d, T, n_tiles, per_xcd, nx, S, part);
            else hipLaunchKernelGGL((hess_syrk_kernel<bf16x8_t, SYRK_WAVES, false>), grid, block, RING_BYTES, s, H, xt, ch, d_pad, d, T, n_tiles, per_xcd, nx, S, part);
        } else {
            if (vec) hipLaunchKernelGGL((hess_syrk_kernel<h16x8_t, SYRK_WAVES, true>), grid, block, RING_BYTES, s, H, xt, ch, d_pad, d, T, n_tiles, per_xcd, nx, S, part);
            else hipLaunchKernelGGL((hess_syrk_kernel<h16x8_t, SYRK_WAVES, false>), grid, block, RING_BYTES, s, H, xt, ch, d_pad, d, T, n_tiles, per_xcd, nx, S, part);
        }
        GPTQ_LAUNCH_CHECK();
        if (S > 1) {
            hipLaunchKernelGGL(syrk_slices_add_kernel, dim3((unsigned)(n_tiles * (BT / 4))), dim3(BT), 0, s, H, part, T,
                               S, d);
            GPTQ_LAUNCH_CHECK();
        }
        if (ev) GPTQ_HIP(hipEventRecord(ev[2 * ci + 1], s));
        if (n_tr > 0) {
            hipLaunchKernelGGL(diag_add_kernel, dgrid, b256, 0, s, slot_part(ci + 1), nblk_next, d, H);
            GPTQ_LAUNCH_CHECK();
        }
    }
    return GPTQ_OK;
}

}  // namespace gptq
