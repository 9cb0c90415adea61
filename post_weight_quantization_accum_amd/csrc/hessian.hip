// Hessian accumulation H += 2 X^T X ("GPTQ量化算法深度解析" §3.1 step 1),
// upper triangle, on the gfx950 matrix cores.
//
// bf16 / fp16 activations.  One workgroup (8 wave64s, two per SIMD) computes
// a 256 x 128 tile of H (rows i0 .. i0+255, columns j0 .. j0+127, j0+127 >=
// i0) over a window of tokens.  Each wave owns 64 x 64 of it as 2 x 2
// v_mfma_f32_32x32x16_{bf16,f16} tiles.
//
// Accuracy: products of bf16/fp16 values are exact in float32, but a float32
// running sum rounds at every MFMA relative to its own size, so long float32
// sums drift.  The MFMA sums run over 256 tokens at a time only (the first
// MFMA of each run starts from zero); each run is then added to float64
// register accumulators, and at the end of the window the tile is added to
// H in float64.  The diagonal is summed separately from exact float64
// squares, so the act-order key diag(H) agrees with a float64 reference to
// rounding order.
//
// Data path: X stays token-major.  Each 64-token stage of the row panel
// (256 features, 512 bytes per token) and the column panel (128 features,
// 256 bytes per token) goes straight from memory into LDS with
// buffer_load ... lds (16 bytes per lane, no VGPR staging); two ring slots
// alternate (one stage in flight while the other is multiplied), and a run
// of 256 tokens covers the ring a whole number of times, so every LDS
// address is a per-lane base plus a constant.  The MFMA operand wants 8 consecutive tokens
// of one feature per lane: ds_read_b64_tr_b16 delivers exactly that from the
// token-major rows (lane i of a 16-lane group receives element i % 4 of the
// 8-byte rows addressed by lanes 4k + i / 4, k = 0..3: four tokens of one
// feature), so no transposed copy of X is ever written.  The 64-byte chunks
// of a token row are XOR-rotated by (token & 3), which spreads the four
// token rows read by one 32-lane half over all LDS banks.
//
// Scheduling: work items are (token window, tile) in window-major order.  A
// launch takes at most n_tiles consecutive items, so no two items of one
// launch touch the same tile and every item adds its window to H directly;
// launches run in stream order, hence every entry of H receives its windows
// in token order (bit-reproducible).  Within a full round of 256 items the
// 32 items that run on one XCD are consecutive tiles of a banded
// enumeration (4 row blocks x ~8 column blocks), which share their panels
// through that XCD's L2.  With fewer than 256 tiles (narrow layers) the
// windows are shorter and every item writes its float64 partial tile to the
// workspace instead; a second kernel adds them to H in window order.
//
// Inputs whose rows are not 16-byte aligned (ld_x or d_in not a multiple of
// 8, or X itself misaligned) are first copied, a bounded number of tokens
// at a time, into an aligned, zero-padded workspace copy.
//
// fp32 activations take a float64 path (products of fp32 values are exact
// in float64): a plain tiled float64 kernel.
#include "internal.hpp"

namespace gptq {
namespace {

constexpr int TR = 256;                        // tile rows (row-panel features)
constexpr int TC = 128;                        // tile columns (column-panel features)
#ifndef GPTQ_HKT
#define GPTQ_HKT 64
#endif
#ifndef GPTQ_HNSTAGE
#define GPTQ_HNSTAGE 2
#endif
constexpr int KT = GPTQ_HKT;                   // tokens per LDS stage
constexpr int NSTAGE = GPTQ_HNSTAGE;           // LDS ring depth
constexpr int KSTEPS = KT / 16;                // MFMA k-steps per stage
constexpr int WROWS = KT / 8;                  // token rows each wave loads per stage
constexpr int ROW_B = TR * 2;                  // bytes of one token of the row panel
constexpr int COL_B = TC * 2;                  // bytes of one token of the column panel
constexpr int STAGE_B = KT * (ROW_B + COL_B);  // 48 KiB
constexpr int RING_B = NSTAGE * STAGE_B;       // 96 KiB
constexpr int SQ_B = 4 * TR * 8;               // float64 sums of squares (4 token groups x 256 features)
constexpr int LDS_B = RING_B + SQ_B;
#ifndef GPTQ_HFOLD
#define GPTQ_HFOLD (256 / GPTQ_HKT)
#endif
constexpr int FOLD = GPTQ_HFOLD;               // stages per float32 run
constexpr int RUN_TOK = FOLD * KT;             // tokens per float32 run
constexpr int DMA_PER_STAGE = WROWS / 2 + WROWS / 4;   // buffer_load ... lds per wave per stage
static_assert(KT == 32 || KT == 64, "stage of 32 or 64 tokens");
static_assert(LDS_B <= 160 * 1024, "LDS of one CU");
// the ring slot of a stage is a compile-time constant in the unrolled run
constexpr bool SLOT_STATIC = FOLD % NSTAGE == 0;
constexpr int BAND = 4;                        // row blocks per band of the tile enumeration
#ifndef GPTQ_HWIN
#define GPTQ_HWIN 32768
#endif
constexpr int64_t WIN_MAX = GPTQ_HWIN / RUN_TOK * RUN_TOK;   // tokens per window (full mode)
constexpr int64_t PART_TILES = 256;            // fewer tiles: partial-tile mode
constexpr int64_t ROUND = 256;                 // work items that run at once (one workgroup per CU)
constexpr size_t PART_ELEMS = (size_t)TR * TC + TR;   // one partial tile + its diagonal sums
constexpr size_t REPACK_BYTES = (size_t)64 << 20;     // aligned copy of a misaligned input

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t* lds_v4_t;

struct Grid {
    int64_t RB, CB, n_tiles;
};

__host__ __device__ inline Grid tile_grid(int64_t d) {
    Grid g;
    g.RB = ceil_div(d, TR);
    g.CB = ceil_div(d, TC);
    g.n_tiles = g.RB * g.CB - g.RB * (g.RB - 1);   // row block a has column blocks 2a .. CB-1
    return g;
}

// Tile k of the banded enumeration: bands of BAND row blocks; inside a band,
// column blocks in order and, per column, the band's rows a with b >= 2a.
__device__ inline void tile_of(int64_t k, int64_t RB, int64_t CB, int64_t& a, int64_t& b) {
    for (int64_t r0 = 0; r0 < RB; r0 += BAND) {
        const int64_t r1 = (r0 + BAND < RB) ? r0 + BAND : RB;
        const int64_t m = (CB < 2 * r1) ? CB : 2 * r1;
        const int64_t n1 = m - 2 * r0;   // columns whose rows are cut by the diagonal
        const int64_t c1 = (n1 % 2 == 0) ? (n1 / 2) * (n1 / 2 + 1) : ((n1 + 1) / 2) * ((n1 + 1) / 2);
        const int64_t cnt = c1 + (CB - m) * (r1 - r0);
        if (k < cnt) {
            for (int64_t bb = 2 * r0;; ++bb) {
                const int64_t top = (bb / 2 < r1 - 1) ? bb / 2 : r1 - 1;
                const int64_t c = top - r0 + 1;
                if (k < c) {
                    a = r0 + k;
                    b = bb;
                    return;
                }
                k -= c;
            }
        }
        k -= cnt;
    }
    a = b = 0;   // unreachable for k < n_tiles
}

template <typename Tag>
__device__ __forceinline__ double elem_f64(uint32_t bits16);
template <>
__device__ __forceinline__ double elem_f64<bf16x8_t>(uint32_t b) { return (double)__uint_as_float(b << 16); }
template <>
__device__ __forceinline__ double elem_f64<h16x8_t>(uint32_t b) {
    return (double)(float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

__device__ __forceinline__ uint64_t tr_read(const char* p) {
    const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_t)(p));
    return __builtin_bit_cast(uint64_t, v);
}
__device__ __forceinline__ u32x4_t pair(uint64_t lo, uint64_t hi) {
    u32x4_t r;
    r.x = (uint32_t)lo;
    r.y = (uint32_t)(lo >> 32);
    r.z = (uint32_t)hi;
    r.w = (uint32_t)(hi >> 32);
    return r;
}

// One wave-wide buffer_load_dwordx4 ... lds: lane l's 16 bytes at buffer
// offset voff land at LDS address lds_addr + 16 l.  Written as inline asm so
// that the compiler does not order every later LDS read behind it (it cannot
// tell which LDS bytes the load writes, and would wait for it before each
// read); the kernel waits for these loads itself (s_waitcnt vmcnt before the
// barrier that publishes a stage).  No register receives data, so nothing is
// left in flight in a register the compiler could reuse.
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, u32x4_t rs) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rs)
                 : "memory");
}

struct HessArgs {
    double* H;          // d x d, upper triangle
    const uint16_t* X;  // token-major, row stride ld (elements), 16-byte aligned rows
    int64_t ld, d, n_tok;
    int64_t win;        // tokens per window (multiple of RUN_TOK)
    int64_t RB, CB, n_tiles;
    int64_t item0, n_items;   // this launch: items item0 .. item0 + n_items - 1
    double* part;       // partial mode: PART_ELEMS doubles per item (indexed by global item); else null
};

template <typename Tag>
__global__ __launch_bounds__(512) void hess_tile_kernel(HessArgs A) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform: scalar branches below
    const int wr = wave >> 1, wc = wave & 1;

    // item of this workgroup: inside a full round of 256, the 32 workgroups
    // of one XCD (b % 8) take 32 consecutive items
    const int64_t bq = blockIdx.x;
    int64_t q = bq;
    if ((bq / 256 + 1) * 256 <= A.n_items) q = (bq / 256) * 256 + (bq % 8) * 32 + (bq % 256) / 8;
    const int64_t item = A.item0 + q;
    const int64_t w = item / A.n_tiles;
    int64_t a, b;
    tile_of(item % A.n_tiles, A.RB, A.CB, a, b);
    const int64_t i0 = a * TR, j0 = b * TC;
    const int64_t t0 = w * A.win;
    const int64_t nt = (A.n_tok - t0 < A.win) ? A.n_tok - t0 : A.win;
    const int n_st = (int)(ceil_div(nt, RUN_TOK) * FOLD);
    // the diagonal tile of the row block: its lower half (waves wr >= 2) lies
    // under the diagonal; those waves sum exact squares instead
    const bool diag_item = (b == 2 * a);
    const bool sq_wave = diag_item && wr >= 2;

    // one buffer resource over the window: tokens past its end and the
    // features past d of its last token read as zero.  The range check works
    // on whole dwords, so the range ends on the last token's last 16-byte
    // granule (d is a multiple of 8, or the rows are a zero-padded aligned
    // copy that holds that granule).
    const uint32_t nrec = (uint32_t)(((nt - 1) * A.ld + ceil_div(A.d, 8) * 8) * 2);
    const uint64_t xbase = (uint64_t)(uintptr_t)(A.X + t0 * A.ld);
    u32x4_t rs;   // raw buffer: base, stride 0, num_records, default format
    rs.x = __builtin_amdgcn_readfirstlane((uint32_t)xbase);
    rs.y = __builtin_amdgcn_readfirstlane((uint32_t)(xbase >> 32) & 0xFFFFu);
    rs.z = __builtin_amdgcn_readfirstlane(nrec);
    rs.w = 0x00020000u;
    const uint32_t ldb = (uint32_t)A.ld * 2;

    // DMA of stage st into ring slot sl: wave w loads token rows WROWS*w ..
    // +WROWS-1 of both panels (row panel: 2 rows per load, column panel: 4).
    // Lane l fills LDS granule slot s of its row, which holds feature
    // granule s ^ (4 * (row & 3)).
    // The per-lane part of each load's offset is the same for every stage; the
    // stage's part is a wave-uniform value made opaque to the compiler, so the
    // offsets of the unrolled stages are not all kept in registers.  (The whole
    // offset stays in the vector offset: the buffer's range check, which reads
    // tokens past the window as zeros, does not see the scalar offset.)
    uint32_t vrow[WROWS / 2], vcol[WROWS / 4];
#pragma unroll
    for (int u = 0; u < WROWS / 2; ++u) {
        const int r = WROWS * wave + 2 * u + (lane >> 5);
        const int g = (lane & 31) ^ ((r & 3) << 2);
        vrow[u] = (uint32_t)r * ldb + (uint32_t)(i0 + 8 * g) * 2;
    }
#pragma unroll
    for (int u = 0; u < WROWS / 4; ++u) {
        const int r = WROWS * wave + 4 * u + (lane >> 4);
        const int g = (lane & 15) ^ ((r & 3) << 2);
        vcol[u] = (uint32_t)r * ldb + (uint32_t)(j0 + 8 * g) * 2;
    }
    auto issue = [&](int st, int sl) {
        const uint32_t sb = (uint32_t)(uintptr_t)(lds + sl * STAGE_B);
        const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)st * KT * ldb);
#pragma unroll
        for (int u = 0; u < WROWS / 2; ++u) dma16(sb + (WROWS * wave + 2 * u) * ROW_B, vrow[u] + so, rs);
#pragma unroll
        for (int u = 0; u < WROWS / 4; ++u) dma16(sb + KT * ROW_B + (WROWS * wave + 4 * u) * COL_B, vcol[u] + so, rs);
    };

    // Operand addressing for ds_read_b64_tr_b16.  Lane (G = lane/16, p =
    // lane%16, k4 = p/4, q4 = p%4) points at token 8*(G/2) + 4h + k4 of the
    // k-step and feature 16*(G%2) + 4*q4 of the 32-feature block; its row's
    // chunk rotation is k4 (k-step bases are multiples of 4).
    const int G = lane >> 4, k4 = (lane >> 2) & 3, q4 = lane & 3;
    const int lrow = 8 * (G >> 1) + k4;
    const int lgr = 2 * (G & 1) + (q4 >> 1);         // granule within the 64-byte chunk
    const int lhalf = 8 * (q4 & 1);
    int offA[2], offB[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        offA[i] = lrow * ROW_B + 16 * (4 * ((2 * wr + i) ^ k4) + lgr) + lhalf;
        offB[i] = KT * ROW_B + lrow * COL_B + 16 * (4 * ((2 * wc + i) ^ k4) + lgr) + lhalf;
    }
    auto read_ops = [&](u32x4_t (&av)[2], u32x4_t (&bv)[2], int sl, int ks) {
        const char* sb = lds + sl * STAGE_B;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const char* pa = sb + offA[i] + 16 * ks * ROW_B;
            av[i] = pair(tr_read(pa), tr_read(pa + 4 * ROW_B));
            const char* pb = sb + offB[i] + 16 * ks * COL_B;
            bv[i] = pair(tr_read(pb), tr_read(pb + 4 * COL_B));
        }
    };

    // exact squares (sq waves): thread u = 0..255 sums features 4*(u%64) ..
    // +3 of the row panel over the token quarter u/64 of each stage into its
    // own four float64 slots past the ring
    const int usq = t - 256;
    const int sfg = usq & 63, stg = usq >> 6;
    double* sqs = (double*)(lds + RING_B) + stg * TR + 4 * sfg;
    if (sq_wave) {
#pragma unroll
        for (int c = 0; c < 4; ++c) sqs[c] = 0.0;
    }
    auto squares = [&](int sl) {
        const char* sb = lds + sl * STAGE_B;
        double sq[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
        for (int r = 0; r < KT / 4; ++r) {
            const int row = (KT / 4) * stg + r;
            const uint64_t v = *(const uint64_t*)(sb + row * ROW_B + 16 * ((sfg >> 1) ^ ((row & 3) << 2)) +
                                                  8 * (sfg & 1));
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const double x = elem_f64<Tag>((uint32_t)(v >> (16 * c)) & 0xFFFFu);
                sq[c] = fma(x, x, sq[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) sqs[c] += sq[c];
    };

    f16_t acc[2][2];
    double acc64[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[i][j][r] = 0.0f;
                acc64[i][j][r] = 0.0;
            }
    const f16_t zero = {};

    // prologue: all ring slots in flight, stage 0 visible to every wave
#pragma unroll
    for (int s = 0; s < NSTAGE; ++s)
        if (s < n_st) issue(s, s);
    if (n_st >= NSTAGE) wait_vmcnt<DMA_PER_STAGE * (NSTAGE - 1)>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();

    if (sq_wave) {
        // the same barriers and refills as the MFMA loop below, one per stage
        for (int st = 0; st < n_st; ++st) {
            squares(st % NSTAGE);
            if (st + 1 < n_st) {
                wait_lgkm0();
                if (st + NSTAGE - 1 < n_st) wait_vmcnt<DMA_PER_STAGE * (NSTAGE - 2)>();
                else wait_vmcnt<0>();
                __builtin_amdgcn_s_barrier();
                if (st + NSTAGE < n_st) issue(st + NSTAGE, st % NSTAGE);
            }
        }
    } else {
        u32x4_t a0[2], b0[2], a1[2], b1[2];
        read_ops(a0, b0, 0, 0);
        // Runs of FOLD stages (256 tokens); inside a stage, KSTEPS k-steps of
        // 16 tokens whose operands are read one k-step ahead, also across the
        // stage barrier (the next stage's first operands are read right after
        // it).
        for (int st0 = 0; st0 < n_st; st0 += FOLD) {
#pragma unroll
            for (int s4 = 0; s4 < FOLD; ++s4) {
                const int st = st0 + s4;
                const int sl = SLOT_STATIC ? s4 % NSTAGE : st % NSTAGE;
                const int sl_next = SLOT_STATIC ? (s4 + 1) % NSTAGE : (st + 1) % NSTAGE;
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    const bool odd = ((s4 * KSTEPS + ks) & 1) != 0;
                    u32x4_t (&ac)[2] = odd ? a1 : a0;
                    u32x4_t (&bc)[2] = odd ? b1 : b0;
                    u32x4_t (&an)[2] = odd ? a0 : a1;
                    u32x4_t (&bn)[2] = odd ? b0 : b1;
                    if (ks + 1 < KSTEPS) read_ops(an, bn, sl, ks + 1);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i][j] = mfma_32x32x16(ac[i], bc[j], (s4 == 0 && ks == 0) ? zero : acc[i][j],
                                                      (Tag*)nullptr);
                    if (ks + 1 == KSTEPS && st + 1 < n_st) {
                        // The stage's last MFMAs are queued before the barrier, so
                        // the matrix pipe keeps working while the wave waits:
                        // this wave's reads of stage st are complete, stage st+1
                        // has landed everywhere after the barrier.
                        wait_lgkm0();
                        if (st + NSTAGE - 1 < n_st) wait_vmcnt<DMA_PER_STAGE * (NSTAGE - 2)>();
                        else wait_vmcnt<0>();
                        __builtin_amdgcn_s_barrier();
                        // the slot of stage st is free: stage st + NSTAGE goes there
                        if (st + NSTAGE < n_st) issue(st + NSTAGE, sl);
                        read_ops(an, bn, sl_next, 0);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc64[i][j][r] += (double)acc[i][j][r];
        }
    }

    // epilogue: lane l holds C[8*(r/4) + 4*(l/32) + r%4][l%32] of each 32x32 tile
    double* part = A.part ? A.part + (size_t)item * PART_ELEMS : nullptr;
    if (!sq_wave) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = 64 * wc + 32 * j + (lane & 31);
                if (part) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = 64 * wr + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        part[row * TC + col] = 2.0 * acc64[i][j][r];
                    }
                } else {
                    // the 16 values of one MFMA tile: all loads in flight
                    // together (entries outside the strict upper triangle read
                    // a valid neighbour and are not written back)
                    const int64_t gj = j0 + col;
                    int64_t idx[16];
                    bool ok[16];
                    double h[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t gi = i0 + 64 * wr + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        ok[r] = gi < gj && gj < A.d;
                        idx[r] = ok[r] ? gi * A.d + gj : 0;
                        h[r] = A.H[idx[r]];
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (ok[r]) A.H[idx[r]] = h[r] + 2.0 * acc64[i][j][r];
                }
            }
    }
    if (diag_item) {
        // the four token groups' sums, in a fixed order
        __syncthreads();
        if (t < TR) {
            const double* red = (const double*)(lds + RING_B);
            const double s = ((red[t] + red[TR + t]) + red[2 * TR + t]) + red[3 * TR + t];
            if (part) part[TR * TC + t] = 2.0 * s;
            else if (i0 + t < A.d) A.H[(i0 + t) * A.d + i0 + t] += 2.0 * s;
        }
    }
}

// H += the partial tiles of every window, in window order (partial mode).
// One workgroup per 4 rows of a tile; thread c takes column c (and, on the
// diagonal tile of a row block, the diagonal sum of feature 4*blk + k).
__global__ __launch_bounds__(TC) void part_add_kernel(double* __restrict__ H, const double* __restrict__ part,
                                                      int64_t d, int64_t RB, int64_t CB, int64_t n_tiles,
                                                      int64_t n_win) {
    const int64_t tile = blockIdx.x / (TR / 4), rq = blockIdx.x % (TR / 4);
    int64_t a, b;
    tile_of(tile, RB, CB, a, b);
    const int c = threadIdx.x;
    const int64_t gj = b * TC + c;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int row = (int)rq * 4 + k;
        const int64_t gi = a * TR + row;
        if (gi < gj && gj < d) {
            double s = 0.0;
            for (int64_t w = 0; w < n_win; ++w) s += part[(size_t)(w * n_tiles + tile) * PART_ELEMS + row * TC + c];
            H[gi * d + gj] += s;
        }
    }
    if (b == 2 * a && c < 4) {
        const int row = (int)rq * 4 + c;
        const int64_t gi = a * TR + row;
        if (gi < d) {
            double s = 0.0;
            for (int64_t w = 0; w < n_win; ++w) s += part[(size_t)(w * n_tiles + tile) * PART_ELEMS + TR * TC + row];
            H[gi * d + gi] += s;
        }
    }
}

// Aligned copy of a misaligned input: dst[t][f] = src[t][f] for f < d, zero
// for d <= f < ldd (grid-stride over the n_tok x ldd destination).
__global__ __launch_bounds__(256) void repack_kernel(const uint16_t* __restrict__ src, int64_t ld, int64_t d,
                                                     int64_t n_tok, uint16_t* __restrict__ dst, int64_t ldd) {
    const int64_t total = n_tok * ldd;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t tok = e / ldd, f = e % ldd;
        dst[e] = f < d ? src[tok * ld + f] : (uint16_t)0;
    }
}

// fp32 activations: float64 products and sums.  64x64 tiles of the upper
// triangle, 256 threads, each thread a 4x4 block, 32 tokens per stage; the
// next stage's loads are in flight while the current one is multiplied
// (each thread's elements of a stage go through registers), so a stage
// costs its arithmetic rather than a memory round trip.
constexpr int FT = 64, FK = 32;
constexpr int FE = FK * FT / 256;   // elements of one operand per thread and stage

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
    // element q of this thread in a stage: token row k = e / FT, column c = e % FT
    auto load = [&](int64_t t0, float (&va)[FE], float (&vb)[FE]) {
#pragma unroll
        for (int q = 0; q < FE; ++q) {
            const int e = t + 256 * q;
            const int k = e / FT, c = e % FT;
            const int64_t tok = t0 + k;
            const int64_t ca = ti * FT + c, cb = tj * FT + c;
            const bool tok_ok = tok < n_tok;
            va[q] = (tok_ok && ca < d) ? X[tok * ld + ca] : 0.0f;
            vb[q] = (tok_ok && cb < d) ? X[tok * ld + cb] : 0.0f;
        }
    };
    double acc[4][4] = {};
    float va[FE], vb[FE];
    load(0, va, vb);
    for (int64_t t0 = 0; t0 < n_tok; t0 += FK) {
#pragma unroll
        for (int q = 0; q < FE; ++q) {
            const int e = t + 256 * q;
            sA[e / FT][e % FT] = (double)va[q];
            sB[e / FT][e % FT] = (double)vb[q];
        }
        __syncthreads();
        if (t0 + FK < n_tok) load(t0 + FK, va, vb);
#pragma unroll
        for (int k = 0; k < FK; ++k) {
            double av[4], bv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                av[u] = sA[k][ty * 4 + u];
                bv[u] = sB[k][tx * 4 + u];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[u][v] = fma(av[u], bv[v], acc[u][v]);
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

// ---------------------------------------------------------------------------
// Host-side planning
// ---------------------------------------------------------------------------

// Workspace budget of one call: at most max_items partial tiles (0: as many
// as the plan wants) and an aligned copy of at most `repack` bytes.
struct Budget {
    int64_t max_items;
    size_t repack;
};
constexpr Budget DEFAULT_BUDGET{0, REPACK_BYTES};

// Work plan of one pass.  Full mode: windows of WIN_MAX tokens; partial
// mode: windows short enough for about 512 items (fewer if the budget
// holds fewer partial tiles; with room for less than one window of them the
// pass runs in full mode, one window of tiles per launch).  win_cap bounds a
// window so that its byte offsets fit in 31 bits.
struct Plan {
    Grid g;
    bool partial;
    int64_t win, n_win, n_items, per_launch;
};

int64_t window_cap(int64_t ld) {
    const int64_t cap = ((int64_t(1) << 31) / (2 * ld)) / RUN_TOK * RUN_TOK;
    return cap < RUN_TOK ? RUN_TOK : cap;
}

Plan make_plan(int64_t n_tok, int64_t d, int64_t win_cap, int64_t max_items) {
    Plan p;
    p.g = tile_grid(d);
    p.partial = p.g.n_tiles < PART_TILES && (max_items == 0 || max_items >= p.g.n_tiles);
    int64_t win = WIN_MAX;
    if (p.partial) {
        // at most about 512 items (and no more than the runs or the
        // budget allow); among those window counts, the one whose rounds
        // of ROUND items (one workgroup per CU) cost least: the time goes
        // as ceil(nw T / ROUND) rounds of n_tok / nw tokens each
        const int64_t T = p.g.n_tiles;
        int64_t nw_max = ceil_div(512, T);
        const int64_t runs = ceil_div(n_tok, RUN_TOK);
        if (nw_max > runs) nw_max = runs;
        if (max_items > 0 && nw_max > max_items / T) nw_max = max_items / T;
        if (nw_max < 1) nw_max = 1;
        int64_t nw = 1;
        for (int64_t c = 2; c <= nw_max; ++c)
            if (ceil_div(c * T, ROUND) * nw < ceil_div(nw * T, ROUND) * c) nw = c;   // cost(c) < cost(nw)
        win = ceil_div(ceil_div(n_tok, nw), RUN_TOK) * RUN_TOK;
    }
    if (win > win_cap) win = win_cap;
    p.win = win;
    p.n_win = ceil_div(n_tok, win);
    p.n_items = p.n_win * p.g.n_tiles;
    if (p.partial) p.per_launch = p.n_items;
    else p.per_launch = p.g.n_tiles >= 256 ? (p.g.n_tiles / 256) * 256 : p.g.n_tiles;
    return p;
}

constexpr int64_t NO_CAP = int64_t(1) << 62;

size_t part_bytes(int64_t n_tok, int64_t d, const Budget& b) {
    const Plan p = make_plan(n_tok, d, NO_CAP, b.max_items);
    return p.partial ? (size_t)p.n_items * PART_ELEMS * sizeof(double) : 0;
}

// Rows are 16-byte aligned and short enough for 32-bit window offsets.
bool aligned_input(const void* X, int64_t d, int64_t ld) {
    return (ld % 8 == 0) && (d % 8 == 0) && ((uintptr_t)X % 16 == 0) && ld <= (int64_t(1) << 21);
}

int64_t repack_tokens(int64_t d, const Budget& b) {
    const int64_t ldd = ceil_div(d, 8) * 8;
    int64_t t = (int64_t)(b.repack / (2 * (size_t)ldd)) / RUN_TOK * RUN_TOK;
    return t < RUN_TOK ? RUN_TOK : t;
}

size_t repack_bytes(int64_t n_tok, int64_t d, const Budget& b) {
    const int64_t ldd = ceil_div(d, 8) * 8;
    int64_t nt = repack_tokens(d, b);
    if (nt > n_tok) nt = n_tok;
    return align_up((size_t)nt * ldd * 2, 256);
}

// Token chunks of one aligned call: one chunk, unless the window cap forces
// partial-mode windows shorter than planned (then chunks of as many capped
// windows as the workspace holds).
int64_t aligned_chunk(int64_t n_tok, int64_t d, int64_t ld, const Budget& b) {
    const Plan p0 = make_plan(n_tok, d, NO_CAP, b.max_items);
    const int64_t cap = window_cap(ld);
    return (p0.partial && p0.win > cap) ? p0.n_win * cap : n_tok;
}

int64_t launches_aligned(int64_t n_tok, int64_t d, int64_t ld, const Budget& b) {
    int64_t n = 0;
    const int64_t chunk = aligned_chunk(n_tok, d, ld, b);
    for (int64_t c0 = 0; c0 < n_tok; c0 += chunk) {
        const Plan p = make_plan((n_tok - c0 < chunk) ? n_tok - c0 : chunk, d, window_cap(ld), b.max_items);
        n += ceil_div(p.n_items, p.per_launch);
    }
    return n;
}

// H += 2 X^T X for 16-byte aligned rows (ld and d multiples of 8).
template <typename Tag>
gptq_status hess_aligned(double* H, const uint16_t* X, int64_t n_tok, int64_t d, int64_t ld, double* part,
                         const Budget& bud, hipStream_t s, hipEvent_t* ev, int64_t& ev_i) {
    if (n_tok <= 0) return GPTQ_OK;
    GPTQ_HIP(ensure_lds_limit((const void*)hess_tile_kernel<Tag>, (int)LDS_B));
    const int64_t chunk = aligned_chunk(n_tok, d, ld, bud);
    for (int64_t c0 = 0; c0 < n_tok; c0 += chunk) {
        const int64_t nt = (n_tok - c0 < chunk) ? n_tok - c0 : chunk;
        const Plan p = make_plan(nt, d, window_cap(ld), bud.max_items);
        HessArgs A{H, X + c0 * ld, ld, d, nt, p.win, p.g.RB, p.g.CB, p.g.n_tiles, 0, 0, p.partial ? part : nullptr};
        for (int64_t i0 = 0; i0 < p.n_items; i0 += p.per_launch) {
            A.item0 = i0;
            A.n_items = (p.n_items - i0 < p.per_launch) ? p.n_items - i0 : p.per_launch;
            if (ev) GPTQ_HIP(hipEventRecord(ev[2 * ev_i], s));
            hipLaunchKernelGGL(hess_tile_kernel<Tag>, dim3((unsigned)A.n_items), dim3(512), LDS_B, s, A);
            GPTQ_LAUNCH_CHECK();
            if (ev) GPTQ_HIP(hipEventRecord(ev[2 * ev_i + 1], s));
            ++ev_i;
        }
        if (p.partial) {
            hipLaunchKernelGGL(part_add_kernel, dim3((unsigned)(p.g.n_tiles * (TR / 4))), dim3(TC), 0, s, H, part, d,
                               p.g.RB, p.g.CB, p.g.n_tiles, p.n_win);
            GPTQ_LAUNCH_CHECK();
        }
    }
    return GPTQ_OK;
}

int64_t launches(int64_t n_tok, gptq_dtype dt, int64_t d, int64_t ld_x, const void* X, const Budget& b) {
    if (n_tok <= 0) return 0;
    if (dt == GPTQ_F32) return 1;
    if (aligned_input(X, d, ld_x)) return launches_aligned(n_tok, d, ld_x, b);
    const int64_t ldd = ceil_div(d, 8) * 8, rt = repack_tokens(d, b);
    int64_t n = 0;
    for (int64_t c0 = 0; c0 < n_tok; c0 += rt) n += launches_aligned((n_tok - c0 < rt) ? n_tok - c0 : rt, d, ldd, b);
    return n;
}

gptq_status launch_with_budget(double* H, const void* X, gptq_dtype dt, int64_t n_tok, int64_t d, int64_t ld_x,
                               void* ws, const Budget& bud, hipStream_t s, hipEvent_t* ev) {
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
    const bool bf = dt == GPTQ_BF16;
    int64_t ev_i = 0;
    if (aligned_input(X, d, ld_x)) {
        double* part = (double*)ws;
        return bf ? hess_aligned<bf16x8_t>(H, (const uint16_t*)X, n_tok, d, ld_x, part, bud, s, ev, ev_i)
                  : hess_aligned<h16x8_t>(H, (const uint16_t*)X, n_tok, d, ld_x, part, bud, s, ev, ev_i);
    }
    // misaligned rows: chunks copied into an aligned, zero-padded buffer
    const int64_t ldd = ceil_div(d, 8) * 8, rt = repack_tokens(d, bud);
    uint16_t* xr = (uint16_t*)ws;
    double* part = (double*)((char*)ws + repack_bytes(n_tok, d, bud));
    for (int64_t c0 = 0; c0 < n_tok; c0 += rt) {
        const int64_t nt = (n_tok - c0 < rt) ? n_tok - c0 : rt;
        const int64_t nblk = ceil_div(nt * ldd, 256);
        hipLaunchKernelGGL(repack_kernel, dim3((unsigned)(nblk < 8192 ? nblk : 8192)), dim3(256), 0, s,
                           (const uint16_t*)X + c0 * ld_x, ld_x, d, nt, xr, ldd);
        GPTQ_LAUNCH_CHECK();
        gptq_status st = bf ? hess_aligned<bf16x8_t>(H, xr, nt, d, ldd, part, bud, s, ev, ev_i)
                            : hess_aligned<h16x8_t>(H, xr, nt, d, ldd, part, bud, s, ev, ev_i);
        if (st != GPTQ_OK) return st;
    }
    return GPTQ_OK;
}

}  // namespace

size_t hessian_workspace_bytes(int64_t n_tok, int64_t d) {
    if (n_tok <= 0) return 0;
    // aligned inputs: the partial tiles of the call; misaligned ones: the
    // aligned copy of one token chunk plus that chunk's partial tiles (the
    // query does not know the alignment of X, so it covers both)
    const Budget& b = DEFAULT_BUDGET;
    const size_t a = part_bytes(n_tok, d, b);
    const int64_t nr = repack_tokens(d, b) < n_tok ? repack_tokens(d, b) : n_tok;
    const size_t r = repack_bytes(n_tok, d, b) + part_bytes(nr, d, b);
    return align_up((a > r ? a : r) + 256, 256);
}

int64_t hessian_syrk_launches(int64_t n_tok, gptq_dtype dt, int64_t d, int64_t ld_x, const void* X) {
    return launches(n_tok, dt, d, ld_x, X, DEFAULT_BUDGET);
}

gptq_status hessian_launch(double* H, const void* X, gptq_dtype dt, int64_t n_tok, int64_t d,
                           int64_t ld_x, void* ws, hipStream_t s, hipEvent_t* ev) {
    return launch_with_budget(H, X, dt, n_tok, d, ld_x, ws, DEFAULT_BUDGET, s, ev);
}

gptq_status hessian_launch_scratch(double* H, const void* X, gptq_dtype dt, int64_t n_tok, int64_t d,
                                   int64_t ld_x, void* scratch, size_t scratch_bytes, hipStream_t s) {
    if (n_tok == 0 || dt == GPTQ_F32) return launch_with_budget(H, X, dt, n_tok, d, ld_x, nullptr, DEFAULT_BUDGET, s,
                                                                nullptr);
    // split the scratch: an aligned copy of a token chunk (misaligned rows
    // only; a chunk of at least one 256-token run must fit), then as many
    // partial tiles as the rest holds
    Budget b{0, 0};
    size_t rest = scratch_bytes;
    if (!aligned_input(X, d, ld_x)) {
        b.repack = scratch_bytes / 4;
        const int64_t ldd = ceil_div(d, 8) * 8;
        if ((size_t)RUN_TOK * ldd * 2 > b.repack) return GPTQ_ERR_WORKSPACE;
        rest -= repack_bytes(n_tok, d, b);
    }
    b.max_items = (int64_t)(rest / (PART_ELEMS * sizeof(double)));
    if (b.max_items < 1) b.max_items = 1;   // below one window of tiles the pass uses no partial tiles
    return launch_with_budget(H, X, dt, n_tok, d, ld_x, scratch, b, s, nullptr);
}

}  // namespace gptq
