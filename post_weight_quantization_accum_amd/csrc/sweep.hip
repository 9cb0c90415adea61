// Blocked column sweep with error compensation and lazy block updates
// ("GPTQ量化算法深度解析" §2.2 compensation, §2.4 fixed order and lazy batch
// updates, §3.1 step 3 blocks of 128 columns; grid per "通义千问...GPTQ-Int4"
// §2.1-2.2), all in float64.
//
// Data layout in HBM (workspace):
//   Wwork  d_out x d_in float64, columns in sweep order (the running W)
//   Err    2 x d_out x S float64, scaled errors of the current superblock (ping-pong)
//   codes_s d_out x d_in uint8, codes in sweep order
//   scale64 / zero64  n_groups x d_out float64
//   row_loss64 d_out float64, pinv d_in int32, flags
//
// sweep_block: sixteen lanes per row (one DPP row), lane p holding block
// columns p, p + 16, ..., p + 112 of that row in registers; 4 rows per wave,
// 16 rows per workgroup.  The upper triangle of the block's U (73 KiB: row c
// from column 16 floor(c / 16) on) is staged in LDS once per workgroup, so
// the serial column loop reads U rows at LDS latency; one such workgroup
// fits on a CU beside a float64 GEMM workgroup of another stream.  Column c
// is quantized by the lane owning it; its scaled error reaches the other
// lanes of the row by a DPP row broadcast, and every lane then applies
// w_j -= err * U[c][j] to its registers from c / 16 on (the earlier ones
// hold finished columns only), so each w_j receives the compensations of
// the earlier columns one by one, in column order.  A finished column keeps
// its error in place: the later updates leave it unchanged because U is zero
// below the diagonal.  The column loop is unrolled, so register indices and
// the broadcast lane are constants.
//
// Lazy updates are two-level (mathematically the same as one update per
// block): after each block, a float64 MFMA GEMM updates the rest of its
// superblock of S = 1024 columns (K = B); after each superblock, one GEMM
// with K = S updates the next superblock, and another (on a second stream,
// overlapping the next superblock's sweep) everything after it.
//
// Static groups: every group's (scale, zero) comes first, from W as given,
// per group of consecutive original columns (one wave per row and group);
// the sweep kernel then holds, per lane, the parameters of the columns it
// owns (loaded once per block through the group of each sweep column) and
// takes none during the sweep.
#include <utility>

#include "internal.hpp"

namespace gptq {
namespace {

constexpr int BMAX = 128;   // largest supported block (columns per lazy update)
constexpr int LPR = 16;     // lanes per row: one DPP row of 16 lanes
constexpr int CPL = BMAX / LPR;  // columns per lane: lane p holds block columns p, p + 16, ..., p + 112
constexpr int SWAVES = 4;        // waves per workgroup
constexpr int ROWS = SWAVES * 64 / LPR;   // rows per workgroup
// U block in LDS: row c = 16 m + j keeps its columns 16 m .. 127 (the
// columns whose lane register a later update still touches; the ones below
// the diagonal are U's zeros), so lane p finds U[c][16 m' + p] (m' >= m) at
// 16 (m' - m) + p of the row; then the reciprocal diagonal.
__host__ __device__ constexpr int seg_len(int m) { return BMAX - LPR * m; }
__host__ __device__ constexpr int seg_base(int m) { return LPR * (BMAX * m - 8 * m * (m - 1)); }
constexpr int UP_DOUBLES = seg_base(CPL);   // 9216
constexpr size_t SWEEP_LDS = (size_t)(UP_DOUBLES + BMAX) * sizeof(double);   // 73 KiB
static_assert(seg_base(1) == LPR * seg_len(0), "row segments of the first register group");
// double pairs staged per thread for register group m, and their running index
__host__ __device__ constexpr int stage_iters(int m) { return (LPR * seg_len(m) / 2 + SWAVES * 64 - 1) / (SWAVES * 64); }
__host__ __device__ constexpr int stage_first(int m) { return m == 0 ? 0 : stage_first(m - 1) + stage_iters(m - 1); }
__host__ __device__ constexpr int stage_group(int k) {   // register group of staged pair slot k
    int m = 0;
    while (m + 1 < CPL && stage_first(m + 1) <= k) ++m;
    return m;
}

struct SweepWs {
    int* flags;
    double* Wwork;
    double* Err;
    double* W0;   // factored form: the weights before the sweep (sweep order)
    uint8_t* codes_s;
    double* scale64;
    double* zero64;
    double* loss64;
    int32_t* pinv;
    int32_t* gsw;   // group of each sweep column (static groups)
};

int64_t n_groups_of(int64_t d_in, int32_t g) { return g > 0 ? ceil_div(d_in, g) : 1; }

// Columns per superblock of the two-level lazy update: blocks are swept one
// by one and update the rest of their superblock (K = B); each finished
// superblock updates everything after it once (K = S).  Where a group may
// cross a superblock end (S % g != 0), the sweep of each superblock waits
// for the previous far update.
int64_t superblock_cols(int64_t d_in, const gptq_config* cfg) {
    const int64_t B = cfg->block_size;
#ifndef GPTQ_SUPER
#define GPTQ_SUPER 1024
#endif
    const int64_t S = B * (GPTQ_SUPER / B > 0 ? GPTQ_SUPER / B : 1);
    const int64_t g = cfg->group_size > 0 ? cfg->group_size : d_in;
    if (cfg->group_size <= 0 || cfg->static_groups || S % g == 0 || g % S == 0) return S;
    // otherwise the largest multiple of lcm(B, g) up to GPTQ_SUPER, so that
    // no group crosses a superblock end (a group crossing a block end reads
    // columns of its own superblock, which the in-superblock updates keep
    // current up to the block being swept)
    int64_t a = B, b = g;
    while (b != 0) {
        const int64_t t = a % b;
        a = b;
        b = t;
    }
    const int64_t l = B / a * g;
    if (l <= GPTQ_SUPER) return GPTQ_SUPER / l * l;
    return B;
}

SweepWs carve(void* ws, int64_t d_out, int64_t d_in, const gptq_config* cfg, bool factored) {
    char* p = (char*)ws;
    SweepWs w;
    size_t off = 0;
    w.flags = (int*)(p + off);
    off += 256;
    w.Wwork = (double*)(p + off);
    off = align_up(off + (size_t)d_out * d_in * 8, 256);
    w.Err = (double*)(p + off);
    off = align_up(off + 2 * (size_t)d_out * superblock_cols(d_in, cfg) * 8, 256);
    w.codes_s = (uint8_t*)(p + off);
    off = align_up(off + (size_t)d_out * d_in, 256);
    const int64_t ng = n_groups_of(d_in, cfg->group_size);
    w.scale64 = (double*)(p + off);
    off = align_up(off + (size_t)ng * d_out * 8, 256);
    w.zero64 = (double*)(p + off);
    off = align_up(off + (size_t)ng * d_out * 8, 256);
    w.loss64 = (double*)(p + off);
    off = align_up(off + (size_t)d_out * 8, 256);
    w.pinv = (int32_t*)(p + off);
    off = align_up(off + (size_t)d_in * 4, 256);
    w.gsw = (int32_t*)(p + off);
    off = align_up(off + (size_t)d_in * 4, 256);
    w.W0 = factored ? (double*)(p + off) : nullptr;
    return w;
}

size_t carve_size(int64_t d_out, int64_t d_in, const gptq_config* cfg, bool factored) {
    size_t off = 256;
    off = align_up(off + (size_t)d_out * d_in * 8, 256);
    off = align_up(off + 2 * (size_t)d_out * superblock_cols(d_in, cfg) * 8, 256);
    off = align_up(off + (size_t)d_out * d_in, 256);
    const int64_t ng = n_groups_of(d_in, cfg->group_size);
    off = align_up(off + (size_t)ng * d_out * 8, 256);
    off = align_up(off + (size_t)ng * d_out * 8, 256);
    off = align_up(off + (size_t)d_out * 8, 256);
    off = align_up(off + (size_t)d_in * 4, 256);
    off = align_up(off + (size_t)d_in * 4, 256);
    if (factored) off = align_up(off + (size_t)d_out * d_in * 8, 256);
    return off;
}

// Wwork[r][k] = W[r][perm[k]] widened to float64; row_loss64 = 0; flags non-finite W.
__global__ __launch_bounds__(256) void convert_kernel(const void* __restrict__ W, gptq_dtype dt, int64_t d_out,
                                                      int64_t d_in, int64_t ld_w, const int32_t* __restrict__ perm,
                                                      double* Wwork, double* loss64, int* flags) {
    const int64_t r = blockIdx.y;
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k == 0) loss64[r] = 0.0;
    if (k >= d_in) return;
    int64_t p = perm[k];
    if (p < 0 || p >= d_in) {
        raise_flag(flags, FLAG_BAD_PERM);
        p = 0;
    }
    const double v = load_as_f64(W, r * ld_w + p, dt);
    if (!isfinite(v)) raise_flag(flags, FLAG_NONFINITE);
    Wwork[r * d_in + k] = v;
}

// The same with one workgroup per row: the row is read in order into LDS
// (its bytes in 4-byte words), then gathered from there, so that the global
// reads are coalesced instead of scattered along the row.
constexpr size_t CONVERT_LDS_MAX = 64 * 1024;
__global__ __launch_bounds__(256) void convert_rows_lds_kernel(const void* __restrict__ W, gptq_dtype dt,
                                                               int64_t d_in, int64_t ld_w,
                                                               const int32_t* __restrict__ perm, double* Wwork,
                                                               double* loss64, int* flags, double* W0) {
    extern __shared__ uint32_t crow[];
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    const size_t esz = dt == GPTQ_F32 ? 4 : 2;
    const uint32_t nw = (uint32_t)((d_in * (int64_t)esz + 3) / 4);   // words holding the row
    const char* src = (const char*)W + r * ld_w * (int64_t)esz;
    const bool aligned = ((uintptr_t)src & 3) == 0;
    for (uint32_t q = tid; q < nw; q += 256) {
        uint32_t v;
        if (aligned && (int64_t)(4 * q + 4) <= d_in * (int64_t)esz) {
            v = ((const uint32_t*)src)[q];
        } else {   // unaligned row start or the last partial word: byte by byte
            v = 0;
            for (int b = 0; b < 4; ++b)
                if ((int64_t)(4 * q + b) < d_in * (int64_t)esz) v |= (uint32_t)(uint8_t)src[4 * q + b] << (8 * b);
        }
        crow[q] = v;
    }
    if (tid == 0) loss64[r] = 0.0;
    __syncthreads();
    bool bad_perm = false, nonfinite = false;
    for (int64_t k = tid; k < d_in; k += 256) {
        int64_t p = perm[k];
        if (p < 0 || p >= d_in) {
            bad_perm = true;
            p = 0;
        }
        const double v = load_as_f64(crow, p, dt);
        nonfinite |= !isfinite(v);
        Wwork[r * d_in + k] = v;
        if (W0) W0[r * d_in + k] = v;   // factored form: the weights before the sweep
    }
    if (bad_perm) raise_flag(flags, FLAG_BAD_PERM);
    if (nonfinite) raise_flag(flags, FLAG_NONFINITE);
}

__global__ void fill_neg_kernel(int32_t* p, int64_t n) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k < n) p[k] = -1;
}

// pinv[perm[k]] = k; g_idx[perm[k]] = k / g, or with static groups
// g_idx[j] = j / g and gsw[k] = perm[k] / g (the group of sweep column k).
// Out-of-range entries are skipped (convert_kernel flags them; gsw then
// names group 0), duplicates leave a -1 that finalize flags.
__global__ void pinv_kernel(const int32_t* __restrict__ perm, int64_t d_in, int64_t g, bool stat, int32_t* pinv,
                            int32_t* g_idx, int32_t* gsw) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= d_in) return;
    const int32_t j = perm[k];
    const bool ok = j >= 0 && j < d_in;
    if (stat) {
        gsw[k] = ok ? (int32_t)(j / g) : 0;
        g_idx[k] = (int32_t)(k / g);
    }
    if (!ok) return;
    pinv[j] = (int32_t)k;
    if (!stat) g_idx[j] = (int32_t)(k / g);
}

struct QParams {
    int bits;
    int sym;
    double maxq;
};

// (scale, zero) of a group whose values span [xmin, xmax] (0 included).
__device__ __forceinline__ void grid_params(double xmin, double xmax, const QParams& qp, double& scale,
                                            double& zero) {
    if (qp.sym) {
        double amax = fmax(-xmin, xmax);
        if (amax == 0.0) amax = 1.0;
        scale = 2.0 * amax / qp.maxq;
        zero = (double)(1 << (qp.bits - 1));
    } else {
        if (xmin == 0.0 && xmax == 0.0) {
            xmin = -1.0;
            xmax = 1.0;
        }
        scale = (xmax - xmin) / qp.maxq;
        zero = rint(-xmin / scale);
    }
}

// Static groups: (scale, zero) of row r and original-order group G (columns
// G*g .. min((G+1)*g, d_in) - 1) from W as given; one wave per (r, G), the
// groups of one row on consecutive waves.
__global__ __launch_bounds__(256) void static_params_kernel(const void* __restrict__ W, gptq_dtype dt,
                                                            int64_t d_out, int64_t d_in, int64_t ld_w, int64_t g,
                                                            int64_t ng, QParams qp, double* __restrict__ scale64,
                                                            double* __restrict__ zero64, float* __restrict__ scales,
                                                            float* __restrict__ zeros) {
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wid >= d_out * ng) return;   // whole waves
    const int64_t r = wid / ng, G = wid % ng;
    const int64_t c0 = G * g, c1 = (c0 + g < d_in) ? c0 + g : d_in;
    double xmin = 0.0, xmax = 0.0;
    for (int64_t c = c0 + lane; c < c1; c += 64) {
        const double v = load_as_f64(W, r * ld_w + c, dt);
        xmin = fmin(xmin, v);
        xmax = fmax(xmax, v);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        xmin = fmin(xmin, __shfl_xor(xmin, o));
        xmax = fmax(xmax, __shfl_xor(xmax, o));
    }
    if (lane == 0) {
        double scale, zero;
        grid_params(xmin, xmax, qp, scale, zero);
        scale64[G * d_out + r] = scale;
        zero64[G * d_out + r] = zero;
        scales[G * d_out + r] = (float)scale;
        zeros[G * d_out + r] = (float)zero;
    }
}

// A non-blocking stream at the default priority plus two events, created
// on first use (layers of at most two superblocks never need them) and
// released when the call returns.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t err_ready = nullptr, far_done = nullptr;
    hipError_t init() {
        if (s) return hipSuccess;
        hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&err_ready, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&far_done, hipEventDisableTiming);
        return e;
    }
    ~SideStream() {
        if (s) {
            (void)hipStreamSynchronize(s);
            (void)hipStreamDestroy(s);
        }
        if (err_ready) (void)hipEventDestroy(err_ready);
        if (far_done) (void)hipEventDestroy(far_done);
    }
};

// DPP helpers on doubles (two 32-bit moves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    // every control used here reads a lane of the same row: the "old" operand
    // is never taken (the source itself, so that no register is cleared)
    const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)b, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(b >> 32), (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm (1,0,3,2)
constexpr int DPP_XOR2 = 0x4E;         // quad_perm (2,3,0,1)
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7-i within each group of 8

constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15-i within each row of 16
constexpr int DPP_ROW_BCAST = 0x150;   // + n: lane n of each row of 16 to the whole row

// f(integral_constant<int, i>) for i = 0 .. N-1, in order.
template <typename F, int... Is>
__device__ __forceinline__ void for_each_seq(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void for_each_n(F&& f) {
    for_each_seq(f, std::make_integer_sequence<int, N>{});
}

// Reductions over the 16 lanes of a row; every lane ends with the same bits
// (each step combines two equal partial results in both orders).
__device__ __forceinline__ double row_sum16(double x) {
    x += dpp_f64<DPP_XOR1>(x);
    x += dpp_f64<DPP_XOR2>(x);
    x += dpp_f64<DPP_HALF_MIRROR>(x);
    return x + dpp_f64<DPP_MIRROR>(x);
}
__device__ __forceinline__ double row_min16(double x) {
    x = fmin(x, dpp_f64<DPP_XOR1>(x));
    x = fmin(x, dpp_f64<DPP_XOR2>(x));
    x = fmin(x, dpp_f64<DPP_HALF_MIRROR>(x));
    return fmin(x, dpp_f64<DPP_MIRROR>(x));
}
__device__ __forceinline__ double row_max16(double x) {
    x = fmax(x, dpp_f64<DPP_XOR1>(x));
    x = fmax(x, dpp_f64<DPP_XOR2>(x));
    x = fmax(x, dpp_f64<DPP_HALF_MIRROR>(x));
    return fmax(x, dpp_f64<DPP_MIRROR>(x));
}

// FACT (the factored form of the lazy updates): the stored per-column value
// is W0_c - q_c (W0: the weights before the sweep) instead of the scaled
// error.  The owner lane keeps q_c in a register of its own (pinned by an
// empty asm: without it the compiler's schedule for the unrolled loop grew
// past 256 VGPRs) and the epilogue subtracts it from W0.
template <int SEG, bool FULL, bool STATIC, bool FACT = false>
__global__ __launch_bounds__(SWAVES * 64) void sweep_block_kernel(double* __restrict__ Wwork, int64_t d_out, int64_t d_in,
                                                         int64_t i1, int nb, const double* __restrict__ U,
                                                         int64_t g, QParams qp, double* __restrict__ Err,
                                                         int ldE, int errc, uint8_t* __restrict__ codes_s,
                                                         double* __restrict__ scale64, double* __restrict__ zero64,
                                                         float* __restrict__ scales, float* __restrict__ zeros,
                                                         double* __restrict__ loss64, const int32_t* __restrict__ gsw,
                                                         const double* __restrict__ W0) {
    extern __shared__ __attribute__((aligned(16))) double sweep_lds[];
    // the sweep is the serial chain of the layer: its waves take issue
    // priority over GEMM waves of the other stream on the same SIMD
    __builtin_amdgcn_s_setprio(3);
    double* rinv = sweep_lds + UP_DOUBLES;
    const int tid = threadIdx.x, lane = tid & 63;
    const int p = lane & (LPR - 1);   // place in the row: block columns p + 16 m
    const int64_t row = (int64_t)blockIdx.x * ROWS + (tid >> 4);
    const bool live = row < d_out;
    const int64_t i2 = i1 + nb;
    const double* Ub = U + i1 * d_in + i1;

    // All global loads of the prologue are issued together (one memory
    // round trip): this row's weights, the parameters of a group begun in
    // an earlier block, the running loss, U's diagonal and the U block.
    double w[CPL];
    {
        const int64_t rr = live ? row : d_out - 1;
        const double* wrow = Wwork + rr * d_in + i1;
#pragma unroll
        for (int mm = 0; mm < CPL; ++mm) {
            const int j = p + LPR * mm;
            const double x = wrow[FULL ? j : (j < nb ? j : 0)];
            w[mm] = (live && (FULL || j < nb)) ? x : 0.0;
        }
    }

    const int64_t rem = i1 % g;
    const int64_t rrow = live ? row : 0;
    const double scale_in = scale64[(i1 / g) * d_out + rrow], zero_in = zero64[(i1 / g) * d_out + rrow];
    double scale = (rem != 0 && live) ? scale_in : 1.0, zero = (rem != 0 && live) ? zero_in : 0.0, rscale = 1.0;
    // static groups: the parameters of this lane's columns (the group of
    // each sweep column, then that group's scale and zero for this row)
    double sc[STATIC ? CPL : 1], ze[STATIC ? CPL : 1];
    if constexpr (STATIC) {
        int32_t gc[CPL];
#pragma unroll
        for (int mm = 0; mm < CPL; ++mm) {
            const int j = p + LPR * mm;
            gc[mm] = gsw[i1 + ((FULL || j < nb) ? j : 0)];
        }
#pragma unroll
        for (int mm = 0; mm < CPL; ++mm) {
            sc[mm] = scale64[(int64_t)gc[mm] * d_out + rrow];
            ze[mm] = zero64[(int64_t)gc[mm] * d_out + rrow];
        }
    }
    const double loss_l = loss64[rrow];
    const double loss_in = (live && p == 0) ? loss_l : 0.0;
    const int dt = tid < nb ? tid : 0;
    const double udiag_l = Ub[(uint32_t)dt * (uint32_t)d_in + dt];
    const double udiag = (tid < nb) ? udiag_l : 1.0;
    // stage the row segments (zeros outside the nb x nb block) and
    // 1 / U[c][c]: every load of a thread issued before the first store
    {
        constexpr int NV = stage_first(CPL);
        double2 v[NV];
        const bool even_rows = ((d_in | i1) & 1) == 0 && ((uintptr_t)U & 15) == 0;
        // slot k of the staging registers: pair q of register group m (both
        // compile-time constants, so the divisions by the segment length fold)
        for_each_n<NV>([&](auto kk) __attribute__((always_inline)) {
            constexpr int k = decltype(kk)::value;
            constexpr int m = stage_group(k), it = k - stage_first(m);
            constexpr int L = seg_len(m);
            const int q = tid + it * SWAVES * 64;          // pair within register group m
            const int off = 2 * q;
            const int r = LPR * m + off / L;               // U row (block index)
            const int j = LPR * m + off % L;               // U column (block index), even
            const bool in = q < LPR * L / 2;
            const bool r_ok = in && r < nb;
            // r < 128 and d_in <= 2^20: the row offset fits 32 bits
            const double* src = Ub + (uint32_t)(r_ok ? r : 0) * (uint32_t)d_in;
            double x, y;
            // loads from clamped (in-range) addresses, unconditionally, so
            // that all of them are in flight together; unused values dropped
            if (FULL && even_rows) {
                // 16-byte aligned: the block starts at an even column and every row
                // at an even offset
                const double2 u2 = *(const double2*)(src + j);
                x = r_ok ? u2.x : 0.0;
                y = r_ok ? u2.y : 0.0;
            } else if (FULL) {
                const double xl = src[j], yl = src[j + 1];
                x = r_ok ? xl : 0.0;
                y = r_ok ? yl : 0.0;
            } else {
                const double xl = src[j < nb ? j : 0], yl = src[j + 1 < nb ? j + 1 : 0];
                x = (r_ok && j < nb) ? xl : 0.0;
                y = (r_ok && j + 1 < nb) ? yl : 0.0;
            }
            v[k] = double2{x, y};
        });
        for_each_n<NV>([&](auto kk) __attribute__((always_inline)) {
            constexpr int k = decltype(kk)::value;
            constexpr int m = stage_group(k), it = k - stage_first(m);
            const int q = tid + it * SWAVES * 64;
            if (q < LPR * seg_len(m) / 2) *(double2*)&sweep_lds[seg_base(m) + 2 * q] = v[k];
        });
    }
    static_assert(BMAX <= SWAVES * 64, "one diagonal entry per thread");
    if (tid < nb) rinv[tid] = 1.0 / udiag;
    if (rem != 0 && live) rscale = 1.0 / scale;
    __syncthreads();
    // U row c's entries for this lane's registers m' >= c / 16
    auto load_urow = [&](double (&u)[CPL], int c) __attribute__((always_inline)) {
        const int m = c / LPR;
        const double* r = sweep_lds + seg_base(m) + (c % LPR) * seg_len(m) + p;
#pragma unroll
        for (int mm = 0; mm < CPL; ++mm)
            if (mm >= m) u[mm] = r[LPR * (mm - m)];
    };

    uint32_t pk[CPL / 4] = {0u, 0u};
    int next_gs = (int)(rem == 0 ? 0 : g - rem);      // block column of the next group start
    int64_t next_gi = i1 / g + (rem == 0 ? 0 : 1);  // and its group index

    double qr[FACT ? CPL : 1] = {};   // FACT: q of this lane's columns
    // U rows of the next two columns in registers
    double ua[CPL], ub[CPL];
    load_urow(ua, 0);
    load_urow(ub, 1);
    double ria = rinv[0], rib = rinv[1];
    double xn = 0.0;   // the next column's weight in its owner lane

    // one call per block column c, as a compile-time constant
    for_each_n<BMAX>([&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        constexpr int m = c / LPR, j = c % LPR;
        if (!FULL && c >= nb) return;
        if (!STATIC && c % SEG == 0 && c == next_gs) {
            // group parameters from the group's current values: block
            // columns [c, cend) in registers, later columns from Wwork
            const int64_t gend = (i1 + c + g < d_in) ? i1 + c + g : d_in;
            const int cend = (gend - i1 < nb) ? (int)(gend - i1) : nb;
            double xmin = 0.0, xmax = 0.0;
#pragma unroll
            for (int mm = 0; mm < CPL; ++mm) {
                const int col = p + LPR * mm;
                const bool in = col >= c && col < cend;
                xmin = fmin(xmin, in ? w[mm] : 0.0);
                xmax = fmax(xmax, in ? w[mm] : 0.0);
            }
            if (live && c > 0 && gend > i2) {
                // a group begun inside the block and running past its end:
                // the columns past the block still lack the compensation of
                // this block's finished columns (their lazy update comes
                // after the block), so it is applied here: v_j = W_j - sum
                // over finished c' of err_c' U[c'][j], each lane summing
                // over its own columns, then the row
                for (int64_t jj = i2; jj < gend; ++jj) {
                    double ps = 0.0;
#pragma unroll
                    for (int mm = 0; mm < CPL; ++mm) {
                        const int col = p + LPR * mm;
                        const bool done = col < c;
                        const double u = Ub[(int64_t)(done ? col : 0) * d_in + (jj - i1)];
                        ps = done ? fma(w[mm], u, ps) : ps;
                    }
                    const double v = Wwork[row * d_in + jj] - row_sum16(ps);
                    xmin = fmin(xmin, v);
                    xmax = fmax(xmax, v);
                }
            } else if (live) {
                for (int64_t jj = i2 + p; jj < gend; jj += LPR) {
                    const double v = Wwork[row * d_in + jj];
                    xmin = fmin(xmin, v);
                    xmax = fmax(xmax, v);
                }
            }
            xmin = row_min16(xmin);
            xmax = row_max16(xmax);
            grid_params(xmin, xmax, qp, scale, zero);
            rscale = 1.0 / scale;
            if (live && p == 0) {
                scale64[next_gi * d_out + row] = scale;
                zero64[next_gi * d_out + row] = zero;
                scales[next_gi * d_out + row] = (float)scale;
                zeros[next_gi * d_out + row] = (float)zero;
            }
            next_gs = c + (int)g;
            ++next_gi;
        }
        // even columns use ua / ria, odd ub / rib; the buffers are refilled
        // with the row two columns ahead once this column has used them
        double (&u)[CPL] = (c & 1) ? ub : ua;
        double& ri = (c & 1) ? rib : ria;
        // quantize column c (meaningful in the owner lane, p == j); the
        // code is decided on the correctly rounded quotient w / scale.
        // y = w * (1/scale) is within 2^-51 |y| of that quotient, so their
        // nearest integers agree unless y lies within 2^-40 max(1, |y|) of
        // a half-integer; only then is the column redone from the quotient
        // (divergent, rare), off the common path's dependency chain.
        // w[m] as the previous column left it before its owner's select
        // (which only changes that owner's lane, not this column's owner)
        const double x = (c == 0) ? w[0] : xn;
        // this column's grid (static groups: the owner lane's column m)
        const double cs = STATIC ? sc[STATIC ? m : 0] : scale;
        const double cz = STATIC ? ze[STATIC ? m : 0] : zero;
        double code, t;
        if constexpr (STATIC) {
            // static groups: the quotient in every column.  With a grid per
            // column the rare branch below made the compiler keep the 128
            // columns' values live across it (256 VGPRs, 256 AGPRs and
            // scratch spills, 16.0 ms for the headline layer's sweep).
            code = fmin(fmax(rint(x / cs) + cz, 0.0), qp.maxq);
            t = (x - cs * (code - cz)) * ri;
        } else {
            const double y = x * rscale;
            const double ry = rint(y);
            code = fmin(fmax(ry + cz, 0.0), qp.maxq);
            t = (x - cs * (code - cz)) * ri;
            // the common path's result is formed before the rare branch, which
            // then stays off the dependency chain
            asm volatile("" : "+v"(t), "+v"(code));
            // distance of y to the nearest half-integer: 0.5 - |y - rint(y)| (exact)
            if (fabs(y - ry) >= fma(-0x1p-40, fmax(1.0, fabs(y)), 0.5)) {
                asm volatile("");   // a real branch: the division is not worth computing in every column
                code = fmin(fmax(rint(x / cs) + cz, 0.0), qp.maxq);
                t = (x - cs * (code - cz)) * ri;
            }
        }
        const bool own = p == j;
        // the owner's scaled error to its whole row (DPP row broadcast)
        const double err = dpp_f64<DPP_ROW_BCAST + j>(t);
        // the code goes into this lane's code bytes now (deferred, every
        // column's code would stay live); the owner's scaled error t stays in
        // w[m] below, and the row loss is summed from those at the end
        pk[m >> 2] = own ? (pk[m >> 2] | ((uint32_t)code << (8 * (m & 3)))) : pk[m >> 2];
        asm volatile("" : "+v"(pk[m >> 2]));
        // compensation of the later columns of the block: registers m' >= m
        // (in register m, the finished columns meet zeros of U below the
        // diagonal; earlier registers hold finished columns only)
#pragma unroll
        for (int mm = 0; mm < CPL; ++mm)
            if (mm >= m) w[mm] = fma(-err, u[mm], w[mm]);
        if (c + 1 < BMAX) xn = w[(c + 1) / LPR];
        if constexpr (FACT) {
            // the owner keeps q of its column (off the dependency chain)
            qr[FACT ? m : 0] = own ? cs * (code - cz) : qr[FACT ? m : 0];
            asm volatile("" : "+v"(qr[FACT ? m : 0]));
        }
        w[m] = own ? err : w[m];
        if (c + 2 < BMAX) {
            load_urow(u, c + 2);
            ri = rinv[c + 2];
        }
        // keep the U row loads two columns ahead, not hoisted further (the
        // unrolled sequence would otherwise hold many rows in registers, and
        // a kernel this wide would keep a GEMM workgroup of the other stream
        // off the CU)
        asm volatile("" ::: "memory");
    });

    // errors (FACT: W0 - q) and codes of this row's columns back to HBM
    if (live) {
        double* erow = Err + row * ldE + errc;
        uint8_t* crow = codes_s + row * d_in + i1;
        const double* w0row = W0 + row * d_in + i1;
#pragma unroll
        for (int mm = 0; mm < CPL; ++mm) {
            const int col = p + LPR * mm;
            if (FULL || col < nb) {
                erow[col] = FACT ? w0row[col] - qr[FACT ? mm : 0] : w[mm];
                crow[col] = (uint8_t)(pk[mm >> 2] >> (8 * (mm & 3)));
            }
        }
    }
    // row loss: sum over the row's columns of t^2 / 2, t = (w - q) / U[c][c]
    // (now in w), each lane over its columns in column order, then the
    // sixteen parts in a fixed order
    double loss = 0.0;
#pragma unroll
    for (int mm = 0; mm < CPL; ++mm) loss = fma(0.5 * w[mm], w[mm], loss);
    loss = row_sum16(loss);
    if (live && p == 0) loss64[row] = loss_in + loss;
}

// codes / w_hat in original column order.
__global__ __launch_bounds__(256) void finalize_kernel(const uint8_t* __restrict__ codes_s, int64_t d_out,
                                                       int64_t d_in, const int32_t* __restrict__ pinv, int64_t g,
                                                       bool stat, const double* __restrict__ scale64,
                                                       const double* __restrict__ zero64, uint8_t* codes,
                                                       float* w_hat, int* flags) {
    const int64_t r = blockIdx.y;
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= d_in) return;
    int64_t k = pinv[j];
    if (k < 0 || k >= d_in) {
        raise_flag(flags, FLAG_BAD_PERM);
        k = 0;
    }
    const uint8_t c = codes_s[r * d_in + k];
    codes[r * d_in + j] = c;
    if (w_hat) {
        const int64_t gi = (stat ? j : k) / g;
        w_hat[r * d_in + j] = (float)(scale64[gi * d_out + r] * ((double)c - zero64[gi * d_out + r]));
    }
}

// The same with one workgroup per row: the row's codes (sweep order) and
// its group parameters are read in order into LDS, then gathered from there.
__global__ __launch_bounds__(256) void finalize_rows_lds_kernel(const uint8_t* __restrict__ codes_s, int64_t d_out,
                                                                int64_t d_in, const int32_t* __restrict__ pinv,
                                                                int64_t g, int64_t ng, bool stat,
                                                                const double* __restrict__ scale64,
                                                                const double* __restrict__ zero64, uint8_t* codes,
                                                                float* w_hat, int* flags) {
    extern __shared__ double fl[];          // [ng] scales, [ng] zeros, then the codes
    uint8_t* cl = (uint8_t*)(fl + 2 * ng);
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    const uint8_t* src = codes_s + r * d_in;
    for (int64_t k = tid; k < d_in; k += 256) cl[k] = src[k];
    if (w_hat)
        for (int64_t q = tid; q < ng; q += 256) {
            fl[q] = scale64[q * d_out + r];
            fl[ng + q] = zero64[q * d_out + r];
        }
    __syncthreads();
    bool bad = false;
    for (int64_t j = tid; j < d_in; j += 256) {
        int64_t k = pinv[j];
        if (k < 0 || k >= d_in) {
            bad = true;
            k = 0;
        }
        const uint8_t c = cl[k];
        codes[r * d_in + j] = c;
        if (w_hat) {
            const int64_t gi = (stat ? j : k) / g;
            w_hat[r * d_in + j] = (float)(fl[gi] * ((double)c - fl[ng + gi]));
        }
    }
    if (bad) raise_flag(flags, FLAG_BAD_PERM);
}

__global__ void copy_loss_kernel(const double* __restrict__ src, double* dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

}  // namespace

size_t sweep_workspace_bytes(int64_t d_out, int64_t d_in, const gptq_config* cfg, bool factored) {
    return carve_size(d_out, d_in, cfg, factored);
}

bool sweep_factored_supported(int64_t d_in, const gptq_config* cfg) {
    if (d_in % BMAX != 0 || cfg->block_size != BMAX) return false;
    if (cfg->static_groups != 0 && cfg->group_size > 0) return true;
    const int64_t g = cfg->group_size > 0 ? cfg->group_size : d_in;
    // every group inside one block (or one group per row), and group starts
    // on multiples of CPL block columns
    if (g % CPL != 0) return false;
    return g >= d_in || BMAX % g == 0;
}

gptq_status sweep_launch(const void* W, gptq_dtype dt, int64_t d_out, int64_t d_in, int64_t ld_w,
                         const double* U, const int32_t* perm, const gptq_config* cfg, uint8_t* codes,
                         float* scales, float* zeros, int32_t* g_idx, float* w_hat, double* row_loss, void* ws,
                         hipStream_t s, int* host_flags, bool factored) {
    if (factored && !sweep_factored_supported(d_in, cfg)) return GPTQ_ERR_UNSUPPORTED;
    SweepWs w = carve(ws, d_out, d_in, cfg, factored);
    const int64_t g = cfg->group_size > 0 ? cfg->group_size : d_in;
    const int B = cfg->block_size;
    // per-row static groups are the dynamic per-row group (taken at column 0
    // from the untouched row either way)
    const bool stat = cfg->static_groups != 0 && cfg->group_size > 0;
    const int64_t ng = n_groups_of(d_in, cfg->group_size);
    // group starts fall on multiples of SEG block columns
    int SEG = CPL;
    while (SEG > 1 && ((B % SEG) != 0 || (cfg->group_size > 0 && (g % SEG) != 0))) SEG >>= 1;
    GPTQ_HIP(hipMemsetAsync(w.flags, 0, 256, s));

    const unsigned gx = (unsigned)ceil_div(d_in, 256);
    const size_t row_bytes = (size_t)d_in * (dt == GPTQ_F32 ? 4 : 2);
    if (row_bytes <= CONVERT_LDS_MAX) {
        const size_t lds = align_up(row_bytes, 4);
        hipLaunchKernelGGL(convert_rows_lds_kernel, dim3((unsigned)d_out), dim3(256), lds, s, W, dt, d_in, ld_w, perm,
                           w.Wwork, w.loss64, w.flags, w.W0);
    } else {
        hipLaunchKernelGGL(convert_kernel, dim3(gx, (unsigned)d_out), dim3(256), 0, s, W, dt, d_out, d_in, ld_w, perm,
                           w.Wwork, w.loss64, w.flags);
    }
    GPTQ_LAUNCH_CHECK();
    if (factored && row_bytes > CONVERT_LDS_MAX)
        GPTQ_HIP(hipMemcpyAsync(w.W0, w.Wwork, (size_t)d_out * d_in * sizeof(double), hipMemcpyDeviceToDevice, s));
    hipLaunchKernelGGL(fill_neg_kernel, dim3(gx), dim3(256), 0, s, w.pinv, d_in);
    GPTQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(pinv_kernel, dim3(gx), dim3(256), 0, s, perm, d_in, g, stat, w.pinv, g_idx, w.gsw);
    GPTQ_LAUNCH_CHECK();

    QParams qp{cfg->bits, cfg->sym, (double)((1 << cfg->bits) - 1)};
    if (stat) {
        if (ceil_div(d_out * ng, 4) > INT32_MAX) return GPTQ_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(static_params_kernel, dim3((unsigned)ceil_div(d_out * ng, 4)), dim3(256), 0, s, W, dt,
                           d_out, d_in, ld_w, g, ng, qp, w.scale64, w.zero64, scales, zeros);
        GPTQ_LAUNCH_CHECK();
    }
    const unsigned grid = (unsigned)ceil_div(d_out, ROWS);
#define SWEEP_ATTR(n, f) GPTQ_HIP(ensure_lds_limit((const void*)sweep_block_kernel<n, f, false>, (int)SWEEP_LDS));
    SWEEP_ATTR(8, true)
    SWEEP_ATTR(8, false)
    SWEEP_ATTR(4, true)
    SWEEP_ATTR(4, false)
    SWEEP_ATTR(2, true)
    SWEEP_ATTR(2, false)
    SWEEP_ATTR(1, true)
    SWEEP_ATTR(1, false)
#undef SWEEP_ATTR
    GPTQ_HIP(ensure_lds_limit((const void*)sweep_block_kernel<CPL, true, true>, (int)SWEEP_LDS));
    GPTQ_HIP(ensure_lds_limit((const void*)sweep_block_kernel<CPL, false, true>, (int)SWEEP_LDS));
    if (factored) {
        GPTQ_HIP(ensure_lds_limit((const void*)sweep_block_kernel<CPL, true, false, true>, (int)SWEEP_LDS));
        GPTQ_HIP(ensure_lds_limit((const void*)sweep_block_kernel<CPL, true, true, true>, (int)SWEEP_LDS));
    }
    // lazy updates: W[:, later] -= Err U[block, later]; factored: W[:, later]
    // += (W0 - Q)[:, block] F[block, later] (the same columns, from the
    // factored form F in U's place)
    const double lz = factored ? 1.0 : -1.0;
    const int64_t S = superblock_cols(d_in, cfg);
    // A group that runs past the end of its superblock (groups wider than a
    // superblock, or superblocks of one block when lcm(B, g) exceeds the
    // superblock cap) reads columns of later superblocks at its first
    // column; the far update that writes those columns must be done first.
    const bool wait_far_before_sweep = !stat && cfg->group_size > 0 && S % g != 0;

    // A second stream runs each superblock's far update (everything past
    // the next superblock) while the next superblock is swept.
    SideStream side;
    bool far_pending = false;
    for (int64_t k = 0, a = 0; a < d_in; ++k, a += S) {
        const int64_t e = (a + S < d_in) ? a + S : d_in;
        double* Ek = w.Err + (k & 1) * d_out * S;
        if (wait_far_before_sweep && far_pending) GPTQ_HIP(hipStreamWaitEvent(s, side.far_done, 0));
        for (int64_t i1 = a; i1 < e; i1 += B) {
            const int nb = (int)((e - i1 < B) ? e - i1 : B);
            const bool full = nb == BMAX;
            switch (factored ? (stat ? -4 : -3) : stat ? -1 - (full ? 1 : 0) : SEG * 2 + (full ? 1 : 0)) {
#define SWEEP_CASE_T(n, f, t, x, label)                                                                      \
    case label:                                                                                               \
        hipLaunchKernelGGL((sweep_block_kernel<n, f, t, x>), dim3(grid), dim3(SWAVES * 64), SWEEP_LDS, s,       \
                           w.Wwork, d_out, d_in, i1,                                                        \
                           nb, U, g, qp, Ek, (int)S, (int)(i1 - a), w.codes_s, w.scale64, w.zero64, scales,  \
                           zeros, w.loss64, w.gsw, w.W0);                                                     \
        break;
#define SWEEP_CASE(n, f) SWEEP_CASE_T(n, f, false, false, n * 2 + f)
                SWEEP_CASE_T(CPL, true, true, true, -4)
                SWEEP_CASE_T(CPL, true, false, true, -3)
                SWEEP_CASE_T(CPL, true, true, false, -2)
                SWEEP_CASE_T(CPL, false, true, false, -1)
                SWEEP_CASE(8, 1)
                SWEEP_CASE(8, 0)
                SWEEP_CASE(4, 1)
                SWEEP_CASE(4, 0)
                SWEEP_CASE(2, 1)
                SWEEP_CASE(2, 0)
                SWEEP_CASE(1, 1)
                SWEEP_CASE(1, 0)
#undef SWEEP_CASE
#undef SWEEP_CASE_T
            }
            GPTQ_LAUNCH_CHECK();
            const int64_t i2 = i1 + nb;
            if (i2 < e) {  // rest of this superblock, K = nb
                gptq_status st = launch_gemm_f64(s, d_out, e - i2, nb, lz, Ek + (i1 - a), S, U + i1 * d_in + i2,
                                                 d_in, false, 1.0, w.Wwork + i2, d_in, false);
                if (st != GPTQ_OK) return st;
            }
        }
        if (e >= d_in) break;
        // near update: the next superblock's columns, on the main stream,
        // after the previous far update (which also wrote them) is done
        if (far_pending) GPTQ_HIP(hipStreamWaitEvent(s, side.far_done, 0));
        const int64_t n_near = (S < d_in - e) ? S : d_in - e;
        gptq_status st = launch_gemm_f64(s, d_out, n_near, e - a, lz, Ek, S, U + a * d_in + e, d_in, false, 1.0,
                                         w.Wwork + e, d_in, false);
        if (st != GPTQ_OK) return st;
        far_pending = false;
        if (e + n_near < d_in) {  // far update on the side stream
            GPTQ_HIP(side.init());
            GPTQ_HIP(hipEventRecord(side.err_ready, s));
            GPTQ_HIP(hipStreamWaitEvent(side.s, side.err_ready, 0));
            st = launch_gemm_f64(side.s, d_out, d_in - e - n_near, e - a, lz, Ek, S, U + a * d_in + e + n_near,
                                 d_in, false, 1.0, w.Wwork + e + n_near, d_in, false, GEMM_TRI_NONE, true);
            if (st != GPTQ_OK) return st;
            GPTQ_HIP(hipEventRecord(side.far_done, side.s));
            far_pending = true;
        }
    }
    if (far_pending) GPTQ_HIP(hipStreamWaitEvent(s, side.far_done, 0));
    const size_t fin_lds = (size_t)ng * 16 + (size_t)d_in;
    if (fin_lds <= CONVERT_LDS_MAX) {
        hipLaunchKernelGGL(finalize_rows_lds_kernel, dim3((unsigned)d_out), dim3(256), fin_lds, s, w.codes_s, d_out,
                           d_in, w.pinv, g, ng, stat, w.scale64, w.zero64, codes, w_hat, w.flags);
    } else {
        hipLaunchKernelGGL(finalize_kernel, dim3(gx, (unsigned)d_out), dim3(256), 0, s, w.codes_s, d_out, d_in,
                           w.pinv, g, stat, w.scale64, w.zero64, codes, w_hat, w.flags);
    }
    GPTQ_LAUNCH_CHECK();
    if (row_loss) {
        hipLaunchKernelGGL(copy_loss_kernel, dim3((unsigned)ceil_div(d_out, 256)), dim3(256), 0, s, w.loss64,
                           row_loss, d_out);
        GPTQ_LAUNCH_CHECK();
    }
    GPTQ_HIP(hipMemcpyAsync(host_flags, w.flags, N_FLAGS * sizeof(int), hipMemcpyDeviceToHost, s));
    GPTQ_HIP(hipStreamSynchronize(s));
    return GPTQ_OK;
}

}  // namespace gptq
