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
// sweep_block: one wave64 per 64 rows, one lane per row.  The block's columns
// of those rows sit in LDS as [column][row] (conflict-free per column), and
// the block's upper triangle of U sits in LDS packed, with reciprocal
// pivots.  The block is walked in sub-blocks of SB columns held in
// registers: inside a sub-block the compensation is applied column by column
// in registers; the sub-block's errors then update the block's remaining
// columns in LDS (SB fused multiply-adds per element).
//
// Lazy updates are two-level (mathematically the same as one update per
// block): after each block, a float64 MFMA GEMM updates the rest of its
// superblock of S = 512 columns (K = B); after each superblock, one GEMM
// with K = S updates the next superblock, and another (on a second stream,
// overlapping the next superblock's sweep) everything after it.
#include "internal.hpp"

namespace gptq {
namespace {

constexpr int BMAX = 128;   // largest supported block (columns per lazy update)
constexpr int ROWS = 64;    // rows per workgroup (one wave)
constexpr int SBMAX = 8;

struct SweepWs {
    int* flags;
    double* Wwork;
    double* Err;
    uint8_t* codes_s;
    double* scale64;
    double* zero64;
    double* loss64;
    int32_t* pinv;
};

int64_t n_groups_of(int64_t d_in, int32_t g) { return g > 0 ? ceil_div(d_in, g) : 1; }

// Columns per superblock of the two-level lazy update: blocks are swept one
// by one and update the rest of their superblock (K = B); each finished
// superblock updates everything after it once (K = S).  Every group must lie
// inside one superblock or start on a superblock boundary; otherwise S = B.
int64_t superblock_cols(int64_t d_in, const gptq_config* cfg) {
    const int64_t B = cfg->block_size;
    const int64_t S = B * (512 / B > 0 ? 512 / B : 1);
    const int64_t g = cfg->group_size > 0 ? cfg->group_size : d_in;
    if (cfg->group_size <= 0 || S % g == 0 || g % S == 0) return S;
    return B;
}

SweepWs carve(void* ws, int64_t d_out, int64_t d_in, const gptq_config* cfg) {
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
    return w;
}

size_t carve_size(int64_t d_out, int64_t d_in, const gptq_config* cfg) {
    size_t off = 256;
    off = align_up(off + (size_t)d_out * d_in * 8, 256);
    off = align_up(off + 2 * (size_t)d_out * superblock_cols(d_in, cfg) * 8, 256);
    off = align_up(off + (size_t)d_out * d_in, 256);
    const int64_t ng = n_groups_of(d_in, cfg->group_size);
    off = align_up(off + (size_t)ng * d_out * 8, 256);
    off = align_up(off + (size_t)ng * d_out * 8, 256);
    off = align_up(off + (size_t)d_out * 8, 256);
    off = align_up(off + (size_t)d_in * 4, 256);
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

__global__ void fill_neg_kernel(int32_t* p, int64_t n) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k < n) p[k] = -1;
}

// pinv[perm[k]] = k, g_idx[perm[k]] = k / g; out-of-range entries are skipped
// (convert_kernel flags them), duplicates leave a -1 that finalize flags.
__global__ void pinv_kernel(const int32_t* __restrict__ perm, int64_t d_in, int64_t g, int32_t* pinv,
                            int32_t* g_idx) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= d_in) return;
    const int32_t j = perm[k];
    if (j < 0 || j >= d_in) return;
    pinv[j] = (int32_t)k;
    g_idx[j] = (int32_t)(k / g);
}

struct QParams {
    int bits;
    int sym;
    double maxq;
};

// A non-blocking stream at the default priority plus two events, released
// when the call returns.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t err_ready = nullptr, far_done = nullptr;
    hipError_t init() {
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

// Packed upper triangle of a BMAX x BMAX block: row a holds columns
// a+1 .. BMAX-1; element (a, b) sits at upper_base(a) + b.
__host__ __device__ __forceinline__ int upper_base(int a) { return a * (BMAX - 1) - a * (a - 1) / 2 - a - 1; }
constexpr int UPACK = BMAX * (BMAX - 1) / 2;

template <int SB>
__global__ __launch_bounds__(256) void sweep_block_kernel(double* __restrict__ Wwork, int64_t d_out, int64_t d_in,
                                                          int64_t i1, int nb, const double* __restrict__ U,
                                                          int64_t g, QParams qp, double* __restrict__ Err,
                                                          int ldE, int errc, uint8_t* __restrict__ codes_s,
                                                          double* __restrict__ scale64, double* __restrict__ zero64,
                                                          float* __restrict__ scales, float* __restrict__ zeros,
                                                          double* __restrict__ loss64) {
    __shared__ double w1[BMAX][ROWS + 1];
    __shared__ double up[UPACK];
    __shared__ double rinv[BMAX];
    __shared__ uint8_t cb[BMAX][ROWS];

    // All four waves stage the block (many loads in flight per thread);
    // wave 0 then sweeps it, one lane per row; all four write it back.
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int64_t r0 = (int64_t)blockIdx.x * ROWS;
    const int64_t row = r0 + lane;
    const bool live = row < d_out;
    const int64_t i2 = i1 + nb;

    // the block's columns of the 64 rows -> LDS [column][row]
#pragma unroll 16
    for (int idx = t; idx < ROWS * BMAX; idx += 256) {
        const int rr = idx / BMAX, j = idx % BMAX;
        const int64_t gr = r0 + rr;
        if (j < nb) w1[j][rr] = (gr < d_out) ? Wwork[gr * d_in + i1 + j] : 0.0;
    }
    // the block's upper triangle of U -> packed LDS; reciprocal pivots
#pragma unroll 16
    for (int idx = t; idx < BMAX * BMAX; idx += 256) {
        const int a = idx / BMAX, b = idx % BMAX;
        if (a < nb && b < nb && b > a) up[upper_base(a) + b] = U[(i1 + a) * d_in + i1 + b];
    }
    if (t < nb) rinv[t] = 1.0 / U[(i1 + t) * d_in + i1 + t];
    __syncthreads();
    if (t < ROWS) {  // wave 0: the sweep (no barriers inside)
        // current group parameters of this row (kept across blocks via scale64/zero64)
        double scale = 1.0, zero = 0.0;
        {
            const int64_t gi = i1 / g;
            if ((i1 % g) != 0 && live) {  // group started in an earlier block
                scale = scale64[gi * d_out + row];
                zero = zero64[gi * d_out + row];
            }
        }
        double loss = 0.0;

        for (int s0 = 0; s0 < nb; s0 += SB) {
            double wv[SB];
#pragma unroll
            for (int k = 0; k < SB; ++k) wv[k] = (s0 + k < nb) ? w1[s0 + k][lane] : 0.0;

            const int64_t c0 = i1 + s0;
            if (c0 % g == 0) {
                // group parameters from the group's current values
                double xmin = 0.0, xmax = 0.0;
                const int64_t gend = (c0 + g < d_in) ? c0 + g : d_in;
                const int64_t inblk_end = (gend < i2) ? gend : i2;
                for (int64_t j = c0; j < inblk_end; ++j) {
                    const double v = w1[j - i1][lane];
                    xmin = fmin(xmin, v);
                    xmax = fmax(xmax, v);
                }
                if (live)
                    for (int64_t j = i2; j < gend; ++j) {
                        const double v = Wwork[row * d_in + j];
                        xmin = fmin(xmin, v);
                        xmax = fmax(xmax, v);
                    }
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
                if (live) {
                    const int64_t gi = c0 / g;
                    scale64[gi * d_out + row] = scale;
                    zero64[gi * d_out + row] = zero;
                    scales[gi * d_out + row] = (float)scale;
                    zeros[gi * d_out + row] = (float)zero;
                }
            }

            double errs[SB];
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                errs[k] = 0.0;
                if (s0 + k < nb) {
                    const int c = s0 + k;
                    const double w = wv[k];
                    // the code is decided on the correctly rounded quotient w / scale
                    double code = rint(w / scale) + zero;
                    code = fmin(fmax(code, 0.0), qp.maxq);
                    const double q = scale * (code - zero);
                    const double ri = rinv[c];
                    const double diff = w - q;
                    const double err = diff * ri;
                    const int ub = upper_base(c);
#pragma unroll
                    for (int kk = k + 1; kk < SB; ++kk) wv[kk] = fma(-err, up[ub + s0 + kk], wv[kk]);
                    errs[k] = err;
                    loss += 0.5 * (diff * ri) * (diff * ri);
                    w1[c][lane] = err;
                    cb[c][lane] = (uint8_t)code;
                }
            }
            // the sub-block's errors update the rest of the block
            int ubk[SB];
#pragma unroll
            for (int k = 0; k < SB; ++k) ubk[k] = upper_base(s0 + k < nb ? s0 + k : 0);
            for (int j = s0 + SB; j < nb; ++j) {
                double v = w1[j][lane];
#pragma unroll
                for (int k = 0; k < SB; ++k) v = fma(-errs[k], up[ubk[k] + j], v);
                w1[j][lane] = v;
            }
        }
        if (live) loss64[row] += loss;
    }
    __syncthreads();
    // Err (now in w1) and codes back to HBM, row-contiguous
#pragma unroll 8
    for (int idx = t; idx < ROWS * BMAX; idx += 256) {
        const int rr = idx / BMAX, j = idx % BMAX;
        const int64_t gr = r0 + rr;
        if (j < nb && gr < d_out) {
            Err[gr * ldE + errc + j] = w1[j][rr];
            codes_s[gr * d_in + i1 + j] = cb[j][rr];
        }
    }
}

// codes / w_hat in original column order.
__global__ __launch_bounds__(256) void finalize_kernel(const uint8_t* __restrict__ codes_s, int64_t d_out,
                                                       int64_t d_in, const int32_t* __restrict__ pinv, int64_t g,
                                                       const double* __restrict__ scale64,
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
        const int64_t gi = k / g;
        w_hat[r * d_in + j] = (float)(scale64[gi * d_out + r] * ((double)c - zero64[gi * d_out + r]));
    }
}

__global__ void copy_loss_kernel(const double* __restrict__ src, double* dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

}  // namespace

size_t sweep_workspace_bytes(int64_t d_out, int64_t d_in, const gptq_config* cfg) {
    return carve_size(d_out, d_in, cfg);
}

gptq_status sweep_launch(const void* W, gptq_dtype dt, int64_t d_out, int64_t d_in, int64_t ld_w,
                         const double* U, const int32_t* perm, const gptq_config* cfg, uint8_t* codes,
                         float* scales, float* zeros, int32_t* g_idx, float* w_hat, double* row_loss, void* ws,
                         hipStream_t s, int* host_flags) {
    SweepWs w = carve(ws, d_out, d_in, cfg);
    const int64_t g = cfg->group_size > 0 ? cfg->group_size : d_in;
    const int B = cfg->block_size;
    GPTQ_HIP(hipMemsetAsync(w.flags, 0, 256, s));

    const unsigned gx = (unsigned)ceil_div(d_in, 256);
    hipLaunchKernelGGL(convert_kernel, dim3(gx, (unsigned)d_out), dim3(256), 0, s, W, dt, d_out, d_in, ld_w, perm,
                       w.Wwork, w.loss64, w.flags);
    GPTQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(fill_neg_kernel, dim3(gx), dim3(256), 0, s, w.pinv, d_in);
    GPTQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(pinv_kernel, dim3(gx), dim3(256), 0, s, perm, d_in, g, w.pinv, g_idx);
    GPTQ_LAUNCH_CHECK();

    // sub-block width: the largest of 8, 4, 2, 1 dividing B and (when
    // grouped) the group size, so every group starts on a sub-block boundary
    int SB = 8;
    while (SB > 1 && ((B % SB) != 0 || (cfg->group_size > 0 && (g % SB) != 0))) SB >>= 1;

    QParams qp{cfg->bits, cfg->sym, (double)((1 << cfg->bits) - 1)};
    const unsigned grid = (unsigned)ceil_div(d_out, ROWS);
    const int64_t S = superblock_cols(d_in, cfg);
    // Groups that span several superblocks read columns past the current
    // superblock at their first column: those must be fully updated first.
    const bool wait_far_before_sweep = cfg->group_size > 0 && g > S;

    // A second stream runs each superblock's far update (everything past
    // the next superblock) while the next superblock is swept.
    SideStream side;
    GPTQ_HIP(side.init());
    bool far_pending = false;
    for (int64_t k = 0, a = 0; a < d_in; ++k, a += S) {
        const int64_t e = (a + S < d_in) ? a + S : d_in;
        double* Ek = w.Err + (k & 1) * d_out * S;
        if (wait_far_before_sweep && far_pending) GPTQ_HIP(hipStreamWaitEvent(s, side.far_done, 0));
        for (int64_t i1 = a; i1 < e; i1 += B) {
            const int nb = (int)((e - i1 < B) ? e - i1 : B);
            switch (SB) {
#define SWEEP_CASE(n)                                                                                           \
    case n:                                                                                                     \
        hipLaunchKernelGGL(sweep_block_kernel<n>, dim3(grid), dim3(256), 0, s, w.Wwork, d_out, d_in, i1, nb, U, \
                           g, qp, Ek, (int)S, (int)(i1 - a), w.codes_s, w.scale64, w.zero64, scales, zeros,    \
                           w.loss64);                                                                           \
        break;
                SWEEP_CASE(8)
                SWEEP_CASE(4)
                SWEEP_CASE(2)
                SWEEP_CASE(1)
#undef SWEEP_CASE
            }
            GPTQ_LAUNCH_CHECK();
            const int64_t i2 = i1 + nb;
            if (i2 < e) {  // rest of this superblock, K = nb
                gptq_status st = launch_gemm_f64(s, d_out, e - i2, nb, -1.0, Ek + (i1 - a), S, U + i1 * d_in + i2,
                                                 d_in, false, 1.0, w.Wwork + i2, d_in, false);
                if (st != GPTQ_OK) return st;
            }
        }
        if (e >= d_in) break;
        // near update: the next superblock's columns, on the main stream,
        // after the previous far update (which also wrote them) is done
        if (far_pending) GPTQ_HIP(hipStreamWaitEvent(s, side.far_done, 0));
        const int64_t n_near = (S < d_in - e) ? S : d_in - e;
        gptq_status st = launch_gemm_f64(s, d_out, n_near, e - a, -1.0, Ek, S, U + a * d_in + e, d_in, false, 1.0,
                                         w.Wwork + e, d_in, false);
        if (st != GPTQ_OK) return st;
        far_pending = false;
        if (e + n_near < d_in) {  // far update on the side stream
            GPTQ_HIP(hipEventRecord(side.err_ready, s));
            GPTQ_HIP(hipStreamWaitEvent(side.s, side.err_ready, 0));
            st = launch_gemm_f64(side.s, d_out, d_in - e - n_near, e - a, -1.0, Ek, S, U + a * d_in + e + n_near,
                                 d_in, false, 1.0, w.Wwork + e + n_near, d_in, false);
            if (st != GPTQ_OK) return st;
            GPTQ_HIP(hipEventRecord(side.far_done, side.s));
            far_pending = true;
        }
    }
    if (far_pending) GPTQ_HIP(hipStreamWaitEvent(s, side.far_done, 0));
    hipLaunchKernelGGL(finalize_kernel, dim3(gx, (unsigned)d_out), dim3(256), 0, s, w.codes_s, d_out, d_in, w.pinv,
                       g, w.scale64, w.zero64, codes, w_hat, w.flags);
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
