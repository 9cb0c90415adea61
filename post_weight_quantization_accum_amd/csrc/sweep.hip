// Blocked column sweep with error compensation and lazy block updates
// ("GPTQ量化算法深度解析" §2.2 compensation, §2.4 fixed order and lazy batch
// updates, §3.1 step 3 blocks of 128 columns; grid per "通义千问...GPTQ-Int4"
// §2.1-2.2), all in float64.
//
// Data layout in HBM (workspace):
//   Wwork  d_out x d_in float64, columns in sweep order (the running W)
//   Err    d_out x B    float64, scaled errors of the current block
//   codes_s d_out x d_in uint8, codes in sweep order
//   scale64 / zero64  n_groups x d_out float64
//   row_loss64 d_out float64, pinv d_in int32, flags
//
// sweep_block: one wave64 per 64 rows, one lane per row.  The block's columns
// of those rows sit in LDS as [column][row] (conflict-free per column).  The
// block is walked in sub-blocks of SB columns held in registers: inside a
// sub-block the compensation is applied column by column in registers; the
// sub-block's errors then update the block's remaining columns in LDS (SB
// fused multiply-adds per element).  The rows of U needed by a sub-block are
// staged in LDS and read as broadcasts.  After the block, a float64 MFMA GEMM
// applies W[:, i2:] -= Err * U[i1:i2, i2:].
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

SweepWs carve(void* ws, int64_t d_out, int64_t d_in, const gptq_config* cfg) {
    char* p = (char*)ws;
    SweepWs w;
    size_t off = 0;
    w.flags = (int*)(p + off);
    off += 256;
    w.Wwork = (double*)(p + off);
    off = align_up(off + (size_t)d_out * d_in * 8, 256);
    w.Err = (double*)(p + off);
    off = align_up(off + (size_t)d_out * cfg->block_size * 8, 256);
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
    off = align_up(off + (size_t)d_out * cfg->block_size * 8, 256);
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

template <int SB>
__global__ __launch_bounds__(ROWS) void sweep_block_kernel(double* __restrict__ Wwork, int64_t d_out, int64_t d_in,
                                                           int64_t i1, int nb, const double* __restrict__ U,
                                                           int64_t g, QParams qp, double* __restrict__ Err,
                                                           int ldE, uint8_t* __restrict__ codes_s,
                                                           double* __restrict__ scale64, double* __restrict__ zero64,
                                                           float* __restrict__ scales, float* __restrict__ zeros,
                                                           double* __restrict__ loss64) {
    __shared__ double w1[BMAX][ROWS + 1];
    __shared__ double us[SBMAX][BMAX];
    __shared__ uint8_t cb[BMAX][ROWS];

    const int lane = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * ROWS;
    const int64_t row = r0 + lane;
    const bool live = row < d_out;
    const int64_t i2 = i1 + nb;

    // block columns of the 64 rows -> LDS [column][row]
    for (int rr = 0; rr < ROWS; ++rr) {
        const int64_t gr = r0 + rr;
        for (int j = lane; j < nb; j += ROWS) w1[j][rr] = (gr < d_out) ? Wwork[gr * d_in + i1 + j] : 0.0;
    }

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
        __syncthreads();
        for (int k = 0; k < SB; ++k) {
            const int64_t c = i1 + s0 + k;
            for (int j = s0 + lane; j < nb; j += ROWS)
                us[k][j] = (s0 + k < nb) ? U[c * d_in + i1 + j] : 0.0;
        }
        __syncthreads();

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
                const double w = wv[k];
                double code = rint(w / scale) + zero;
                code = fmin(fmax(code, 0.0), qp.maxq);
                const double q = scale * (code - zero);
                const double ucc = us[k][s0 + k];
                const double diff = w - q;
                const double err = diff / ucc;
#pragma unroll
                for (int kk = k + 1; kk < SB; ++kk) wv[kk] = fma(-err, us[k][s0 + kk], wv[kk]);
                errs[k] = err;
                loss += diff * diff / (2.0 * ucc * ucc);
                w1[s0 + k][lane] = err;
                cb[s0 + k][lane] = (uint8_t)code;
            }
        }
        // the sub-block's errors update the rest of the block
        for (int j = s0 + SB; j < nb; ++j) {
            double v = w1[j][lane];
#pragma unroll
            for (int k = 0; k < SB; ++k) v = fma(-errs[k], us[k][j], v);
            w1[j][lane] = v;
        }
    }
    __syncthreads();

    // Err (now in w1) and codes back to HBM, row-contiguous
    for (int rr = 0; rr < ROWS; ++rr) {
        const int64_t gr = r0 + rr;
        if (gr >= d_out) break;
        for (int j = lane; j < nb; j += ROWS) {
            Err[gr * ldE + j] = w1[j][rr];
            codes_s[gr * d_in + i1 + j] = cb[j][rr];
        }
    }
    if (live) loss64[row] += loss;
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
    for (int64_t i1 = 0; i1 < d_in; i1 += B) {
        const int nb = (int)((d_in - i1 < B) ? d_in - i1 : B);
        switch (SB) {
#define SWEEP_CASE(n)                                                                                           \
    case n:                                                                                                     \
        hipLaunchKernelGGL(sweep_block_kernel<n>, dim3(grid), dim3(ROWS), 0, s, w.Wwork, d_out, d_in, i1, nb, U, \
                           g, qp, w.Err, B, w.codes_s, w.scale64, w.zero64, scales, zeros, w.loss64);          \
        break;
            SWEEP_CASE(8)
            SWEEP_CASE(4)
            SWEEP_CASE(2)
            SWEEP_CASE(1)
#undef SWEEP_CASE
        }
        GPTQ_LAUNCH_CHECK();
        const int64_t i2 = i1 + nb;
        if (i2 < d_in) {
            gptq_status st = launch_gemm_f64(s, d_out, d_in - i2, nb, -1.0, w.Err, B, U + i1 * d_in + i2, d_in,
                                             false, 1.0, w.Wwork + i2, d_in, false);
            if (st != GPTQ_OK) return st;
        }
    }
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
