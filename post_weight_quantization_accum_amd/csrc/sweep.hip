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
// sweep_block: eight lanes per row, each holding 16 of the block's (up to)
// 128 columns of that row in registers; 8 rows per wave, 16 rows per
// workgroup.  The upper triangle of the block's U (73 KiB with the zero
// padding of its 16-column panels) is staged in LDS once per workgroup, so
// the serial column loop reads U rows at LDS latency; one such workgroup
// fits on a CU beside a float64 GEMM workgroup of another stream.  Column c
// is quantized by the lane owning it; its scaled error reaches the other
// lanes of the row through a masked 8-lane sum (DPP), and every lane then
// applies w_j -= err * U[c][j] to its 16 columns, so each w_j receives the
// compensations of the earlier columns one by one, in column order.  A
// finished column keeps its error in place: the later updates leave it
// unchanged because U is zero below the diagonal.
//
// Lazy updates are two-level (mathematically the same as one update per
// block): after each block, a float64 MFMA GEMM updates the rest of its
// superblock of S = 1024 columns (K = B); after each superblock, one GEMM
// with K = S updates the next superblock, and another (on a second stream,
// overlapping the next superblock's sweep) everything after it.
#include "internal.hpp"

namespace gptq {
namespace {

constexpr int BMAX = 128;   // largest supported block (columns per lazy update)
constexpr int LPR = 8;      // lanes per row
constexpr int CPL = BMAX / LPR;  // columns per lane
constexpr int SWAVES = 2;        // waves per workgroup
constexpr int ROWS = SWAVES * 64 / LPR;   // rows per workgroup
// U block in LDS, one panel per lane part p (block columns 16p..16p+15):
// rows 0..16p+15 of the panel (the rows below are zero in U), 16 doubles
// each; then one zero row for the parts whose panel has ended; then the
// reciprocal diagonal.
constexpr int UP_DOUBLES = CPL * CPL * LPR * (LPR + 1) / 2;   // 9216
constexpr int UZERO = UP_DOUBLES;
constexpr size_t SWEEP_LDS = (size_t)(UP_DOUBLES + CPL + BMAX) * sizeof(double);   // 73 KiB
__host__ __device__ constexpr int panel_base(int p) { return CPL * CPL * p * (p + 1) / 2; }

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
#ifndef GPTQ_SUPER
#define GPTQ_SUPER 1024
#endif
    const int64_t S = B * (GPTQ_SUPER / B > 0 ? GPTQ_SUPER / B : 1);
    const int64_t g = cfg->group_size > 0 ? cfg->group_size : d_in;
    if (cfg->group_size <= 0 || S % g == 0 || g % S == 0) return S;
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

// DPP helpers on doubles (two 32-bit moves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm (1,0,3,2)
constexpr int DPP_XOR2 = 0x4E;         // quad_perm (2,3,0,1)
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7-i within each group of 8

__device__ __forceinline__ double row_sum8(double x) {
    x += dpp_f64<DPP_XOR1>(x);
    x += dpp_f64<DPP_XOR2>(x);
    return x + dpp_f64<DPP_HALF_MIRROR>(x);
}
__device__ __forceinline__ double row_min8(double x) {
    x = fmin(x, dpp_f64<DPP_XOR1>(x));
    x = fmin(x, dpp_f64<DPP_XOR2>(x));
    return fmin(x, dpp_f64<DPP_HALF_MIRROR>(x));
}
__device__ __forceinline__ double row_max8(double x) {
    x = fmax(x, dpp_f64<DPP_XOR1>(x));
    x = fmax(x, dpp_f64<DPP_XOR2>(x));
    return fmax(x, dpp_f64<DPP_HALF_MIRROR>(x));
}

template <int SEG, bool FULL>
__global__ __launch_bounds__(SWAVES * 64) void sweep_block_kernel(double* __restrict__ Wwork, int64_t d_out, int64_t d_in,
                                                         int64_t i1, int nb, const double* __restrict__ U,
                                                         int64_t g, QParams qp, double* __restrict__ Err,
                                                         int ldE, int errc, uint8_t* __restrict__ codes_s,
                                                         double* __restrict__ scale64, double* __restrict__ zero64,
                                                         float* __restrict__ scales, float* __restrict__ zeros,
                                                         double* __restrict__ loss64) {
    extern __shared__ __attribute__((aligned(16))) double sweep_lds[];
    // the sweep is the serial chain of the layer: its waves take issue
    // priority over GEMM waves of the other stream on the same SIMD
    __builtin_amdgcn_s_setprio(3);
    double* rinv = sweep_lds + UP_DOUBLES + CPL;
    const int tid = threadIdx.x, lane = tid & 63;
    const int part = lane & (LPR - 1);
    const int64_t row = (int64_t)blockIdx.x * ROWS + (tid >> 3);
    const bool live = row < d_out;
    const int64_t i2 = i1 + nb;
    const int cbase = part * CPL;  // first block column of this lane
    const int nbm = nb - 1;
    const double* Ub = U + i1 * d_in + i1;

    // stage the panels (zeros outside the nb x nb block) and 1 / U[c][c]:
    // every load of a thread issued before the first store
    constexpr int NSTG = UP_DOUBLES / 2 / (SWAVES * 64);   // 36 double pairs per thread
    static_assert(NSTG * SWAVES * 64 * 2 == UP_DOUBLES, "staging covers the panels");
    {
        double2 v[NSTG];
#pragma unroll
        for (int it = 0; it < NSTG; ++it) {
            const int e = tid + it * SWAVES * 64;
            int p = 0;
#pragma unroll
            for (int q = 1; q < LPR; ++q) p += (2 * e >= panel_base(q)) ? 1 : 0;
            const int off = 2 * e - panel_base(p);
            const int r = off / CPL, j = CPL * p + off % CPL;
            const bool rok = r < nb;
            const double* src = Ub + (int64_t)(rok ? r : 0) * d_in + j;
            if (FULL) {
                v[it].x = rok ? src[0] : 0.0;
                v[it].y = rok ? src[1] : 0.0;
            } else {
                v[it].x = (rok && j < nb) ? src[0] : 0.0;
                v[it].y = (rok && j + 1 < nb) ? src[1] : 0.0;
            }
        }
#pragma unroll
        for (int it = 0; it < NSTG; ++it) *(double2*)&sweep_lds[2 * (tid + it * SWAVES * 64)] = v[it];
    }
    if (tid < CPL) sweep_lds[UZERO + tid] = 0.0;
    for (int c = tid; c < nb; c += SWAVES * 64) rinv[c] = 1.0 / Ub[(int64_t)c * d_in + c];
    __syncthreads();
    // this lane's part of U row c: its panel row, or the zero row once the
    // panel has ended (c > 16 part + 15)
    const double* my_panel = sweep_lds + panel_base(part);
    auto load_urow = [&](double (&u)[CPL], int c) {
        const double* p = (c < cbase + CPL) ? my_panel + c * CPL : sweep_lds + UZERO;
#pragma unroll
        for (int kk = 0; kk < CPL; kk += 2) {
            const double2 v = *(const double2*)(p + kk);
            u[kk] = v.x;
            u[kk + 1] = v.y;
        }
    };

    double w[CPL];
    {
        const int64_t rr = live ? row : d_out - 1;
        const double* wrow = Wwork + rr * d_in + i1;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const int j = cbase + k;
            const double x = wrow[FULL ? j : (j < nbm ? j : nbm)];
            w[k] = (live && (FULL || j < nb)) ? x : 0.0;
        }
    }
    uint32_t pk[CPL / 4];
#pragma unroll
    for (int k = 0; k < CPL / 4; ++k) pk[k] = 0u;

    // current group parameters of this row (a group begun in an earlier
    // block is continued)
    double scale = 1.0, zero = 0.0, rscale = 1.0;
    const int64_t rem = i1 % g;
    if (rem != 0 && live) {
        scale = scale64[(i1 / g) * d_out + row];
        rscale = 1.0 / scale;
        zero = zero64[(i1 / g) * d_out + row];
    }
    int next_gs = (int)(rem == 0 ? 0 : g - rem);      // block column of the next group start
    int64_t next_gi = i1 / g + (rem == 0 ? 0 : 1);  // and its group index
    double loss = 0.0;

    // U rows of the next two columns in registers
    double ua[CPL], ub[CPL];
    load_urow(ua, 0);
    load_urow(ub, 1);

    for (int P = 0; P < LPR; ++P) {
        if (P * CPL >= nb) break;
#pragma unroll
        for (int s0 = 0; s0 < CPL; s0 += SEG) {
            const int cs = P * CPL + s0;
            if (!FULL && cs >= nb) break;
            if (cs == next_gs) {
                // group parameters from the group's current values: block
                // columns [cs, cend) in registers, later columns from Wwork
                const int64_t gend = (i1 + cs + g < d_in) ? i1 + cs + g : d_in;
                const int cend = (gend - i1 < nb) ? (int)(gend - i1) : nb;
                double xmin = 0.0, xmax = 0.0;
#pragma unroll
                for (int kk = 0; kk < CPL; ++kk) {
                    const int j = cbase + kk;
                    const bool in = j >= cs && j < cend;
                    xmin = fmin(xmin, in ? w[kk] : 0.0);
                    xmax = fmax(xmax, in ? w[kk] : 0.0);
                }
                if (live && cs > 0 && gend > i2) {
                    // a group begun inside the block and running past its
                    // end: the columns past the block still lack the
                    // compensation of this block's finished columns (their
                    // lazy update comes after the block), so it is applied
                    // here: v_j = W_j - sum over finished c of err_c U[c][j],
                    // each lane summing over its own columns, then the row
                    for (int64_t j = i2; j < gend; ++j) {
                        double p = 0.0;
#pragma unroll
                        for (int kk = 0; kk < CPL; ++kk) {
                            const int col = cbase + kk;
                            const bool done = col < cs;
                            const double u = Ub[(int64_t)(done ? col : 0) * d_in + (j - i1)];
                            p = done ? fma(w[kk], u, p) : p;
                        }
                        const double v = Wwork[row * d_in + j] - row_sum8(p);
                        xmin = fmin(xmin, v);
                        xmax = fmax(xmax, v);
                    }
                } else if (live) {
                    for (int64_t j = i2 + part; j < gend; j += LPR) {
                        const double v = Wwork[row * d_in + j];
                        xmin = fmin(xmin, v);
                        xmax = fmax(xmax, v);
                    }
                }
                xmin = row_min8(xmin);
                xmax = row_max8(xmax);
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
                rscale = 1.0 / scale;
                if (live && part == 0) {
                    scale64[next_gi * d_out + row] = scale;
                    zero64[next_gi * d_out + row] = zero;
                    scales[next_gi * d_out + row] = (float)scale;
                    zeros[next_gi * d_out + row] = (float)zero;
                }
                next_gs = cs + (int)g;
                ++next_gi;
            }
#pragma unroll
            for (int kq = 0; kq < SEG; ++kq) {
                const int k = s0 + kq;
                const int c = P * CPL + k;
                if (!FULL && c >= nb) break;
                // even columns use ua, odd ub; the buffer is refilled with
                // the row two columns ahead once this column has used it
                double (&u)[CPL] = (k & 1) ? ub : ua;
                const double ri = rinv[c];
                // quantize column c (meaningful in the owner lane, part == P);
                // the code is decided on the correctly rounded quotient w / scale.
                // y = w * (1/scale) is within 2^-51 |y| of that quotient, so
                // their nearest integers agree unless y lies within 2^-40
                // max(1, |y|) of a half-integer; only then is the quotient
                // formed (divergent, rare).
                const double x = w[k];
                double y = x * rscale;
                if (fabs(y - floor(y) - 0.5) <= 0x1p-40 * fmax(1.0, fabs(y))) y = x / scale;
                double code = rint(y) + zero;
                code = fmin(fmax(code, 0.0), qp.maxq);
                const double q = scale * (code - zero);
                const double diff = x - q;
                const double t = diff * ri;
                const bool own = part == P;
                const double err = row_sum8(own ? t : 0.0);
                loss = own ? fma(0.5 * t, t, loss) : loss;
                pk[k >> 2] = own ? (pk[k >> 2] | ((uint32_t)code << (8 * (k & 3)))) : pk[k >> 2];
                // compensation of the later columns of the block (earlier
                // columns meet zeros of U below the diagonal)
#pragma unroll
                for (int kk = 0; kk < CPL; ++kk) w[kk] = fma(-err, u[kk], w[kk]);
                w[k] = own ? err : w[k];
                load_urow(u, c + 2);
            }
        }
    }

    // errors and codes of this row's columns back to HBM
    if (live) {
        double* erow = Err + row * ldE + errc + cbase;
        uint8_t* crow = codes_s + row * d_in + i1 + cbase;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            if (FULL || cbase + k < nb) {
                erow[k] = w[k];
                crow[k] = (uint8_t)(pk[k >> 2] >> (8 * (k & 3)));
            }
        }
    }
    // row loss: the eight parts summed in a fixed order
    loss = row_sum8(loss);
    if (live && part == 0) loss64[row] += loss;
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
    // group starts fall on multiples of SEG block columns
    int SEG = CPL;
    while (SEG > 1 && ((B % SEG) != 0 || (cfg->group_size > 0 && (g % SEG) != 0))) SEG >>= 1;
    GPTQ_HIP(hipMemsetAsync(w.flags, 0, 256, s));

    const unsigned gx = (unsigned)ceil_div(d_in, 256);
    hipLaunchKernelGGL(convert_kernel, dim3(gx, (unsigned)d_out), dim3(256), 0, s, W, dt, d_out, d_in, ld_w, perm,
                       w.Wwork, w.loss64, w.flags);
    GPTQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(fill_neg_kernel, dim3(gx), dim3(256), 0, s, w.pinv, d_in);
    GPTQ_LAUNCH_CHECK();
    hipLaunchKernelGGL(pinv_kernel, dim3(gx), dim3(256), 0, s, perm, d_in, g, w.pinv, g_idx);
    GPTQ_LAUNCH_CHECK();

    QParams qp{cfg->bits, cfg->sym, (double)((1 << cfg->bits) - 1)};
    const unsigned grid = (unsigned)ceil_div(d_out, ROWS);
#define SWEEP_ATTR(n, f)                                                                                        \
    GPTQ_HIP(hipFuncSetAttribute((const void*)sweep_block_kernel<n, f>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                 (int)SWEEP_LDS));
    SWEEP_ATTR(16, true)
    SWEEP_ATTR(16, false)
    SWEEP_ATTR(8, true)
    SWEEP_ATTR(8, false)
    SWEEP_ATTR(4, true)
    SWEEP_ATTR(4, false)
    SWEEP_ATTR(2, true)
    SWEEP_ATTR(2, false)
    SWEEP_ATTR(1, true)
    SWEEP_ATTR(1, false)
#undef SWEEP_ATTR
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
            const bool full = nb == BMAX;
            switch (SEG * 2 + (full ? 1 : 0)) {
#define SWEEP_CASE(n, f)                                                                                      \
    case n * 2 + f:                                                                                           \
        hipLaunchKernelGGL((sweep_block_kernel<n, f>), dim3(grid), dim3(SWAVES * 64), SWEEP_LDS, s, w.Wwork,     \
                           d_out, d_in, i1,                                                                 \
                           nb, U, g, qp, Ek, (int)S, (int)(i1 - a), w.codes_s, w.scale64, w.zero64, scales,  \
                           zeros, w.loss64);                                                                  \
        break;
                SWEEP_CASE(16, 1)
                SWEEP_CASE(16, 0)
                SWEEP_CASE(8, 1)
                SWEEP_CASE(8, 0)
                SWEEP_CASE(4, 1)
                SWEEP_CASE(4, 0)
                SWEEP_CASE(2, 1)
                SWEEP_CASE(2, 0)
                SWEEP_CASE(1, 1)
                SWEEP_CASE(1, 0)
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
                                 d_in, false, 1.0, w.Wwork + e + n_near, d_in, false, GEMM_TRI_NONE, true);
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
