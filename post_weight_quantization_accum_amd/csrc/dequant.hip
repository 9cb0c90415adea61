// Products with the quantized weights, Y = X W_hat^T, computed straight from
// the packed codes ("通义千问1.5-1.8B-Chat-GPTQ-Int4模型压缩技术解析" §2.2: INT4
// weights with a scale / zero point per group are turned back into weights
// for the computation while activations keep their precision;
// "gptq-for-llama" article, "工程细节": dedicated matrix-product kernels over
// packed 4-bit codes; "GPTQ论文复现指南" §5.2: a dedicated kernel for speed;
// "GPTQ量化算法深度解析" §3.3: act-order needs an extra gather at
// inference).
//
//   W_hat[r][j] = scale[g(j)][r] * (code[r][j] - zero[g(j)][r]),
//   Y[t][r]     = sum_j X[t][j] * W_hat[r][j].
//
// Decode-sized token counts: the packed words are the bytes that matter.  A
// workgroup owns RW = 8 output rows and reads each of their words once;
// thread k takes the 32-column blocks k, k + 256, ... (32 columns are
// exactly `bits` words of a row).  Partial sums meet at the end (halving
// exchange inside each wave, then LDS).  Two inner loops:
//
// * block path (each 32-column block inside one group: no g_idx, group size
//   a multiple of 32 or one group per row).  The codes of a row are turned
//   into pairs of half-precision values 2^b + c by placing c in the top b
//   mantissa bits under the exponent of 2^b (exact), and multiplied with the
//   matching pair of activations by one v_dot2 (float32 accumulation):
//     D = sum_blk x (2^b + c),   Y += s * (D - (2^b + z) * sum_blk x),
//   which equals s * sum x (c - z).  About 1.5 vector instructions per
//   weight for one token.  With `perm` the packed stream is in sorted
//   (group-contiguous) order and the activations are gathered through perm.
//
// * column path (g_idx in the original column order, any group size, fp32
//   activations, 8-bit codes with bf16 activations): per column the group is
//   looked up, the scales and zeros of the workgroup's rows come from LDS
//   ([group][row]), w = s * (c - z) in float32 and one FMA per token.
#include "internal.hpp"

namespace gptq {
namespace {

constexpr int RW = 8;                      // output rows per workgroup
constexpr int DQ_THREADS = 256;
constexpr int DQ_WAVES = DQ_THREADS / 64;
constexpr int64_t DQ_MAX_GROUPS = 2048;    // column path: 8 rows x 2 floats x 2048 groups = 128 KiB of LDS

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));

struct DqArgs {
    const void* X;
    int64_t n_tok, d_in, ld_x;
    const uint32_t* packed;
    int64_t wpr;                 // words per packed row
    const float* scales;         // [n_groups][d_out]
    const float* zeros;          // [n_groups][d_out]
    const int32_t* g_idx;        // column path only; null: g = position / gsize
    const int32_t* perm;         // null, or stream position -> activation column
    int64_t gsize;               // d_in when there is one group per row
    int64_t n_groups, d_out;
    float* Y;
    int64_t ld_y;
    int xvec;                    // X 16-byte aligned rows (bf16 / f16 only)
    int wvec;                    // packed rows aligned for vector word loads
};

// Activation storage types: raw 16-bit patterns for bf16 and f16, float for f32.
struct Bf16 {
    typedef uint16_t store;
    static constexpr int MB = 7, BIAS = 127;
    static constexpr uint32_t NAN_BITS = 0x7FC0u, ONES = 0x3F803F80u;
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a), __builtin_bit_cast(b2_t, b), c, false);
    }
    static __device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }
};
struct F16 {
    typedef uint16_t store;
    static constexpr int MB = 10, BIAS = 15;
    static constexpr uint32_t NAN_BITS = 0x7E00u, ONES = 0x3C003C00u;
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c, false);
    }
    static __device__ __forceinline__ float to_f32(uint16_t v) { return (float)__builtin_bit_cast(_Float16, v); }
};
struct F32 {
    typedef float store;
    static __device__ __forceinline__ float to_f32(float v) { return v; }
};

// code k (0..31) of a 32-column block held in `bits` words
template <int BITS>
__device__ __forceinline__ uint32_t block_code(const uint32_t (&w)[BITS], int k) {
    const int pos = BITS * k, wi = pos >> 5, sh = pos & 31;
    uint32_t v = w[wi] >> sh;
    if (sh + BITS > 32) v |= w[wi + 1] << (32 - sh);
    return v & ((1u << BITS) - 1u);
}

// Columns (a, b) of pair i (0..15) in the block path: for 2-, 4- and 8-bit
// codes the pair is code ii and code ii + H of word m (16 bits apart, so one
// shift and one mask place both); for 3-bit codes, codes i and i + 16.
template <int BITS>
__device__ __forceinline__ int pair_col_a(int i) {
    if constexpr (BITS == 3) {
        return i;
    } else {
        constexpr int CPW = 32 / BITS, H = CPW / 2;
        return (i / H) * CPW + (i % H);
    }
}
template <int BITS>
__device__ __forceinline__ int pair_col_b(int i) {
    if constexpr (BITS == 3) {
        return i + 16;
    } else {
        return pair_col_a<BITS>(i) + 16 / BITS;
    }
}

// Pair i of one row's block as two half-precision values (2^b + c_a, 2^b + c_b).
template <int BITS, typename T>
__device__ __forceinline__ uint32_t code_pair(const uint32_t (&w)[BITS], int i) {
    constexpr int SH = T::MB - BITS;
    static_assert(SH >= 0, "codes must fit the mantissa");
    constexpr uint32_t E = (uint32_t)(T::BIAS + BITS) << T::MB;
    constexpr uint32_t EXPO = E | (E << 16);
    if constexpr (BITS == 3) {
        const uint32_t ca = block_code<3>(w, i), cb = block_code<3>(w, i + 16);
        return (ca << SH) | (cb << (SH + 16)) | EXPO;
    } else {
        constexpr int CPW = 32 / BITS, H = CPW / 2;
        constexpr uint32_t M1 = ((1u << BITS) - 1u) << SH;
        constexpr uint32_t MASK = M1 | (M1 << 16);
        const int m = i / H, p = BITS * (i % H);
        const uint32_t v = (p >= SH) ? (w[m] >> (p - SH)) : (w[m] << (SH - p));
        return (v & MASK) | EXPO;
    }
}

// The `bits` words of block blk of one row (zeros past the row's end).
template <int BITS>
__device__ __forceinline__ void load_words(const DqArgs& a, int64_t row, bool row_ok, int64_t blk,
                                           uint32_t (&w)[BITS]) {
    const int64_t w0 = blk * BITS;
    const uint32_t* p = a.packed + row * a.wpr + w0;
    if (row_ok && a.wvec && w0 + BITS <= a.wpr) {
        if constexpr (BITS == 2) {
            const uint2 v = *(const uint2*)p;
            w[0] = v.x;
            w[1] = v.y;
        } else if constexpr (BITS == 4 || BITS == 8) {
#pragma unroll
            for (int q = 0; q < BITS; q += 4) {
                const uint4 v = *(const uint4*)(p + q);
                w[q] = v.x;
                w[q + 1] = v.y;
                w[q + 2] = v.z;
                w[q + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < BITS; ++q) w[q] = p[q];
        }
    } else {
#pragma unroll
        for (int q = 0; q < BITS; ++q) w[q] = (row_ok && w0 + q < a.wpr) ? p[q] : 0u;
    }
}

// Activation column of stream position j (j < d_in), or -1 if perm names a
// column outside [0, d_in).
__device__ __forceinline__ int64_t act_col(const DqArgs& a, int64_t j) {
    if (!a.perm) return j;
    const int32_t c = a.perm[j];
    return ((uint32_t)c < (uint64_t)a.d_in) ? (int64_t)c : -1;
}

// Sum of NV per-thread values over the workgroup; thread i < NV returns value i.
template <int NV>
__device__ __forceinline__ float wg_reduce(float (&v)[NV], float (*red)[64], int tid, bool& have) {
    static_assert((NV & (NV - 1)) == 0 && NV <= 64, "power of two, one per lane");
    const int lane = tid & 63, wave = tid >> 6;
    // halving exchange: after the level with distance h a lane keeps half of
    // its values (the upper half if bit h of its lane is set) plus the
    // partner's copy of the same half; lane l ends with value (l mod NV)
#pragma unroll
    for (int h = NV / 2; h >= 1; h >>= 1) {
        const bool up = (lane & h) != 0;
#pragma unroll
        for (int e = 0; e < h; ++e) {
            const float keep = up ? v[e + h] : v[e];
            const float give = up ? v[e] : v[e + h];
            v[e] = keep + __shfl_xor(give, h, 64);
        }
    }
#pragma unroll
    for (int m = NV; m < 64; m <<= 1) v[0] += __shfl_xor(v[0], m, 64);
    red[wave][lane] = v[0];
    __syncthreads();
    have = tid < NV;
    float s = 0.0f;
    if (have) {
#pragma unroll
        for (int w = 0; w < DQ_WAVES; ++w) s += red[w][tid];
    }
    return s;
}

template <int TM>
__device__ __forceinline__ void store_y(const DqArgs& a, float (&acc)[TM][RW], float (*red)[64], int tid,
                                        int64_t r0, int nr, int64_t t0, int nt) {
    constexpr int NV = TM * RW;
    float v[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) v[e] = acc[e / RW][e % RW];
    bool have;
    const float s = wg_reduce<NV>(v, red, tid, have);
    if (have) {
        const int t = tid / RW, rr = tid % RW;
        if (t < nt && rr < nr) a.Y[(t0 + t) * a.ld_y + r0 + rr] = s;
    }
}

// ---------------------------------------------------------------------------
// Block path.
// ---------------------------------------------------------------------------
template <int BITS, int TM, typename T>
__global__ __launch_bounds__(DQ_THREADS) void dequant_block_kernel(DqArgs a) {
    __shared__ float red[DQ_WAVES][64];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * RW, t0 = (int64_t)blockIdx.y * TM;
    const int nr = (a.d_out - r0 < RW) ? (int)(a.d_out - r0) : RW;
    const int nt = (a.n_tok - t0 < TM) ? (int)(a.n_tok - t0) : TM;
    const uint16_t* X = (const uint16_t*)a.X;
    constexpr float OFF = (float)(1 << BITS);

    float acc[TM][RW];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) acc[t][rr] = 0.0f;

    const int64_t nblk = ceil_div(a.d_in, 32);
    for (int64_t blk = tid; blk < nblk; blk += DQ_THREADS) {
        const int64_t j0 = blk * 32;
        uint32_t wd[RW][BITS];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) load_words<BITS>(a, r0 + rr, rr < nr, blk, wd[rr]);
        const int64_t g = j0 / a.gsize;
        float sv[RW], ov[RW];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            sv[rr] = rr < nr ? a.scales[g * a.d_out + r0 + rr] : 0.0f;
            ov[rr] = OFF + (rr < nr ? a.zeros[g * a.d_out + r0 + rr] : 0.0f);
        }
        // activation pairs matching the code pairs, per token
        const bool full = j0 + 32 <= a.d_in;
        const bool vec = a.xvec && full && !a.perm;
        int32_t col[32];
        if (!vec) {
#pragma unroll
            for (int k = 0; k < 32; ++k) col[k] = (j0 + k < a.d_in) ? (int32_t)act_col(a, j0 + k) : -2;
        }
        uint32_t xp[TM][16];
        float xs[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const bool tok = t < nt;
            const uint16_t* xr = X + (t0 + t) * a.ld_x;
            if (vec) {
                uint32_t dd[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 v = tok ? *(const uint4*)(xr + j0 + 8 * q) : make_uint4(0, 0, 0, 0);
                    dd[4 * q] = v.x;
                    dd[4 * q + 1] = v.y;
                    dd[4 * q + 2] = v.z;
                    dd[4 * q + 3] = v.w;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int ca = pair_col_a<BITS>(i), cb = pair_col_b<BITS>(i);
                    xp[t][i] = __builtin_amdgcn_perm(dd[cb >> 1], dd[ca >> 1], (ca & 1) ? 0x07060302u : 0x05040100u);
                }
            } else {
                uint32_t u[32];
#pragma unroll
                for (int k = 0; k < 32; ++k)
                    u[k] = (!tok || col[k] == -2) ? 0u : (col[k] < 0 ? T::NAN_BITS : (uint32_t)xr[col[k]]);
#pragma unroll
                for (int i = 0; i < 16; ++i) xp[t][i] = u[pair_col_a<BITS>(i)] | (u[pair_col_b<BITS>(i)] << 16);
            }
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) s = T::dot2(xp[t][i], T::ONES, s);
            xs[t] = s;
        }
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            uint32_t cp[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) cp[i] = code_pair<BITS, T>(wd[rr], i);
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                float d = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) d = T::dot2(xp[t][i], cp[i], d);
                acc[t][rr] = fmaf(sv[rr], fmaf(-ov[rr], xs[t], d), acc[t][rr]);
            }
        }
    }
    store_y<TM>(a, acc, red, tid, r0, nr, t0, nt);
}

// ---------------------------------------------------------------------------
// Column path.
// ---------------------------------------------------------------------------
// One token per workgroup row of the grid (blockIdx.y): the per-column
// group indices and activations of a block are gathered first (32 + 32
// independent loads), then each column costs two LDS reads of 32 bytes
// (scales and zeros of the 8 rows) and per row one dequantization and one FMA.
template <int BITS, typename T>
__global__ __launch_bounds__(DQ_THREADS) void dequant_col_kernel(DqArgs a) {
    extern __shared__ __attribute__((aligned(16))) float sz[];   // scales [n_groups][RW], then zeros
    __shared__ float red[DQ_WAVES][64];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * RW, t0 = blockIdx.y;
    const int nr = (a.d_out - r0 < RW) ? (int)(a.d_out - r0) : RW;
    const typename T::store* xr = (const typename T::store*)a.X + t0 * a.ld_x;
    float* s_lds = sz;
    float* z_lds = sz + a.n_groups * RW;
    for (int64_t e = tid; e < a.n_groups * RW; e += DQ_THREADS) {
        const int64_t g = e / RW;
        const int rr = (int)(e % RW);
        s_lds[e] = rr < nr ? a.scales[g * a.d_out + r0 + rr] : 0.0f;
        z_lds[e] = rr < nr ? a.zeros[g * a.d_out + r0 + rr] : 0.0f;
    }
    __syncthreads();

    float acc[1][RW];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) acc[0][rr] = 0.0f;

    const int64_t nblk = ceil_div(a.d_in, 32);
    for (int64_t blk = tid; blk < nblk; blk += DQ_THREADS) {
        const int64_t j0 = blk * 32;
        uint32_t wd[RW][BITS];
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) load_words<BITS>(a, r0 + rr, rr < nr, blk, wd[rr]);
        // group (LDS row offset) and activation of each column of the block
        int32_t gk[32];
        float xk[32];
        {
            // without g_idx: the group of the block's first position, advanced
            // by one at each boundary (at most one per column)
            int64_t g_run = j0 / a.gsize, g_end = (g_run + 1) * a.gsize;
#pragma unroll
            for (int k = 0; k < 32; ++k) {
                const int64_t j = j0 + k;
                if (j >= g_end) {
                    ++g_run;
                    g_end += a.gsize;
                }
                const bool jok = j < a.d_in;
                int32_t g = (int32_t)g_run;
                if (a.g_idx) g = jok ? a.g_idx[j] : 0;
                const bool bad_g = (uint32_t)g >= (uint64_t)a.n_groups;
                const int64_t c = jok ? act_col(a, j) : 0;
                gk[k] = bad_g || !jok ? 0 : g * RW;
                xk[k] = !jok ? 0.0f : ((c < 0 || bad_g) ? __builtin_nanf("") : T::to_f32(xr[c]));
            }
        }
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            const float4 s0 = *(const float4*)&s_lds[gk[k]], s1 = *(const float4*)&s_lds[gk[k] + 4];
            const float4 z0 = *(const float4*)&z_lds[gk[k]], z1 = *(const float4*)&z_lds[gk[k] + 4];
            const float sv[RW] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
            const float zv[RW] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
            for (int rr = 0; rr < RW; ++rr) {
                const float w = sv[rr] * ((float)block_code<BITS>(wd[rr], k) - zv[rr]);
                acc[0][rr] = fmaf(xk[k], w, acc[0][rr]);
            }
        }
    }
    store_y<1>(a, acc, red, tid, r0, nr, t0, 1);
}

template <int BITS, typename T>
gptq_status launch_col(const DqArgs& a, hipStream_t s) {
    const size_t lds = (size_t)a.n_groups * RW * 2 * sizeof(float);
    if (lds > 48 * 1024) {
        static const hipError_t attr = hipFuncSetAttribute(
            (const void*)dequant_col_kernel<BITS, T>, hipFuncAttributeMaxDynamicSharedMemorySize,
            (int)(DQ_MAX_GROUPS * RW * 2 * sizeof(float)));
        if (attr != hipSuccess) return GPTQ_ERR_HIP;
    }
    const dim3 grid((unsigned)ceil_div(a.d_out, RW), (unsigned)a.n_tok);
    hipLaunchKernelGGL((dequant_col_kernel<BITS, T>), grid, dim3(DQ_THREADS), lds, s, a);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

template <int BITS, int TM, typename T>
gptq_status launch_block(const DqArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)ceil_div(a.d_out, RW), (unsigned)ceil_div(a.n_tok, TM));
    hipLaunchKernelGGL((dequant_block_kernel<BITS, TM, T>), grid, dim3(DQ_THREADS), 0, s, a);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

template <typename T>
gptq_status by_bits_col(const DqArgs& a, int bits, hipStream_t s) {
    switch (bits) {
        case 2: return launch_col<2, T>(a, s);
        case 3: return launch_col<3, T>(a, s);
        case 4: return launch_col<4, T>(a, s);
        case 8: return launch_col<8, T>(a, s);
    }
    return GPTQ_ERR_INVALID_ARG;
}

template <int TM, typename T>
gptq_status by_bits_block(const DqArgs& a, int bits, hipStream_t s) {
    switch (bits) {
        case 2: return launch_block<2, TM, T>(a, s);
        case 3: return launch_block<3, TM, T>(a, s);
        case 4: return launch_block<4, TM, T>(a, s);
        case 8:
            if constexpr (T::MB - 8 >= 0) return launch_block<8, TM, T>(a, s);
            break;
    }
    return GPTQ_ERR_INVALID_ARG;
}

template <int TM>
gptq_status dispatch_block(const DqArgs& a, gptq_dtype dt, int bits, hipStream_t s) {
    if (dt == GPTQ_BF16) return by_bits_block<TM, Bf16>(a, bits, s);
    return by_bits_block<TM, F16>(a, bits, s);
}

}  // namespace

int64_t dequant_max_groups() { return DQ_MAX_GROUPS; }

bool dequant_uses_block_path(gptq_dtype dt, int32_t bits, int64_t d_in, int64_t group_size, bool has_g_idx) {
    if (has_g_idx || dt == GPTQ_F32) return false;
    if (dt == GPTQ_BF16 && bits == 8) return false;
    return group_size <= 0 || group_size >= d_in || (group_size % 32) == 0;
}

gptq_status dequant_matmul_launch(const void* X, gptq_dtype dt, int64_t n_tok, int64_t d_in, int64_t ld_x,
                                  const uint32_t* packed, int32_t bits, const float* scales, const float* zeros,
                                  int64_t n_groups, const int32_t* g_idx, const int32_t* perm, int64_t group_size,
                                  int64_t d_out, float* Y, int64_t ld_y, hipStream_t s) {
    if (n_tok == 0 || d_out == 0) return GPTQ_OK;
    DqArgs a;
    a.X = X;
    a.n_tok = n_tok;
    a.d_in = d_in;
    a.ld_x = ld_x;
    a.packed = packed;
    a.wpr = ceil_div(d_in * bits, 32);
    a.scales = scales;
    a.zeros = zeros;
    a.g_idx = g_idx;
    a.perm = perm;
    a.gsize = (group_size > 0 && group_size < d_in) ? group_size : (d_in > 0 ? d_in : 1);
    a.n_groups = n_groups;
    a.d_out = d_out;
    a.Y = Y;
    a.ld_y = ld_y;
    const size_t xb = dt == GPTQ_F32 ? 4 : 2;
    a.xvec = (dt != GPTQ_F32) && ((uintptr_t)X % 16 == 0) && ((ld_x * (int64_t)xb) % 16 == 0);
    const size_t wal = bits == 2 ? 8 : (bits == 3 ? 4 : 16);
    const int64_t wmul = bits == 2 ? 2 : (bits == 3 ? 1 : 4);
    a.wvec = ((uintptr_t)packed % wal == 0) && (a.wpr % wmul == 0);
    const bool block_path = dequant_uses_block_path(dt, bits, d_in, group_size, g_idx != nullptr);
    if (!block_path && n_groups > DQ_MAX_GROUPS) return GPTQ_ERR_UNSUPPORTED;
    // the grid's y dimension (token tiles) stays below 65536: larger token
    // counts go in several launches
    const int64_t tm = block_path ? (n_tok == 1 ? 1 : 4) : 1;
    const int64_t chunk = 65535 * tm;
    for (int64_t t0 = 0; t0 < n_tok; t0 += chunk) {
        DqArgs c = a;
        c.n_tok = (n_tok - t0 < chunk) ? n_tok - t0 : chunk;
        c.X = (const char*)X + t0 * ld_x * (int64_t)xb;
        c.Y = Y + t0 * ld_y;
        gptq_status st;
        if (!block_path) {
            if (dt == GPTQ_BF16) st = by_bits_col<Bf16>(c, bits, s);
            else if (dt == GPTQ_F16) st = by_bits_col<F16>(c, bits, s);
            else st = by_bits_col<F32>(c, bits, s);
        } else if (tm == 1) {
            st = dispatch_block<1>(c, dt, bits, s);
        } else {
            st = dispatch_block<4>(c, dt, bits, s);
        }
        if (st != GPTQ_OK) return st;
    }
    return GPTQ_OK;
}

}  // namespace gptq
