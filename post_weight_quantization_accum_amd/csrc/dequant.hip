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
#include <type_traits>

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
};

// Activation storage types: raw 16-bit patterns for bf16 and f16, float for f32.
struct Bf16 {
    typedef uint16_t store;
    typedef bf16x8_t mfma_tag;
    static constexpr int MB = 7, BIAS = 127;
    static constexpr uint32_t NAN_BITS = 0x7FC0u, ONES = 0x3F803F80u;
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a), __builtin_bit_cast(b2_t, b), c, false);
    }
    static __device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }
};
struct F16 {
    typedef uint16_t store;
    typedef h16x8_t mfma_tag;
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

// (x & m) | c in one instruction (VOP3 v_and_or_b32: the mask from an SGPR,
// the exponent bits from a VGPR).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
    return r;
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
        const uint32_t v = (p == SH) ? w[m] : ((p > SH) ? (w[m] >> (p - SH)) : (w[m] << (SH - p)));
        return and_or(v, MASK, EXPO);
    }
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));

// Buffer resource over the packed rows from r0 to the end of the matrix (at
// most 2 GiB: a workgroup reads 8 rows).  Offsets past its end read zeros,
// so the loads need no branches: rows past d_out read zeros, and a block
// that runs past the end of a row reads words of the next row, which meet
// activations that are zero there.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t words_rsrc(const DqArgs& a, int64_t r0) {
    const int64_t bytes = (a.d_out - r0) * a.wpr * 4;
    const int n = bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(a.packed + r0 * a.wpr), (short)0, n, 0x00020000);
}

// the `bits` words of block blk of the 8 rows; a block past the row's last
// (blk >= nblk) gets an offset past the buffer's end: zeros, no memory access
template <int BITS>
__device__ __forceinline__ void load_block_words(__amdgpu_buffer_rsrc_t rs, uint32_t row_bytes, uint32_t blk,
                                                 uint32_t nblk, uint32_t (&w)[RW][BITS]) {
    const uint32_t off = blk < nblk ? blk * (uint32_t)(BITS * 4) : 0x80000000u;
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
        const uint32_t o = off + (uint32_t)rr * row_bytes;
        if constexpr (BITS == 2) {
            const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0);
            w[rr][0] = v.x;
            w[rr][1] = v.y;
        } else if constexpr (BITS == 3) {
            const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(rs, o, 0, 0);
            w[rr][0] = v.x;
            w[rr][1] = v.y;
            w[rr][2] = v.z;
        } else {
#pragma unroll
            for (int q = 0; q < BITS; q += 4) {
                const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, o + 4 * q, 0, 0);
                w[rr][q] = v.x;
                w[rr][q + 1] = v.y;
                w[rr][q + 2] = v.z;
                w[rr][q + 3] = v.w;
            }
        }
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
    const __amdgpu_buffer_rsrc_t rs = words_rsrc(a, r0);
    const uint32_t row_bytes = (uint32_t)a.wpr * 4;

    float acc[TM][RW];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) acc[t][rr] = 0.0f;

    const int64_t nblk = ceil_div(a.d_in, 32);
    for (int64_t blk = tid; blk < nblk; blk += DQ_THREADS) {
        const int64_t j0 = blk * 32;
        uint32_t wd[RW][BITS];
        load_block_words<BITS>(rs, row_bytes, (uint32_t)blk, (uint32_t)nblk, wd);
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
    const __amdgpu_buffer_rsrc_t rs = words_rsrc(a, r0);
    const uint32_t row_bytes = (uint32_t)a.wpr * 4;
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
        load_block_words<BITS>(rs, row_bytes, (uint32_t)blk, (uint32_t)nblk, wd);
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
        GPTQ_HIP(ensure_lds_limit((const void*)dequant_col_kernel<BITS, T>, (int)(DQ_MAX_GROUPS * RW * 2 * sizeof(float))));
    }
    const dim3 grid((unsigned)ceil_div(a.d_out, RW), (unsigned)a.n_tok);
    hipLaunchKernelGGL((dequant_col_kernel<BITS, T>), grid, dim3(DQ_THREADS), lds, s, a);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

// ---------------------------------------------------------------------------
// Block route with the activations and the group parameters staged in LDS.
//
// Each workgroup first copies, with coalesced loads, the scales and
// (2^b + zero) of its 8 rows ([group][row] floats) and the activations of its
// tokens in stream order (gathered through perm when given: the activation
// row goes to LDS whole, then each stream position reads its column from
// there) into LDS; 32-column blocks sit 80 bytes apart, which keeps the
// 16-byte LDS reads of consecutive lanes on distinct banks.  The lanes then
// read only their packed words from global memory (one block ahead) and
// everything else from LDS.  Used whenever the staging fits in LDS.
// ---------------------------------------------------------------------------
constexpr int XS_STRIDE = 40;                   // 16-bit slots per 32-column block (64 B + 16 B pad)
constexpr size_t STAGED_LDS_MAX = 150 * 1024;

struct StagedLayout {
    size_t o_off, xs_off, xf_off, total;
};

__host__ __device__ inline StagedLayout staged_layout(int64_t n_groups, int64_t nblk, int64_t d_in, int tm,
                                                      bool perm) {
    StagedLayout L;
    L.o_off = (size_t)n_groups * 2 * RW * sizeof(float);
    L.xs_off = align_up(2 * L.o_off, 16);
    L.xf_off = L.xs_off + align_up((size_t)tm * nblk * XS_STRIDE * 2, 16);
    L.total = L.xf_off + (perm ? align_up((size_t)d_in * 2, 16) : 0);
    return L;
}

// One activation row (d_in 16-bit values, zeros up to n) from global memory
// into LDS: element k goes to dst[(k / 32) * XS_STRIDE + k % 32] (blocked) or
// dst[k] (flat).  Loads are issued in batches (clamped addresses, unused
// values dropped) so that their latencies overlap.
template <bool BLOCKED>
__device__ __forceinline__ uint16_t* slot(uint16_t* dst, uint32_t k) {
    return BLOCKED ? dst + (k >> 5) * XS_STRIDE + (k & 31) : dst + k;
}

// skip_pc: whole pieces [0, skip_pc) are already stored (vector route only).
template <bool BLOCKED, int NT>
__device__ __forceinline__ void copy_row(const DqArgs& a, const uint16_t* __restrict__ xr, uint16_t* dst,
                                         uint32_t n, int tid, uint32_t skip_pc) {
    const uint32_t d_in = (uint32_t)a.d_in;
    uint32_t done = 0;
    if (a.xvec) {
        // whole 16-byte pieces of 8 columns
        const uint32_t npc = d_in / 8;
        constexpr int B = 8;
        for (uint32_t p0 = skip_pc + tid; p0 < npc; p0 += NT * B) {
            uint4 v[B];
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const uint32_t p = p0 + NT * i;
                v[i] = *(const uint4*)(xr + 8 * (p < npc ? p : 0));
            }
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const uint32_t p = p0 + NT * i;
                if (p < npc) *(uint4*)slot<BLOCKED>(dst, 8 * p) = v[i];
            }
        }
        done = 8 * npc;
    }
    constexpr int B = 8;
    for (uint32_t k0 = done + tid; k0 < n; k0 += NT * B) {
        uint16_t v[B];
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const uint32_t k = k0 + NT * i;
            v[i] = xr[k < d_in ? k : 0];
        }
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const uint32_t k = k0 + NT * i;
            if (k < n) *slot<BLOCKED>(dst, k) = k < d_in ? v[i] : (uint16_t)0;
        }
    }
}

// 512 threads: two halves of 256 lanes, each half owning 8 of the
// workgroup's 16 rows and sharing the staged activations.
constexpr int ST_THREADS = 512;
constexpr int ST_ROWS = 2 * RW;

template <int BITS, int TM, typename T>
__global__ __launch_bounds__(ST_THREADS) void dequant_staged_kernel(DqArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ float red[ST_THREADS / 64][64];
    const int tid = threadIdx.x, half = tid >> 8;
    // lane index within the half; the second half counts down, so that lanes
    // with one block more than the others (the low lane indices) sit in waves
    // 0-1 of the first half and waves 6-7 of the second: on different SIMDs
    const int tl = half ? 255 - (tid & 255) : tid;
    const int64_t rw0 = (int64_t)blockIdx.x * ST_ROWS;              // first row of the workgroup
    const int64_t r0 = rw0 + half * RW;                             // first row of this half
    const int nrw = (a.d_out - rw0 < ST_ROWS) ? (int)(a.d_out - rw0) : ST_ROWS;
    const int nr = (a.d_out - r0 < RW) ? (a.d_out - r0 > 0 ? (int)(a.d_out - r0) : 0) : RW;
    const int64_t t0 = (int64_t)blockIdx.y * TM;
    const int nt = (a.n_tok - t0 < TM) ? (int)(a.n_tok - t0) : TM;
    const uint32_t nblk = (uint32_t)ceil_div(a.d_in, 32);
    const StagedLayout Ly = staged_layout(a.n_groups, nblk, a.d_in, TM, a.perm != nullptr);
    float* s_l = (float*)lds;                                       // [group][16] scales
    float* o_l = (float*)(lds + Ly.o_off);                          // [group][16] 2^b + zero
    uint16_t* xs = (uint16_t*)(lds + Ly.xs_off);
    uint16_t* xf = (uint16_t*)(lds + Ly.xf_off);
    const uint16_t* X = (const uint16_t*)a.X;
    constexpr float OFF = (float)(1 << BITS);
    const __amdgpu_buffer_rsrc_t rs = words_rsrc(a, r0 < a.d_out ? r0 : a.d_out);
    const uint32_t row_bytes = (uint32_t)a.wpr * 4;
    const uint32_t d_in = (uint32_t)a.d_in;
    const uint32_t ncol = nblk * 32;
    const uint32_t nsz = (uint32_t)a.n_groups * ST_ROWS;
    const uint32_t npc = a.xvec ? d_in / 8 : 0;       // whole 16-byte pieces of an activation row

    // Phase 1: the first batch of every staging load, then the packed words of
    // the lane's first two blocks, all in flight together.
    constexpr int BS = 4, BX = 4, BP = 24;
    float sv0[BS], zv0[BS];
#pragma unroll
    for (int i = 0; i < BS; ++i) {
        const uint32_t e = tid + ST_THREADS * i;
        const int64_t idx = (e < nsz && (int)(e % ST_ROWS) < nrw) ? (int64_t)(e / ST_ROWS) * a.d_out + rw0 + e % ST_ROWS : 0;
        sv0[i] = a.scales[idx];
        zv0[i] = a.zeros[idx];
    }
    // token t0 (it exists: nt >= 1); whole 16-byte pieces through a
    // bounds-checked buffer, so that the loads need no branch
    const uint16_t* xr0 = X + t0 * a.ld_x;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)xr0, (short)0, (int)(npc * 16),
                                                                       0x00020000);
    u32x4_t xv0[BX];
#pragma unroll
    for (int i = 0; i < BX; ++i) xv0[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, (tid + ST_THREADS * i) * 16, 0, 0);
    int32_t cp[BP];
    if (a.perm) {
#pragma unroll
        for (int i = 0; i < BP; ++i) {
            const uint32_t k = tid + ST_THREADS * i;
            cp[i] = a.perm[k < d_in ? k : 0];
        }
    }
    uint32_t blk = tl;
    uint32_t wd[RW][BITS], wn[RW][BITS];
    load_block_words<BITS>(rs, row_bytes, blk, nblk, wd);
    load_block_words<BITS>(rs, row_bytes, blk + 256, nblk, wn);

    // Phase 2: LDS stores; anything past the first batch is staged in batches.
#pragma unroll
    for (int i = 0; i < BS; ++i) {
        const uint32_t e = tid + ST_THREADS * i;
        const bool ok = e < nsz && (int)(e % ST_ROWS) < nrw;
        if (e < nsz) {
            s_l[e] = ok ? sv0[i] : 0.0f;
            o_l[e] = OFF + (ok ? zv0[i] : 0.0f);
        }
    }
    for (uint32_t e0 = tid + ST_THREADS * BS; e0 < nsz; e0 += ST_THREADS * BS) {
        float sv[BS], zv[BS];
#pragma unroll
        for (int i = 0; i < BS; ++i) {
            const uint32_t e = e0 + ST_THREADS * i;
            const bool ok = e < nsz && (int)(e % ST_ROWS) < nrw;
            const int64_t idx = ok ? (int64_t)(e / ST_ROWS) * a.d_out + rw0 + e % ST_ROWS : 0;
            const float sl = a.scales[idx], zl = a.zeros[idx];
            sv[i] = ok ? sl : 0.0f;
            zv[i] = ok ? zl : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < BS; ++i) {
            const uint32_t e = e0 + ST_THREADS * i;
            if (e < nsz) {
                s_l[e] = sv[i];
                o_l[e] = OFF + zv[i];
            }
        }
    }
    // activations in stream order.  Token t0: its row (natural order: straight
    // into the blocked slots; with perm: flat, then gathered) from the
    // registers of phase 1.
    {
        uint16_t* dst0 = a.perm ? xf : xs;
#pragma unroll
        for (int i = 0; i < BX; ++i) {
            const uint32_t p = tid + ST_THREADS * i;
            if (p < npc) {
                uint16_t* q = a.perm ? xf + 8 * p : slot<true>(xs, 8 * p);
                *(u32x4_t*)q = xv0[i];
            }
        }
        if (a.perm) copy_row<false, ST_THREADS>(a, xr0, dst0, d_in, tid, ST_THREADS * BX);
        else copy_row<true, ST_THREADS>(a, xr0, dst0, ncol, tid, ST_THREADS * BX);
    }
    for (int t = 0; t < TM; ++t) {
        const bool tok = t < nt;
        const uint16_t* xr = X + (t0 + t) * a.ld_x;
        uint16_t* xst = xs + (size_t)t * nblk * XS_STRIDE;
        if (!a.perm) {
            if (t == 0) continue;
            if (tok) copy_row<true, ST_THREADS>(a, xr, xst, ncol, tid, 0);
            else
                for (uint32_t k = tid; k < ncol; k += ST_THREADS) *slot<true>(xst, k) = 0;
        } else {
            if (t > 0) {
                __syncthreads();               // the previous token's gather is done with xf
                if (tok) copy_row<false, ST_THREADS>(a, xr, xf, d_in, tid, 0);
            }
            __syncthreads();
            if (t > 0) {
#pragma unroll
                for (int i = 0; i < BP; ++i) {
                    const uint32_t k = tid + ST_THREADS * i;
                    cp[i] = a.perm[k < d_in ? k : 0];
                }
            }
#pragma unroll
            for (int i = 0; i < BP; ++i) {
                const uint32_t k = tid + ST_THREADS * i;
                if (k < ncol) {
                    uint16_t v = 0;
                    if (tok && k < d_in) v = ((uint32_t)cp[i] < d_in) ? xf[cp[i]] : (uint16_t)T::NAN_BITS;
                    *slot<true>(xst, k) = v;
                }
            }
            constexpr int B = 8;
            for (uint32_t k0 = tid + ST_THREADS * BP; k0 < ncol; k0 += ST_THREADS * B) {
                int32_t c[B];
#pragma unroll
                for (int i = 0; i < B; ++i) {
                    const uint32_t k = k0 + ST_THREADS * i;
                    c[i] = a.perm[k < d_in ? k : 0];
                }
#pragma unroll
                for (int i = 0; i < B; ++i) {
                    const uint32_t k = k0 + ST_THREADS * i;
                    if (k < ncol) {
                        uint16_t v = 0;
                        if (tok && k < d_in) v = ((uint32_t)c[i] < d_in) ? xf[c[i]] : (uint16_t)T::NAN_BITS;
                        *slot<true>(xst, k) = v;
                    }
                }
            }
        }
    }
    __syncthreads();

    float acc[TM][RW];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) acc[t][rr] = 0.0f;

    const bool one_group = a.gsize >= a.d_in;
    const uint32_t bpg = (uint32_t)(a.gsize >> 5);   // blocks per group (a multiple of 32 columns here)
    const float* s_h = s_l + half * RW;
    const float* o_h = o_l + half * RW;
    for (; blk < nblk; blk += 256) {
        const uint32_t g = one_group ? 0u : blk / bpg;
        const float4 s0 = *(const float4*)&s_h[g * ST_ROWS], s1 = *(const float4*)&s_h[g * ST_ROWS + 4];
        const float4 o0 = *(const float4*)&o_h[g * ST_ROWS], o1 = *(const float4*)&o_h[g * ST_ROWS + 4];
        const float sv[RW] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const float ov[RW] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
        uint32_t xp[TM][16];
        float xsum[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const uint4* q = (const uint4*)(xs + ((size_t)t * nblk + blk) * XS_STRIDE);
            uint32_t dd[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 v = q[i];
                dd[4 * i] = v.x;
                dd[4 * i + 1] = v.y;
                dd[4 * i + 2] = v.z;
                dd[4 * i + 3] = v.w;
            }
            float sx = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int ca = pair_col_a<BITS>(i), cb = pair_col_b<BITS>(i);
                xp[t][i] = __builtin_amdgcn_perm(dd[cb >> 1], dd[ca >> 1], (ca & 1) ? 0x07060302u : 0x05040100u);
                sx = T::dot2(xp[t][i], T::ONES, sx);
            }
            xsum[t] = sx;
        }
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            uint32_t cpr[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) cpr[i] = code_pair<BITS, T>(wd[rr], i);
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                float d = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) d = T::dot2(xp[t][i], cpr[i], d);
                acc[t][rr] = fmaf(sv[rr], fmaf(-ov[rr], xsum[t], d), acc[t][rr]);
            }
        }
#pragma unroll
        for (int rr = 0; rr < RW; ++rr)
#pragma unroll
            for (int q = 0; q < BITS; ++q) wd[rr][q] = wn[rr][q];
        load_block_words<BITS>(rs, row_bytes, blk + 2 * 256, nblk, wn);
    }

    // per half: exchange inside each wave, then the half's 4 waves meet in LDS
    constexpr int NV = TM * RW;
    float v[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) v[e] = acc[e / RW][e % RW];
    const int lane = tid & 63, wave = tid >> 6;
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
    if (tl < NV) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) sum += red[half * 4 + w][tl];
        const int t = tl / RW, rr = tl % RW;
        if (t < nt && rr < nr) a.Y[(t0 + t) * a.ld_y + r0 + rr] = sum;
    }
}

// ---------------------------------------------------------------------------
// Many tokens: the same arithmetic on the matrix cores.
//
// A workgroup computes 128 tokens x 128 rows.  Per 32-column block it stages
// the activations (A operands) and the rows' codes as exact half-precision
// values 2^b + c (B operands) in LDS, in MFMA operand order, and each of its
// four waves runs a 64x64 tile with v_mfma_f32_32x32x16.  The products of one
// group accumulate in float32 by themselves; at the group's end each lane
// adds s * (P - (2^b + z) * sum x) to its float32 output, with sum x taken
// from the A operands (v_dot2 with ones) and moved to the output layout by
// lane shuffles.  The next block's global loads are in flight while the
// current block computes (two LDS buffers, one barrier per block).
// ---------------------------------------------------------------------------
constexpr int MM_TILE = 128;
constexpr int MM_THREADS = 256;
constexpr int MM_OP_BYTES = 2 * 4 * 64 * 16;       // [k-step][32-wide tile][lane][16 B]
constexpr int MM_STAGE_BYTES = 2 * MM_OP_BYTES;    // A, then B
constexpr int64_t MM_MIN_TOKENS = 128;

// The 16 codes 16h .. 16h+15 of a 32-column block (h = 0, 1), as two B
// operands: op[q] holds codes 8q .. 8q+7 as values 2^b + c.
template <int BITS, typename T>
__device__ __forceinline__ void mm_code_operands(const uint32_t (&w)[BITS], int h, u32x4_t (&op)[2]) {
    constexpr int SH = T::MB - BITS;
    constexpr uint32_t E = (uint32_t)(T::BIAS + BITS) << T::MB;
    constexpr uint32_t M = (1u << BITS) - 1u;
    if constexpr (BITS == 4) {
        // a word holds 8 consecutive codes; even / odd nibbles to bytes, then
        // one byte permute pairs codes (2j, 2j+1) into the two halves
        constexpr uint32_t EE = E | (E << 16);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t wq = h ? w[2 + q] : w[q];
            const uint32_t ev = wq & 0x0F0F0F0Fu, od = (wq >> 4) & 0x0F0F0F0Fu;
            uint32_t v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // bytes: ev.byte j, zero, od.byte j, zero
                const uint32_t pr = __builtin_amdgcn_perm(od, ev, 0x0C000C00u | (uint32_t)j | ((uint32_t)(4 + j) << 16));
                v[j] = (pr << SH) | EE;
            }
            op[q] = u32x4_t{v[0], v[1], v[2], v[3]};
        }
        return;
    }
    uint64_t win0, win1 = 0;
    if constexpr (BITS == 2) {
        win0 = h ? w[1] : w[0];
    } else if constexpr (BITS == 3) {
        const uint64_t lo = ((uint64_t)w[1] << 32) | w[0], hi = ((uint64_t)w[2] << 32) | w[1];
        win0 = h ? (hi >> 16) : lo;
    } else if constexpr (BITS == 4) {
        win0 = h ? (((uint64_t)w[3] << 32) | w[2]) : (((uint64_t)w[1] << 32) | w[0]);
    } else {
        win0 = h ? (((uint64_t)w[5] << 32) | w[4]) : (((uint64_t)w[1] << 32) | w[0]);
        win1 = h ? (((uint64_t)w[7] << 32) | w[6]) : (((uint64_t)w[3] << 32) | w[2]);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        uint32_t v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e0 = 8 * q + 2 * j, e1 = e0 + 1;
            uint32_t c0, c1;
            if constexpr (BITS == 8) {
                c0 = (uint32_t)(((e0 < 8 ? win0 : win1) >> (8 * (e0 & 7))) & M);
                c1 = (uint32_t)(((e1 < 8 ? win0 : win1) >> (8 * (e1 & 7))) & M);
            } else {
                c0 = (uint32_t)((win0 >> (BITS * e0)) & M);
                c1 = (uint32_t)((win0 >> (BITS * e1)) & M);
            }
            v[j] = (E | (c0 << SH)) | ((E | (c1 << SH)) << 16);
        }
        op[q] = u32x4_t{v[0], v[1], v[2], v[3]};
    }
}

// XV: activation rows 16-byte aligned and d_in a multiple of 8, so every
// 16-byte piece is either whole or past the row's end (vector loads, no
// branches); otherwise element-wise loads.
template <int BITS, typename T, bool XV>
__global__ __launch_bounds__(MM_THREADS, 2) void dequant_mfma_kernel(DqArgs a, int64_t n_mt, int64_t n_rt,
                                                                     int64_t per_xcd) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_u8[];
    char* lds = (char*)lds_u8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // XCD-grouped order: the row tiles of one token tile run on one XCD
    const int64_t b = blockIdx.x;
    const int64_t lin = (b % 8) * per_xcd + b / 8;
    if (lin >= n_mt * n_rt) return;
    const int64_t mt = lin / n_rt, rt = lin % n_rt;
    const int64_t t0 = mt * MM_TILE, n0 = rt * MM_TILE;
    const uint16_t* X = (const uint16_t*)a.X;
    const uint32_t d_in = (uint32_t)a.d_in;
    const uint32_t nkb = (uint32_t)ceil_div(a.d_in, 32);
    const uint32_t bpg = a.gsize >= a.d_in ? nkb : (uint32_t)(a.gsize >> 5);
    const uint32_t ngr = (uint32_t)ceil_div(nkb, bpg);
    constexpr float OFF = (float)(1 << BITS);
    const __amdgpu_buffer_rsrc_t rs = words_rsrc(a, n0 < a.d_out ? n0 : a.d_out);
    const uint32_t row_bytes = (uint32_t)a.wpr * 4;

    // staging assignments: two 16-byte activation pieces per thread (token
    // p >> 2, columns 8 (p & 3) ..), and one row's half block of codes
    const int srow = tid >> 1, sh = tid & 1;
    const uint16_t* xrow[2];
    bool tok_ok[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int p = tid + MM_THREADS * j, t = p >> 2;
        const int64_t tok = t0 + t;
        tok_ok[j] = tok < a.n_tok;
        xrow[j] = X + (tok_ok[j] ? tok : 0) * a.ld_x + 8 * (p & 3);
    }
    auto load_x = [&](uint32_t kb, u32x4_t (&xv)[2]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t k = kb * 32 + 8 * ((tid + MM_THREADS * j) & 3);
            if constexpr (XV) {
                const bool ok = tok_ok[j] && k < d_in;
                const u32x4_t v = *(const u32x4_t*)(xrow[j] + (ok ? kb * 32 : 0));
                xv[j] = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
            } else {
                uint32_t e[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) e[i] = (tok_ok[j] && k + i < d_in) ? xrow[j][kb * 32 + i] : 0u;
                xv[j] = u32x4_t{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
            }
        }
    };
    auto load_w = [&](uint32_t kb, uint32_t (&w)[BITS]) {
        const uint32_t o = (uint32_t)srow * row_bytes + kb * (uint32_t)(BITS * 4);
        if constexpr (BITS == 2) {
            const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0);
            w[0] = v.x;
            w[1] = v.y;
        } else if constexpr (BITS == 3) {
            const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(rs, o, 0, 0);
            w[0] = v.x;
            w[1] = v.y;
            w[2] = v.z;
        } else {
#pragma unroll
            for (int q = 0; q < BITS; q += 4) {
                const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, o + 4 * q, 0, 0);
                w[q] = v.x;
                w[q + 1] = v.y;
                w[q + 2] = v.z;
                w[q + 3] = v.w;
            }
        }
    };
    auto store_stage = [&](int buf, const u32x4_t (&xv)[2], const uint32_t (&w)[BITS]) {
        char* st = lds + buf * MM_STAGE_BYTES;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int p = tid + MM_THREADS * j, t = p >> 2, q = p & 3;
            const int ks = q >> 1, kh = q & 1;
            *(u32x4_t*)(st + (((ks * 4 + (t >> 5)) * 64) + (t & 31) + 32 * kh) * 16) = xv[j];
        }
        u32x4_t op[2];
        mm_code_operands<BITS, T>(w, sh, op);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
            *(u32x4_t*)(st + MM_OP_BYTES + (((sh * 4 + (srow >> 5)) * 64) + (srow & 31) + 32 * kh) * 16) = op[kh];
    };

    const int wm = wave >> 1, wn = wave & 1;     // the wave's 64x64: token tiles 2wm, 2wm+1; row tiles 2wn, 2wn+1
    f16_t acc[2][2], accg[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const f16_t zero16 = {};

    // one k-block from LDS buffer `buf`; FIRST: the group's first block (its
    // first MFMA starts from zero)
    auto compute = [&](int buf, float (&xpart)[2], auto first) {
        const char* st = lds + buf * MM_STAGE_BYTES;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            u32x4_t av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) av[i] = *(const u32x4_t*)(st + ((ks * 4 + 2 * wm + i) * 64 + lane) * 16);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bv[j] = *(const u32x4_t*)(st + MM_OP_BYTES + ((ks * 4 + 2 * wn + j) * 64 + lane) * 16);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    accg[i][j] = mfma_32x32x16(av[i], bv[j], (decltype(first)::value && ks == 0) ? zero16 : accg[i][j],
                                               (typename T::mfma_tag*)nullptr);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                float x = (decltype(first)::value && ks == 0) ? 0.0f : xpart[i];
                x = T::dot2(av[i].x, T::ONES, x);
                x = T::dot2(av[i].y, T::ONES, x);
                x = T::dot2(av[i].z, T::ONES, x);
                xpart[i] = T::dot2(av[i].w, T::ONES, x);
            }
        }
    };

    u32x4_t xv[2];
    uint32_t w[BITS];
    load_x(0, xv);
    load_w(0, w);
    store_stage(0, xv, w);
    __syncthreads();
    uint32_t kb = 0;
    for (uint32_t g = 0; g < ngr; ++g) {
        // the group's scales and 2^b + zero for the wave's two row tiles
        float sv[2], ov[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t row = n0 + (2 * wn + j) * 32 + (lane & 31);
            const bool ok = row < a.d_out;
            const int64_t idx = ok ? (int64_t)g * a.d_out + row : 0;
            const float sl = a.scales[idx], zl = a.zeros[idx];
            sv[j] = ok ? sl : 0.0f;
            ov[j] = OFF + (ok ? zl : 0.0f);
        }
        const uint32_t kend = (kb + bpg < nkb) ? kb + bpg : nkb;
        float xpart[2];
        for (bool first = true; kb < kend; ++kb, first = false) {
            // next block's loads in flight (the last block reloads itself)
            const uint32_t kn = (kb + 1 < nkb) ? kb + 1 : kb;
            load_x(kn, xv);
            load_w(kn, w);
            if (first) compute(kb & 1, xpart, std::true_type{});
            else compute(kb & 1, xpart, std::false_type{});
            if (kb + 1 < nkb) store_stage((kb + 1) & 1, xv, w);
            __syncthreads();
        }
        // group end: acc += s * (P - (2^b + z) * sum x); the token of element
        // r of lane l is 8 (r / 4) + 4 (l / 32) + r % 4
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float xt = xpart[i] + __shfl_xor(xpart[i], 32, 64);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float x = __shfl(xt, 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), 64);
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j][r] = fmaf(sv[j], fmaf(-ov[j], x, accg[i][j][r]), acc[i][j][r]);
            }
        }
    }
    // outputs: element r of lane l of tile (i, j) is token 8 (r / 4) + 4 (l / 32) + r % 4, row l % 32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t row = n0 + (2 * wn + j) * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t tok = t0 + (2 * wm + i) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (tok < a.n_tok && row < a.d_out) a.Y[tok * a.ld_y + row] = acc[i][j][r];
            }
        }
}

template <int BITS, typename T>
gptq_status launch_mfma(const DqArgs& a, hipStream_t s) {
    const int64_t n_mt = ceil_div(a.n_tok, MM_TILE), n_rt = ceil_div(a.d_out, MM_TILE);
    const int64_t per_xcd = ceil_div(n_mt * n_rt, 8);
    const dim3 grid((unsigned)(per_xcd * 8)), block(MM_THREADS);
    if (a.xvec && a.d_in % 8 == 0)
        hipLaunchKernelGGL((dequant_mfma_kernel<BITS, T, true>), grid, block, 2 * MM_STAGE_BYTES, s, a, n_mt, n_rt,
                           per_xcd);
    else
        hipLaunchKernelGGL((dequant_mfma_kernel<BITS, T, false>), grid, block, 2 * MM_STAGE_BYTES, s, a, n_mt, n_rt,
                           per_xcd);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

template <typename T>
gptq_status by_bits_mfma(const DqArgs& a, int bits, hipStream_t s) {
    switch (bits) {
        case 2: return launch_mfma<2, T>(a, s);
        case 3: return launch_mfma<3, T>(a, s);
        case 4: return launch_mfma<4, T>(a, s);
        case 8:
            if constexpr (T::MB - 8 >= 0) return launch_mfma<8, T>(a, s);
            break;
    }
    return GPTQ_ERR_INVALID_ARG;
}

// ---------------------------------------------------------------------------
// Few tokens (2 .. 127) on the matrix cores.
//
// The weights are read once per 16 TT tokens (TT = 1, 2 or 4 tiles of 16),
// so the packed words are again the bytes that matter; the matrix cores only
// spare the per-token dot products.  A workgroup owns 16 weight rows and up
// to 16 TT tokens, and its FW_WAVES waves split the 32-column blocks of the
// rows between them (contiguous ranges; a group cut by a range end is
// corrected per part, which is exact since s (P - (2^b + z) sum x) is linear
// in P and sum x).  Each wave runs TT 16x16 tiles with v_mfma_f32_16x16x32
// (one instruction per tile and block, all sharing the block's B operand)
// and takes its operands straight from memory into registers, several blocks
// ahead, without LDS: lane l holds token l % 16 (of each tile) and columns
// 8 (l / 16) .. + 7 of the block (A: 16 bytes of the activation row) and row
// l % 16 with the same columns (B: the codes as exact half-precision values
// 2^b + c, from one load of the packed row).  At the end the waves' tiles
// are added in wave order through LDS (deterministic).
// ---------------------------------------------------------------------------
constexpr int FW_WAVES = 8;
constexpr int FW_THREADS = 64 * FW_WAVES;
#ifndef GPTQ_FW_MIN
#define GPTQ_FW_MIN 2
#endif
constexpr int64_t FW_MIN_TOKENS = GPTQ_FW_MIN;   // below: the per-token kernels

typedef float f4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f4_t c, bf16x8_t*) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f4_t c, h16x8_t*) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h16x8_t, a), __builtin_bit_cast(h16x8_t, b), c,
                                                  0, 0, 0);
}

// The 8 codes held in the low 8 * BITS bits of `win` as a B operand of
// exact values 2^b + c (pairs of half-precision lanes).
template <int BITS, typename T>
__device__ __forceinline__ u32x4_t codes8_operand(uint64_t win) {
    constexpr int SH = T::MB - BITS;
    constexpr uint32_t E = (uint32_t)(T::BIAS + BITS) << T::MB;
    constexpr uint32_t EE = E | (E << 16);
    constexpr uint32_t M = (1u << BITS) - 1u;
    uint32_t v[4];
    if constexpr (BITS == 4) {
        const uint32_t x = (uint32_t)win;
        const uint32_t ev = x & 0x0F0F0F0Fu, od = (x >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // bytes: ev.byte j, zero, od.byte j, zero
            const uint32_t pr = __builtin_amdgcn_perm(od, ev, 0x0C000C00u | (uint32_t)j | ((uint32_t)(4 + j) << 16));
            v[j] = (pr << SH) | EE;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t c0 = (uint32_t)(win >> (BITS * (2 * j))) & M;
            const uint32_t c1 = (uint32_t)(win >> (BITS * (2 * j + 1))) & M;
            v[j] = (c0 << SH) | (c1 << (SH + 16)) | EE;
        }
    }
    return u32x4_t{v[0], v[1], v[2], v[3]};
}

// blocks whose loads are in flight per wave
__host__ __device__ constexpr int fw_depth(int tt) { return tt >= 4 ? 4 : 8; }

template <int BITS, typename T, bool XV, int TT>
__global__ __launch_bounds__(FW_THREADS) void dequant_mfma_few_kernel(DqArgs a, int64_t n_rt, int64_t n_mt,
                                                                      int64_t per_xcd) {
    constexpr int DEPTH = fw_depth(TT);
    __shared__ float red[FW_WAVES - 1][TT][4][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // XCD-grouped order: the token tiles of one row tile run on one XCD
    const int64_t b = blockIdx.x;
    const int64_t lin = (b % 8) * per_xcd + b / 8;
    if (lin >= n_rt * n_mt) return;
    const int64_t rt = lin / n_mt, mt = lin % n_mt;
    const int64_t n0 = rt * 16, t0 = mt * 16 * TT;
    const int li = lane & 15, q = lane >> 4;          // token / row, and the lane's 8-column part of a block
    const uint32_t d_in = (uint32_t)a.d_in;
    const uint32_t nkb = (uint32_t)ceil_div(a.d_in, 32);
    const uint32_t bpg = a.gsize >= a.d_in ? nkb : (uint32_t)(a.gsize >> 5);
    const uint32_t kb_lo = (uint32_t)((uint64_t)nkb * wave / FW_WAVES);
    const uint32_t kb_hi = (uint32_t)((uint64_t)nkb * (wave + 1) / FW_WAVES);
    constexpr float OFF = (float)(1 << BITS);

    bool tok_ok[TT];
    const uint16_t* xrow[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const int64_t tok = t0 + 16 * t + li;
        tok_ok[t] = tok < a.n_tok;
        xrow[t] = (const uint16_t*)a.X + (tok_ok[t] ? tok : 0) * a.ld_x;
    }
    const __amdgpu_buffer_rsrc_t rs = words_rsrc(a, n0 < a.d_out ? n0 : a.d_out);
    const uint32_t row_off = (uint32_t)li * (uint32_t)a.wpr * 4;   // rows past d_out: past the buffer's end
    const int64_t row = n0 + li;
    const bool row_ok = row < a.d_out;

    // raw loads of block kb for this lane: its 8 activations of each token
    // tile, the words holding its 8 codes, and its row's scale and zero point
    // of the block's group.  Every load is unconditional (clamped addresses)
    // and its value is only used (masked, shifted) when the block is
    // computed, so that a ring slot is consumed before it is refilled and
    // keeps its registers.
    struct Ops {
        u32x4_t x[TT];
        u32x2_t w;
        float s, z;
    };
    auto load = [&](uint32_t kb, Ops& o) {
        const uint32_t k = kb * 32 + 8 * q;   // first column of the lane's 8
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if constexpr (XV) {
                o.x[t] = *(const u32x4_t*)(xrow[t] + (k < d_in ? k : 0));
            } else {
                uint32_t e[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) e[i] = xrow[t][k + i < d_in ? k + i : 0];
                o.x[t] = u32x4_t{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
            }
        }
        const uint32_t bit = (uint32_t)BITS * k;   // bit offset of the lane's first code in its row
        if constexpr (BITS == 4) {
            o.w.x = __builtin_amdgcn_raw_buffer_load_b32(rs, row_off + (bit >> 5) * 4, 0, 0);
        } else {
            o.w = __builtin_amdgcn_raw_buffer_load_b64(rs, row_off + (bit >> 5) * 4, 0, 0);
        }
        const int64_t idx = (int64_t)(kb / bpg) * a.d_out + (row_ok ? row : 0);
        o.s = a.scales[idx];
        o.z = a.zeros[idx];
    };
    // the lane's activations of block kb in tile t (zeros past d_in or past the last token)
    auto acts = [&](uint32_t kb, const Ops& o, int t) -> u32x4_t {
        const uint32_t k = kb * 32 + 8 * q;
        if constexpr (XV) {
            return (tok_ok[t] && k < d_in) ? o.x[t] : u32x4_t{0u, 0u, 0u, 0u};
        } else {
            // element i of the lane's 8 is zero past d_in
            uint32_t m[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                m[i] = (tok_ok[t] && k + 2 * i < d_in ? 0x0000FFFFu : 0u) |
                       (tok_ok[t] && k + 2 * i + 1 < d_in ? 0xFFFF0000u : 0u);
            return u32x4_t{o.x[t].x & m[0], o.x[t].y & m[1], o.x[t].z & m[2], o.x[t].w & m[3]};
        }
    };
    auto window = [&](uint32_t kb, const Ops& o) -> uint64_t {
        if constexpr (BITS == 4) {
            return o.w.x;
        } else {
            const uint32_t bit = (uint32_t)BITS * (kb * 32 + 8 * q);
            return ((((uint64_t)o.w.y) << 32) | o.w.x) >> (bit & 31);
        }
    };

    f4_t acc[TT], accg[TT];
    float xpart[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        acc[t] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
        accg[t] = acc[t];
        xpart[t] = 0.0f;
    }
    float sv = 0.0f, ov = 0.0f;

    // group end (or the end of this wave's part of a group): acc += s (P -
    // (2^b + z) sum x); element r of lane l is token 4 (l / 16) + r of the tile
    auto close_group = [&]() {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float xt = xpart[t] + __shfl_xor(xpart[t], 16, 64);
            xt += __shfl_xor(xt, 32, 64);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = __shfl(xt, 4 * q + r, 64);
                acc[t][r] = fmaf(sv, fmaf(-ov, x, accg[t][r]), acc[t][r]);
            }
        }
    };

    Ops ring[DEPTH];
    const uint32_t kb_last = kb_hi > kb_lo ? kb_hi - 1 : kb_lo;
#pragma unroll
    for (int p = 0; p < DEPTH; ++p) load(kb_lo + p < kb_hi ? kb_lo + p : kb_last, ring[p]);
    bool open = false;
    for (uint32_t kb0 = kb_lo; kb0 < kb_hi; kb0 += DEPTH) {
#pragma unroll
        for (int p = 0; p < DEPTH; ++p) {
            const uint32_t kb = kb0 + p;
            if (kb < kb_hi) {
                if (kb == kb_lo || kb % bpg == 0) {
                    if (open) close_group();
                    sv = row_ok ? ring[p].s : 0.0f;
                    ov = OFF + (row_ok ? ring[p].z : 0.0f);
                    open = true;
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        xpart[t] = 0.0f;
                        accg[t] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
                    }
                }
                const u32x4_t bop = codes8_operand<BITS, T>(window(kb, ring[p]));
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    const u32x4_t xa = acts(kb, ring[p], t);
                    accg[t] = mfma_16x16x32(xa, bop, accg[t], (typename T::mfma_tag*)nullptr);
                    float x = T::dot2(xa.x, T::ONES, xpart[t]);
                    x = T::dot2(xa.y, T::ONES, x);
                    x = T::dot2(xa.z, T::ONES, x);
                    xpart[t] = T::dot2(xa.w, T::ONES, x);
                }
            }
            // refill this slot DEPTH blocks ahead (past the range: reload the last block)
            load(kb + DEPTH < kb_hi ? kb + DEPTH : kb_last, ring[p]);
        }
    }
    if (open) close_group();

    // the waves' tiles added in wave order; element r of lane l is token
    // 4 (l / 16) + r of the tile, row l % 16
    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave - 1][t][r][lane] = acc[t][r];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float y = acc[t][r];
#pragma unroll
                for (int w = 0; w < FW_WAVES - 1; ++w) y += red[w][t][r][lane];
                const int64_t tk = t0 + 16 * t + 4 * q + r;
                if (tk < a.n_tok && row_ok) a.Y[tk * a.ld_y + row] = y;
            }
    }
}

template <int BITS, typename T, int TT>
gptq_status launch_mfma_few_tt(const DqArgs& a, hipStream_t s) {
    const int64_t n_rt = ceil_div(a.d_out, 16), n_mt = ceil_div(a.n_tok, 16 * TT);
    const int64_t per_xcd = ceil_div(n_rt * n_mt, 8);
    if (per_xcd * 8 > INT32_MAX) return GPTQ_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)(per_xcd * 8)), block(FW_THREADS);
    if (a.xvec && a.d_in % 8 == 0)
        hipLaunchKernelGGL((dequant_mfma_few_kernel<BITS, T, true, TT>), grid, block, 0, s, a, n_rt, n_mt, per_xcd);
    else
        hipLaunchKernelGGL((dequant_mfma_few_kernel<BITS, T, false, TT>), grid, block, 0, s, a, n_rt, n_mt, per_xcd);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

// The same with whole 128-column super-blocks (4 blocks) per lane step,
// when every group is made of whole super-blocks (group size a multiple of
// 128, or one group per row): lane l holds, for super-block sb, row l % 16's
// whole block 4 sb + l / 16 (one load of 4 b contiguous bytes, so the four
// lanes of a row read 16 b contiguous bytes instead of four scattered
// b-byte pieces) and token l % 16's 32 activations of that block. MFMA j
// (j = 0..3) takes the lane's codes and activations 8j .. 8j + 7: its 32
// K-values are columns 8j .. 8j + 7 of the four blocks, all in one group.
template <int BITS, typename T, bool XV, int TT>
__global__ __launch_bounds__(FW_THREADS) void dequant_mfma_few4_kernel(DqArgs a, int64_t n_rt, int64_t n_mt,
                                                                       int64_t per_xcd) {
    constexpr int DEPTH = TT >= 4 ? 1 : 2;   // super-blocks whose loads are in flight per wave
    __shared__ float red[FW_WAVES - 1][TT][4][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t b = blockIdx.x;
    const int64_t lin = (b % 8) * per_xcd + b / 8;
    if (lin >= n_rt * n_mt) return;
    const int64_t rt = lin / n_mt, mt = lin % n_mt;
    const int64_t n0 = rt * 16, t0 = mt * 16 * TT;
    const int li = lane & 15, q = lane >> 4;          // token / row, and the lane's block of a super-block
    const uint32_t d_in = (uint32_t)a.d_in;
    const uint32_t nkb = (uint32_t)ceil_div(a.d_in, 32);
    const uint32_t nsb = (nkb + 3) / 4;
    const uint32_t bpg = a.gsize >= a.d_in ? 4 * nsb : (uint32_t)(a.gsize >> 5);   // a multiple of 4
    const uint32_t sb_lo = (uint32_t)((uint64_t)nsb * wave / FW_WAVES);
    const uint32_t sb_hi = (uint32_t)((uint64_t)nsb * (wave + 1) / FW_WAVES);
    constexpr float OFF = (float)(1 << BITS);

    bool tok_ok[TT];
    const uint16_t* xrow[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const int64_t tok = t0 + 16 * t + li;
        tok_ok[t] = tok < a.n_tok;
        xrow[t] = (const uint16_t*)a.X + (tok_ok[t] ? tok : 0) * a.ld_x;
    }
    const __amdgpu_buffer_rsrc_t rs = words_rsrc(a, n0 < a.d_out ? n0 : a.d_out);
    const uint32_t row_off = (uint32_t)li * (uint32_t)a.wpr * 4;   // rows past d_out: past the buffer's end
    const int64_t row = n0 + li;
    const bool row_ok = row < a.d_out;

    // raw loads of super-block sb for this lane (unconditional, clamped;
    // masked and decoded only when used, as in the block-wise kernel)
    struct Ops {
        u32x4_t x[TT][4];
        uint32_t w[BITS];
        float s, z;
    };
    auto load = [&](uint32_t sb, Ops& o) {
        const uint32_t blk = 4 * sb + q;
        const uint32_t k0 = 32 * blk;
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t k = k0 + 8 * j;
                if constexpr (XV) {
                    o.x[t][j] = *(const u32x4_t*)(xrow[t] + (k < d_in ? k : 0));
                } else {
                    uint32_t e[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) e[i] = xrow[t][k + i < d_in ? k + i : 0];
                    o.x[t][j] = u32x4_t{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
                }
            }
        const uint32_t off = row_off + blk * (uint32_t)(BITS * 4);
        if constexpr (BITS == 2) {
            const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
            o.w[0] = v.x;
            o.w[1] = v.y;
        } else if constexpr (BITS == 3) {
            const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, 0);
            o.w[0] = v.x;
            o.w[1] = v.y;
            o.w[2] = v.z;
        } else {
#pragma unroll
            for (int u = 0; u < BITS; u += 4) {
                const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 4 * u, 0, 0);
                o.w[u] = v.x;
                o.w[u + 1] = v.y;
                o.w[u + 2] = v.z;
                o.w[u + 3] = v.w;
            }
        }
        const int64_t idx = (int64_t)((4 * sb) / bpg) * a.d_out + (row_ok ? row : 0);
        o.s = a.scales[idx];
        o.z = a.zeros[idx];
    };
    // the lane's activations 8j .. 8j + 7 of its block (zeros past d_in or past the last token)
    auto acts = [&](uint32_t sb, const Ops& o, int t, int j) -> u32x4_t {
        const uint32_t k = 32 * (4 * sb + q) + 8 * j;
        if constexpr (XV) {
            return (tok_ok[t] && k < d_in) ? o.x[t][j] : u32x4_t{0u, 0u, 0u, 0u};
        } else {
            uint32_t m[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                m[i] = (tok_ok[t] && k + 2 * i < d_in ? 0x0000FFFFu : 0u) |
                       (tok_ok[t] && k + 2 * i + 1 < d_in ? 0xFFFF0000u : 0u);
            return u32x4_t{o.x[t][j].x & m[0], o.x[t][j].y & m[1], o.x[t][j].z & m[2], o.x[t][j].w & m[3]};
        }
    };
    // the 64-bit window whose low bits hold codes 8j .. 8j + 7 of the lane's block
    auto window = [&](const Ops& o, int j) -> uint64_t {
        const int bit = BITS * 8 * j, wi = bit >> 5, sh = bit & 31;
        const uint64_t lo = o.w[wi];
        const uint64_t hi = (wi + 1 < BITS) ? (uint64_t)o.w[wi + 1 < BITS ? wi + 1 : wi] : 0u;
        return ((hi << 32) | lo) >> sh;
    };

    f4_t acc[TT], accg[TT];
    float xpart[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        acc[t] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
        accg[t] = acc[t];
        xpart[t] = 0.0f;
    }
    float sv = 0.0f, ov = 0.0f;
    auto close_group = [&]() {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float xt = xpart[t] + __shfl_xor(xpart[t], 16, 64);
            xt += __shfl_xor(xt, 32, 64);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = __shfl(xt, 4 * q + r, 64);
                acc[t][r] = fmaf(sv, fmaf(-ov, x, accg[t][r]), acc[t][r]);
            }
        }
    };

    Ops ring[DEPTH];
    const uint32_t sb_last = sb_hi > sb_lo ? sb_hi - 1 : sb_lo;
#pragma unroll
    for (int p = 0; p < DEPTH; ++p) load(sb_lo + p < sb_hi ? sb_lo + p : sb_last, ring[p]);
    bool open = false;
    for (uint32_t sb0 = sb_lo; sb0 < sb_hi; sb0 += DEPTH) {
#pragma unroll
        for (int p = 0; p < DEPTH; ++p) {
            const uint32_t sb = sb0 + p;
            if (sb < sb_hi) {
                if (sb == sb_lo || (4 * sb) % bpg == 0) {
                    if (open) close_group();
                    sv = row_ok ? ring[p].s : 0.0f;
                    ov = OFF + (row_ok ? ring[p].z : 0.0f);
                    open = true;
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        xpart[t] = 0.0f;
                        accg[t] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x4_t bop = codes8_operand<BITS, T>(window(ring[p], j));
#pragma unroll
                    for (int t = 0; t < TT; ++t) {
                        const u32x4_t xa = acts(sb, ring[p], t, j);
                        accg[t] = mfma_16x16x32(xa, bop, accg[t], (typename T::mfma_tag*)nullptr);
                        float x = T::dot2(xa.x, T::ONES, xpart[t]);
                        x = T::dot2(xa.y, T::ONES, x);
                        x = T::dot2(xa.z, T::ONES, x);
                        xpart[t] = T::dot2(xa.w, T::ONES, x);
                    }
                }
            }
            load(sb + DEPTH < sb_hi ? sb + DEPTH : sb_last, ring[p]);
        }
    }
    if (open) close_group();

    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave - 1][t][r][lane] = acc[t][r];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float y = acc[t][r];
#pragma unroll
                for (int w = 0; w < FW_WAVES - 1; ++w) y += red[w][t][r][lane];
                const int64_t tk = t0 + 16 * t + 4 * q + r;
                if (tk < a.n_tok && row_ok) a.Y[tk * a.ld_y + row] = y;
            }
    }
}

template <int BITS, typename T, int TT>
gptq_status launch_mfma_few4_tt(const DqArgs& a, hipStream_t s) {
    const int64_t n_rt = ceil_div(a.d_out, 16), n_mt = ceil_div(a.n_tok, 16 * TT);
    const int64_t per_xcd = ceil_div(n_rt * n_mt, 8);
    if (per_xcd * 8 > INT32_MAX) return GPTQ_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)(per_xcd * 8)), block(FW_THREADS);
    if (a.xvec && a.d_in % 8 == 0)
        hipLaunchKernelGGL((dequant_mfma_few4_kernel<BITS, T, true, TT>), grid, block, 0, s, a, n_rt, n_mt, per_xcd);
    else
        hipLaunchKernelGGL((dequant_mfma_few4_kernel<BITS, T, false, TT>), grid, block, 0, s, a, n_rt, n_mt, per_xcd);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

#ifndef GPTQ_FEW4
#define GPTQ_FEW4 1
#endif
// 16 tokens per tile; up to 16: one tile, up to 32: two, more: four per
// workgroup.  Groups of whole 128-column super-blocks take the super-block
// kernel.
template <int BITS, typename T>
gptq_status launch_mfma_few(const DqArgs& a, hipStream_t s) {
    const bool whole = a.gsize >= a.d_in || a.gsize % 128 == 0;
    if (GPTQ_FEW4 && whole) {
        if (a.n_tok <= 16) return launch_mfma_few4_tt<BITS, T, 1>(a, s);
        if (a.n_tok <= 32) return launch_mfma_few4_tt<BITS, T, 2>(a, s);
        return launch_mfma_few4_tt<BITS, T, 4>(a, s);
    }
    if (a.n_tok <= 16) return launch_mfma_few_tt<BITS, T, 1>(a, s);
    if (a.n_tok <= 32) return launch_mfma_few_tt<BITS, T, 2>(a, s);
    return launch_mfma_few_tt<BITS, T, 4>(a, s);
}

template <typename T>
gptq_status by_bits_mfma_few(const DqArgs& a, int bits, hipStream_t s) {
    switch (bits) {
        case 2: return launch_mfma_few<2, T>(a, s);
        case 3: return launch_mfma_few<3, T>(a, s);
        case 4: return launch_mfma_few<4, T>(a, s);
        case 8:
            if constexpr (T::MB - 8 >= 0) return launch_mfma_few<8, T>(a, s);
            break;
    }
    return GPTQ_ERR_INVALID_ARG;
}

template <int BITS, int TM, typename T>
gptq_status launch_block(const DqArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)ceil_div(a.d_out, RW), (unsigned)ceil_div(a.n_tok, TM));
    const StagedLayout Ly = staged_layout(a.n_groups, ceil_div(a.d_in, 32), a.d_in, TM, a.perm != nullptr);
    if (Ly.total <= STAGED_LDS_MAX) {
        GPTQ_HIP(ensure_lds_limit((const void*)dequant_staged_kernel<BITS, TM, T>, (int)STAGED_LDS_MAX));
        const dim3 grid_s((unsigned)ceil_div(a.d_out, ST_ROWS), (unsigned)ceil_div(a.n_tok, TM));
        hipLaunchKernelGGL((dequant_staged_kernel<BITS, TM, T>), grid_s, dim3(ST_THREADS), Ly.total, s, a);
    } else {
        hipLaunchKernelGGL((dequant_block_kernel<BITS, TM, T>), grid, dim3(DQ_THREADS), 0, s, a);
    }
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

// ---------------------------------------------------------------------------
// Column gather Xg[t][k] = X[t][perm[k]] ("GPTQ量化算法深度解析" §3.3: with
// act-order, inference gathers the activations into the quantization order).
// A workgroup owns `rows` token rows and one chunk of `chunk` columns (a
// grid of token tiles x chunks): the chunk's perm entries go to LDS once,
// then every row is gathered with coalesced writes (the reads stay inside
// one row).  Many tokens: 16 rows x 4096 columns, which spreads the perm
// reads over many rows; fewer than 1024 tokens: 4 rows x 512 columns, so
// that a few long rows still spread over the chip.
// ---------------------------------------------------------------------------
constexpr int GA_CHUNK_MAX = 4096;

template <typename E>
__global__ __launch_bounds__(256) void gather_columns_kernel(const E* __restrict__ X, int64_t n_tok, int64_t d_in,
                                                             int64_t ld_x, const int32_t* __restrict__ perm,
                                                             E* __restrict__ Xg, int64_t ld_g, E nan_value, int rows,
                                                             int chunk) {
    __shared__ int32_t pl[GA_CHUNK_MAX];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * rows;
    const int64_t c0 = (int64_t)blockIdx.y * chunk;
    const int nc = (d_in - c0 < chunk) ? (int)(d_in - c0) : chunk;
    for (int k = tid; k < nc; k += 256) pl[k] = perm[c0 + k];
    __syncthreads();
    for (int rr = 0; rr < rows; ++rr) {
        const int64_t t = r0 + rr;
        if (t >= n_tok) break;
        const E* xr = X + t * ld_x;
        E* gr = Xg + t * ld_g + c0;
        for (int k = tid; k < nc; k += 256) {
            const int32_t p = pl[k];
            gr[k] = ((uint32_t)p < (uint64_t)d_in) ? xr[p] : nan_value;
        }
    }
}

}  // namespace

gptq_status gather_columns_launch(const void* X, gptq_dtype dt, int64_t n_tok, int64_t d_in, int64_t ld_x,
                                  const int32_t* perm, void* Xg, int64_t ld_g, hipStream_t s) {
    if (n_tok == 0) return GPTQ_OK;
    const int rows = n_tok >= 1024 ? 16 : 4;
    const int chunk = n_tok >= 1024 ? GA_CHUNK_MAX : 512;
    if (ceil_div(d_in, chunk) > 65535 || ceil_div(n_tok, rows) > INT32_MAX) return GPTQ_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)ceil_div(n_tok, rows), (unsigned)ceil_div(d_in, chunk));
    if (dt == GPTQ_F32) {
        hipLaunchKernelGGL(gather_columns_kernel<float>, grid, dim3(256), 0, s, (const float*)X, n_tok, d_in, ld_x,
                           perm, (float*)Xg, ld_g, __builtin_nanf(""), rows, chunk);
    } else {
        const uint16_t nan16 = dt == GPTQ_BF16 ? (uint16_t)Bf16::NAN_BITS : (uint16_t)F16::NAN_BITS;
        hipLaunchKernelGGL(gather_columns_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)X, n_tok, d_in,
                           ld_x, perm, (uint16_t*)Xg, ld_g, nan16, rows, chunk);
    }
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

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
    const bool block_path = dequant_uses_block_path(dt, bits, d_in, group_size, g_idx != nullptr);
    if (!block_path && n_groups > DQ_MAX_GROUPS) return GPTQ_ERR_UNSUPPORTED;
    if (block_path && !perm && n_tok >= MM_MIN_TOKENS) {
        // many tokens in natural order: matrix cores (grid in x only)
        if (dt == GPTQ_BF16) return by_bits_mfma<Bf16>(a, bits, s);
        return by_bits_mfma<F16>(a, bits, s);
    }
    if (block_path && !perm && n_tok >= FW_MIN_TOKENS) {
        // a few tokens in natural order: matrix cores, 32 rows x 32 tokens per workgroup
        if (dt == GPTQ_BF16) return by_bits_mfma_few<Bf16>(a, bits, s);
        return by_bits_mfma_few<F16>(a, bits, s);
    }
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
