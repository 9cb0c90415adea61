// Packing of b-bit codes into 32-bit words ("gptq-for-llama" article,
// "工程细节": four 4-bit codes share one 16-bit integer).  Per output row the
// codes form a little-endian bit stream: code k occupies bits
// [b*k, b*k + b), bit 0 being the least significant bit of word 0.
//
// Optional column order (perm): stream position k then holds the code of
// column perm[k], which puts the groups of an act-order layer back into
// consecutive positions for the product kernels.
//
// One thread per 32 consecutive stream positions of a row: their codes
// fill exactly `bits` words (32 codes x b bits), so no word is shared
// between threads and no thread searches for its codes.  Rows whose 32
// codes sit 16-byte aligned are read with two 16-byte loads; otherwise (and
// with perm) code by code.  Reads are contiguous bytes of one row, writes
// contiguous words: the kernel streams HBM once in each direction.
#include "internal.hpp"

namespace gptq {
namespace {

template <int BITS>
__global__ __launch_bounds__(256) void pack32_kernel(const uint8_t* __restrict__ codes, int64_t d_out, int64_t d_in,
                                                     int64_t cpr, int64_t wpr, const int32_t* __restrict__ perm,
                                                     uint32_t* __restrict__ packed) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = d_out * cpr;
    if (idx >= n) return;
    int64_t r, c;
    if (n <= (int64_t)UINT32_MAX) {
        r = (uint32_t)idx / (uint32_t)cpr;
        c = (uint32_t)idx - (uint32_t)r * (uint32_t)cpr;
    } else {
        r = idx / cpr;
        c = idx - r * cpr;
    }
    const uint8_t* row = codes + r * d_in;
    const int64_t k0 = 32 * c;
    uint32_t v[8];   // the 32 codes, four bytes per entry (byte j % 4 of v[j / 4] is code k0 + j)
    if (!perm && k0 + 32 <= d_in && ((uintptr_t)(row + k0) & 15) == 0) {
        const uint4 a = *(const uint4*)(row + k0);
        const uint4 b = *(const uint4*)(row + k0 + 16);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = 0u;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int64_t k = k0 + j;
            if (k < d_in) {
                int64_t col = k;
                if (perm) {
                    const int32_t p = perm[k];
                    col = ((uint32_t)p < (uint64_t)d_in) ? (int64_t)p : -1;
                }
                const uint32_t x = col >= 0 ? row[col] : 0u;
                v[j >> 2] |= x << (8 * (j & 3));
            }
        }
    }
    constexpr uint32_t mask = (1u << BITS) - 1u;
    uint32_t w[BITS];
#pragma unroll
    for (int q = 0; q < BITS; ++q) w[q] = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const uint32_t x = (v[j >> 2] >> (8 * (j & 3))) & mask;
        const int bit = BITS * j;   // compile-time after unrolling
        w[bit >> 5] |= x << (bit & 31);
        if ((bit & 31) + BITS > 32) w[(bit >> 5) + 1] |= x >> (32 - (bit & 31));
    }
    uint32_t* out = packed + r * wpr + c * BITS;
#pragma unroll
    for (int q = 0; q < BITS; ++q)
        if (c * BITS + q < wpr) out[q] = w[q];
}

}  // namespace

gptq_status pack_launch(const uint8_t* codes, int64_t d_out, int64_t d_in, int32_t bits, const int32_t* perm,
                        uint32_t* packed, hipStream_t s) {
    const int64_t wpr = ceil_div(d_in * bits, 32);
    const int64_t cpr = ceil_div(d_in, 32);
    const int64_t n = d_out * cpr;
    if (n == 0) return GPTQ_OK;
    if (ceil_div(n, 256) > INT32_MAX) return GPTQ_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)ceil_div(n, 256)), block(256);
    switch (bits) {
        case 2: hipLaunchKernelGGL(pack32_kernel<2>, grid, block, 0, s, codes, d_out, d_in, cpr, wpr, perm, packed); break;
        case 3: hipLaunchKernelGGL(pack32_kernel<3>, grid, block, 0, s, codes, d_out, d_in, cpr, wpr, perm, packed); break;
        case 4: hipLaunchKernelGGL(pack32_kernel<4>, grid, block, 0, s, codes, d_out, d_in, cpr, wpr, perm, packed); break;
        case 8: hipLaunchKernelGGL(pack32_kernel<8>, grid, block, 0, s, codes, d_out, d_in, cpr, wpr, perm, packed); break;
        default: return GPTQ_ERR_INVALID_ARG;
    }
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

}  // namespace gptq
