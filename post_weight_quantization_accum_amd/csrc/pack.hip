// Packing of b-bit codes into 32-bit words ("gptq-for-llama" article,
// "工程细节": four 4-bit codes share one 16-bit integer).  Per output row the
// codes form a little-endian bit stream: code k occupies bits
// [b*k, b*k + b), bit 0 being the least significant bit of word 0.
//
// Optional column order (perm): stream position k then holds the code of
// column perm[k], which puts the groups of an act-order layer back into
// consecutive positions for the product kernels.
//
// One thread per output word: it gathers the (at most 33/b + 1) codes that
// overlap its 32 bits.  Reads are contiguous bytes of one row, writes are
// contiguous words: the kernel streams HBM once in each direction.
#include "internal.hpp"

namespace gptq {
namespace {

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes, int64_t d_out, int64_t d_in,
                                                   int bits, int64_t wpr, const int32_t* __restrict__ perm,
                                                   uint32_t* __restrict__ packed) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= d_out * wpr) return;
    const int64_t r = idx / wpr, m = idx - r * wpr;
    const uint8_t* row = codes + r * d_in;
    const uint32_t mask = (1u << bits) - 1u;
    const int64_t bit0 = 32 * m;
    int64_t k_lo = bit0 / bits;
    int64_t k_hi = (bit0 + 31) / bits;
    if (k_hi >= d_in) k_hi = d_in - 1;
    uint32_t word = 0;
    for (int64_t k = k_lo; k <= k_hi; ++k) {
        int64_t col = k;
        if (perm) {
            const int32_t p = perm[k];
            col = ((uint32_t)p < (uint64_t)d_in) ? (int64_t)p : -1;
        }
        const uint32_t c = col >= 0 ? (row[col] & mask) : 0u;
        const int64_t sh = bits * k - bit0;
        if (sh >= 0) word |= c << sh;
        else word |= c >> (-sh);
    }
    packed[idx] = word;
}

}  // namespace

gptq_status pack_launch(const uint8_t* codes, int64_t d_out, int64_t d_in, int32_t bits, const int32_t* perm,
                        uint32_t* packed, hipStream_t s) {
    const int64_t wpr = ceil_div(d_in * bits, 32);
    const int64_t n = d_out * wpr;
    if (n == 0) return GPTQ_OK;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, codes, d_out, d_in, bits, wpr,
                       perm, packed);
    GPTQ_LAUNCH_CHECK();
    return GPTQ_OK;
}

}  // namespace gptq
