// Shared device/host helpers of libgptq_mi355x (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/gptq.h"

namespace gptq {

// ---------------------------------------------------------------------------
// MFMA operand types (wave64).
// ---------------------------------------------------------------------------
typedef double d4_t __attribute__((ext_vector_type(4)));
typedef float f16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// v_mfma_f64_16x16x4_f64.  Lane l supplies A[l%16][l/16] and B[l/16][l%16];
// result element r of lane l is C[4*r + l/16][l%16].
__device__ __forceinline__ d4_t mfma_f64_16x16x4(double a, double b, d4_t c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_{bf16,f16}.  Lane l supplies A[l%32][8*(l/32) + 0..7]
// and B[8*(l/32) + 0..7][l%32]; result element r of lane l is
// C[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f16_t c, bf16x8_t*) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f16_t c, h16x8_t*) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h16x8_t, a),
                                                  __builtin_bit_cast(h16x8_t, b), c, 0, 0, 0);
}

// Widen one stored element to double (exact for every input type).
__device__ __forceinline__ double to_f64(float x) { return (double)x; }
__device__ __forceinline__ double bf16_bits_to_f64(uint16_t b) {
    return (double)__uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ double f16_bits_to_f64(uint16_t b) {
    _Float16 h = __builtin_bit_cast(_Float16, b);
    return (double)(float)h;
}
__device__ __forceinline__ double load_as_f64(const void* p, int64_t idx, gptq_dtype dt) {
    if (dt == GPTQ_F32) return (double)((const float*)p)[idx];
    uint16_t b = ((const uint16_t*)p)[idx];
    return dt == GPTQ_BF16 ? bf16_bits_to_f64(b) : f16_bits_to_f64(b);
}

// Device-side status words written by kernels and read back by the
// synchronous calls.
enum : int { FLAG_NONFINITE = 0, FLAG_NOT_PD = 1, FLAG_BAD_PERM = 2, N_FLAGS = 4 };

__device__ __forceinline__ void raise_flag(int* flags, int which) {
    // Any lane may set it; a plain store of the constant 1 is race-free in effect.
    __hip_atomic_store(&flags[which], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ __forceinline__ size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

}  // namespace gptq

// Host-side HIP error check inside functions that return gptq_status.
#define GPTQ_HIP(call)                                   \
    do {                                                 \
        hipError_t e_ = (call);                          \
        if (e_ != hipSuccess) return GPTQ_ERR_HIP;       \
    } while (0)

#define GPTQ_LAUNCH_CHECK() GPTQ_HIP(hipGetLastError())
