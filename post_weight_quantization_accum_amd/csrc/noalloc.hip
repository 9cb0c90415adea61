// gptq_hessian_accumulate_noalloc: the Hessian accumulation with all of its
// scratch memory in a fixed device array, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The declaration and contract are in include/gptq.h.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy until the process ends.  In host code its name only stands in
// for the symbol, so its device address is looked up once per device (with
// that device current) by hipGetSymbolAddress, and that address is what the
// kernels receive.  Every call on one GPU shares that GPU's array; the
// kernels write every scratch byte they later read, so nothing needs
// clearing between calls, and calls that overlap on one GPU race.
#include <mutex>

#include "internal.hpp"

namespace {

constexpr size_t SCRATCH_BYTES = GPTQ_NOALLOC_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;

static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

// Device address of this device's scratch array (null on failure).
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" {

gptq_status gptq_hessian_accumulate_noalloc(double* H, const void* X, gptq_dtype x_dtype, int64_t n_tok,
                                            int64_t d_in, int64_t ld_x, hipStream_t stream) {
    if (!H || !(x_dtype == GPTQ_F32 || x_dtype == GPTQ_F16 || x_dtype == GPTQ_BF16)) return GPTQ_ERR_INVALID_ARG;
    if (d_in <= 0 || d_in > (int64_t(1) << 20) || n_tok < 0 || ld_x < d_in) return GPTQ_ERR_INVALID_ARG;
    if (n_tok > 0 && !X) return GPTQ_ERR_INVALID_ARG;
    void* p = scratch_ptr();
    if (!p) return GPTQ_ERR_HIP;
    return gptq::hessian_launch_scratch(H, X, x_dtype, n_tok, d_in, ld_x, p, SCRATCH_BYTES, stream);
}

}  // extern "C"
