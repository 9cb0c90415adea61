// The C ABI of libgptq_mi355x: argument validation, workspace sizing and
// dispatch to the kernels.  Declarations and contracts are in include/gptq.h.
#include <mutex>
#include <tuple>
#include <vector>

#include "internal.hpp"

using namespace gptq;

namespace gptq {

hipError_t ensure_lds_limit(const void* kernel, int bytes) {
    static std::mutex mu;
    static std::vector<std::tuple<int, const void*, int>> done;   // (device, kernel, bytes) already set
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(mu);
    for (const auto& t : done)
        if (std::get<0>(t) == dev && std::get<1>(t) == kernel && std::get<2>(t) >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done.emplace_back(dev, kernel, bytes);
    return e;
}

}  // namespace gptq

namespace {

constexpr int64_t MAX_DIM = int64_t(1) << 20;   // per-dimension sanity bound

bool valid_dtype(gptq_dtype dt) { return dt == GPTQ_F32 || dt == GPTQ_F16 || dt == GPTQ_BF16; }

bool valid_bits(int32_t b) { return b == 2 || b == 3 || b == 4 || b == 8; }

gptq_status check_config(const gptq_config* cfg) {
    if (!cfg) return GPTQ_ERR_INVALID_ARG;
    if (!valid_bits(cfg->bits)) return GPTQ_ERR_INVALID_ARG;
    if (cfg->block_size < 1) return GPTQ_ERR_INVALID_ARG;
    if (cfg->block_size > 128) return GPTQ_ERR_UNSUPPORTED;
    if (cfg->static_groups != 0 && cfg->static_groups != 1) return GPTQ_ERR_INVALID_ARG;
    if (!(cfg->damp >= 0.0) || !(cfg->damp < 1e300)) return GPTQ_ERR_INVALID_ARG;
    return GPTQ_OK;
}

}  // namespace

extern "C" {

void gptq_config_default(gptq_config* cfg) {
    if (!cfg) return;
    cfg->bits = 4;
    cfg->group_size = 128;
    cfg->sym = 0;
    cfg->act_order = 0;
    cfg->block_size = 128;
    cfg->static_groups = 0;
    cfg->damp = 0.01;
}

const char* gptq_status_string(gptq_status st) {
    switch (st) {
        case GPTQ_OK: return "ok";
        case GPTQ_ERR_INVALID_ARG: return "invalid argument";
        case GPTQ_ERR_NOT_PD: return "damped Hessian is not positive definite";
        case GPTQ_ERR_NONFINITE: return "non-finite value (NaN/Inf) in the input";
        case GPTQ_ERR_WORKSPACE: return "workspace missing or too small";
        case GPTQ_ERR_HIP: return "HIP runtime error";
        case GPTQ_ERR_UNSUPPORTED: return "unsupported by this build";
    }
    return "unknown status";
}

const char* gptq_version(void) { return "0.1.0"; }

size_t gptq_hessian_workspace(int64_t n_tok, int64_t d_in) {
    if (d_in <= 0 || d_in > MAX_DIM || n_tok < 0) return 0;
    return hessian_workspace_bytes(n_tok, d_in);
}

gptq_status gptq_hessian_accumulate(double* H, const void* X, gptq_dtype x_dtype, int64_t n_tok, int64_t d_in,
                                    int64_t ld_x, void* workspace, size_t ws_bytes, hipStream_t stream) {
    if (!H || !valid_dtype(x_dtype)) return GPTQ_ERR_INVALID_ARG;
    if (d_in <= 0 || d_in > MAX_DIM || n_tok < 0 || ld_x < d_in) return GPTQ_ERR_INVALID_ARG;
    if (n_tok > 0 && !X) return GPTQ_ERR_INVALID_ARG;
    if (x_dtype != GPTQ_F32 && n_tok > 0 && (!workspace || ws_bytes < hessian_workspace_bytes(n_tok, d_in)))
        return GPTQ_ERR_WORKSPACE;
    return hessian_launch(H, X, x_dtype, n_tok, d_in, ld_x, workspace, stream);
}

gptq_status gptq_hessian_accumulate_timed(double* H, const void* X, gptq_dtype x_dtype, int64_t n_tok,
                                          int64_t d_in, int64_t ld_x, void* workspace, size_t ws_bytes,
                                          hipStream_t stream, double* syrk_ms, int64_t* n_launches) {
    if (!syrk_ms || !n_launches) return GPTQ_ERR_INVALID_ARG;
    if (!H || !valid_dtype(x_dtype)) return GPTQ_ERR_INVALID_ARG;
    if (d_in <= 0 || d_in > MAX_DIM || n_tok < 0 || ld_x < d_in) return GPTQ_ERR_INVALID_ARG;
    if (n_tok > 0 && !X) return GPTQ_ERR_INVALID_ARG;
    if (x_dtype != GPTQ_F32 && n_tok > 0 && (!workspace || ws_bytes < hessian_workspace_bytes(n_tok, d_in)))
        return GPTQ_ERR_WORKSPACE;
    const int64_t n = hessian_syrk_launches(n_tok, x_dtype, d_in, ld_x, X);
    *syrk_ms = 0.0;
    *n_launches = n;
    if (n == 0) return GPTQ_OK;
    std::vector<hipEvent_t> ev((size_t)(2 * n), nullptr);
    gptq_status st = GPTQ_OK;
    for (auto& e : ev)
        if (hipEventCreate(&e) != hipSuccess) st = GPTQ_ERR_HIP;
    if (st == GPTQ_OK) st = hessian_launch(H, X, x_dtype, n_tok, d_in, ld_x, workspace, stream, ev.data());
    if (st == GPTQ_OK && hipStreamSynchronize(stream) != hipSuccess) st = GPTQ_ERR_HIP;
    double total = 0.0;
    for (int64_t i = 0; st == GPTQ_OK && i < n; ++i) {
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]) != hipSuccess) st = GPTQ_ERR_HIP;
        total += ms;
    }
    for (auto& e : ev)
        if (e) (void)hipEventDestroy(e);
    if (st == GPTQ_OK) *syrk_ms = total / (double)n;
    return st;
}

size_t gptq_prepare_hinv_workspace(int64_t d_in) {
    if (d_in <= 0 || d_in > MAX_DIM) return 0;
    return hinv_workspace_bytes(d_in);
}

gptq_status gptq_prepare_hinv(double* H, int64_t d_in, const gptq_config* cfg, int32_t* perm, void* workspace,
                              size_t ws_bytes, hipStream_t stream) {
    if (!H || !perm) return GPTQ_ERR_INVALID_ARG;
    if (d_in <= 0 || d_in > MAX_DIM) return GPTQ_ERR_INVALID_ARG;
    gptq_status st = check_config(cfg);
    if (st != GPTQ_OK) return st;
    if (!workspace || ws_bytes < hinv_workspace_bytes(d_in)) return GPTQ_ERR_WORKSPACE;
    int flags[N_FLAGS] = {0, 0, 0, 0};
    st = hinv_launch(H, d_in, cfg, perm, workspace, stream, flags);
    if (st != GPTQ_OK) return st;
    if (flags[FLAG_NONFINITE]) return GPTQ_ERR_NONFINITE;
    if (flags[FLAG_NOT_PD]) return GPTQ_ERR_NOT_PD;
    return GPTQ_OK;
}

size_t gptq_prepare_hinv_factored_workspace(int64_t d_in) {
    if (d_in <= 0 || d_in > MAX_DIM || d_in % 128 != 0) return 0;
    return hinv_workspace_bytes(d_in, true);
}

gptq_status gptq_prepare_hinv_factored(double* H, int64_t d_in, const gptq_config* cfg, int32_t* perm,
                                       void* workspace, size_t ws_bytes, hipStream_t stream) {
    if (!H || !perm) return GPTQ_ERR_INVALID_ARG;
    if (d_in <= 0 || d_in > MAX_DIM) return GPTQ_ERR_INVALID_ARG;
    gptq_status st = check_config(cfg);
    if (st != GPTQ_OK) return st;
    if (d_in % 128 != 0) return GPTQ_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < hinv_workspace_bytes(d_in, true)) return GPTQ_ERR_WORKSPACE;
    int flags[N_FLAGS] = {0, 0, 0, 0};
    st = hinv_launch(H, d_in, cfg, perm, workspace, stream, flags, true);
    if (st != GPTQ_OK) return st;
    if (flags[FLAG_NONFINITE]) return GPTQ_ERR_NONFINITE;
    if (flags[FLAG_NOT_PD]) return GPTQ_ERR_NOT_PD;
    return GPTQ_OK;
}

size_t gptq_quantize_layer_factored_workspace(int64_t d_out, int64_t d_in, const gptq_config* cfg) {
    if (d_out <= 0 || d_in <= 0 || d_out > MAX_DIM || d_in > MAX_DIM) return 0;
    if (check_config(cfg) != GPTQ_OK || !sweep_factored_supported(d_in, cfg)) return 0;
    return sweep_workspace_bytes(d_out, d_in, cfg, true);
}

gptq_status gptq_quantize_layer_factored(const void* W, gptq_dtype w_dtype, int64_t d_out, int64_t d_in,
                                         int64_t ld_w, const double* F, const int32_t* perm,
                                         const gptq_config* cfg, uint8_t* codes, float* scales, float* zeros,
                                         int32_t* g_idx, float* w_hat, double* row_loss, void* workspace,
                                         size_t ws_bytes, hipStream_t stream) {
    if (!W || !F || !perm || !codes || !scales || !zeros || !g_idx) return GPTQ_ERR_INVALID_ARG;
    if (!valid_dtype(w_dtype)) return GPTQ_ERR_INVALID_ARG;
    if (d_out <= 0 || d_in <= 0 || d_out > MAX_DIM || d_in > MAX_DIM || ld_w < d_in) return GPTQ_ERR_INVALID_ARG;
    gptq_status st = check_config(cfg);
    if (st != GPTQ_OK) return st;
    if (!sweep_factored_supported(d_in, cfg)) return GPTQ_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < sweep_workspace_bytes(d_out, d_in, cfg, true)) return GPTQ_ERR_WORKSPACE;
    int flags[N_FLAGS] = {0, 0, 0, 0};
    st = sweep_launch(W, w_dtype, d_out, d_in, ld_w, F, perm, cfg, codes, scales, zeros, g_idx, w_hat, row_loss,
                      workspace, stream, flags, true);
    if (st != GPTQ_OK) return st;
    if (flags[FLAG_BAD_PERM]) return GPTQ_ERR_INVALID_ARG;
    if (flags[FLAG_NONFINITE]) return GPTQ_ERR_NONFINITE;
    return GPTQ_OK;
}

size_t gptq_quantize_layer_workspace(int64_t d_out, int64_t d_in, const gptq_config* cfg) {
    if (d_out <= 0 || d_in <= 0 || d_out > MAX_DIM || d_in > MAX_DIM) return 0;
    if (check_config(cfg) != GPTQ_OK) return 0;
    return sweep_workspace_bytes(d_out, d_in, cfg);
}

gptq_status gptq_quantize_layer(const void* W, gptq_dtype w_dtype, int64_t d_out, int64_t d_in, int64_t ld_w,
                                const double* U, const int32_t* perm, const gptq_config* cfg, uint8_t* codes,
                                float* scales, float* zeros, int32_t* g_idx, float* w_hat, double* row_loss,
                                void* workspace, size_t ws_bytes, hipStream_t stream) {
    if (!W || !U || !perm || !codes || !scales || !zeros || !g_idx) return GPTQ_ERR_INVALID_ARG;
    if (!valid_dtype(w_dtype)) return GPTQ_ERR_INVALID_ARG;
    if (d_out <= 0 || d_in <= 0 || d_out > MAX_DIM || d_in > MAX_DIM || ld_w < d_in) return GPTQ_ERR_INVALID_ARG;
    gptq_status st = check_config(cfg);
    if (st != GPTQ_OK) return st;
    if (!workspace || ws_bytes < sweep_workspace_bytes(d_out, d_in, cfg)) return GPTQ_ERR_WORKSPACE;
    int flags[N_FLAGS] = {0, 0, 0, 0};
    st = sweep_launch(W, w_dtype, d_out, d_in, ld_w, U, perm, cfg, codes, scales, zeros, g_idx, w_hat, row_loss,
                      workspace, stream, flags);
    if (st != GPTQ_OK) return st;
    if (flags[FLAG_BAD_PERM]) return GPTQ_ERR_INVALID_ARG;
    if (flags[FLAG_NONFINITE]) return GPTQ_ERR_NONFINITE;
    return GPTQ_OK;
}

int64_t gptq_packed_words_per_row(int64_t d_in, int32_t bits) {
    if (d_in < 0 || !valid_bits(bits)) return -1;
    return ceil_div(d_in * bits, 32);
}

gptq_status gptq_pack(const uint8_t* codes, int64_t d_out, int64_t d_in, int32_t bits, uint32_t* packed,
                      hipStream_t stream) {
    if (!codes || !packed || !valid_bits(bits)) return GPTQ_ERR_INVALID_ARG;
    if (d_out <= 0 || d_in <= 0 || d_out > MAX_DIM || d_in > MAX_DIM) return GPTQ_ERR_INVALID_ARG;
    return pack_launch(codes, d_out, d_in, bits, nullptr, packed, stream);
}

gptq_status gptq_pack_permuted(const uint8_t* codes, int64_t d_out, int64_t d_in, int32_t bits, const int32_t* perm,
                               uint32_t* packed, hipStream_t stream) {
    if (!codes || !packed || !perm || !valid_bits(bits)) return GPTQ_ERR_INVALID_ARG;
    if (d_out <= 0 || d_in <= 0 || d_out > MAX_DIM || d_in > MAX_DIM) return GPTQ_ERR_INVALID_ARG;
    return pack_launch(codes, d_out, d_in, bits, perm, packed, stream);
}

int64_t gptq_dequant_max_groups(void) { return dequant_max_groups(); }

gptq_status gptq_gather_columns(const void* X, gptq_dtype x_dtype, int64_t n_tok, int64_t d_in, int64_t ld_x,
                                const int32_t* perm, void* Xg, int64_t ld_g, hipStream_t stream) {
    if (!valid_dtype(x_dtype)) return GPTQ_ERR_INVALID_ARG;
    if (n_tok < 0 || d_in <= 0 || n_tok > (int64_t(1) << 32) || d_in > MAX_DIM) return GPTQ_ERR_INVALID_ARG;
    if (ld_x < d_in || ld_g < d_in) return GPTQ_ERR_INVALID_ARG;
    if (n_tok == 0) return GPTQ_OK;
    if (!X || !perm || !Xg) return GPTQ_ERR_INVALID_ARG;
    return gather_columns_launch(X, x_dtype, n_tok, d_in, ld_x, perm, Xg, ld_g, stream);
}

gptq_status gptq_dequant_matmul(const void* X, gptq_dtype x_dtype, int64_t n_tok, int64_t d_in, int64_t ld_x,
                                const uint32_t* packed, int32_t bits, const float* scales, const float* zeros,
                                int64_t n_groups, const int32_t* g_idx, const int32_t* perm, int32_t group_size,
                                int64_t d_out, float* Y, int64_t ld_y, hipStream_t stream) {
    if (!valid_dtype(x_dtype) || !valid_bits(bits)) return GPTQ_ERR_INVALID_ARG;
    if (n_tok < 0 || d_in <= 0 || d_out < 0 || n_tok > MAX_DIM || d_in > MAX_DIM || d_out > MAX_DIM)
        return GPTQ_ERR_INVALID_ARG;
    if (ld_x < d_in || ld_y < d_out) return GPTQ_ERR_INVALID_ARG;
    if (g_idx && perm) return GPTQ_ERR_INVALID_ARG;
    const int64_t expect = (group_size > 0) ? ceil_div(d_in, group_size) : 1;
    if (g_idx ? (n_groups < 1 || n_groups > d_in) : (n_groups != expect)) return GPTQ_ERR_INVALID_ARG;
    if (n_tok == 0 || d_out == 0) return GPTQ_OK;
    if (!X || !packed || !scales || !zeros || !Y) return GPTQ_ERR_INVALID_ARG;
    return dequant_matmul_launch(X, x_dtype, n_tok, d_in, ld_x, packed, bits, scales, zeros, n_groups, g_idx, perm,
                                 group_size, d_out, Y, ld_y, stream);
}

}  // extern "C"
