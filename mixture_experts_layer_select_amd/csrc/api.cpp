// C ABI of libmoe.so: argument validation and dispatch to the kernels.
// Every check happens before anything is enqueued; a rejected call leaves
// the stream untouched.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <vector>

#include "moe_internal.h"

namespace moe {

static thread_local char g_msg[512] = "";

moe_status set_error(moe_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return s;
}

moe_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_error(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

const DeviceInfo& device_info() {
    static std::mutex mu;
    static std::vector<DeviceInfo> cache;
    static std::vector<bool> known;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)cache.size() <= dev) {
        cache.resize(dev + 1);
        known.resize(dev + 1, false);
    }
    if (!known[dev]) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
            cu = 256;
        cache[dev].cu_count = cu;
        known[dev] = true;
    }
    return cache[dev];
}

}  // namespace moe

using namespace moe;

#define REQUIRE(cond, code, ...)                        \
    do {                                                \
        if (!(cond)) return set_error(code, __VA_ARGS__); \
    } while (0)

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        default: return "MOE_ERR_UNKNOWN";
    }
}

const char* moe_last_error_message(void) { return g_msg; }

moe_status moe_route(const void* x, const void* w_router, const float* bias, moe_dtype dt, int T,
                     int H, int E, int k, moe_scoring scoring, int renormalize, float* logits,
                     int32_t* topk_ids, float* topk_w, void* stream) {
    g_msg[0] = 0;
    REQUIRE(T >= 0 && H >= 1 && E >= 1 && k >= 1, MOE_ERR_INVALID_ARG,
            "moe_route: need T >= 0, H >= 1, E >= 1, k >= 1 (T=%d H=%d E=%d k=%d)", T, H, E, k);
    REQUIRE(k <= E, MOE_ERR_INVALID_ARG, "moe_route: k=%d > E=%d", k, E);
    REQUIRE(E <= 256, MOE_ERR_UNSUPPORTED, "moe_route: E=%d > 256", E);
    REQUIRE(dt == MOE_F32 || dt == MOE_BF16, MOE_ERR_UNSUPPORTED,
            "moe_route: dt must be MOE_F32 or MOE_BF16");
    REQUIRE(scoring == MOE_SOFTMAX || scoring == MOE_SIGMOID, MOE_ERR_INVALID_ARG,
            "moe_route: unknown scoring %d", (int)scoring);
    if (T == 0) return MOE_OK;
    REQUIRE(x && w_router && logits && topk_ids && topk_w, MOE_ERR_INVALID_ARG,
            "moe_route: null pointer");
    return launch_route(x, w_router, bias, dt, T, H, E, k, scoring, renormalize ? 1 : 0, logits,
                        topk_ids, topk_w, (hipStream_t)stream);
}

size_t moe_route_select_workspace_size(int T, int E) {
    if (T < 0 || E < 1) return 0;
    return route_select_workspace_bytes(T, E);
}

moe_status moe_route_select(const void* x, const void* w_router, const float* bias, moe_dtype dt,
                            int T, int H, int E, int k, moe_scoring scoring, int renormalize,
                            int32_t* topk_ids, float* topk_w, void* workspace, size_t ws_bytes,
                            void* stream) {
    g_msg[0] = 0;
    REQUIRE(T >= 0 && H >= 1 && E >= 1 && k >= 1, MOE_ERR_INVALID_ARG,
            "moe_route_select: need T >= 0, H >= 1, E >= 1, k >= 1 (T=%d H=%d E=%d k=%d)", T, H, E, k);
    REQUIRE(k <= E, MOE_ERR_INVALID_ARG, "moe_route_select: k=%d > E=%d", k, E);
    REQUIRE(scoring == MOE_SOFTMAX || scoring == MOE_SIGMOID, MOE_ERR_INVALID_ARG,
            "moe_route_select: unknown scoring %d", (int)scoring);
    REQUIRE(E <= 256, MOE_ERR_UNSUPPORTED, "moe_route_select: E=%d > 256", E);
    REQUIRE(dt == MOE_BF16, MOE_ERR_UNSUPPORTED, "moe_route_select: dt must be MOE_BF16");
    REQUIRE(H % 32 == 0 && H <= 8192, MOE_ERR_UNSUPPORTED,
            "moe_route_select: need H %% 32 == 0 and H <= 8192 (H=%d)", H);
    REQUIRE(scoring == MOE_SIGMOID || renormalize, MOE_ERR_UNSUPPORTED,
            "moe_route_select: softmax without renormalisation needs every logit (use moe_route)");
    if (T == 0) return MOE_OK;
    REQUIRE(x && w_router && topk_ids && topk_w, MOE_ERR_INVALID_ARG, "moe_route_select: null pointer");
    const size_t need = route_select_workspace_bytes(T, E);
    REQUIRE(workspace && ws_bytes >= need, MOE_ERR_WORKSPACE,
            "moe_route_select: workspace %zu < %zu bytes", ws_bytes, need);
    return launch_route_select(x, w_router, bias, T, H, E, k, scoring, renormalize ? 1 : 0, topk_ids,
                               topk_w, workspace, (hipStream_t)stream);
}

size_t moe_permute_workspace_size(int T, int k, int E_local) {
    if (T < 0 || k < 1 || E_local < 1) return 0;
    return permute_workspace_bytes(T, k, E_local);
}

moe_status moe_permute(const int32_t* topk_ids, int T, int k, int expert_base, int E_local,
                       int include_shared, const void* x, moe_dtype x_dt, int H, moe_dtype perm_dt,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_to_slot,
                       int32_t* slot_to_row, void* x_perm, float* x_perm_scale, void* workspace,
                       size_t ws_bytes, void* stream) {
    g_msg[0] = 0;
    REQUIRE(T >= 0 && k >= 1 && E_local >= 1, MOE_ERR_INVALID_ARG,
            "moe_permute: need T >= 0, k >= 1, E_local >= 1 (T=%d k=%d E_local=%d)", T, k, E_local);
    REQUIRE(E_local <= 256, MOE_ERR_UNSUPPORTED, "moe_permute: E_local=%d > 256", E_local);
    REQUIRE((long)T * k + T < (1L << 31), MOE_ERR_UNSUPPORTED, "moe_permute: T*k+T exceeds int32");
    if (T == 0) return MOE_OK;
    REQUIRE(topk_ids && expert_counts && expert_offsets && row_to_slot && slot_to_row,
            MOE_ERR_INVALID_ARG, "moe_permute: null pointer");
    if (x_perm) {
        REQUIRE(x && H >= 1, MOE_ERR_INVALID_ARG, "moe_permute: x_perm given without x / H");
        if (perm_dt == MOE_FP8_E4M3) {
            REQUIRE(x_dt == MOE_BF16, MOE_ERR_UNSUPPORTED, "moe_permute: fp8 x_perm needs bf16 x");
            REQUIRE(H % 128 == 0, MOE_ERR_UNSUPPORTED, "moe_permute: fp8 needs H %% 128 == 0 (H=%d)", H);
            REQUIRE(x_perm_scale, MOE_ERR_INVALID_ARG, "moe_permute: fp8 needs x_perm_scale");
        } else {
            REQUIRE(perm_dt == x_dt && (x_dt == MOE_BF16 || x_dt == MOE_F32), MOE_ERR_UNSUPPORTED,
                    "moe_permute: perm_dt must equal x_dt (bf16/f32) or be fp8");
        }
    }
    const size_t need = permute_workspace_bytes(T, k, E_local);
    REQUIRE(workspace && ws_bytes >= need, MOE_ERR_WORKSPACE,
            "moe_permute: workspace %zu < %zu bytes", ws_bytes, need);
    return launch_permute(topk_ids, T, k, expert_base, E_local, include_shared ? 1 : 0, x, x_dt, H,
                          perm_dt, expert_counts, expert_offsets, row_to_slot, slot_to_row, x_perm,
                          x_perm_scale, workspace, (hipStream_t)stream);
}

static moe_status check_weights(const moe_expert_weights* w) {
    REQUIRE(w, MOE_ERR_INVALID_ARG, "moe_expert_ffn: null weights");
    REQUIRE(w->E_local >= 1 && w->H >= 1 && w->I >= 1, MOE_ERR_INVALID_ARG,
            "moe_expert_ffn: need E_local, H, I >= 1");
    REQUIRE(w->E_local <= 1024, MOE_ERR_UNSUPPORTED, "moe_expert_ffn: E_local > 1024");
    REQUIRE(w->w13 && w->w2, MOE_ERR_INVALID_ARG, "moe_expert_ffn: null w13/w2");
    if (w->dt == MOE_BF16) {
        REQUIRE(w->H % 128 == 0 && w->I % 128 == 0, MOE_ERR_UNSUPPORTED,
                "moe_expert_ffn: bf16 needs H, I multiples of 128 (H=%d I=%d)", w->H, w->I);
    } else if (w->dt == MOE_FP8_E4M3) {
        REQUIRE(w->H % 256 == 0 && w->I % 128 == 0, MOE_ERR_UNSUPPORTED,
                "moe_expert_ffn: fp8 needs H %% 256 == 0 and I %% 128 == 0 (H=%d I=%d)", w->H, w->I);
        REQUIRE(w->H <= 16384 && w->I <= 16384, MOE_ERR_UNSUPPORTED,
                "moe_expert_ffn: fp8 needs H, I <= 16384 (H=%d I=%d)", w->H, w->I);
        REQUIRE(w->w13_scale && w->w2_scale, MOE_ERR_INVALID_ARG, "moe_expert_ffn: fp8 needs scales");
    } else {
        REQUIRE(w->dt == MOE_F32, MOE_ERR_UNSUPPORTED, "moe_expert_ffn: unknown dt %d", (int)w->dt);
    }
    return MOE_OK;
}

size_t moe_expert_ffn_workspace_size(const moe_expert_weights* w, int max_rows) {
    if (max_rows < 0 || check_weights(w) != MOE_OK) return 0;
    return ffn_workspace_bytes(w, max_rows);
}

static moe_status check_ffn_call(const char* fn, const moe_expert_weights* w, int n_groups,
                                 int max_rows, const int32_t* expert_offsets, void* workspace,
                                 size_t ws_bytes) {
    moe_status s = check_weights(w);
    if (s) return s;
    REQUIRE(max_rows >= 0, MOE_ERR_INVALID_ARG, "%s: max_rows < 0", fn);
    REQUIRE(n_groups == w->E_local || n_groups == w->E_local + 1, MOE_ERR_INVALID_ARG,
            "%s: n_groups=%d must be E_local or E_local+1", fn, n_groups);
    if (n_groups == w->E_local + 1) {
        REQUIRE(w->ws13 && w->ws2, MOE_ERR_INVALID_ARG, "%s: shared group without weights", fn);
        REQUIRE(w->dt != MOE_FP8_E4M3 || (w->ws13_scale && w->ws2_scale), MOE_ERR_INVALID_ARG,
                "%s: fp8 shared expert needs scales", fn);
    }
    if (max_rows == 0) return MOE_OK;
    REQUIRE(expert_offsets, MOE_ERR_INVALID_ARG, "%s: null expert_offsets", fn);
    const size_t need = ffn_workspace_bytes(w, max_rows);
    REQUIRE(workspace && ws_bytes >= need, MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn,
            ws_bytes, need);
    return MOE_OK;
}

moe_status moe_expert_ffn_gate_up(const moe_expert_weights* w, const void* x_perm,
                                  const float* x_perm_scale, const int32_t* expert_offsets,
                                  int n_groups, int max_rows, void* workspace, size_t ws_bytes,
                                  void* stream) {
    g_msg[0] = 0;
    moe_status s = check_ffn_call("moe_expert_ffn_gate_up", w, n_groups, max_rows, expert_offsets,
                                  workspace, ws_bytes);
    if (s || max_rows == 0) return s;
    REQUIRE(x_perm, MOE_ERR_INVALID_ARG, "moe_expert_ffn_gate_up: null x_perm");
    REQUIRE(w->dt != MOE_FP8_E4M3 || x_perm_scale, MOE_ERR_INVALID_ARG,
            "moe_expert_ffn_gate_up: fp8 needs x_perm_scale");
    return launch_ffn_gate_up(w, x_perm, x_perm_scale, expert_offsets, n_groups, max_rows, workspace,
                              (hipStream_t)stream);
}

moe_status moe_quantize_tokens(const void* x, moe_dtype x_dt, int T, int H, void* codes,
                               float* scales, void* stream) {
    g_msg[0] = 0;
    REQUIRE(T >= 0 && H >= 1, MOE_ERR_INVALID_ARG, "moe_quantize_tokens: T=%d H=%d", T, H);
    REQUIRE(x_dt == MOE_BF16, MOE_ERR_UNSUPPORTED, "moe_quantize_tokens: x must be bf16");
    REQUIRE(H % 128 == 0, MOE_ERR_UNSUPPORTED, "moe_quantize_tokens: H=%d not a multiple of 128", H);
    REQUIRE((long)T * H < (1L << 31), MOE_ERR_UNSUPPORTED, "moe_quantize_tokens: T*H >= 2^31");
    if (T == 0) return MOE_OK;
    REQUIRE(x && codes && scales, MOE_ERR_INVALID_ARG, "moe_quantize_tokens: null pointer");
    return launch_quantize_tokens(x, T, H, codes, scales, (hipStream_t)stream);
}

moe_status moe_expert_ffn_gate_up_tokens(const moe_expert_weights* w, const void* x_tokens,
                                         const float* x_tokens_scale, int T, int k,
                                         const int32_t* row_to_slot, const int32_t* expert_offsets,
                                         int n_groups, int max_rows, void* workspace,
                                         size_t ws_bytes, void* stream) {
    g_msg[0] = 0;
    moe_status s = check_ffn_call("moe_expert_ffn_gate_up_tokens", w, n_groups, max_rows,
                                  expert_offsets, workspace, ws_bytes);
    if (s) return s;
    REQUIRE(w->dt == MOE_FP8_E4M3, MOE_ERR_UNSUPPORTED, "moe_expert_ffn_gate_up_tokens: fp8 only");
    REQUIRE(T >= 0 && k >= 1, MOE_ERR_INVALID_ARG, "moe_expert_ffn_gate_up_tokens: T=%d k=%d", T, k);
    REQUIRE((long)T * w->H < (1L << 31) && (long)T * (k + 1) < (1L << 31), MOE_ERR_UNSUPPORTED,
            "moe_expert_ffn_gate_up_tokens: T*H or T*(k+1) >= 2^31");
    if (max_rows == 0 || T == 0) return MOE_OK;
    REQUIRE(x_tokens && x_tokens_scale && row_to_slot, MOE_ERR_INVALID_ARG,
            "moe_expert_ffn_gate_up_tokens: null pointer");
    return launch_ffn_gate_up(w, x_tokens, x_tokens_scale, expert_offsets, n_groups, max_rows,
                              workspace, (hipStream_t)stream, ActSrc{row_to_slot, k, T * k, T, T});
}

moe_status moe_expert_ffn_down(const moe_expert_weights* w, const int32_t* expert_offsets,
                               int n_groups, int max_rows, void* y_perm, void* workspace,
                               size_t ws_bytes, void* stream) {
    g_msg[0] = 0;
    moe_status s = check_ffn_call("moe_expert_ffn_down", w, n_groups, max_rows, expert_offsets,
                                  workspace, ws_bytes);
    if (s || max_rows == 0) return s;
    REQUIRE(y_perm, MOE_ERR_INVALID_ARG, "moe_expert_ffn_down: null y_perm");
    return launch_ffn_down(w, expert_offsets, n_groups, max_rows, y_perm, workspace,
                           (hipStream_t)stream);
}

moe_status moe_expert_ffn(const moe_expert_weights* w, const void* x_perm, const float* x_perm_scale,
                          const int32_t* expert_offsets, int n_groups, int max_rows, void* y_perm,
                          void* workspace, size_t ws_bytes, void* stream) {
    g_msg[0] = 0;
    moe_status s = check_ffn_call("moe_expert_ffn", w, n_groups, max_rows, expert_offsets, workspace,
                                  ws_bytes);
    if (s || max_rows == 0) return s;
    REQUIRE(x_perm && y_perm, MOE_ERR_INVALID_ARG, "moe_expert_ffn: null pointer");
    REQUIRE(w->dt != MOE_FP8_E4M3 || x_perm_scale, MOE_ERR_INVALID_ARG,
            "moe_expert_ffn: fp8 needs x_perm_scale");
    s = launch_ffn_gate_up(w, x_perm, x_perm_scale, expert_offsets, n_groups, max_rows, workspace,
                           (hipStream_t)stream);
    if (s) return s;
    return launch_ffn_down(w, expert_offsets, n_groups, max_rows, y_perm, workspace,
                           (hipStream_t)stream);
}

moe_status moe_expert_ffn_noalloc(const moe_expert_weights* w, const void* x_perm,
                                  const float* x_perm_scale, const int32_t* expert_offsets,
                                  int n_groups, int max_rows, void* y_perm, void* stream) {
    g_msg[0] = 0;
    moe_status s = check_weights(w);
    if (s) return s;
    REQUIRE(max_rows >= 0, MOE_ERR_INVALID_ARG, "moe_expert_ffn_noalloc: max_rows < 0");
    const size_t need = ffn_workspace_bytes(w, max_rows);
    REQUIRE(need <= (size_t)MOE_NOALLOC_SCRATCH_BYTES, MOE_ERR_WORKSPACE,
            "moe_expert_ffn_noalloc: max_rows=%d needs %zu bytes of scratch, the static array "
            "holds %zu (use moe_expert_ffn with a workspace)",
            max_rows, need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    void* scratch = nullptr;
    if (max_rows > 0 && (s = ffn_noalloc_scratch(&scratch))) return s;
    s = check_ffn_call("moe_expert_ffn_noalloc", w, n_groups, max_rows, expert_offsets, scratch,
                       (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    if (s || max_rows == 0) return s;
    REQUIRE(x_perm && y_perm, MOE_ERR_INVALID_ARG, "moe_expert_ffn_noalloc: null pointer");
    REQUIRE(w->dt != MOE_FP8_E4M3 || x_perm_scale, MOE_ERR_INVALID_ARG,
            "moe_expert_ffn_noalloc: fp8 needs x_perm_scale");
    s = launch_ffn_gate_up(w, x_perm, x_perm_scale, expert_offsets, n_groups, max_rows, scratch,
                           (hipStream_t)stream);
    if (s) return s;
    return launch_ffn_down(w, expert_offsets, n_groups, max_rows, y_perm, scratch,
                           (hipStream_t)stream);
}

size_t moe_layer_fused_workspace_size(const moe_expert_weights* w, int T, int E, int k) {
    if (T < 0 || E < 1 || k < 1 || check_weights(w) != MOE_OK) return 0;
    return layer_fused_workspace_bytes(w, T, E, k);
}

moe_status moe_layer_fused(const void* x, const void* w_router, const float* bias, int T, int E,
                           int k, moe_scoring scoring, int renormalize,
                           const moe_expert_weights* w, int32_t* topk_ids, float* topk_w,
                           void* out, void* workspace, size_t ws_bytes, void* stream) {
    g_msg[0] = 0;
    moe_status s = check_weights(w);
    if (s) return s;
    REQUIRE(T >= 0 && E >= 1 && k >= 1 && k <= E, MOE_ERR_INVALID_ARG,
            "moe_layer_fused: need T >= 0, 1 <= k <= E (T=%d E=%d k=%d)", T, E, k);
    REQUIRE(scoring == MOE_SOFTMAX || scoring == MOE_SIGMOID, MOE_ERR_INVALID_ARG,
            "moe_layer_fused: unknown scoring %d", (int)scoring);
    REQUIRE(T <= 256 && k <= 8 && E <= 256, MOE_ERR_UNSUPPORTED,
            "moe_layer_fused: needs T <= 256, k <= 8, E <= 256 (T=%d k=%d E=%d)", T, k, E);
    REQUIRE(w->E_local == E, MOE_ERR_INVALID_ARG,
            "moe_layer_fused: all experts must be local (E_local=%d, E=%d)", w->E_local, E);
    REQUIRE(w->dt == MOE_BF16 || w->dt == MOE_FP8_E4M3, MOE_ERR_UNSUPPORTED,
            "moe_layer_fused: bf16 or fp8 experts");
    REQUIRE(w->H % 256 == 0 && w->I % 128 == 0, MOE_ERR_UNSUPPORTED,
            "moe_layer_fused: needs H %% 256 == 0 and I %% 128 == 0 (H=%d I=%d)", w->H, w->I);
    REQUIRE(!w->ws13 == !w->ws2, MOE_ERR_INVALID_ARG, "moe_layer_fused: shared w13 without w2 or back");
    REQUIRE(w->dt != MOE_FP8_E4M3 || !w->ws13 || (w->ws13_scale && w->ws2_scale), MOE_ERR_INVALID_ARG,
            "moe_layer_fused: fp8 shared expert needs scales");
    if (T == 0) return MOE_OK;
    REQUIRE(x && w_router && topk_ids && topk_w && out, MOE_ERR_INVALID_ARG,
            "moe_layer_fused: null pointer");
    const size_t need = layer_fused_workspace_bytes(w, T, E, k);
    REQUIRE(workspace && ws_bytes >= need, MOE_ERR_WORKSPACE, "moe_layer_fused: workspace %zu < %zu bytes",
            ws_bytes, need);
    return launch_layer_fused(x, w_router, bias, T, E, k, scoring, renormalize ? 1 : 0, w, topk_ids,
                              topk_w, out, workspace, (hipStream_t)stream);
}

moe_status moe_combine(const void* y_perm, moe_dtype y_dt, const int32_t* slot_to_row,
                       const float* topk_w, int T, int k, int H, const int32_t* expert_offsets,
                       int shared_group, void* out, moe_dtype out_dt, void* stream) {
    g_msg[0] = 0;
    REQUIRE(T >= 0 && k >= 1 && H >= 1, MOE_ERR_INVALID_ARG, "moe_combine: need T >= 0, k >= 1, H >= 1");
    REQUIRE(k <= 256, MOE_ERR_UNSUPPORTED, "moe_combine: k=%d > 256", k);
    REQUIRE((y_dt == MOE_BF16 || y_dt == MOE_F32) && (out_dt == MOE_BF16 || out_dt == MOE_F32),
            MOE_ERR_UNSUPPORTED, "moe_combine: y_dt/out_dt must be bf16 or f32");
    if (T == 0) return MOE_OK;
    REQUIRE(y_perm && slot_to_row && topk_w && out, MOE_ERR_INVALID_ARG, "moe_combine: null pointer");
    REQUIRE(shared_group < 0 || expert_offsets, MOE_ERR_INVALID_ARG,
            "moe_combine: shared_group needs expert_offsets");
    return launch_combine(y_perm, y_dt, slot_to_row, topk_w, T, k, H, expert_offsets, shared_group,
                          out, out_dt, (hipStream_t)stream);
}

moe_status moe_balanced_partition(const int64_t* counts, int E, int G, int32_t* new_to_old,
                                  int32_t* old_to_new, int64_t* group_loads) {
    g_msg[0] = 0;
    REQUIRE(counts && new_to_old && old_to_new && group_loads, MOE_ERR_INVALID_ARG,
            "moe_balanced_partition: null pointer");
    REQUIRE(E >= 1 && G >= 1 && E % G == 0, MOE_ERR_INVALID_ARG,
            "moe_balanced_partition: need E %% G == 0 (E=%d G=%d)", E, G);
    for (int e = 0; e < E; ++e)
        REQUIRE(counts[e] >= 0, MOE_ERR_INVALID_ARG, "moe_balanced_partition: counts[%d] < 0", e);
    return balanced_partition(counts, E, G, new_to_old, old_to_new, group_loads);
}

moe_status moe_count_accumulate(const int32_t* counts, int n, int64_t* acc, void* stream) {
    g_msg[0] = 0;
    REQUIRE(n >= 0, MOE_ERR_INVALID_ARG, "moe_count_accumulate: n < 0");
    if (n == 0) return MOE_OK;
    REQUIRE(counts && acc, MOE_ERR_INVALID_ARG, "moe_count_accumulate: null pointer");
    return launch_count_accumulate(counts, n, acc, (hipStream_t)stream);
}

moe_status moe_coactivation(const int32_t* topk_ids, int T, int k, int E, int64_t* hist,
                            void* stream) {
    g_msg[0] = 0;
    REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "moe_coactivation: T < 0");
    REQUIRE(T <= (1 << 24), MOE_ERR_UNSUPPORTED, "moe_coactivation: T=%d above 2^24", T);
    REQUIRE(k >= 1 && k <= 256, MOE_ERR_UNSUPPORTED, "moe_coactivation: k=%d outside [1, 256]", k);
    REQUIRE(E >= 1 && E <= 1024, MOE_ERR_UNSUPPORTED, "moe_coactivation: E=%d outside [1, 1024]", E);
    if (T == 0) return MOE_OK;
    REQUIRE(topk_ids && hist, MOE_ERR_INVALID_ARG, "moe_coactivation: null pointer");
    return launch_coactivation(topk_ids, T, k, E, hist, (hipStream_t)stream);
}

moe_status moe_affinity_partition(const int64_t* counts, const int64_t* aff, int E, int G,
                                  int tol_permille, int32_t* new_to_old, int32_t* old_to_new,
                                  int64_t* group_loads, int64_t* intra_affinity) {
    g_msg[0] = 0;
    REQUIRE(counts && aff && new_to_old && old_to_new && group_loads && intra_affinity,
            MOE_ERR_INVALID_ARG, "moe_affinity_partition: null pointer");
    REQUIRE(E >= 1 && G >= 1 && E % G == 0, MOE_ERR_INVALID_ARG,
            "moe_affinity_partition: need E %% G == 0 (E=%d G=%d)", E, G);
    REQUIRE(tol_permille >= 0, MOE_ERR_INVALID_ARG, "moe_affinity_partition: tol_permille < 0");
    for (int e = 0; e < E; ++e)
        REQUIRE(counts[e] >= 0, MOE_ERR_INVALID_ARG, "moe_affinity_partition: counts[%d] < 0", e);
    return affinity_partition(counts, aff, E, G, tol_permille, new_to_old, old_to_new, group_loads,
                              intra_affinity);
}

moe_status moe_gather_rows(const void* src, int n_src_rows, void* dst, const int32_t* index,
                           int n_rows, size_t row_bytes, void* stream) {
    g_msg[0] = 0;
    REQUIRE(n_rows >= 0 && n_src_rows >= 0, MOE_ERR_INVALID_ARG, "moe_gather_rows: negative size");
    REQUIRE(row_bytes % 4 == 0 && row_bytes > 0, MOE_ERR_UNSUPPORTED,
            "moe_gather_rows: row_bytes must be a positive multiple of 4");
    if (n_rows == 0) return MOE_OK;
    REQUIRE(src && dst && index, MOE_ERR_INVALID_ARG, "moe_gather_rows: null pointer");
    return launch_gather_rows(src, dst, index, n_src_rows, n_rows, row_bytes, (hipStream_t)stream);
}

}  // extern "C"
