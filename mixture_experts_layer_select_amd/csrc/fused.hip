// The whole MoE layer for a small batch in one persistent launch ([Moreh-EP]
// Library optimization: a fused MoE kernel for small batch sizes; Use of HIP
// Graphs: static sizes, so the launch can be captured).
//
// One workgroup of 512 threads per CU runs the layer's steps as phases, with
// a grid-wide barrier between them:
//   1. router logits (one token-expert pair per wave up to 64 tokens, else
//      8 x 8 tiles per wave; the fixed fp32 order of moe_route) barrier
//   2. top-k and combine weights (one wave per token)          barrier
//   3. the permutation in workgroup 0; fp8: every token quantised once (1x128
//      blocks) by the other workgroups                       barrier
//   4. bf16: x_perm rows copied from their tokens             barrier
//   5. gate/up + SwiGLU as the grouped GEMM of moe_expert_ffn  barrier
//   6. down projection                                         barrier
//   7. routing-weighted combine
// Every phase runs the device code of the separate kernels, so the results are
// bit for bit those of moe_route, moe_permute, moe_expert_ffn (fp8: the token-row
// gate/up) and moe_combine on the same inputs.
//
// Grid barrier: an arrival counter and a generation word in the workspace.
// The last workgroup to arrive resets the counter and bumps the generation;
// the others poll the generation with a sleep between polls, for a bounded
// number of polls. Agent-scope release before arriving (the L2 write-back of
// this XCD) and acquire after leaving (the invalidation of this CU's vector
// cache and of its XCD's L2), each by one thread of the workgroup after a
// workgroup barrier, make each phase's global writes visible to every XCD.
// The grid is
// one workgroup per CU, all resident at once on an otherwise idle device; if
// a poll limit is reached (the grid was not resident), the error word is set,
// the waves carry on, and the outputs are invalid.
#include "combine_dev.h"
#include "ffn_dev.h"
#include "permute_dev.h"
#include "route_dev.h"

namespace moe {
namespace {

constexpr int kFusedThreads = 512;
constexpr int kFusedRowsMaxT = 64;  // batches routed one (token, expert) pair per wave
constexpr unsigned kPollLimit = 1u << 20;  // polls before a barrier gives up (about a second)

struct GridBar {
    unsigned count;  // arrivals at the current barrier
    unsigned gen;    // barriers completed
    unsigned error;  // nonzero: a poll limit was reached
};

__device__ __forceinline__ void grid_sync(GridBar* b) {
    __syncthreads();  // every wave of this workgroup is done with the phase
    if (threadIdx.x == 0) {
        const unsigned g0 = __hip_atomic_load(&b->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned arrived =
            __hip_atomic_fetch_add(&b->count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) + 1u;
        if (arrived == gridDim.x) {
            __hip_atomic_store(&b->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&b->gen, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            for (unsigned i = 0;
                 __hip_atomic_load(&b->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g0; ++i) {
                if (i >= kPollLimit) {
                    __hip_atomic_store(&b->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        // one acquire per workgroup: the invalidation it issues covers this
        // CU's vector cache and its XCD's L2, which every wave here reads
        // through (one per wave tripled the barrier's cost)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

struct FusedArgs {
    const uint16_t* x;        // [T][H] bf16
    const uint16_t* wr;       // [E][H] bf16
    const float* bias;        // [E] or null
    int T, H, E, k, I, scoring, renorm, has_shared;
    const void* w13;
    const float* w13s;
    const void* w2;
    const float* w2s;
    const void* ws13;
    const float* ws13s;
    const void* ws2;
    const float* ws2s;
    int32_t* ids;             // [T][k] out
    float* topk_w;            // [T][k] out
    uint16_t* out;            // [T][H] bf16 out
    // workspace
    GridBar* bar;
    float* logits;            // [T][E]
    int32_t* counts;          // [E+1]
    int32_t* offsets;         // [E+2]
    int32_t* row_to_slot;     // [cap]
    int32_t* slot_to_row;     // [T*k]
    void* xact;               // bf16: x_perm [cap][H]; fp8: token codes [T][H]
    float* xact_scale;        // fp8: [H/128][T]
    void* a;                  // intermediate [cap][I] (bf16, or e4m3 codes)
    float* a_scale;           // fp8: [I/128][cap]
    uint16_t* y;              // [cap][H] bf16
};

template <bool kFp8>
__global__ __launch_bounds__(kFusedThreads) void moe_layer_fused_kernel(FusedArgs p) {
    __shared__ PermLds pl;
    __shared__ TileMap tm;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int S = p.T * p.k;
    const int cap = S + p.T;
    const int n_groups = p.E + (p.has_shared ? 1 : 0);
    const int gw = blockIdx.x * (kFusedThreads / 64) + wave;  // wave index in the grid
    const int nw = gridDim.x * (kFusedThreads / 64);

    // 1. router logits: one (token, expert) pair per wave for small batches,
    // 8 x 8 tiles otherwise (the same logits bit for bit)
    if (p.T <= kFusedRowsMaxT && p.H <= 16 * kStep) {
        for (int q = gw; q < p.T * p.E; q += nw)
            route_logits_row<16>(p.x, p.wr, p.bias, p.H, p.E, p.logits, q / p.E, q % p.E);
    } else {
        const int n_et = (p.E + kWE - 1) / kWE;
        const int tasks = (p.T + kWT - 1) / kWT * n_et;
        for (int q = gw; q < tasks; q += nw)
            route_logits_tile(p.x, p.wr, p.bias, p.T, p.H, p.E, p.logits, q / n_et * kWT, q % n_et * kWE);
    }
    grid_sync(p.bar);
    // 2. selection and weights
    for (int t = gw; t < p.T; t += nw)
        route_topk_token(p.logits, p.T, p.E, p.k, p.scoring, p.renorm, p.ids, p.topk_w, t);
    grid_sync(p.bar);
    // 3. permutation (workgroup 0); fp8: the tokens quantised by the others
    if (blockIdx.x == 0) {
        perm_block(p.ids, S, p.T, 0, p.E, p.has_shared ? p.T : 0, p.counts, p.offsets, p.row_to_slot,
                   p.slot_to_row, pl);
    } else if constexpr (kFp8) {
        const int vb = (blockIdx.x - 1) * 2 + (tid >> 8), nvb = (gridDim.x - 1) * 2;
        for (int t = vb; t < p.T; t += nvb)
            quant_row_fp8(p.x + (size_t)t * p.H, p.H, p.T, t, (uint8_t*)p.xact, p.xact_scale, tid & 255);
    }
    grid_sync(p.bar);
    if constexpr (!kFp8) {
        // 4. x_perm: the rows of every group (shared rows included) from their tokens
        const int used = p.offsets[n_groups];
        for (int r = blockIdx.x; r < used; r += gridDim.x) {
            const int slot = p.row_to_slot[r];
            const int t = slot < S ? slot / p.k : slot - S;
            const u32x4* src = reinterpret_cast<const u32x4*>(p.x + (size_t)t * p.H);
            u32x4* dst = reinterpret_cast<u32x4*>((uint16_t*)p.xact + (size_t)r * p.H);
            for (int i = tid; i < p.H / 8; i += kFusedThreads) dst[i] = src[i];
        }
        grid_sync(p.bar);
        __shared__ __attribute__((aligned(16))) uint8_t xs[2][kBigTile * kLdsRowBf16];
        // 5. gate/up + SwiGLU, 6. down
        ffn_gemm_bf16_body<true, kBigTile, 8>((const uint16_t*)p.xact, (const uint16_t*)p.w13,
                                              (const uint16_t*)p.ws13, p.E, p.offsets, n_groups, cap,
                                              p.H, 2 * p.I, p.I / 128, (uint16_t*)p.a, p.I, xs, tm,
                                              blockIdx.x, gridDim.x);
        grid_sync(p.bar);
        ffn_gemm_bf16_body<false, kBigTile, 8>((const uint16_t*)p.a, (const uint16_t*)p.w2,
                                               (const uint16_t*)p.ws2, p.E, p.offsets, n_groups, cap,
                                               p.I, p.H, p.H / 256, p.y, p.H, xs, tm, blockIdx.x,
                                               gridDim.x);
    } else {
        __shared__ __attribute__((aligned(1024))) XStage st0;
        __shared__ __attribute__((aligned(1024))) XStage st1;
        __shared__ __attribute__((aligned(1024))) XStage st2;
        __shared__ float wsc[2][kLMaxSteps];
        __shared__ float red[kLWaves * kLTM];
        // 5. gate/up + SwiGLU from the token rows, A quantised per 1x128 block
        ffn_gemm_fp8_lds_body<true, true>((const uint8_t*)p.xact, p.xact_scale, (const uint8_t*)p.w13,
                                          p.w13s, (const uint8_t*)p.ws13, p.ws13s, p.E, p.offsets,
                                          n_groups, cap, p.H, 2 * p.I, p.I / 128, p.a, p.a_scale, p.I,
                                          ActSrc{p.row_to_slot, p.k, S, p.T, p.T}, st0, st1, st2, tm,
                                          wsc, red, blockIdx.x, gridDim.x);
        grid_sync(p.bar);
        // 6. down
        ffn_gemm_fp8_lds_body<false, false>((const uint8_t*)p.a, p.a_scale, (const uint8_t*)p.w2, p.w2s,
                                            (const uint8_t*)p.ws2, p.ws2s, p.E, p.offsets, n_groups,
                                            cap, p.I, p.H, p.H / 256, p.y, nullptr, p.H,
                                            ActSrc{nullptr, 0, 0, 0, 0}, st0, st1, st2, tm, wsc, red,
                                            blockIdx.x, gridDim.x);
    }
    grid_sync(p.bar);
    // 7. combine: four blocks of 128 threads per workgroup
    combine_small_k_units(p.y, p.slot_to_row, p.topk_w, p.T, p.k, p.H, p.offsets,
                          p.has_shared ? p.E : -1, p.out, blockIdx.x * 4 + (tid >> 7),
                          (long)gridDim.x * 4, tid & 127);
}

// workspace: barrier words (256 B) | logits | counts | offsets | row_to_slot |
// slot_to_row | activations (+ scales) | intermediate (+ scales) | y_perm
struct FusedWs {
    GridBar* bar;
    float* logits;
    int32_t *counts, *offsets, *row_to_slot, *slot_to_row;
    void* xact;
    float* xact_scale;
    void* a;
    float* a_scale;
    uint16_t* y;
    size_t bytes;
};

FusedWs carve_fused(const moe_expert_weights* w, int T, int E, int k, void* base) {
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes, 256);
        return base ? (void*)((uint8_t*)base + o) : nullptr;
    };
    const bool fp8 = w->dt == MOE_FP8_E4M3;
    const size_t cap = (size_t)T * k + T;
    FusedWs r{};
    r.bar = (GridBar*)take(256);
    r.logits = (float*)take((size_t)T * E * 4);
    r.counts = (int32_t*)take((size_t)(E + 1) * 4);
    r.offsets = (int32_t*)take((size_t)(E + 2) * 4);
    r.row_to_slot = (int32_t*)take(cap * 4);
    r.slot_to_row = (int32_t*)take((size_t)T * k * 4);
    if (fp8) {
        r.xact = take((size_t)T * w->H);
        r.xact_scale = (float*)take((size_t)(w->H / 128) * T * 4);
        r.a = take(cap * w->I);
        r.a_scale = (float*)take((size_t)(w->I / 128) * cap * 4);
    } else {
        r.xact = take(cap * w->H * 2);
        r.a = take(cap * w->I * 2);
    }
    r.y = (uint16_t*)take(cap * w->H * 2);
    r.bytes = off;
    return r;
}

}  // namespace

size_t layer_fused_workspace_bytes(const moe_expert_weights* w, int T, int E, int k) {
    return carve_fused(w, T, E, k, nullptr).bytes;
}

moe_status launch_layer_fused(const void* x, const void* w_router, const float* bias, int T, int E, int k,
                              int scoring, int renorm, const moe_expert_weights* w, int32_t* topk_ids,
                              float* topk_w, void* out, void* ws, hipStream_t st) {
    const FusedWs s = carve_fused(w, T, E, k, ws);
    FusedArgs p{};
    p.x = (const uint16_t*)x;
    p.wr = (const uint16_t*)w_router;
    p.bias = bias;
    p.T = T;
    p.H = w->H;
    p.E = E;
    p.k = k;
    p.I = w->I;
    p.scoring = scoring;
    p.renorm = renorm;
    p.has_shared = w->ws13 != nullptr;
    p.w13 = w->w13;
    p.w13s = w->w13_scale;
    p.w2 = w->w2;
    p.w2s = w->w2_scale;
    p.ws13 = w->ws13;
    p.ws13s = w->ws13_scale;
    p.ws2 = w->ws2;
    p.ws2s = w->ws2_scale;
    p.ids = topk_ids;
    p.topk_w = topk_w;
    p.out = (uint16_t*)out;
    p.bar = s.bar;
    p.logits = s.logits;
    p.counts = s.counts;
    p.offsets = s.offsets;
    p.row_to_slot = s.row_to_slot;
    p.slot_to_row = s.slot_to_row;
    p.xact = s.xact;
    p.xact_scale = s.xact_scale;
    p.a = s.a;
    p.a_scale = s.a_scale;
    p.y = s.y;
    // one workgroup per CU (a multiple of the 8 XCDs): the whole grid is resident
    const int grid = device_info().cu_count / 8 * 8;
    if (w->dt == MOE_FP8_E4M3)
        hipLaunchKernelGGL(moe_layer_fused_kernel<true>, dim3(grid), dim3(kFusedThreads), 0, st, p);
    else
        hipLaunchKernelGGL(moe_layer_fused_kernel<false>, dim3(grid), dim3(kFusedThreads), 0, st, p);
    return check_launch("moe_layer_fused_kernel");
}

}  // namespace moe
