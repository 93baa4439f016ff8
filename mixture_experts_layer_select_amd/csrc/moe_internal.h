// Internal declarations of libmoe.so (gfx950 / CDNA4). Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------- buffer access
// Raw buffer access: a 128-bit descriptor in SGPRs (base, size in bytes) plus
// a 32-bit lane offset and a scalar offset. Loads need no 64-bit VGPR address
// arithmetic, and accesses at or beyond `bytes` read zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    // dword 3 = 0x00020000: 32-bit data format, the raw-buffer setting on gfx9
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t clamp_bytes(size_t n) { return n < 0xffffffffu ? (uint32_t)n : 0xffffffffu; }

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// round-to-nearest-even fp32 -> bf16 bits (NaN kept quiet)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// four fp32 values (already within +-448) -> four e4m3fn codes, round to nearest even
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
    return (uint32_t)v;
}

__device__ __forceinline__ float clamp_e4m3(float v) { return fminf(fmaxf(v, -kE4M3Max), kE4M3Max); }

// per-1x128-block scale: amax/448 in fp32, 1 for an all-zero block
__device__ __forceinline__ float block_scale(float amax) { return amax == 0.0f ? 1.0f : amax / kE4M3Max; }

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// ---------------------------------------------------------------- host side
struct DeviceInfo {
    int cu_count;
};
const DeviceInfo& device_info();  // of the current device (cached per device)

moe_status set_error(moe_status s, const char* fmt, ...);
moe_status check_launch(const char* what);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- launchers
moe_status launch_route(const void* x, const void* w, const float* bias, moe_dtype dt, int T, int H,
                        int E, int k, int scoring, int renorm, float* logits, int32_t* ids,
                        float* topk_w, hipStream_t st);
size_t route_select_workspace_bytes(int T, int E);
moe_status launch_route_select(const void* x, const void* w, const float* bias, int T, int H, int E,
                               int k, int scoring, int renorm, int32_t* ids, float* topk_w, void* ws,
                               hipStream_t st);

size_t permute_workspace_bytes(int T, int k, int E_local);
moe_status launch_permute(const int32_t* ids, int T, int k, int base, int E_local, int include_shared,
                          const void* x, moe_dtype x_dt, int H, moe_dtype perm_dt, int32_t* counts,
                          int32_t* offsets, int32_t* row_to_slot, int32_t* slot_to_row,
                          void* x_perm, float* x_perm_scale, void* ws, hipStream_t st);

size_t ffn_workspace_bytes(const moe_expert_weights* w, int max_rows);
// device address of the static scratch of moe_expert_ffn_noalloc on the
// current device (looked up on the first call per device)
moe_status ffn_noalloc_scratch(void** ptr);
// Where the fp8 gate/up GEMM reads permuted row r's activations: row r of
// x_perm (row_slot null), or the row of its token in a [rows][H] token
// buffer, token = slot < S ? slot / k : slot - S with slot = row_slot[r];
// the scales are K-major with s_ld rows per K block.
struct ActSrc {
    const int32_t* row_slot;
    int k, S, rows, s_ld;
};
moe_status launch_ffn_gate_up(const moe_expert_weights* w, const void* x_perm,
                              const float* x_perm_scale, const int32_t* offsets, int n_groups,
                              int max_rows, void* ws, hipStream_t st,
                              const ActSrc& src = ActSrc{nullptr, 0, 0, 0, 0});
size_t layer_fused_workspace_bytes(const moe_expert_weights* w, int T, int E, int k);
moe_status launch_layer_fused(const void* x, const void* w_router, const float* bias, int T, int E, int k,
                              int scoring, int renorm, const moe_expert_weights* w, int32_t* topk_ids,
                              float* topk_w, void* out, void* ws, hipStream_t st);
moe_status launch_quantize_tokens(const void* x, int T, int H, void* codes, float* scales,
                                  hipStream_t st);
moe_status launch_ffn_down(const moe_expert_weights* w, const int32_t* offsets, int n_groups,
                           int max_rows, void* y_perm, void* ws, hipStream_t st);

moe_status launch_combine(const void* y_perm, moe_dtype y_dt, const int32_t* slot_to_row,
                          const float* topk_w, int T, int k, int H, const int32_t* offsets,
                          int shared_group, void* out, moe_dtype out_dt, hipStream_t st);

moe_status launch_gather_rows(const void* src, void* dst, const int32_t* index, int n_src_rows,
                              int n_rows, size_t row_bytes, hipStream_t st);

moe_status balanced_partition(const int64_t* counts, int E, int G, int32_t* new_to_old,
                              int32_t* old_to_new, int64_t* group_loads);
moe_status affinity_partition(const int64_t* counts, const int64_t* aff, int E, int G,
                              int tol_permille, int32_t* new_to_old, int32_t* old_to_new,
                              int64_t* group_loads, int64_t* intra_affinity);

moe_status launch_count_accumulate(const int32_t* counts, int n, int64_t* acc, hipStream_t st);
moe_status launch_coactivation(const int32_t* ids, int T, int k, int E, int64_t* hist,
                               hipStream_t st);

}  // namespace moe
