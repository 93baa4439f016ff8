// Device code of the routing-weighted combine for k <= 8 (bf16 rows, bf16
// output), shared by the combine kernel and the fused small-batch layer.
// Internal to libmoe.so.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
    u32x4 q = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_lo(q[i]);
        v[2 * i + 1] = bf16_hi(q[i]);
    }
}
__device__ __forceinline__ void load8(const float* p, float* v) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = a[i];
        v[4 + i] = b[i];
    }
}
__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
    *reinterpret_cast<u32x4*>(p) = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                         pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}
__device__ __forceinline__ void store8(float* p, const float* v) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ float load1(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ void store1(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16_bits(v); }
__device__ __forceinline__ void store1(float* p, float v) { *p = v; }

constexpr int kCombineThreads = 128;
constexpr int kChunkH = kCombineThreads * 8;  // columns per unit

// bf16 rows and output, k <= kSmallK, 8-column vectors: the unit's token is the same for the
// whole workgroup, so its pick rows and weights are uniform loads kept in
// scalar registers (no LDS staging, no barriers), and the next unit's are
// loaded before the current unit's rows are summed, so the index latency of
// one unit hides under the row loads of the previous one. Same summation
// order as combine_kernel: slots 0..k-1, then the shared row.
// The units u = bid, bid + nblk, ... of a block of kCombineThreads threads
// (tid = its thread index).
constexpr int kSmallK = 8;
__device__ __forceinline__ void combine_small_k_units(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ slot_to_row,
    const float* __restrict__ topk_w, int T, int k, int H, const int32_t* __restrict__ offsets,
    int shared_group, uint16_t* __restrict__ out, long bid, long nblk, int tid) {
    const int nch = (H + kChunkH - 1) / kChunkH;
    const long n_units = (long)T * nch;
    const int shared0 = shared_group >= 0 ? offsets[shared_group] : -1;
    auto fetch = [&](long u, int* rows, float* wts) {
        const int t = (int)(u / nch);
#pragma unroll
        for (int j = 0; j < kSmallK; ++j) {
            rows[j] = j < k ? slot_to_row[(size_t)t * k + j] : -1;
            wts[j] = j < k ? topk_w[(size_t)t * k + j] : 0.f;
        }
    };
    int rows[kSmallK];
    float wts[kSmallK];
    long u = bid;
    if (u < n_units) fetch(u, rows, wts);
    for (; u < n_units; u += nblk) {
        const int t = (int)(u / nch);
        const int h = (int)(u % nch) * kChunkH + tid * 8;
        // every row load is issued before the first sum; a non-local pick
        // (row -1) or an absent shared row issues none (a uniform branch
        // around the load only: the values are unpacked after all loads, so
        // they stay in flight together)
        u32x4 q[kSmallK], qs;
        if (h < H) {
#pragma unroll
            for (int j = 0; j < kSmallK; ++j)
                if (rows[j] >= 0)
                    q[j] = buffer_load16(buffer_rsrc(y + (size_t)rows[j] * H, (uint32_t)H * 2u),
                                         (uint32_t)h * 2u, 0);
            if (shared0 >= 0)
                qs = buffer_load16(buffer_rsrc(y + (size_t)(shared0 + t) * H, (uint32_t)H * 2u),
                                   (uint32_t)h * 2u, 0);
        }
        float wc[kSmallK];
        int rc[kSmallK];
#pragma unroll
        for (int j = 0; j < kSmallK; ++j) {
            wc[j] = wts[j];
            rc[j] = rows[j];
        }
        if (u + nblk < n_units) fetch(u + nblk, rows, wts);
        if (h < H) {
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kSmallK; ++j)
                if (rc[j] >= 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[2 * i] = __builtin_fmaf(wc[j], bf16_lo(q[j][i]), acc[2 * i]);
                        acc[2 * i + 1] = __builtin_fmaf(wc[j], bf16_hi(q[j][i]), acc[2 * i + 1]);
                    }
                }
            if (shared0 >= 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] += bf16_lo(qs[i]);
                    acc[2 * i + 1] += bf16_hi(qs[i]);
                }
            }
            store8(out + (size_t)t * H + h, acc);
        }
    }
}

}  // namespace
}  // namespace moe
