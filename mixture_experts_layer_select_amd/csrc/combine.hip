// Routing-weighted combine back to token order ([Moreh-EP] Overview:
// dispatch/combine -- this is the GPU-local half) and the row gather used to
// apply a new expert order ([Moreh-EP] Inter-GPU load balancing).
//
// Combine is a memory-bound gather. The unit of work is (token, 1024-column
// chunk) so a small batch still spreads over every CU (T = 256, H = 7168:
// 1792 units); a workgroup of 128 threads takes units grid-stride, 8 bf16
// (16 bytes) per thread per row read, fp32 accumulation in slot order
// j = 0..k-1 followed by the shared-expert row, then one rounding.
#include "moe_internal.h"

namespace moe {
namespace {

template <typename TY, typename TO>
struct CombineIO;

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

constexpr int kMaxK = 256;
constexpr int kCombineThreads = 128;
constexpr int kChunkH = kCombineThreads * 8;  // columns per unit

template <typename TY, typename TO>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const TY* __restrict__ y, const int32_t* __restrict__ slot_to_row,
    const float* __restrict__ topk_w, int T, int k, int H, const int32_t* __restrict__ offsets,
    int shared_group, TO* __restrict__ out) {
    __shared__ int rows[kMaxK + 1];
    __shared__ float wts[kMaxK];
    const bool vec = (H & 7) == 0;
    const int nch = (H + kChunkH - 1) / kChunkH;
    const long n_units = (long)T * nch;
    for (long u = blockIdx.x; u < n_units; u += gridDim.x) {
        const int t = (int)(u / nch);
        const int h_lo = (int)(u % nch) * kChunkH;
        const int h_hi = min(H, h_lo + kChunkH);
        __syncthreads();
        for (int j = threadIdx.x; j < k; j += blockDim.x) {
            rows[j] = slot_to_row[(size_t)t * k + j];
            wts[j] = topk_w[(size_t)t * k + j];
        }
        if (threadIdx.x == 0) rows[k] = shared_group >= 0 ? offsets[shared_group] + t : -1;
        __syncthreads();
        if (vec) {
            for (int h = h_lo + threadIdx.x * 8; h < h_hi; h += blockDim.x * 8) {
                float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                // picks in slot order, 8 at a time: all 8 row loads are issued
                // before the first multiply-add so their latencies overlap
                for (int j0 = 0; j0 < k; j0 += 8) {
                    float v[8][8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const int j = j0 + q;
                        const int r = j < k ? rows[j] : -1;
                        if (r >= 0) load8(y + (size_t)r * H + h, v[q]);
                    }
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const int j = j0 + q;
                        if (j < k && rows[j] >= 0) {
                            const float wj = wts[j];
#pragma unroll
                            for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj, v[q][i], acc[i]);
                        }
                    }
                }
                if (rows[k] >= 0) {
                    float v[8];
                    load8(y + (size_t)rows[k] * H + h, v);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] += v[i];
                }
                store8(out + (size_t)t * H + h, acc);
            }
        } else {
            for (int h = h_lo + threadIdx.x; h < h_hi; h += blockDim.x) {
                float acc = 0.f;
                for (int j = 0; j < k; ++j) {
                    const int r = rows[j];
                    if (r >= 0) acc = __builtin_fmaf(wts[j], load1(y + (size_t)r * H + h), acc);
                }
                if (rows[k] >= 0) acc += load1(y + (size_t)rows[k] * H + h);
                store1(out + (size_t)t * H + h, acc);
            }
        }
    }
}

// bf16 rows and output, k <= kSmallK, 8-column vectors: the unit's token is the same for the
// whole workgroup, so its pick rows and weights are uniform loads kept in
// scalar registers (no LDS staging, no barriers), and the next unit's are
// loaded before the current unit's rows are summed, so the index latency of
// one unit hides under the row loads of the previous one. Same summation
// order as combine_kernel: slots 0..k-1, then the shared row.
constexpr int kSmallK = 8;
__global__ __launch_bounds__(kCombineThreads) void combine_small_k_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ slot_to_row,
    const float* __restrict__ topk_w, int T, int k, int H, const int32_t* __restrict__ offsets,
    int shared_group, uint16_t* __restrict__ out) {
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
    long u = blockIdx.x;
    if (u < n_units) fetch(u, rows, wts);
    for (; u < n_units; u += gridDim.x) {
        const int t = (int)(u / nch);
        const int h = (int)(u % nch) * kChunkH + threadIdx.x * 8;
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
        if (u + gridDim.x < n_units) fetch(u + gridDim.x, rows, wts);
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

__global__ void gather_rows_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                   const int32_t* __restrict__ index, int n_src_rows, int n_rows,
                                   long row_words) {
    for (long r = blockIdx.x; r < n_rows; r += gridDim.x) {
        const int s = index[r];
        if (s < 0 || s >= n_src_rows) continue;  // out-of-range index: row left untouched
        const uint32_t* a = src + (size_t)s * row_words;
        uint32_t* b = dst + (size_t)r * row_words;
        if ((row_words & 3) == 0) {
            for (long i = threadIdx.x; i < row_words / 4; i += blockDim.x)
                reinterpret_cast<u32x4*>(b)[i] = reinterpret_cast<const u32x4*>(a)[i];
        } else {
            for (long i = threadIdx.x; i < row_words; i += blockDim.x) b[i] = a[i];
        }
    }
}

}  // namespace

moe_status launch_combine(const void* y_perm, moe_dtype y_dt, const int32_t* slot_to_row,
                          const float* topk_w, int T, int k, int H, const int32_t* offsets,
                          int shared_group, void* out, moe_dtype out_dt, hipStream_t st) {
    const long units = (long)T * ((H + kChunkH - 1) / kChunkH);
    const int blocks = (int)std::max(1L, std::min(units, (long)device_info().cu_count * 16));
    if (k <= kSmallK && (H & 7) == 0 && y_dt == MOE_BF16 && out_dt == MOE_BF16) {
        hipLaunchKernelGGL(combine_small_k_kernel, dim3(blocks), dim3(kCombineThreads), 0,
                           st, (const uint16_t*)y_perm, slot_to_row, topk_w, T, k, H, offsets,
                           shared_group, (uint16_t*)out);
        return check_launch("combine_small_k_kernel");
    }
    if (y_dt == MOE_BF16 && out_dt == MOE_BF16)
        hipLaunchKernelGGL((combine_kernel<uint16_t, uint16_t>), dim3(blocks), dim3(kCombineThreads), 0, st,
                           (const uint16_t*)y_perm, slot_to_row, topk_w, T, k, H, offsets,
                           shared_group, (uint16_t*)out);
    else if (y_dt == MOE_BF16)
        hipLaunchKernelGGL((combine_kernel<uint16_t, float>), dim3(blocks), dim3(kCombineThreads), 0, st,
                           (const uint16_t*)y_perm, slot_to_row, topk_w, T, k, H, offsets,
                           shared_group, (float*)out);
    else if (out_dt == MOE_BF16)
        hipLaunchKernelGGL((combine_kernel<float, uint16_t>), dim3(blocks), dim3(kCombineThreads), 0, st,
                           (const float*)y_perm, slot_to_row, topk_w, T, k, H, offsets,
                           shared_group, (uint16_t*)out);
    else
        hipLaunchKernelGGL((combine_kernel<float, float>), dim3(blocks), dim3(kCombineThreads), 0, st,
                           (const float*)y_perm, slot_to_row, topk_w, T, k, H, offsets,
                           shared_group, (float*)out);
    return check_launch("combine_kernel");
}

moe_status launch_gather_rows(const void* src, void* dst, const int32_t* index, int n_src_rows,
                              int n_rows, size_t row_bytes, hipStream_t st) {
    const int blocks = std::min(n_rows, device_info().cu_count * 8);
    hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks), dim3(256), 0, st, (const uint32_t*)src,
                       (uint32_t*)dst, index, n_src_rows, n_rows, (long)(row_bytes / 4));
    return check_launch("gather_rows_kernel");
}

}  // namespace moe
