// Routing-weighted combine back to token order ([Moreh-EP] Overview:
// dispatch/combine -- this is the GPU-local half) and the row gather used to
// apply a new expert order ([Moreh-EP] Inter-GPU load balancing).
//
// Combine is a memory-bound gather. The unit of work is (token, 1024-column
// chunk) so a small batch still spreads over every CU (T = 256, H = 7168:
// 1792 units); a workgroup of 128 threads takes units grid-stride, 8 bf16
// (16 bytes) per thread per row read, fp32 accumulation in slot order
// j = 0..k-1 followed by the shared-expert row, then one rounding.
#include "combine_dev.h"

namespace moe {
namespace {

template <typename TY, typename TO>
struct CombineIO;

constexpr int kMaxK = 256;

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

__global__ __launch_bounds__(kCombineThreads) void combine_small_k_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ slot_to_row,
    const float* __restrict__ topk_w, int T, int k, int H, const int32_t* __restrict__ offsets,
    int shared_group, uint16_t* __restrict__ out) {
    combine_small_k_units(y, slot_to_row, topk_w, T, k, H, offsets, shared_group, out, blockIdx.x,
                          gridDim.x, threadIdx.x);
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
