// Measurements for online rebalancing, accumulated on the device across
// steps ([Moreh-EP] Inter-GPU load balancing: activation frequencies
// re-measured periodically; [SGLang-H20] Expert Affinity EPLB: top-k
// co-activation tracked in an affinity matrix).
//
// Both kernels only add integers, so the result does not depend on the order
// in which the additions land.
#include "moe_internal.h"

namespace moe {
namespace {

__global__ void count_accumulate_kernel(const int32_t* __restrict__ counts, int n,
                                        int64_t* __restrict__ acc) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        acc[i] += counts[i];
}

// Row-owned histogram: workgroup (a, s) owns row a of the matrix for the
// s-th slice of the tokens. For one token with occ(x) valid picks of expert
// x, the pair rule gives row a occ(a) on the diagonal and occ(a) * occ(b) at
// every b != a; so a thread that finds a among its token's picks adds occ(a)
// at each other valid pick b (LDS atomics) and occ(a) to a register for the
// diagonal. Popular experts make many lanes add to one entry at once, which
// LDS atomics serialise: the row is kept in kCopies copies, lane l adding to
// copy l % kCopies. The copies are summed at the end and added to the matrix:
// with plain stores when one workgroup owns the whole row, else with global
// 64-bit atomics (the additions commute, so the result is the same).
constexpr int kRowThreads = 1024;
constexpr int kRowUnroll = 4;     // tokens per thread with their loads in flight together
constexpr int kCopies = 16;
constexpr int kSliceTokens = kRowThreads * kRowUnroll;
constexpr int kMaxCoactE = 1024;

__device__ inline unsigned add_token_picks(unsigned* row, const int* p, int k, int a, int E) {
    unsigned occ = 0;
    for (int j = 0; j < k; ++j) occ += p[j] == a;
    if (occ == 0) return 0;
    for (int j = 0; j < k; ++j) {
        const int b = p[j];
        if (b < 0 || b >= E || b == a) continue;
        atomicAdd(&row[(size_t)b * kCopies], occ);
    }
    return occ;
}

// kVec8: k == 8 with a 16-byte aligned id array (two 16-byte loads a token)
template <bool kVec8>
__global__ __launch_bounds__(kRowThreads) void coactivation_row_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int n_slices,
    int64_t* __restrict__ hist) {
    __shared__ unsigned rows[kMaxCoactE * kCopies];  // [E][kCopies], 64 KiB
    __shared__ unsigned long long diag_sum;
    const int a = blockIdx.x / n_slices, slice = blockIdx.x % n_slices;
    const int per = (T + n_slices - 1) / n_slices;
    const int t_begin = slice * per, t_end = min(T, t_begin + per);
    for (int c = threadIdx.x; c < E * kCopies; c += blockDim.x) rows[c] = 0;
    if (threadIdx.x == 0) diag_sum = 0;
    __syncthreads();
    unsigned* row = rows + (threadIdx.x % kCopies);
    unsigned long long diag = 0;
    if constexpr (kVec8) {
        const int4* q = reinterpret_cast<const int4*>(ids);
        for (int t0 = t_begin + threadIdx.x; t0 < t_end; t0 += kSliceTokens) {
            int4 u[kRowUnroll][2];
            // unconditional loads (a token past the end re-reads the last one
            // and is skipped), so all of them are in flight at once
#pragma unroll
            for (int r = 0; r < kRowUnroll; ++r) {
                const size_t t = (size_t)min(t0 + r * kRowThreads, t_end - 1);
                u[r][0] = q[t * 2];
                u[r][1] = q[t * 2 + 1];
            }
#pragma unroll
            for (int r = 0; r < kRowUnroll; ++r) {
                if (t0 + r * kRowThreads >= t_end) break;
                const int p[8] = {u[r][0].x, u[r][0].y, u[r][0].z, u[r][0].w,
                                  u[r][1].x, u[r][1].y, u[r][1].z, u[r][1].w};
                diag += add_token_picks(row, p, 8, a, E);
            }
        }
    } else {
        for (int t = t_begin + threadIdx.x; t < t_end; t += blockDim.x)
            diag += add_token_picks(row, ids + (size_t)t * k, k, a, E);
    }
    if (diag) atomicAdd(&diag_sum, diag);
    __syncthreads();
    int64_t* h = hist + (size_t)a * E;
    for (int c = threadIdx.x; c < E; c += blockDim.x) {
        unsigned long long v = 0;
#pragma unroll
        for (int i = 0; i < kCopies; ++i) v += rows[c * kCopies + i];
        if (c == a) v = diag_sum;
        if (n_slices == 1)
            h[c] += (int64_t)v;
        else if (v)
            atomicAdd(reinterpret_cast<unsigned long long*>(&h[c]), v);
    }
}

}  // namespace

moe_status launch_count_accumulate(const int32_t* counts, int n, int64_t* acc, hipStream_t st) {
    const int blocks = std::min((n + 255) / 256, 1024);
    hipLaunchKernelGGL(count_accumulate_kernel, dim3(blocks), dim3(256), 0, st, counts, n, acc);
    return check_launch("count_accumulate_kernel");
}

moe_status launch_coactivation(const int32_t* ids, int T, int k, int E, int64_t* hist,
                               hipStream_t st) {
    // one workgroup per (row, token slice); a slice is one pass of the
    // unrolled loop up to 64 slices. The 32-bit LDS counters hold a slice's
    // sums: at most 2^24 / 64 tokens a slice, 1/16 of them per copy, times
    // at most (k/2)^2 <= 2^14 per token, stays below 2^32.
    const int n_slices = std::min((T + kSliceTokens - 1) / kSliceTokens, 64);
    const dim3 grid((unsigned)(E * n_slices));
    const bool vec8 = k == 8 && (reinterpret_cast<uintptr_t>(ids) & 15) == 0;
    if (vec8)
        hipLaunchKernelGGL(coactivation_row_kernel<true>, grid, dim3(kRowThreads), 0, st, ids, T,
                           k, E, n_slices, hist);
    else
        hipLaunchKernelGGL(coactivation_row_kernel<false>, grid, dim3(kRowThreads), 0, st, ids,
                           T, k, E, n_slices, hist);
    return check_launch("coactivation_row_kernel");
}

}  // namespace moe
