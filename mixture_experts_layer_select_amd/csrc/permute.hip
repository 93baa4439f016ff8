// Token -> expert grouping ([Moreh-EP] Library optimization: the fused MoE
// kernel consumes tokens grouped by expert; Inter-GPU load balancing: the
// per-expert activation counts). Deterministic, with atomics used only to
// count or to set bits, never to hand out positions.
//
//   hist     one workgroup per chunk of 1024 slots: LDS histogram of the
//            local experts -> chunk_counts[chunk][e]
//   scan     one workgroup: per expert an exclusive scan over chunks, then an
//            exclusive scan over experts (+ the shared group) -> counts,
//            offsets, and chunk_base[chunk][e] = first row of that chunk's
//            slots of expert e
//   scatter  one workgroup per chunk: an LDS bitmap of the chunk's slots per
//            expert; the rank of a slot among its expert's slots is a popcount
//            of the bits below it, so rows come out in (expert, slot) order
//   fill     rows past the routed ones: shared-expert rows, then -1
//   gather   x_perm[row] = x[token(row)] (bit copy or 1x128 e4m3 quantisation)
#include "permute_dev.h"

namespace moe {
namespace {

constexpr int kChunk = 1024;   // slots per chunk

__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t* __restrict__ ids, long S,
                                                        int base, int E_local,
                                                        int32_t* __restrict__ chunk_counts) {
    __shared__ int cnt[kMaxLocal];
    for (int e = threadIdx.x; e < E_local; e += 256) cnt[e] = 0;
    __syncthreads();
    const long s0 = (long)blockIdx.x * kChunk;
    for (int i = threadIdx.x; i < kChunk; i += 256) {
        long s = s0 + i;
        if (s < S) {
            int e = ids[s] - base;
            if (e >= 0 && e < E_local) atomicAdd(&cnt[e], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E_local; e += 256)
        chunk_counts[(size_t)blockIdx.x * E_local + e] = cnt[e];
}

// single workgroup of 256 threads
__global__ __launch_bounds__(256) void perm_scan_kernel(int32_t* __restrict__ chunk_counts,
                                                        int n_chunks, int E_local, int n_shared,
                                                        int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets) {
    __shared__ int tot[kMaxLocal + 1];
    __shared__ int excl[kMaxLocal + 2];
    const int e = threadIdx.x;
    // each thread walks its expert's column of chunk counts in batches of 16
    // independent loads (one memory latency per batch, not per chunk)
    constexpr int kB = 16;
    if (e < E_local) {
        int run = 0;
        for (int c0 = 0; c0 < n_chunks; c0 += kB) {
            int v[kB];
#pragma unroll
            for (int i = 0; i < kB; ++i)
                v[i] = c0 + i < n_chunks ? chunk_counts[(size_t)(c0 + i) * E_local + e] : 0;
#pragma unroll
            for (int i = 0; i < kB; ++i)
                if (c0 + i < n_chunks) {
                    chunk_counts[(size_t)(c0 + i) * E_local + e] = run;
                    run += v[i];
                }
        }
        tot[e] = run;
    }
    if (e == 0) tot[E_local] = n_shared;
    __syncthreads();
    if (e == 0) {  // E_local + 1 <= 257 values: a serial scan is cheapest here
        int run = 0;
        for (int g = 0; g <= E_local; ++g) {
            excl[g] = run;
            run += tot[g];
        }
        excl[E_local + 1] = run;
    }
    __syncthreads();
    if (e < E_local) {
        counts[e] = tot[e];
        offsets[e] = excl[e];
        const int o = excl[e];
        for (int c0 = 0; c0 < n_chunks; c0 += kB) {
            int v[kB];
#pragma unroll
            for (int i = 0; i < kB; ++i)
                v[i] = c0 + i < n_chunks ? chunk_counts[(size_t)(c0 + i) * E_local + e] : 0;
#pragma unroll
            for (int i = 0; i < kB; ++i)
                if (c0 + i < n_chunks) chunk_counts[(size_t)(c0 + i) * E_local + e] = v[i] + o;
        }
    }
    if (e == 0) {
        counts[E_local] = n_shared;
        offsets[E_local] = excl[E_local];
        offsets[E_local + 1] = excl[E_local + 1];
    }
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ ids, long S,
                                                           int base, int E_local,
                                                           const int32_t* __restrict__ chunk_base,
                                                           int32_t* __restrict__ row_to_slot,
                                                           int32_t* __restrict__ slot_to_row) {
    constexpr int kWords = kChunk / 32;
    __shared__ uint32_t bits[kMaxLocal][kWords];
    __shared__ int pre[kMaxLocal][kWords];
    for (int i = threadIdx.x; i < E_local * kWords; i += 256) bits[i / kWords][i % kWords] = 0;
    __syncthreads();
    const long s0 = (long)blockIdx.x * kChunk;
    int my_e[kChunk / 256];
#pragma unroll
    for (int q = 0; q < kChunk / 256; ++q) {
        const int p = threadIdx.x + 256 * q;
        const long s = s0 + p;
        int e = -1;
        if (s < S) {
            e = ids[s] - base;
            if (e < 0 || e >= E_local) e = -1;
        }
        my_e[q] = e;
        if (e >= 0) atomicOr(&bits[e][p >> 5], 1u << (p & 31));
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E_local; e += 256) {
        int run = 0;
        for (int w = 0; w < kWords; ++w) {
            pre[e][w] = run;
            run += __popc(bits[e][w]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kChunk / 256; ++q) {
        const int p = threadIdx.x + 256 * q;
        const long s = s0 + p;
        if (s >= S) continue;
        const int e = my_e[q];
        if (e < 0) {
            slot_to_row[s] = -1;
            continue;
        }
        const int w = p >> 5;
        const int rank = pre[e][w] + __popc(bits[e][w] & ((1u << (p & 31)) - 1u));
        const int row = chunk_base[(size_t)blockIdx.x * E_local + e] + rank;
        row_to_slot[row] = (int32_t)s;
        slot_to_row[s] = row;
    }
}

// All of hist + scan + scatter + fill in one workgroup of 1024 threads when
// the slots fit one LDS bitmap: per local expert a bitmap over all slots
// (nw = ceil(S/32) words), 16-bit popcount prefixes per word, an exclusive
// scan over experts. Used when S <= kSmallSlots and the bitmap fits kSmallLds.
constexpr int kSmallSlots = 8192;
constexpr size_t kSmallLds = 96 * 1024;

__global__ __launch_bounds__(1024) void perm_small_kernel(const int32_t* __restrict__ ids, int S,
                                                          int T, int base, int E_local,
                                                          int n_shared, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ row_to_slot,
                                                          int32_t* __restrict__ slot_to_row) {
    const int nw = (S + 31) / 32;
    const int kWords = nw;  // row stride of both tables
    extern __shared__ uint32_t smem[];
    uint32_t* bits = smem;                                              // [E_local][nw]
    uint16_t* pre = reinterpret_cast<uint16_t*>(smem + E_local * nw);  // [E_local][nw]
    __shared__ int excl[kMaxLocal + 2];
    for (int i = threadIdx.x; i < E_local * kWords; i += blockDim.x) bits[i] = 0;
    __syncthreads();
    for (int s = threadIdx.x; s < S; s += blockDim.x) {
        const int e = ids[s] - base;
        if (e >= 0 && e < E_local) atomicOr(&bits[e * kWords + (s >> 5)], 1u << (s & 31));
    }
    __syncthreads();
    if (threadIdx.x < E_local) {
        const int e = threadIdx.x;
        int run = 0;
        for (int w = 0; w < nw; ++w) {
            pre[e * kWords + w] = (uint16_t)run;
            run += __popc(bits[e * kWords + w]);
        }
        excl[e] = run;  // count for now
    }
    __syncthreads();
    {
        // exclusive scan of the counts over experts: an inclusive scan within
        // each wave (shuffles), then over the wave totals
        __shared__ int wave_tot[1024 / 64];
        const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
        const int c = threadIdx.x < E_local ? excl[threadIdx.x] : 0;
        int v = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int n = __shfl_up(v, d);
            if (lane >= d) v += n;
        }
        if (lane == 63) wave_tot[wv] = v;
        __syncthreads();
        int before = 0;
        for (int u = 0; u < wv; ++u) before += wave_tot[u];
        const int incl = before + v;
        if (threadIdx.x < E_local) {
            counts[threadIdx.x] = c;
            offsets[threadIdx.x] = incl - c;
            excl[threadIdx.x] = incl - c;
        }
        if (threadIdx.x == E_local - 1) {
            counts[E_local] = n_shared;
            offsets[E_local] = incl;
            offsets[E_local + 1] = incl + n_shared;
            excl[E_local] = incl;
        }
    }
    __syncthreads();
    const int R = excl[E_local];
    for (int s = threadIdx.x; s < S; s += blockDim.x) {
        const int e = ids[s] - base;
        if (e >= 0 && e < E_local) {
            const int w = s >> 5;
            const int row = excl[e] + pre[e * kWords + w] +
                            __popc(bits[e * kWords + w] & ((1u << (s & 31)) - 1u));
            row_to_slot[row] = s;
            slot_to_row[s] = row;
        } else {
            slot_to_row[s] = -1;
        }
    }
    const int cap = S + T;
    for (int r = R + threadIdx.x; r < cap; r += blockDim.x)
        row_to_slot[r] = r < R + n_shared ? S + (r - R) : -1;
}

__global__ void perm_fill_kernel(const int32_t* __restrict__ offsets, int E_local, long S,
                                 long cap, int32_t* __restrict__ row_to_slot) {
    const long R = offsets[E_local];
    const long used = offsets[E_local + 1];
    for (long r = R + (long)blockIdx.x * blockDim.x + threadIdx.x; r < cap;
         r += (long)gridDim.x * blockDim.x)
        row_to_slot[r] = r < used ? (int32_t)(S + (r - R)) : -1;
}

__device__ __forceinline__ long token_of(int32_t slot, long S, int k) {
    return slot < S ? slot / k : slot - S;
}

// bit copy of rows; elem_bytes in {2, 4}
__global__ __launch_bounds__(256) void perm_gather_copy_kernel(
    const uint8_t* __restrict__ x, const int32_t* __restrict__ row_to_slot,
    const int32_t* __restrict__ offsets, int E_local, long S, int k, long row_bytes,
    uint8_t* __restrict__ x_perm) {
    const long used = offsets[E_local + 1];
    for (long r = blockIdx.x; r < used; r += gridDim.x) {
        const long t = token_of(row_to_slot[r], S, k);
        const uint8_t* src = x + t * row_bytes;
        uint8_t* dst = x_perm + r * row_bytes;
        if ((row_bytes & 15) == 0) {
            for (long i = threadIdx.x; i < row_bytes / 16; i += blockDim.x)
                reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(src)[i];
        } else {
            for (long i = threadIdx.x; i < row_bytes / 2; i += blockDim.x)
                reinterpret_cast<uint16_t*>(dst)[i] = reinterpret_cast<const uint16_t*>(src)[i];
        }
    }
}

// one pass: every used row quantises its token's row (the next row's token
// index is loaded before this row's work)
__global__ __launch_bounds__(256) void perm_gather_fp8_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ row_to_slot,
    const int32_t* __restrict__ offsets, int E_local, long S, int k, int H, long cap,
    uint8_t* __restrict__ x_perm, float* __restrict__ x_scale) {
    const long used = offsets[E_local + 1];
    long r = blockIdx.x;
    int32_t slot = r < used ? row_to_slot[r] : 0;
    for (; r < used; r += gridDim.x) {
        const long t = token_of(slot, S, k);
        if (r + gridDim.x < used) slot = row_to_slot[r + gridDim.x];
        quant_row_fp8(x + t * H, H, cap, r, x_perm, x_scale, threadIdx.x);
    }
}

// Two passes (with a shared group): each token is quantised once into the
// shared group's rows [R, R + T), which hold the tokens in order anyway, and
// the routed rows copy their token's codes and scales from there. Without a
// shared group the staging rows would be [T*k, T*k + T), which no routed row
// reaches (R <= T*k).
__device__ __forceinline__ long stage_row0(const int32_t* __restrict__ offsets, int E_local, long S) {
    const long R = offsets[E_local];
    return offsets[E_local + 1] > R ? R : S;
}

// pass 1: every token quantised once, into its staging row
__global__ __launch_bounds__(256) void perm_quant_tokens_fp8_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ offsets, int E_local, long S, int T,
    int H, long cap, uint8_t* __restrict__ x_perm, float* __restrict__ x_scale) {
    const long q0 = stage_row0(offsets, E_local, S);
    for (long t = blockIdx.x; t < T; t += gridDim.x)
        quant_row_fp8(x + t * H, H, cap, q0 + t, x_perm, x_scale, threadIdx.x);
}

// pass 2: routed row r takes the codes and scales of its token's staging row.
// A workgroup copies 16 consecutive rows: their tokens go to LDS once, the
// codes move as 16-byte chunks over all (row, chunk) pairs, eight loads in
// flight per thread, and each scale block is written for 16 consecutive rows
// at once.
constexpr int kCopyRows = 16;
__global__ __launch_bounds__(256) void perm_copy_fp8_kernel(
    const int32_t* __restrict__ row_to_slot, const int32_t* __restrict__ offsets, int E_local,
    long S, int k, int H, long cap, uint8_t* __restrict__ x_perm, float* __restrict__ x_scale) {
    __shared__ long tok[kCopyRows];
    const long R = offsets[E_local];
    const long q0 = stage_row0(offsets, E_local, S);
    const int nb = H / 128;
    const int nc = H / 16;
    for (long r0 = (long)blockIdx.x * kCopyRows; r0 < R; r0 += (long)gridDim.x * kCopyRows) {
        const int n = (int)min((long)kCopyRows, R - r0);
        __syncthreads();
        if (threadIdx.x < n) tok[threadIdx.x] = token_of(row_to_slot[r0 + threadIdx.x], S, k);
        __syncthreads();
        {
            const int j = threadIdx.x & (kCopyRows - 1);
            if (j < n) {
                const long src = q0 + tok[j];
                for (int b = threadIdx.x / kCopyRows; b < nb; b += 256 / kCopyRows)
                    x_scale[b * cap + r0 + j] = x_scale[b * cap + src];
            }
        }
        const int total = n * nc;
        for (int i0 = threadIdx.x; i0 < total; i0 += 8 * 256) {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + 256 * u;
                if (i < total) {
                    const int rr = i / nc, c = i - rr * nc;
                    v[u] = *reinterpret_cast<const u32x4*>(x_perm + (q0 + tok[rr]) * H + 16 * c);
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + 256 * u;
                if (i < total) {
                    const int rr = i / nc, c = i - rr * nc;
                    *reinterpret_cast<u32x4*>(x_perm + (r0 + rr) * H + 16 * c) = v[u];
                }
            }
        }
    }
}

// every token quantised once into row t of a [T][H] token buffer, scales
// K-major [H/128][T]
__global__ __launch_bounds__(256) void quant_tokens_fp8_kernel(const uint16_t* __restrict__ x, int T,
                                                               int H, uint8_t* __restrict__ codes,
                                                               float* __restrict__ scales) {
    for (long t = blockIdx.x; t < T; t += gridDim.x) quant_row_fp8(x + t * H, H, T, t, codes, scales, threadIdx.x);
}

}  // namespace

moe_status launch_quantize_tokens(const void* x, int T, int H, void* codes, float* scales,
                                  hipStream_t st) {
    if (T == 0) return MOE_OK;
    const int blocks = (int)std::min<long>(T, (long)device_info().cu_count * 8);
    hipLaunchKernelGGL(quant_tokens_fp8_kernel, dim3(blocks), dim3(256), 0, st, (const uint16_t*)x, T,
                       H, (uint8_t*)codes, scales);
    return check_launch("quant_tokens_fp8_kernel");
}

static moe_status launch_gather(const void* x, moe_dtype x_dt, int H, moe_dtype perm_dt,
                                const int32_t* row_to_slot, const int32_t* offsets, int E_local,
                                long S, int k, long cap, int include_shared, void* x_perm,
                                float* x_perm_scale, hipStream_t st);

size_t permute_workspace_bytes(int T, int k, int E_local) {
    long S = (long)T * k;
    long n_chunks = (S + kChunk - 1) / kChunk;
    return align_up((size_t)(n_chunks > 0 ? n_chunks : 1) * E_local * sizeof(int32_t), 256);
}

moe_status launch_permute(const int32_t* ids, int T, int k, int base, int E_local, int include_shared,
                          const void* x, moe_dtype x_dt, int H, moe_dtype perm_dt, int32_t* counts,
                          int32_t* offsets, int32_t* row_to_slot, int32_t* slot_to_row,
                          void* x_perm, float* x_perm_scale, void* ws, hipStream_t st) {
    const long S = (long)T * k;
    const long cap = S + T;
    const int n_chunks = (int)((S + kChunk - 1) / kChunk);
    int32_t* chunk_counts = (int32_t*)ws;
    moe_status s;
    const size_t small_lds = (size_t)E_local * ((S + 31) / 32) * (4 + 2);
    if (S <= kSmallSlots && small_lds <= kSmallLds) {
        const size_t smem = small_lds;
        static bool lds_opt_in = [] {  // dynamic LDS above 64 KB needs the attribute
            return hipFuncSetAttribute((const void*)perm_small_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)kSmallLds) == hipSuccess;
        }();
        if (!lds_opt_in) return set_error(MOE_ERR_HIP, "perm_small_kernel: LDS attribute refused");
        hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(1024), smem, st, ids, (int)S, T, base,
                           E_local, include_shared ? T : 0, counts, offsets, row_to_slot,
                           slot_to_row);
        if ((s = check_launch("perm_small_kernel"))) return s;
        return launch_gather(x, x_dt, H, perm_dt, row_to_slot, offsets, E_local, S, k, cap,
                             include_shared, x_perm, x_perm_scale, st);
    }
    hipLaunchKernelGGL(perm_hist_kernel, dim3(n_chunks), dim3(256), 0, st, ids, S, base, E_local,
                       chunk_counts);
    if ((s = check_launch("perm_hist_kernel"))) return s;
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(256), 0, st, chunk_counts, n_chunks, E_local,
                       include_shared ? T : 0, counts, offsets);
    if ((s = check_launch("perm_scan_kernel"))) return s;
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(n_chunks), dim3(256), 0, st, ids, S, base, E_local,
                       chunk_counts, row_to_slot, slot_to_row);
    if ((s = check_launch("perm_scatter_kernel"))) return s;
    const int fill_blocks = (int)std::min<long>((cap + 255) / 256, 1024);
    hipLaunchKernelGGL(perm_fill_kernel, dim3(fill_blocks), dim3(256), 0, st, offsets, E_local, S, cap,
                       row_to_slot);
    if ((s = check_launch("perm_fill_kernel"))) return s;
    return launch_gather(x, x_dt, H, perm_dt, row_to_slot, offsets, E_local, S, k, cap,
                         include_shared, x_perm, x_perm_scale, st);
}

static moe_status launch_gather(const void* x, moe_dtype x_dt, int H, moe_dtype perm_dt,
                                const int32_t* row_to_slot, const int32_t* offsets, int E_local,
                                long S, int k, long cap, int include_shared, void* x_perm,
                                float* x_perm_scale, hipStream_t st) {
    if (!x_perm) return MOE_OK;
    const int cu = device_info().cu_count;
    const int gather_blocks = (int)std::min<long>(cap, (long)cu * 8);
    if (perm_dt == MOE_FP8_E4M3 && !include_shared) {
        hipLaunchKernelGGL(perm_gather_fp8_kernel, dim3(gather_blocks), dim3(256), 0, st,
                           (const uint16_t*)x, row_to_slot, offsets, E_local, S, k, H, cap,
                           (uint8_t*)x_perm, x_perm_scale);
        return check_launch("perm_gather_fp8_kernel");
    }
    if (perm_dt == MOE_FP8_E4M3) {
        // with the shared group: each token is quantised once (into its shared
        // row), then routed rows copy their token's codes and scales
        const int T = (int)(cap - S);
        hipLaunchKernelGGL(perm_quant_tokens_fp8_kernel, dim3((int)std::min<long>(T, (long)cu * 8)),
                           dim3(256), 0, st, (const uint16_t*)x, offsets, E_local, S, T, H, cap,
                           (uint8_t*)x_perm, x_perm_scale);
        moe_status s = check_launch("perm_quant_tokens_fp8_kernel");
        if (s != MOE_OK) return s;
        const int copy_blocks = (int)std::max<long>(1, std::min<long>((S + kCopyRows - 1) / kCopyRows, (long)cu * 8));
        hipLaunchKernelGGL(perm_copy_fp8_kernel, dim3(copy_blocks), dim3(256), 0, st, row_to_slot, offsets,
                           E_local, S, k, H, cap, (uint8_t*)x_perm, x_perm_scale);
        return check_launch("perm_copy_fp8_kernel");
    }
    const long eb = x_dt == MOE_F32 ? 4 : 2;
    hipLaunchKernelGGL(perm_gather_copy_kernel, dim3(gather_blocks), dim3(256), 0, st,
                       (const uint8_t*)x, row_to_slot, offsets, E_local, S, k, eb * H,
                       (uint8_t*)x_perm);
    return check_launch("perm_gather_copy_kernel");
}

}  // namespace moe
