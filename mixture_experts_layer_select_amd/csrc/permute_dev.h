// Device code of the token permutation shared by the permute kernels and the
// fused small-batch layer: the 1x128 e4m3 quantisation of a bf16 row, and the
// whole permutation in one workgroup. Internal to libmoe.so.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kMaxLocal = 256;  // local experts handled per launch

// bf16 rows -> e4m3 codes + one fp32 scale per 128 elements; H % 128 == 0.
// 16 lanes own one 128-element block, 8 elements each; a pass of four rounds
// issues all of its row loads before the first block is quantised. Scales are
// K-major: block b of row r at b * cap + r.
// tid: the thread's index in a block of 256 threads.
__device__ __forceinline__ void quant_row_fp8(const uint16_t* __restrict__ src, int H, long cap,
                                              long r, uint8_t* __restrict__ x_perm,
                                              float* __restrict__ x_scale, int tid) {
    const int nb = H / 128;
    const int sub = tid & 15;
    for (int b0 = tid >> 4; b0 < nb; b0 += 64) {
        u32x4 q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = b0 + 16 * i;
            if (b < nb) q[i] = *reinterpret_cast<const u32x4*>(src + b * 128 + sub * 8);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = b0 + 16 * i;
            if (b >= nb) break;
            const int h0 = b * 128 + sub * 8;
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = bf16_lo(q[i][e]);
                v[2 * e + 1] = bf16_hi(q[i][e]);
            }
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[e]));
#pragma unroll
            for (int m = 8; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m));
            const float sc = block_scale(a);
            float qv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[e] = clamp_e4m3(v[e] / sc);
            const uint32_t lo = pack_e4m3x4(qv[0], qv[1], qv[2], qv[3]);
            const uint32_t hi = pack_e4m3x4(qv[4], qv[5], qv[6], qv[7]);
            *reinterpret_cast<uint2*>(x_perm + r * H + h0) = make_uint2(lo, hi);
            if (sub == 0) x_scale[b * cap + r] = sc;
        }
    }
}

// ---------------------------------------------------------------- one-workgroup permute
// The maps of the permute kernels for one workgroup of 512 threads and LDS of
// about 10 KB: per local expert a count (LDS atomics), an exclusive scan over
// the experts, then the slots in chunks of 512, in slot order: a slot's rank
// among the earlier slots of its expert is the count of earlier chunks, of
// the lower waves of its chunk, and of the lower lanes of its wave (found by
// matching lanes on the expert id). Same outputs as the permute kernels:
// counts[E_local+1], offsets[E_local+2], row_to_slot (shared rows S + t,
// unused rows -1), slot_to_row (-1 = not local).
constexpr int kPermThreads = 512;
struct PermLds {
    int excl[kMaxLocal + 2];  // first row of each expert; excl[E_local] = R
    int run[kMaxLocal];       // counts, then the slots of each expert in earlier chunks
    int wc[kPermThreads / 64][kMaxLocal];  // per-wave counts of the current chunk
    int tot[kPermThreads / 64];
};

__device__ __forceinline__ void perm_block(const int32_t* __restrict__ ids, int S, int T, int base,
                                           int E_local, int n_shared, int32_t* __restrict__ counts,
                                           int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ row_to_slot,
                                           int32_t* __restrict__ slot_to_row, PermLds& L) {
    constexpr int kWaves = kPermThreads / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < E_local; e += kPermThreads) L.run[e] = 0;
    __syncthreads();
    for (int s = tid; s < S; s += kPermThreads) {
        const int e = ids[s] - base;
        if (e >= 0 && e < E_local) atomicAdd(&L.run[e], 1);
    }
    __syncthreads();
    {
        // exclusive scan over the experts (E_local <= 256: waves 0..3)
        const int c = tid < E_local ? L.run[tid] : 0;
        int v = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int n = __shfl_up(v, d);
            if (lane >= d) v += n;
        }
        if (lane == 63) L.tot[wave] = v;
        __syncthreads();
        int before = 0;
        for (int u = 0; u < wave; ++u) before += L.tot[u];
        const int incl = before + v;
        if (tid < E_local) {
            counts[tid] = c;
            offsets[tid] = incl - c;
            L.excl[tid] = incl - c;
        }
        if (tid == E_local - 1) {
            counts[E_local] = n_shared;
            offsets[E_local] = incl;
            offsets[E_local + 1] = incl + n_shared;
            L.excl[E_local] = incl;
        }
    }
    __syncthreads();
    for (int e = tid; e < E_local; e += kPermThreads) L.run[e] = 0;
    for (int c0 = 0; c0 < S; c0 += kPermThreads) {
        for (int i = tid; i < kWaves * kMaxLocal; i += kPermThreads) (&L.wc[0][0])[i] = 0;
        __syncthreads();
        const int s = c0 + tid;
        const int e = s < S ? ids[s] - base : -1;
        const bool loc = e >= 0 && e < E_local;
        int rank = 0;
        uint64_t todo = __ballot(loc);
        while (todo) {  // one round per distinct expert of the wave
            const int leader = __builtin_ctzll(todo);
            const int e0 = __shfl(e, leader);
            const uint64_t m = __ballot(loc && e == e0);
            if (loc && e == e0) rank = __popcll(m & ((1ull << lane) - 1ull));
            if (lane == leader) L.wc[wave][e0] = __popcll(m);
            todo &= ~m;
        }
        __syncthreads();
        if (loc) {
            int r = L.excl[e] + L.run[e] + rank;
            for (int w = 0; w < wave; ++w) r += L.wc[w][e];
            row_to_slot[r] = s;
            slot_to_row[s] = r;
        } else if (s < S) {
            slot_to_row[s] = -1;
        }
        __syncthreads();
        for (int x = tid; x < E_local; x += kPermThreads) {
            int add = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) add += L.wc[w][x];
            L.run[x] += add;
        }
        __syncthreads();
    }
    const int R = L.excl[E_local];
    for (int r = R + tid; r < S + T; r += kPermThreads) row_to_slot[r] = r < R + n_shared ? S + (r - R) : -1;
}

}  // namespace
}  // namespace moe
