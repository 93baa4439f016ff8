// Device code of the gating (router logits in a fixed fp32 order, top-k
// selection and combine weights), shared by the gating kernels and the fused
// small-batch layer. Internal to libmoe.so.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {


constexpr int kWT = 8;        // tokens per wave
constexpr int kWE = 8;        // experts per wave
constexpr int kStep = 512;    // h per step: 64 lanes x 8

// 8 consecutive inputs as fp32 (zeros past H)
template <typename TIn>
struct Chunk;

template <>
struct Chunk<uint16_t> {  // bf16 bit patterns: 8 values in one 16-byte load
    u32x4 raw;
    __device__ __forceinline__ void load(const uint16_t* row, int h0, int H, bool vec) {
        if (vec && h0 + 8 <= H) {
            raw = *reinterpret_cast<const u32x4*>(row + h0);
        } else {
            uint32_t v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t lo = h0 + 2 * i < H ? row[h0 + 2 * i] : 0u;
                uint32_t hi = h0 + 2 * i + 1 < H ? row[h0 + 2 * i + 1] : 0u;
                v[i] = lo | (hi << 16);
            }
            raw = u32x4{v[0], v[1], v[2], v[3]};
        }
    }
    __device__ __forceinline__ float at(int i) const {
        return (i & 1) ? bf16_hi(raw[i >> 1]) : bf16_lo(raw[i >> 1]);
    }
};

template <>
struct Chunk<float> {
    f32x4 lo, hi;
    __device__ __forceinline__ void load(const float* row, int h0, int H, bool vec) {
        if (vec && h0 + 8 <= H) {
            lo = *reinterpret_cast<const f32x4*>(row + h0);
            hi = *reinterpret_cast<const f32x4*>(row + h0 + 4);
        } else {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = h0 + i < H ? row[h0 + i] : 0.0f;
            lo = f32x4{v[0], v[1], v[2], v[3]};
            hi = f32x4{v[4], v[5], v[6], v[7]};
        }
    }
    __device__ __forceinline__ float at(int i) const { return i < 4 ? lo[i] : hi[i - 4]; }
};

// A wave owns 8 tokens x 8 experts = 64 (t, e) pairs; a workgroup of 4 waves
// covers 8 tokens x 32 experts. Lane j reads its 16-byte chunk of each of the
// 16 rows straight from global memory (a wave reads 1 KB contiguous per row
// and step), one step ahead in registers; no LDS. Every input row is read
// whole by every wave that needs it, so reuse happens in L2. Rows past T or E
// read a valid row; those pairs are never written. Zero padding past H adds
// fma(0, 0, p) = p exactly (a partial that starts at +0 is never -0).
// Vector loads need H % 8 == 0 (bf16) / H % 4 == 0 (fp32) for alignment;
// other H take the element path for every chunk.
// the 8 x 8 tile of tokens t0.. and experts e0.. (one wave)
template <typename TIn>
__device__ __forceinline__ void route_logits_tile(const TIn* __restrict__ x, const TIn* __restrict__ w,
                                                  const float* __restrict__ bias, int T, int H, int E,
                                                  float* __restrict__ logits, int t0, int e0) {
    const int lane = threadIdx.x & 63;
    const bool aligned = sizeof(TIn) == 2 ? (H & 7) == 0 : (H & 3) == 0;

    const TIn* xr[kWT];
    const TIn* wr[kWE];
#pragma unroll
    for (int a = 0; a < kWT; ++a) xr[a] = x + (size_t)min(t0 + a, T - 1) * H;
#pragma unroll
    for (int b = 0; b < kWE; ++b) wr[b] = w + (size_t)min(e0 + b, E - 1) * H;

    float acc[kWT][kWE];
#pragma unroll
    for (int a = 0; a < kWT; ++a)
#pragma unroll
        for (int b = 0; b < kWE; ++b) acc[a][b] = 0.0f;

    Chunk<TIn> cx[2][kWT], cw[2][kWE];
    auto load = [&](int buf, int hs) {
        const int h0 = hs + 8 * lane;
#pragma unroll
        for (int a = 0; a < kWT; ++a) cx[buf][a].load(xr[a], h0, H, aligned);
#pragma unroll
        for (int b = 0; b < kWE; ++b) cw[buf][b].load(wr[b], h0, H, aligned);
    };
    auto fma_step = [&](int buf) {
        // partial of lane j, ascending h inside its chunk, every pair
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float xv[kWT], wv[kWE];
#pragma unroll
            for (int a = 0; a < kWT; ++a) xv[a] = cx[buf][a].at(i);
#pragma unroll
            for (int b = 0; b < kWE; ++b) wv[b] = cw[buf][b].at(i);
#pragma unroll
            for (int a = 0; a < kWT; ++a)
#pragma unroll
                for (int b = 0; b < kWE; ++b) acc[a][b] = __builtin_fmaf(xv[a], wv[b], acc[a][b]);
        }
    };
    load(0, 0);
    int hs = 0;
    for (;;) {
        const bool more = hs + kStep < H;
        if (more) load(1, hs + kStep);
        __builtin_amdgcn_sched_barrier(0);
        fma_step(0);
        __builtin_amdgcn_sched_barrier(0);
        if (!more) break;
        hs += kStep;
        const bool more2 = hs + kStep < H;
        if (more2) load(0, hs + kStep);
        __builtin_amdgcn_sched_barrier(0);
        fma_step(1);
        __builtin_amdgcn_sched_barrier(0);
        if (!more2) break;
        hs += kStep;
    }

    // transposing pairwise reduction: pair p = a*8 + b ends in lane p
    float v[64];
#pragma unroll
    for (int a = 0; a < kWT; ++a)
#pragma unroll
        for (int b = 0; b < kWE; ++b) v[a * kWE + b] = acc[a][b];
#pragma unroll
    for (int s = 32, n = 64; s >= 1; s >>= 1, n >>= 1) {
        const bool hi = (lane & s) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
            float keep = hi ? v[n / 2 + i] : v[i];
            float give = hi ? v[i] : v[n / 2 + i];
            float got = __shfl_xor(give, s);
            v[i] = keep + got;
        }
    }
    const int t = t0 + (lane >> 3);
    const int e = e0 + (lane & 7);
    if (t < T && e < E) {
        float l = v[0];
        if (bias) l = l + bias[e];
        logits[(size_t)t * E + e] = l;
    }
}

// Small batches: one wave computes one (token, expert) logit with both rows
// read whole into registers up front (kSteps chunks of 16 bytes per lane and
// row), so it waits for one memory latency instead of one per 512-element
// step. Lane j runs the same fma chain over its chunks as route_logits_tile,
// and the butterfly below adds the 64 partials over lane bits 5..0 in the
// same tree as its transposing reduction (each level adds the same two
// values; fp32 addition commutes), so the logit is bit-identical. Rows are
// read through descriptors of the row's size: chunks past H read zeros
// (H % 8 == 0, so a chunk is either inside the row or past it) and the steps
// past ceil(H/512) are skipped. Needs H <= kSteps * 512.
template <int kSteps>
__device__ __forceinline__ void route_logits_row(const uint16_t* __restrict__ x,
                                                 const uint16_t* __restrict__ w,
                                                 const float* __restrict__ bias, int H, int E,
                                                 float* __restrict__ logits, int t, int e) {
    const int lane = threadIdx.x & 63;
    const uint32_t row_bytes = (uint32_t)H * 2u;
    const __amdgpu_buffer_rsrc_t wd = buffer_rsrc(w + (size_t)e * H, row_bytes);
    const __amdgpu_buffer_rsrc_t xd = buffer_rsrc(x + (size_t)t * H, row_bytes);
    u32x4 wc[kSteps], xc[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) wc[s] = buffer_load16(wd, (uint32_t)(512 * s + 8 * lane) * 2u, 0);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) xc[s] = buffer_load16(xd, (uint32_t)(512 * s + 8 * lane) * 2u, 0);
    const int nsteps = (H + kStep - 1) / kStep;
    float p = 0.0f;
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
        if (s < nsteps) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                p = __builtin_fmaf(bf16_lo(xc[s][q]), bf16_lo(wc[s][q]), p);
                p = __builtin_fmaf(bf16_hi(xc[s][q]), bf16_hi(wc[s][q]), p);
            }
        }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) p = p + __shfl_xor(p, s);
    if (lane == 0) logits[(size_t)t * E + e] = bias ? p + bias[e] : p;
}

__device__ __forceinline__ uint32_t ordered_bits(float l) {
    uint32_t u = (l == 0.0f) ? 0u : __float_as_uint(l);  // -0 ties with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return __uint_as_float(u);
}

// The maximum of v over the wave's 64 lanes. Each row of 16 lanes by DPP
// moves (partners lane ^ 1, lane ^ 2, then the mirrored half-rows and rows),
// which leaves the row's maximum in all of its lanes; then the four row
// maxima are read into scalar registers. No LDS round trips; the result is
// wave-uniform. (Integer keys: any order of comparisons gives the same max.)
template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, kCtrl, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), kCtrl, 0xf, 0xf, false);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > v ? o : v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = dpp_max_u64<0xb1>(v);   // quad_perm [1, 0, 3, 2]
    v = dpp_max_u64<0x4e>(v);   // quad_perm [2, 3, 0, 1]
    v = dpp_max_u64<0x141>(v);  // row_half_mirror: lane i <-> 7 - i in each half-row
    v = dpp_max_u64<0x140>(v);  // row_mirror: lane i <-> 15 - i in each row
    uint64_t m = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        m = o > m ? o : m;
    }
    return m;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s);
    return v;
}

// selection and weights of token t (one wave); E <= 256, k <= E
__device__ __forceinline__ void route_topk_token(const float* __restrict__ logits, int T, int E, int k,
                                                 int scoring, int renorm, int32_t* __restrict__ ids,
                                                 float* __restrict__ topk_w, int t) {
    const int lane = threadIdx.x & 63;
    if (t >= T) return;
    const float* l = logits + (size_t)t * E;
    uint64_t key[4];
    float lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int e = lane + 64 * i;
        lv[i] = e < E ? l[e] : 0.0f;
        key[i] = e < E ? (((uint64_t)ordered_bits(lv[i]) << 32) | (0xffffffffu - (uint32_t)e)) : 0;
    }
    int my_id[4] = {0, 0, 0, 0};
    float my_l[4] = {0.f, 0.f, 0.f, 0.f};
    float lmax = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int e = (int)(0xffffffffu - (uint32_t)best);
        const float lb = from_ordered((uint32_t)(best >> 32));
        if (j == 0) lmax = lb;
        if ((e & 63) == lane) key[e >> 6] = 0;  // taken
        if ((j & 63) == lane) {
            my_id[j >> 6] = e;
            my_l[j >> 6] = lb;
        }
    }
    // weights
    float num[4], part = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool mine = lane + 64 * i < k;
        float v;
        if (scoring == MOE_SIGMOID) v = 1.0f / (1.0f + expf(-my_l[i]));
        else v = expf(my_l[i] - lmax);
        num[i] = mine ? v : 0.0f;
        part += num[i];
    }
    float den;
    if (renorm) {
        den = wave_sum(part);
    } else if (scoring == MOE_SOFTMAX) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + 64 * i < E) s += expf(lv[i] - lmax);
        den = wave_sum(s);
    } else {
        den = 1.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        if (j < k) {
            ids[(size_t)t * k + j] = my_id[i];
            topk_w[(size_t)t * k + j] = num[i] / den;
        }
    }
}

}  // namespace
}  // namespace moe
