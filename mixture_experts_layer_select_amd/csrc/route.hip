// Gating: router logits in a fixed fp32 order, then top-k selection and
// combine weights ([Moreh-EP] Overview: a lightweight gating network picks a
// small subset of experts per token; Parallelization: top-8 of 256 for R1).
//
// Logits. A wavefront of 64 lanes owns an 8-token x 8-expert tile of (t, e)
// pairs. Lane j accumulates, for all 64 pairs, the 8-element chunks of h with
// floor(h/8) mod 64 == j in ascending h with fused multiply-adds -- the same
// lane/partial assignment the reduction order is defined by. The partials are
// then combined pairwise (p[j] += p[j+s], s = 32..1) by a transposing
// butterfly: at every level each lane hands half of its pairs to its partner,
// so after 6 levels lane l holds the finished logit of pair l (63 exchanges
// instead of 6 per pair).
//
// Selection. One wavefront per token, up to 4 logits per lane; k rounds of a
// wave-wide maximum over a 64-bit key (order-preserving logit bits, then the
// complemented expert index) pick the experts in (logit desc, index asc)
// order.
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
template <typename TIn>
__global__ __launch_bounds__(256) void route_logits_kernel(const TIn* __restrict__ x,
                                                           const TIn* __restrict__ w,
                                                           const float* __restrict__ bias, int T,
                                                           int H, int E,
                                                           float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kWT;
    const int e0 = (blockIdx.y * 4 + wave) * kWE;
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

__device__ __forceinline__ uint32_t ordered_bits(float l) {
    uint32_t u = (l == 0.0f) ? 0u : __float_as_uint(l);  // -0 ties with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, s);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), s);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s);
    return v;
}

// one wave per token; E <= 256, k <= E
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int scoring, int renorm,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ topk_w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
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

// ---------------------------------------------------------------- candidate routing
// Selection without every fixed-order logit (large token batches). The set of
// the k largest fixed-order logits is found from approximate logits and a
// rigorous bound on their distance to the fixed-order ones:
//   1. route_approx_kernel: a_e = sum_h x_h w_eh and s_e = sum_h |x_h| |w_eh|
//      on bf16 MFMAs (bf16 products are exact in fp32).
//   2. route_refine_kernel, one wave per token: every bound below is taken in
//      fp64 with a margin. Whatever the MFMA's internal summation order, with
//      fp32-or-better intermediates and at most 2 units of fp32 rounding per
//      step (u = 2^-22: twice truncation), |a_e - S_e| <= g(H) s_e/(1 - g(H))
//      (S_e the exact dot product, g(n) = n u/(1 - n u)), plus H * 2^-126 for
//      flushed tiny products. The fixed-order value c_e differs from S_e by at
//      most g'(8 ceil(H/512) + 6) s_e (round to nearest, 2^-24: each lane's
//      partial adds 8 ceil(H/512) products, the tree adds 6 levels). The
//      bias add rounds both once. With D_e bounding |approx_e - logit_e|,
//      lo_e = approx_e - D_e <= logit_e <= hi_e = approx_e + D_e. If L is the
//      k-th largest lo, every expert with hi_e < L has a logit below the k-th
//      largest logit, so it cannot be picked (not even on an index tie). The
//      remaining candidates (at least k) get their fixed-order logit, the rest
//      -inf, written over the approximations.
//   3. route_topk_kernel as in moe_route: ids and weights are those of moe_route.
constexpr int kApproxT = 32;   // tokens per workgroup
constexpr int kApproxE = 64;   // experts per wave (4 waves: 256 experts)
constexpr int kApproxK = 32;   // K per MFMA

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                     __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// H % 32 == 0; blockIdx.x: 32-token block; wave w: experts 64w + [0, 64).
// A operand = 16 expert rows, B = 16 token rows; lane (li, lk) supplies
// k = 32c + 8lk + [0, 8) of row li, and holds D[4lk + r][li] (expert 4lk + r
// of the block, token li). Operands of K steps c+1 and c+2 are in flight
// while step c computes (a 3-slot ring). Rows past T or E read a valid row;
// never stored.
__global__ __launch_bounds__(256) void route_approx_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ w, int T,
                                                           int H, int E, float* __restrict__ approx,
                                                           float* __restrict__ sabs) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15, lk = lane >> 4;
    const int t0 = blockIdx.x * kApproxT;
    const int e0 = wave * kApproxE;
    if (e0 >= E) return;
    const uint16_t* xr[2];
    const uint16_t* wr[4];
#pragma unroll
    for (int b = 0; b < 2; ++b) xr[b] = x + (size_t)min(t0 + 16 * b + li, T - 1) * H + 8 * lk;
#pragma unroll
    for (int b = 0; b < 4; ++b) wr[b] = w + (size_t)min(e0 + 16 * b + li, E - 1) * H + 8 * lk;
    f32x4 acc[4][2], aab[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            aab[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    const int nk = H / kApproxK;
    u32x4 fa[3][4], fb[3][2];
    auto load = [&](int slot, int c) {
        const int k0 = (c < nk ? c : nk - 1) * kApproxK;  // past the end: a reload, never used
#pragma unroll
        for (int b = 0; b < 4; ++b) fa[slot][b] = *reinterpret_cast<const u32x4*>(wr[b] + k0);
#pragma unroll
        for (int b = 0; b < 2; ++b) fb[slot][b] = *reinterpret_cast<const u32x4*>(xr[b] + k0);
    };
    auto step = [&](int slot) {
        u32x4 ga[4], gb[2];
#pragma unroll
        for (int b = 0; b < 4; ++b) ga[b] = fa[slot][b] & 0x7fff7fffu;  // |bf16| pairs
#pragma unroll
        for (int b = 0; b < 2; ++b) gb[b] = fb[slot][b] & 0x7fff7fffu;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                acc[i][j] = mfma16x16x32(fa[slot][i], fb[slot][j], acc[i][j]);
                aab[i][j] = mfma16x16x32(ga[i], gb[j], aab[i][j]);
            }
    };
    // the scheduling barriers keep each step's loads ahead of the previous
    // step's MFMAs (the compiler would otherwise sink them next to their use)
    load(0, 0);
    load(1, 1);
    for (int c = 0;; c += 3) {
        load(2, c + 2);
        __builtin_amdgcn_sched_barrier(0);
        step(0);
        __builtin_amdgcn_sched_barrier(0);
        if (c + 1 >= nk) break;
        load(0, c + 3);
        __builtin_amdgcn_sched_barrier(0);
        step(1);
        __builtin_amdgcn_sched_barrier(0);
        if (c + 2 >= nk) break;
        load(1, c + 4);
        __builtin_amdgcn_sched_barrier(0);
        step(2);
        __builtin_amdgcn_sched_barrier(0);
        if (c + 3 >= nk) break;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = t0 + 16 * j + li;
            const int e = e0 + 16 * i + 4 * lk;
            if (t < T) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (e + r < E) {
                        approx[(size_t)t * E + e + r] = acc[i][j][r];
                        sabs[(size_t)t * E + e + r] = aab[i][j][r];
                    }
            }
        }
}

__device__ __forceinline__ double gamma_n(double n, double u) { return n * u / (1.0 - n * u); }

// one wave per token; E <= 256, H % 32 == 0, H <= 16 * 512 (the token's row
// stays in 16 registers per lane)
__global__ __launch_bounds__(256) void route_refine_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ w,
                                                           const float* __restrict__ bias, int T,
                                                           int H, int E, int k,
                                                           float* __restrict__ logits,
                                                           const float* __restrict__ sabs) {
    constexpr int kMaxSteps = 16;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int nsteps = (H + 511) / 512;
    const double gm = gamma_n((double)H, 0x1p-22);
    const double gc = gamma_n(8.0 * nsteps + 6.0, 0x1p-24);
    // bounds of every expert's logit, rounded outward to fp32
    float lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        lo[i] = -__builtin_inff();
        hi[i] = -__builtin_inff();
        if (e < E) {
            const double a = logits[(size_t)t * E + e];
            const double sa = sabs[(size_t)t * E + e];
            const double b = bias ? (double)bias[e] : 0.0;
            const double s_true = sa / (1.0 - gm) + (double)H * 0x1p-126;  // >= sum |x w|
            const double d_sum = gm * s_true + gc * s_true + (double)H * 0x1p-126;
            const double v = a + b;
            // both sides round once more when the bias is added
            const double d = (d_sum + (fabs(v) + d_sum) * 0x1p-23) * (1.0 + 0x1p-20) + 0x1p-100;
            lo[i] = __double2float_rd(v - d);
            hi[i] = __double2float_ru(v + d);
        }
    }
    // L = k-th largest lower bound (k rounds of a wave maximum over (lo, e))
    uint64_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < E ? (((uint64_t)ordered_bits(lo[i]) << 32) | (0xffffffffu - (uint32_t)e)) : 0;
    }
    uint64_t kth = 0;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int e = (int)(0xffffffffu - (uint32_t)best);
        if ((e & 63) == lane) key[e >> 6] = 0;
        kth = best;
    }
    const float L = from_ordered((uint32_t)(kth >> 32));
    // this token's row of x, one 8-element chunk per lane and step
    const uint16_t* xrow = x + (size_t)t * H;
    u32x4 xc[kMaxSteps];
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s)
        if (s < nsteps) {
            const int h0 = 512 * s + 8 * lane;
            xc[s] = h0 < H ? *reinterpret_cast<const u32x4*>(xrow + h0) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e_lane = lane + 64 * i;
        uint64_t cand = __ballot(e_lane < E && hi[i] >= L);
        float mine = -__builtin_inff();
        // candidates two at a time: two independent multiply-add chains
        while (cand) {
            const int c0 = __builtin_ctzll(cand);
            cand &= cand - 1;
            const bool two = cand != 0;
            const int c1 = two ? __builtin_ctzll(cand) : c0;
            if (two) cand &= cand - 1;
            // fixed-order logit: lane j sums its chunks in ascending h with
            // fused multiply-adds from +0, then p[j] += p[j + s], s = 32..1
            const uint16_t* w0 = w + (size_t)(64 * i + c0) * H;
            const uint16_t* w1 = w + (size_t)(64 * i + c1) * H;
            float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
            for (int s = 0; s < kMaxSteps; ++s)
                if (s < nsteps) {
                    const int h0 = 512 * s + 8 * lane;
                    if (h0 < H) {
                        const u32x4 a0 = *reinterpret_cast<const u32x4*>(w0 + h0);
                        const u32x4 a1 = *reinterpret_cast<const u32x4*>(w1 + h0);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            p0 = __builtin_fmaf(bf16_lo(xc[s][q]), bf16_lo(a0[q]), p0);
                            p1 = __builtin_fmaf(bf16_lo(xc[s][q]), bf16_lo(a1[q]), p1);
                            p0 = __builtin_fmaf(bf16_hi(xc[s][q]), bf16_hi(a0[q]), p0);
                            p1 = __builtin_fmaf(bf16_hi(xc[s][q]), bf16_hi(a1[q]), p1);
                        }
                    }
                }
#pragma unroll
            for (int s = 32; s >= 1; s >>= 1) {
                p0 = p0 + __shfl_xor(p0, s);
                p1 = p1 + __shfl_xor(p1, s);
            }
            float l0 = __shfl(p0, 0), l1 = __shfl(p1, 0);
            if (bias) {
                l0 = l0 + bias[64 * i + c0];
                l1 = l1 + bias[64 * i + c1];
            }
            if (lane == c0) mine = l0;
            if (two && lane == c1) mine = l1;
        }
        if (e_lane < E) logits[(size_t)t * E + e_lane] = mine;
    }
}

}  // namespace

moe_status launch_route(const void* x, const void* w, const float* bias, moe_dtype dt, int T, int H,
                        int E, int k, int scoring, int renorm, float* logits, int32_t* ids,
                        float* topk_w, hipStream_t st) {
    dim3 grid((T + kWT - 1) / kWT, (E + 4 * kWE - 1) / (4 * kWE));
    if (dt == MOE_BF16)
        hipLaunchKernelGGL(route_logits_kernel<uint16_t>, grid, dim3(256), 0, st,
                           (const uint16_t*)x, (const uint16_t*)w, bias, T, H, E, logits);
    else
        hipLaunchKernelGGL(route_logits_kernel<float>, grid, dim3(256), 0, st, (const float*)x,
                           (const float*)w, bias, T, H, E, logits);
    moe_status s = check_launch("route_logits_kernel");
    if (s != MOE_OK) return s;
    hipLaunchKernelGGL(route_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E, k,
                       scoring, renorm, ids, topk_w);
    return check_launch("route_topk_kernel");
}

}  // namespace moe

namespace moe {

size_t route_select_workspace_bytes(int T, int E) {
    return 2 * align_up((size_t)T * E * sizeof(float), 256);
}

moe_status launch_route_select(const void* x, const void* w, const float* bias, int T, int H, int E,
                               int k, int scoring, int renorm, int32_t* ids, float* topk_w, void* ws,
                               hipStream_t st) {
    float* approx = (float*)ws;
    float* sabs = (float*)((uint8_t*)ws + align_up((size_t)T * E * sizeof(float), 256));
    hipLaunchKernelGGL(route_approx_kernel, dim3((T + kApproxT - 1) / kApproxT), dim3(256), 0, st,
                       (const uint16_t*)x, (const uint16_t*)w, T, H, E, approx, sabs);
    moe_status s = check_launch("route_approx_kernel");
    if (s != MOE_OK) return s;
    hipLaunchKernelGGL(route_refine_kernel, dim3((T + 3) / 4), dim3(256), 0, st, (const uint16_t*)x,
                       (const uint16_t*)w, bias, T, H, E, k, approx, sabs);
    s = check_launch("route_refine_kernel");
    if (s != MOE_OK) return s;
    hipLaunchKernelGGL(route_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, approx, T, E, k, scoring,
                       renorm, ids, topk_w);
    return check_launch("route_topk_kernel");
}

}  // namespace moe
