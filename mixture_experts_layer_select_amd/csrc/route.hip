// Gating: router logits in a fixed fp32 order, then top-k selection and
// combine weights ([Moreh-EP] Overview: a lightweight gating network picks a
// small subset of experts per token; Parallelization: top-8 of 256 for R1).
//
// Logits. A wavefront of 64 lanes owns a 4-token x 16-expert tile of (t, e)
// pairs. Lane j accumulates, for all 64 pairs, the 8-element chunks of h with
// floor(h/8) mod 64 == j in ascending h with fused multiply-adds -- the same
// lane/partial assignment the reduction order is defined by. The partials are
// then combined pairwise (p[j] += p[j+s], s = 32..1) by a transposing
// butterfly: at every level each lane hands half of its pairs to its partner,
// so after 6 levels lane l holds the finished logit of pair l (63 exchanges
// instead of 6 per pair). Tiles of x and w_router for one 512-wide h step
// are staged in LDS and shared by the 4 waves of a workgroup (16 tokens x 16
// experts per workgroup).
//
// Selection. One wavefront per token, up to 4 logits per lane; k rounds of a
// wave-wide maximum over a 64-bit key (order-preserving logit bits, then the
// complemented expert index) pick the experts in (logit desc, index asc)
// order.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokTile = 16;   // tokens per workgroup (4 per wave)
constexpr int kExpTile = 16;   // experts per workgroup
constexpr int kStep = 512;     // h per step: 64 lanes x 8

template <typename TIn>
struct RouteIO;

template <>
struct RouteIO<uint16_t> {  // bf16 bit patterns
    static constexpr int kBytes = 2;
    // load the 8-element chunk [h0, h0+8) of a row, zero beyond H
    static __device__ __forceinline__ void load8(const uint16_t* row, int h0, int H, float* v) {
        if (h0 + 8 <= H && (H & 7) == 0) {
            u32x4 q = *reinterpret_cast<const u32x4*>(row + h0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = bf16_lo(q[i]);
                v[2 * i + 1] = bf16_hi(q[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = (h0 + i < H) ? bf16_to_f32(row[h0 + i]) : 0.0f;
        }
    }
};

template <>
struct RouteIO<float> {
    static constexpr int kBytes = 4;
    static __device__ __forceinline__ void load8(const float* row, int h0, int H, float* v) {
        if (h0 + 8 <= H && (H & 3) == 0) {
            f32x4 a = *reinterpret_cast<const f32x4*>(row + h0);
            f32x4 b = *reinterpret_cast<const f32x4*>(row + h0 + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] = a[i];
                v[4 + i] = b[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = (h0 + i < H) ? row[h0 + i] : 0.0f;
        }
    }
};

// LDS tile: rows of 512 elements stored as fp32 (converted once while
// staging). Element 8j + 4q + i of a row (chunk j, half q) sits at
// [q*256 + 4j + i], so the 64 lanes of a wave read two contiguous 1 KB runs.
template <typename TIn>
__global__ __launch_bounds__(256) void route_logits_kernel(const TIn* __restrict__ x,
                                                           const TIn* __restrict__ w,
                                                           const float* __restrict__ bias, int T,
                                                           int H, int E,
                                                           float* __restrict__ logits) {
    __shared__ float xs[kTokTile][kStep];
    __shared__ float ws[kExpTile][kStep];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kTokTile;
    const int e0 = blockIdx.y * kExpTile;

    float acc[4][kExpTile];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < kExpTile; ++b) acc[a][b] = 0.0f;

    for (int hs = 0; hs < H; hs += kStep) {
        // stage: 32 rows x 64 chunks of 8; thread i loads chunks i, i+256, ...
        for (int c = threadIdx.x; c < (kTokTile + kExpTile) * 64; c += 256) {
            int r = c >> 6, j = c & 63;
            float v[8];
            int h0 = hs + 8 * j;
            if (r < kTokTile) {
                int t = t0 + r;
                if (t < T) RouteIO<TIn>::load8(x + (size_t)t * H, h0, H, v);
                else
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xs[r][4 * j + i] = v[i];
                    xs[r][256 + 4 * j + i] = v[4 + i];
                }
            } else {
                int e = e0 + r - kTokTile;
                if (e < E) RouteIO<TIn>::load8(w + (size_t)e * H, h0, H, v);
                else
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ws[r - kTokTile][4 * j + i] = v[i];
                    ws[r - kTokTile][256 + 4 * j + i] = v[4 + i];
                }
            }
        }
        __syncthreads();
        float xv[4][8];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x4 lo = *reinterpret_cast<const f32x4*>(&xs[wave * 4 + a][4 * lane]);
            f32x4 hi = *reinterpret_cast<const f32x4*>(&xs[wave * 4 + a][256 + 4 * lane]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xv[a][i] = lo[i];
                xv[a][4 + i] = hi[i];
            }
        }
#pragma unroll
        for (int b = 0; b < kExpTile; ++b) {
            f32x4 lo = *reinterpret_cast<const f32x4*>(&ws[b][4 * lane]);
            f32x4 hi = *reinterpret_cast<const f32x4*>(&ws[b][256 + 4 * lane]);
            float wv[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int a = 0; a < 4; ++a) acc[a][b] = __builtin_fmaf(xv[a][i], wv[i], acc[a][b]);
        }
        __syncthreads();
    }

    // transposing pairwise reduction: pair p = a*16 + b ends in lane p
    float v[64];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < kExpTile; ++b) v[a * kExpTile + b] = acc[a][b];
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
    const int t = t0 + wave * 4 + (lane >> 4);
    const int e = e0 + (lane & 15);
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

}  // namespace

moe_status launch_route(const void* x, const void* w, const float* bias, moe_dtype dt, int T, int H,
                        int E, int k, int scoring, int renorm, float* logits, int32_t* ids,
                        float* topk_w, hipStream_t st) {
    dim3 grid((T + kTokTile - 1) / kTokTile, (E + kExpTile - 1) / kExpTile);
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
