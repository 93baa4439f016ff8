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
// instead of 6 per pair). Small batches (up to 64 bf16 tokens) have too few
// tiles to fill the GPU: there one wave computes one (token, expert) pair
// with both rows in registers, the same lane partials and the same addition
// tree, so the logits are the same bit for bit.
//
// Selection. One wavefront per token, up to 4 logits per lane; k rounds of a
// wave-wide maximum over a 64-bit key (order-preserving logit bits, then the
// complemented expert index) pick the experts in (logit desc, index asc)
// order.
#include "route_dev.h"

namespace moe {
namespace {

template <typename TIn>
__global__ __launch_bounds__(256) void route_logits_kernel(const TIn* __restrict__ x,
                                                           const TIn* __restrict__ w,
                                                           const float* __restrict__ bias, int T,
                                                           int H, int E,
                                                           float* __restrict__ logits) {
    const int wave = threadIdx.x >> 6;
    route_logits_tile(x, w, bias, T, H, E, logits, blockIdx.x * kWT, (blockIdx.y * 4 + wave) * kWE);
}

// Small batches: wave w of workgroup (x, y) computes expert 4x + w for token
// y (route_logits_row). The workgroups of one expert quadruple differ in y
// only; with E a multiple of 32 their index mod 8, and so their XCD, is the
// same, and the expert rows cross HBM once.
template <int kSteps>
__global__ __launch_bounds__(256) void route_logits_rows_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ w,
                                                                const float* __restrict__ bias, int H,
                                                                int E, float* __restrict__ logits) {
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    route_logits_row<kSteps>(x, w, bias, H, E, logits, blockIdx.y, e);
}

// one wave per token
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int scoring, int renorm,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ topk_w) {
    route_topk_token(logits, T, E, k, scoring, renorm, ids, topk_w, blockIdx.x * 4 + (threadIdx.x >> 6));
}

// ---------------------------------------------------------------- candidate routing
// Selection without every fixed-order logit (large token batches). The set of
// the k largest fixed-order logits is found from approximate logits and a
// rigorous bound on their distance to the fixed-order ones:
//   1. route_approx_kernel: a_e = sum_h x_h w_eh and s_e = sum_h |x_h| |w_eh|
//      on bf16 MFMAs (bf16 products are exact in fp32 unless they underflow).
//      Every 64-deep stage is summed by two chained MFMAs from zero; the stage
//      results are added on the VALU in ascending K. It also writes max_h |w_eh| per expert
//      and max_h |x_th| per token.
//   2. route_refine_kernel, one wave per token: every bound below is taken in
//      fp64 with a margin. The MFMA part of the error only depends on a
//      64-term sum being within gamma(64, 2^-16) of exact relative to the sum
//      of magnitudes (16 significant bits per addition in any order or
//      alignment; fp32 arithmetic has 24), the chunk sums on IEEE fp32 adds,
//      and flushed tiny values (a denormal input, product or partial) costing
//      at most 2^-126 (1 + |w| + |x|) per product and 2^-126 per addition;
//      max |x| of the token and max |w| of the expert bound the latter. The
//      fixed-order value c_e differs from S_e (the exact dot product) by at
//      most g'(8 ceil(H/512) + 6) s_e (round to nearest, 2^-24: each lane's
//      partial adds 8 ceil(H/512) products, the tree adds 6 levels). The
//      bias add rounds both once. With D_e bounding |approx_e - logit_e|,
//      lo_e = approx_e - D_e <= logit_e <= hi_e = approx_e + D_e. If L is the
//      k-th largest lo, every expert with hi_e < L has a logit below the k-th
//      largest logit, so it cannot be picked (not even on an index tie). The
//      remaining candidates (at least k) get their fixed-order logit, the rest
//      -inf, written over the approximations.
//   3. route_topk_kernel as in moe_route: ids and weights are those of moe_route.
constexpr int kApproxT = 128;  // tokens per workgroup
constexpr int kApproxE = 128;  // experts per workgroup
constexpr int kApproxK = 64;   // K per stage

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                     __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// this wave's LDS accesses done (lgkmcnt 0), then a workgroup barrier without
// the release fence of __syncthreads(), which would also wait for every load
// in flight (the register ring)
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    __builtin_amdgcn_s_barrier();
}

struct ApproxStage {
    uint16_t x[kApproxT * kApproxK];  // 16 KB: 128 rows of 128 bytes
    uint16_t w[kApproxE * kApproxK];  // 16 KB
};

// Tile of 128 tokens x 128 experts, 8 waves: wave (wt, we) = tokens 32wt +
// [0, 32), experts 64we + [0, 64). Each K stage (64) of both operand tiles is
// loaded by all 512 threads into registers one stage ahead, then stored to
// one of two LDS buffers; rows are 128 bytes and chunk c (16 bytes) of row r
// sits at physical chunk c ^ ((r >> 1) & 7). A operand = 16 expert rows, B =
// 16 token rows; lane (li, lk) supplies k = 32 sub + 8 lk + [0, 8) of row li
// and holds D[4lk + r][li] (expert 4lk + r of the block, token li). Rows past
// T or E read a valid row and columns past H read zeros (their products add
// exact zeros); neither is stored.
__global__ __launch_bounds__(512) void route_approx_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ w, int T,
                                                           int H, int E, float* __restrict__ approx,
                                                           float* __restrict__ sabs,
                                                           float* __restrict__ wmax,
                                                           float* __restrict__ xmax) {
    __shared__ __attribute__((aligned(1024))) ApproxStage st[2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wt = wave & 3, we = wave >> 2;
    const int li = lane & 15, lk = lane >> 4;
    const int t0 = blockIdx.x * kApproxT;
    const int e0 = blockIdx.y * kApproxE;
    const int nst = (H + kApproxK - 1) / kApproxK;

    // this thread's 2 + 2 chunks of a stage: chunk q = tid + 512 i -> row q / 8,
    // chunk q % 8; a 3-slot register ring holds stages s+1 and s+2 (in flight)
    // while stage s is computed from LDS
    u32x4 rx[3][2], rw[3][2];
    // rows through descriptors of the tile's rows: columns past H read zeros
    const int xrows = min(kApproxT, T - t0), wrows = min(kApproxE, E - e0);
    const __amdgpu_buffer_rsrc_t xd = buffer_rsrc(x + (size_t)t0 * H, (uint32_t)((size_t)xrows * H * 2));
    const __amdgpu_buffer_rsrc_t wd = buffer_rsrc(w + (size_t)e0 * H, (uint32_t)((size_t)wrows * H * 2));
    uint32_t xo[2], wo[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = tid + 512 * i;
        const int r = q >> 3, c = q & 7;
        xo[i] = (uint32_t)(min(r, xrows - 1) * H + 8 * c) * 2u;
        wo[i] = (uint32_t)(min(r, wrows - 1) * H + 8 * c) * 2u;
    }
    auto load = [&](int slot, int sidx) {
        const int k0 = min(sidx, nst - 1) * kApproxK;  // past the end: a reload, never stored
        // a chunk past H (only in a last stage of 32 columns) is masked out
        // by zeroing its value below, never by a branch around the load
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            rx[slot][i] = buffer_load16(xd, xo[i], (uint32_t)k0 * 2u);
            rw[slot][i] = buffer_load16(wd, wo[i], (uint32_t)k0 * 2u);
        }
        if (k0 + kApproxK > H) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int c = (tid + 512 * i) & 7;
                if (k0 + 8 * c >= H) {
                    rx[slot][i] = u32x4{0u, 0u, 0u, 0u};
                    rw[slot][i] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
    };
    // the first token tile's workgroups also take max |w| of each expert row,
    // the first expert tile's max |x| of each token row (bf16 magnitudes
    // compare as integers once the sign bit is cleared)
    const bool row_max = blockIdx.x == 0;
    const bool tok_max = blockIdx.y == 0;
    uint32_t wm_bits[2] = {0u, 0u};
    uint32_t xm_bits[2] = {0u, 0u};
    auto store = [&](int slot, ApproxStage& S) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = tid + 512 * i;
            const int r = q >> 3, c = q & 7;
            const int o = r * kApproxK + ((c ^ ((r >> 1) & 7)) << 3);
            *reinterpret_cast<u32x4*>(&S.x[o]) = rx[slot][i];
            *reinterpret_cast<u32x4*>(&S.w[o]) = rw[slot][i];
            if (row_max) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint32_t u = rw[slot][i][v];
                    wm_bits[i] = max(wm_bits[i], max(u & 0x7fffu, (u >> 16) & 0x7fffu));
                }
            }
            if (tok_max) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint32_t u = rx[slot][i][v];
                    xm_bits[i] = max(xm_bits[i], max(u & 0x7fffu, (u >> 16) & 0x7fffu));
                }
            }
        }
    };
    f32x4 acc[4][2], aab[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            aab[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    auto frag = [&](const uint16_t* base, int row, int sub) {
        const int c = 4 * sub + lk;
        return *reinterpret_cast<const u32x4*>(&base[row * kApproxK + ((c ^ ((row >> 1) & 7)) << 3)]);
    };
    // Each stage (64 deep) is one chain of two MFMAs from zero, added to its
    // sum on the VALU, stage after stage in ascending K: an MFMA only ever
    // sums exact products of one stage, whatever its internal order.
    auto compute = [&](const ApproxStage& S) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 ta[4][2], tb[4][2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            u32x4 fa[4], fb[2], ga[4], gb[2];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                fa[b] = frag(S.w, 64 * we + 16 * b + li, sub);
                ga[b] = fa[b] & 0x7fff7fffu;  // |bf16| pairs: sign bits cleared
            }
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                fb[b] = frag(S.x, 32 * wt + 16 * b + li, sub);
                gb[b] = fb[b] & 0x7fff7fffu;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    ta[i][j] = mfma16x16x32(fa[i], fb[j], sub ? ta[i][j] : z);
                    tb[i][j] = mfma16x16x32(ga[i], gb[j], sub ? tb[i][j] : z);
                }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                acc[i][j] += ta[i][j];
                aab[i][j] += tb[i][j];
            }
    };
    // step s (u = s mod 6 fixes the register slot and the LDS buffer):
    // compute stage s from LDS buffer s%2, store stage s+1 from its register
    // slot into the other buffer (read two steps ago), meet, then load stage
    // s+3 into the slot stage s came from. The loop leaves from the middle.
    load(0, 0);
    load(1, 1);
    load(2, 2);
    store(0, st[0]);
    lds_barrier();
    auto step = [&](int sidx, auto u_c) {
        constexpr int u = decltype(u_c)::value;
        compute(st[u & 1]);
        if (sidx + 1 < nst) store((u + 1) % 3, st[(u + 1) & 1]);
        lds_barrier();
        load(u % 3, sidx + 3);
    };
    for (int sidx = 0;; sidx += 6) {
        step(sidx, std::integral_constant<int, 0>{});
        if (sidx + 1 >= nst) break;
        step(sidx + 1, std::integral_constant<int, 1>{});
        if (sidx + 2 >= nst) break;
        step(sidx + 2, std::integral_constant<int, 2>{});
        if (sidx + 3 >= nst) break;
        step(sidx + 3, std::integral_constant<int, 3>{});
        if (sidx + 4 >= nst) break;
        step(sidx + 4, std::integral_constant<int, 4>{});
        if (sidx + 5 >= nst) break;
        step(sidx + 5, std::integral_constant<int, 5>{});
        if (sidx + 6 >= nst) break;
    }
    if (row_max) {
        // the 8 threads of a row are 8 consecutive lanes
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint32_t m = wm_bits[i];
            m = max(m, (uint32_t)__shfl_xor((int)m, 1));
            m = max(m, (uint32_t)__shfl_xor((int)m, 2));
            m = max(m, (uint32_t)__shfl_xor((int)m, 4));
            const int r = (tid + 512 * i) >> 3;
            if ((tid & 7) == 0 && e0 + r < E) wmax[e0 + r] = __uint_as_float(m << 16);
        }
    }
    if (tok_max) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint32_t m = xm_bits[i];
            m = max(m, (uint32_t)__shfl_xor((int)m, 1));
            m = max(m, (uint32_t)__shfl_xor((int)m, 2));
            m = max(m, (uint32_t)__shfl_xor((int)m, 4));
            const int r = (tid + 512 * i) >> 3;
            if ((tid & 7) == 0 && t0 + r < T) xmax[t0 + r] = __uint_as_float(m << 16);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int t = t0 + 32 * wt + 16 * j + li;
            const int e = e0 + 64 * we + 16 * i + 4 * lk;
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

// one wave per token; E <= 256, H % 32 == 0, H <= kMaxSteps * 512 (the
// token's row stays in registers: kMaxSteps chunks per lane)
template <int kMaxSteps>
__global__ __launch_bounds__(256) void route_refine_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ w,
                                                           const float* __restrict__ bias, int T,
                                                           int H, int E, int k,
                                                           float* __restrict__ logits,
                                                           const float* __restrict__ sabs,
                                                           const float* __restrict__ wmax,
                                                           const float* __restrict__ xmax,
                                                           int32_t* __restrict__ ncand) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int nsteps = (H + 511) / 512;  // steps with data; the rest read zeros
    const double mx = (double)xmax[t];  // max |x| of the token
    // Distance of the approximate sums from the exact dot product S = sum x w,
    // with A = sum |x w| (the same bound for every internal MFMA order):
    //  - each stage's sum (two chained 32-deep MFMAs from zero: 64 products
    //    and at most 64 additions) is within gamma(64, 2^-16) * A_stage of its
    //    exact sum: at least 16 significant bits per addition, in any order or
    //    operand alignment (fp32 keeps 24);
    //  - the nc = ceil(H/64) stage sums are added on the VALU in IEEE fp32
    //    (gamma(nc, 2^-24)), the signed sums and the absolute sums alike;
    //  - flushes: a tiny product, a tiny chunk result, or a tiny (denormal)
    //    input x_h or w_h dropped by the MFMA loses at most 2^-126 (1 + |w_h|
    //    + |x_h|) per product plus 2^-126 per addition: F below.
    // The absolute sums give A <= (s_a + 2F) / (1 - g). The fixed-order logit
    // is within gamma(8 ceil(H/512) + 6, 2^-24) A of S (fma chains per lane,
    // then the 6-level tree), plus F should the VALU flush as well.
    const double nc = (double)((H + 63) / 64);
    const double g = gamma_n(64.0, 0x1p-16) + 2.0 * gamma_n(nc, 0x1p-24);
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
            const double F = 0x1p-126 * ((double)H * (1.0 + (double)wmax[e] + mx) + 64.0 * nc + 64.0);
            const double a_up = (sa + 2.0 * F) / (1.0 - g);  // >= sum |x w|
            const double d_sum = (g + gc) * a_up + 3.0 * F;
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
    // the candidates: experts whose upper bound reaches L (wave-uniform masks)
    uint64_t cmask[4];
    int n_cand = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        cmask[i] = __ballot(lane + 64 * i < E && hi[i] >= L);
        n_cand += __builtin_popcountll(cmask[i]);
    }
    // this token's row of x, one 8-element chunk per lane and step. Rows are
    // read through a descriptor of the row's size: chunks past H read zeros,
    // whose products add exact zeros to a partial (which is never -0), so all
    // kMaxSteps steps run unguarded and every load can be issued up front
    const __amdgpu_buffer_rsrc_t xd = buffer_rsrc(x + (size_t)t * H, (uint32_t)H * 2u);
    u32x4 xc[kMaxSteps];
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s) xc[s] = buffer_load16(xd, (uint32_t)(512 * s + 8 * lane) * 2u, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e_lane = lane + 64 * i;
        uint64_t cand = cmask[i];
        float mine = -__builtin_inff();
        // one candidate at a time; the next candidate's row is loaded while
        // the current one is summed (after the last, the same row again, so
        // every step issues the same number of loads)
        auto load_row = [&](int c, u32x4* r) {
            const __amdgpu_buffer_rsrc_t d = buffer_rsrc(w + (size_t)(64 * i + c) * H, (uint32_t)H * 2u);
#pragma unroll
            for (int s = 0; s < kMaxSteps; ++s) r[s] = buffer_load16(d, (uint32_t)(512 * s + 8 * lane) * 2u, 0);
        };
        // fixed-order logit: lane j sums its chunks in ascending h with
        // fused multiply-adds from +0, then p[j] += p[j + s], s = 32..1
        auto logit = [&](int c, const u32x4* r) {
            float p = 0.0f;
#pragma unroll
            for (int s = 0; s < kMaxSteps; ++s)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    p = __builtin_fmaf(bf16_lo(xc[s][q]), bf16_lo(r[s][q]), p);
                    p = __builtin_fmaf(bf16_hi(xc[s][q]), bf16_hi(r[s][q]), p);
                }
#pragma unroll
            for (int s = 32; s >= 1; s >>= 1) p = p + __shfl_xor(p, s);
            float l = __shfl(p, 0);
            if (bias) l = l + bias[64 * i + c];
            if (lane == c) mine = l;
        };
        if (cand) {
            u32x4 ra[kMaxSteps], rb[kMaxSteps];
            int ca = __builtin_ctzll(cand);
            cand &= cand - 1;
            load_row(ca, ra);
            for (;;) {
                const bool hb = cand != 0;
                const int cb = hb ? __builtin_ctzll(cand) : ca;
                if (hb) cand &= cand - 1;
                load_row(cb, rb);
                logit(ca, ra);
                if (!hb) break;
                const bool ha = cand != 0;
                const int cn = ha ? __builtin_ctzll(cand) : cb;
                if (ha) cand &= cand - 1;
                load_row(cn, ra);
                logit(cb, rb);
                if (!ha) break;
                ca = cn;
            }
        }
        if (e_lane < E) logits[(size_t)t * E + e_lane] = mine;
    }
    if (lane == 0) ncand[t] = n_cand;
}

}  // namespace

// Batches of up to kRowsMaxT bf16 tokens take the row kernels: at the R1
// shape (H = 7168, E = 256) a call takes about 10 us against 33 us for the
// tile kernel at T = 1, 23 against 34 us at T = 64, and about the same at
// T = 128.
#ifndef MOE_ROUTE_ROWS_MAX_T
#define MOE_ROUTE_ROWS_MAX_T 64
#endif
constexpr int kRowsMaxT = MOE_ROUTE_ROWS_MAX_T;

moe_status launch_route(const void* x, const void* w, const float* bias, moe_dtype dt, int T, int H,
                        int E, int k, int scoring, int renorm, float* logits, int32_t* ids,
                        float* topk_w, hipStream_t st) {
    if (dt == MOE_BF16 && T <= kRowsMaxT && H % 8 == 0 && H <= 16 * kStep) {
        const int nsteps = (H + kStep - 1) / kStep;
        auto kern = nsteps <= 4    ? route_logits_rows_kernel<4>
                    : nsteps <= 8  ? route_logits_rows_kernel<8>
                    : nsteps <= 14 ? route_logits_rows_kernel<14>
                                   : route_logits_rows_kernel<16>;
        hipLaunchKernelGGL(kern, dim3((E + 3) / 4, T), dim3(256), 0, st, (const uint16_t*)x,
                           (const uint16_t*)w, bias, H, E, logits);
        moe_status s = check_launch("route_logits_rows_kernel");
        if (s != MOE_OK) return s;
        hipLaunchKernelGGL(route_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E, k,
                           scoring, renorm, ids, topk_w);
        return check_launch("route_topk_kernel");
    }
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

// workspace: approximate sums [T][E] | absolute sums [T][E] | max |w| per
// expert [E] | max |x| per token [T] | candidates per token [T] (int32, a
// diagnostic)
size_t route_select_workspace_bytes(int T, int E) {
    return 2 * align_up((size_t)T * E * sizeof(float), 256) + align_up((size_t)E * sizeof(float), 256) +
           2 * align_up((size_t)T * sizeof(int32_t), 256);
}

moe_status launch_route_select(const void* x, const void* w, const float* bias, int T, int H, int E,
                               int k, int scoring, int renorm, int32_t* ids, float* topk_w, void* ws,
                               hipStream_t st) {
    const size_t te = align_up((size_t)T * E * sizeof(float), 256);
    float* approx = (float*)ws;
    float* sabs = (float*)((uint8_t*)ws + te);
    float* wmax = (float*)((uint8_t*)ws + 2 * te);
    float* xmax = (float*)((uint8_t*)ws + 2 * te + align_up((size_t)E * sizeof(float), 256));
    int32_t* ncand = (int32_t*)((uint8_t*)xmax + align_up((size_t)T * sizeof(float), 256));
    hipLaunchKernelGGL(route_approx_kernel,
                       dim3((T + kApproxT - 1) / kApproxT, (E + kApproxE - 1) / kApproxE), dim3(512), 0, st,
                       (const uint16_t*)x, (const uint16_t*)w, T, H, E, approx, sabs, wmax, xmax);
    moe_status s = check_launch("route_approx_kernel");
    if (s != MOE_OK) return s;
    // the smallest register-resident row that holds H (H <= 8192)
    const int nsteps = (H + 511) / 512;
    auto refine = nsteps <= 4 ? route_refine_kernel<4>
                : nsteps <= 8 ? route_refine_kernel<8>
                : nsteps <= 14 ? route_refine_kernel<14> : route_refine_kernel<16>;
    hipLaunchKernelGGL(refine, dim3((T + 3) / 4), dim3(256), 0, st, (const uint16_t*)x,
                       (const uint16_t*)w, bias, T, H, E, k, approx, sabs, wmax, xmax, ncand);
    s = check_launch("route_refine_kernel");
    if (s != MOE_OK) return s;
    hipLaunchKernelGGL(route_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, approx, T, E, k, scoring,
                       renorm, ids, topk_w);
    return check_launch("route_topk_kernel");
}

}  // namespace moe
