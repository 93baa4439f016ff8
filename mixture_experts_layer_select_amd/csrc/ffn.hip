// Expert FFNs as grouped GEMMs with a device-resident row count per group
// ([SGLang-H20] SwapAB GEMM: the per-expert M varies from token to token;
// [Moreh-EP] Library optimization: fused MoE kernel, the shared expert's GEMMs
// joined into the same launch, and kernel selection by problem size).
//
// Work decomposition. expert_offsets (device) define m-tiles per group; a
// persistent grid walks the (m-tile, n-block) work items. Every workgroup
// builds the tile map in LDS from the offsets, so there is no host sync.
//
// bf16 (ffn_gemm_bf16_kernel): 64-row m-tiles, 4 or 8 waves. The activation tile
//   of each K step (128) is staged in LDS, double buffered, and shared by the
//   waves; each wave streams its own weight rows from HBM into registers one
//   step ahead of v_mfma_f32_16x16x32_bf16. Weights are the A operand (16 rows
//   of N), tokens B (16 rows of M): m-subtiles past a group's rows are
//   skipped, so a sparsely hit expert costs one 16-row MFMA side.
// fp8, groups of at most 256 rows (ffn_gemm_fp8_lds_kernel): the whole group
//   is one tile, so its weights cross HBM once; weights stream into a
//   register ring per wave, activations through a 3-stage LDS ring filled by
//   direct global->LDS loads.
// fp8, larger groups (ffn_gemm_fp8_big_kernel, a second launch): 256 x 256
//   tiles with both operands through a 2-stage LDS ring (buffer loads into
//   LDS), MFMA-bound. Items go in panels of 4 m-tiles x all n-blocks, so the
//   workgroups of one XCD share both operands' K slices through L2; inside a
//   K step each 16-token block's operand is read from LDS one block ahead and
//   the fp32 scaling of each product runs under the next MFMA.
// fp8 MFMAs are v_mfma_scale_f32_16x16x128_f8f6f4 with unit E8M0 scales, one
//   per K step of 128 = one 128x128 weight block and one 1x128 activation
//   block; the fp32 block scales multiply each partial product.
//
// The lane -> K assignment of the loaded pieces is a permutation of the K
// step; A and B use the same one, so the dot products are unchanged.
#include "ffn_dev.h"

#include <mutex>
#include <type_traits>
#include <vector>

namespace moe {
namespace {

template <bool kSwiGLU, int kTM, int kW>
__global__ __launch_bounds__(kW * 64) __attribute__((amdgpu_waves_per_eu(kBf16Occ, kBf16Occ))) void ffn_gemm_bf16_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, const uint16_t* __restrict__ Ws,
    int n_routed, const int32_t* __restrict__ offsets, int n_groups, int max_rows, int K, int Nw,
    int NB, uint16_t* __restrict__ out, int ldo) {
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][kTM * kLdsRowBf16];
    __shared__ TileMap tm;
    ffn_gemm_bf16_body<kSwiGLU, kTM, kW>(X, W, Ws, n_routed, offsets, n_groups, max_rows, K, Nw, NB, out,
                                         ldo, xs, tm, blockIdx.x, gridDim.x);
}

template <bool kSwiGLU, bool kGather>
__global__ __launch_bounds__(kLThreads) void ffn_gemm_fp8_lds_kernel(
    const uint8_t* __restrict__ X, const float* __restrict__ Xs, const uint8_t* __restrict__ W,
    const float* __restrict__ Wsc, const uint8_t* __restrict__ Wsh, const float* __restrict__ Wsh_sc,
    int n_routed, const int32_t* __restrict__ offsets, int n_groups, int max_rows, int K, int Nw,
    int NB, void* __restrict__ out, float* __restrict__ out_scale, int ldo, ActSrc src) {
    __shared__ __attribute__((aligned(1024))) XStage st0;
    __shared__ __attribute__((aligned(1024))) XStage st1;
    __shared__ __attribute__((aligned(1024))) XStage st2;
    __shared__ TileMap tm;
    __shared__ float wsc[2][kLMaxSteps];
    __shared__ float red[kSwiGLU ? kLWaves * kLTM : 1];
    ffn_gemm_fp8_lds_body<kSwiGLU, kGather>(X, Xs, W, Wsc, Wsh, Wsh_sc, n_routed, offsets, n_groups,
                                            max_rows, K, Nw, NB, out, out_scale, ldo, src, st0, st1, st2,
                                            tm, wsc, red, blockIdx.x, gridDim.x);
}

// ============================================================================ fp8, large groups
// Groups of more than 256 rows are compute-bound: tiles of 256 tokens x 256
// weight rows with both operand tiles of each K step arriving by direct
// global->LDS loads into one of two stages (distinct __shared__ objects);
// the next step's loads overlap the current step's MFMAs. 8 waves in a 2 x 4
// grid: wave (wm, wn) owns tokens wm*128 + [0,128) and 64 weight rows,
// 8 x 4 blocks of 16x16 accumulators, so each weight row is read from LDS by
// 2 waves and each activation row by 4 (fewer LDS bytes per MFMA than one
// wave per 32 weight rows). Every wait drains the wave's loads (vmcnt 0), so
// the number of loads may differ between waves: activation pieces beyond the
// tile's rows are skipped.
//   SwiGLU: LDS weight rows q < 128 are gate rows nb*128 + q, q >= 128 the up
//     rows I + nb*128 + q - 128; wave wn owns gate q = 32wn + [0,32) (s = 0, 1)
//     and the up rows 128 + the same (s = 2, 3).
//   Down: q -> w2 row nb*256 + q; wave wn owns q = 64wn + 16s + [0,16).
// LDS rows are 128 bytes; chunk c of row q sits at physical chunk
// c ^ ((q >> 1) & 7).
constexpr int kGTM = 256;  // tokens per tile
constexpr int kGTN = 256;  // weight rows per tile
#ifndef MOE_GPANEL
#define MOE_GPANEL 4
#endif
constexpr int kGPanel = MOE_GPANEL;  // m-tiles per item panel

struct BigStage {
    uint8_t w[kGTN * kBK];  // 32 KB
    uint8_t x[kGTM * kBK];  // 32 KB
    float xs[kGTM];         // activation scales of the step
};

template <bool kSwiGLU, bool kGather>
__global__ __launch_bounds__(kLThreads) void ffn_gemm_fp8_big_kernel(
    const uint8_t* __restrict__ X, const float* __restrict__ Xs, const uint8_t* __restrict__ W,
    const float* __restrict__ Wsc, const uint8_t* __restrict__ Wsh, const float* __restrict__ Wsh_sc,
    int n_routed, const int32_t* __restrict__ offsets, int n_groups, int max_rows, int K, int Nw,
    int NB, void* __restrict__ out, float* __restrict__ out_scale, int ldo, ActSrc src) {
    __shared__ __attribute__((aligned(1024))) BigStage st0;
    __shared__ __attribute__((aligned(1024))) BigStage st1;
    __shared__ TileMap tm;
    __shared__ float wsc[2][kLMaxSteps];  // weight block scales of the item: [block][k step]
    __shared__ float red[kSwiGLU ? 4 * kGTM : 1];  // SwiGLU row amax per weight quarter

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15;
    const int lk = lane >> 4;
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int nk = K / kBK;
    const int n_items = build_tile_map(tm, offsets, n_groups, max_rows, kGTM, kLTM) * NB;
    const int xcd = blockIdx.x & 7;
    const int per_xcd = gridDim.x >> 3;
    const int i_lo = (int)((long)n_items * xcd / 8);
    const int i_hi = (int)((long)n_items * (xcd + 1) / 8);

    for (int item = i_lo + (blockIdx.x >> 3); item < i_hi; item += per_xcd) {
        int nb_v;
        const MTile tile_v = item_at(tm, offsets, n_groups, max_rows, item, NB, kGTM, nb_v, kGPanel);
        // the item is the same for every lane: scalar registers, and scalar
        // branches on the tile's height
        const int nb = __builtin_amdgcn_readfirstlane(nb_v);
        const MTile tile{__builtin_amdgcn_readfirstlane(tile_v.group),
                         __builtin_amdgcn_readfirstlane(tile_v.row0),
                         __builtin_amdgcn_readfirstlane(tile_v.rows)};
        const bool routed = tile.group < n_routed;
        const uint8_t* Wg = routed ? W + (size_t)tile.group * Nw * K : Wsh;
        const float* Sg = routed ? Wsc + (size_t)tile.group * (Nw / kBK) * nk : Wsh_sc;
        const int blk0 = kSwiGLU ? nb : 2 * nb;
        const int blk1 = kSwiGLU ? Nw / 2 / kBK + nb : 2 * nb + 1;
        for (int i = threadIdx.x; i < 2 * nk; i += kLThreads) {
            const int h = i / nk, kc = i % nk;
            wsc[h][kc] = Sg[(size_t)(h ? blk1 : blk0) * nk + kc];
        }
        // piece p = 8i + wave holds LDS rows 8p + [0,8) of both operands; lane:
        // row 8p + lane/8, physical chunk lane%8
        // piece i covers LDS rows q0 + 64i with q0 = 8*wave + lane/8; the
        // swizzled chunk c depends on q0 only. Piece i's weight row is piece
        // 0's plus a uniform distance (64 rows, or the gate->up distance for
        // SwiGLU's upper half), and its activation row is recomputed at issue
        // time, so one lane offset of each kind stays live through the loop
        const int q0 = wave * 8 + (lane >> 3);
        const int c16 = ((lane & 7) ^ ((q0 >> 1) & 7)) * 16;
        // kGather: activation rows are the tokens' rows of a token buffer,
        // token = slot < S ? slot / k : slot - S for slot = row_slot[row];
        // their four lane offsets are fixed for the item
        auto src_row = [&](int rr) -> int {
            const int slot = src.row_slot[tile.row0 + rr];
            return slot < src.S ? slot / src.k : slot - src.S;
        };
        uint32_t xg[kGather ? 4 : 1];
        if constexpr (kGather) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = q0 + 64 * i;
                xg[i] = (uint32_t)src_row(r < tile.rows ? r : tile.rows - 1) * K + c16;
            }
        }
        const int s_ld = kGather ? src.s_ld : max_rows;
        const __amdgpu_buffer_rsrc_t wr_d = buffer_rsrc(Wg, clamp_bytes((size_t)Nw * K));
        const __amdgpu_buffer_rsrc_t xr_d =
            kGather ? buffer_rsrc(X, clamp_bytes((size_t)src.rows * K))
                    : buffer_rsrc(X + (size_t)tile.row0 * K, clamp_bytes((size_t)tile.rows * K));
        const __amdgpu_buffer_rsrc_t sr_d =
            kGather ? buffer_rsrc(Xs, clamp_bytes(((size_t)(nk - 1) * s_ld + src.rows) * 4))
                    : buffer_rsrc(Xs + tile.row0,
                                  clamp_bytes(((size_t)(nk - 1) * max_rows + tile.rows) * 4));
        const uint32_t woff0 = (uint32_t)(kSwiGLU ? nb * 128 + q0 : nb * 256 + q0) * K + c16;
        auto wdist = [&](int i) -> uint32_t {  // uniform: piece i's weight row - piece 0's
            if (kSwiGLU) return (uint32_t)(i < 2 ? 64 * i : Nw / 2 + 64 * (i - 2)) * K;
            return (uint32_t)(64 * i) * K;
        };
        // scales: waves 0..3 load rows 64w + lane (clamped to the tile)
        const int sr = 64 * wave + lane;
        const int sr_c = sr < tile.rows ? sr : tile.rows - 1;
        const uint32_t soff = (uint32_t)(kGather ? src_row(sr_c) : sr_c) * 4;
        const bool s_on = wave < 4 && 64 * wave < tile.rows;
        const int nms = max(0, min(8, (tile.rows - wm * 128 + 15) >> 4));

        auto issue = [&](int kc, BigStage& S) {
            const uint32_t ko = (uint32_t)kc * kBK;
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_buf16(wr_d, woff0, wdist(i) + ko, &S.w[(i * 8 + wave) * 1024]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (64 * i + 8 * wave < tile.rows) {
                    const int r = q0 + 64 * i;
                    const uint32_t xo =
                        kGather ? xg[i] : (uint32_t)(r < tile.rows ? r : tile.rows - 1) * K + c16;
                    lds_buf16(xr_d, xo, ko, &S.x[(i * 8 + wave) * 1024]);
                }
            if (s_on) lds_buf4(sr_d, soff, (uint32_t)kc * s_ld * 4, &S.xs[64 * wave]);
        };

        f32x4 acc[4][8];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int ms = 0; ms < 8; ++ms) acc[s][ms] = f32x4{0.f, 0.f, 0.f, 0.f};

        // activation row wm*128 + 16ms + li: its swizzle depends on li only
        const int bo0 = (wm * 128 + li) * kBK + ((lk ^ ((li >> 1) & 7)) << 4);
        const int bo1 = (wm * 128 + li) * kBK + (((lk + 4) ^ ((li >> 1) & 7)) << 4);
        auto load_b = [&](const BigStage& S, int ms) {
            const uint8_t* base = &S.x[ms * 16 * kBK];
            return __builtin_shufflevector(*reinterpret_cast<const u32x4*>(base + bo0),
                                           *reinterpret_cast<const u32x4*>(base + bo1), 0, 1, 2, 3,
                                           4, 5, 6, 7);
        };
        // Over the 16-token blocks ms of a K step: block ms+1's activation
        // fragment is read from LDS while block ms's MFMAs run, and each
        // product is scaled into its accumulator while the next MFMA runs.
        // Rows past the tile read stale LDS bytes whose products are never
        // kept.
        auto compute = [&](int kc, const BigStage& S) {
            if (nms == 0) return;
            u32x8 a[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int q = kSwiGLU ? (s >> 1) * 128 + 32 * wn + 16 * (s & 1) + li : 64 * wn + 16 * s + li;
                const uint8_t* row = &S.w[q * kBK];
                a[s] = __builtin_shufflevector(*reinterpret_cast<const u32x4*>(row + swz(q, lk)),
                                               *reinterpret_cast<const u32x4*>(row + swz(q, lk + 4)),
                                               0, 1, 2, 3, 4, 5, 6, 7);
            }
            // constant first index: the compiler keeps the table apart from the ring.
            // Weight scale of block s: SwiGLU g0 for gate (s < 2), g1 for up;
            // down: one block per wave pair
            const float g0 = wsc[0][kc], g1 = wsc[1][kc];
            const float gd = (wn >> 1) ? g1 : g0;
            auto wsc_of = [&](int s) { return kSwiGLU ? ((s >> 1) ? g1 : g0) : gd; };
            // activation fragments are read kAhead blocks ahead; gate/up keeps
            // its MFMA/scaling interleave below, which measured faster there,
            // while the down GEMM runs 4% faster two blocks ahead and left to
            // the compiler's own schedule
            constexpr int kAhead = kSwiGLU ? 1 : 2;
            u32x8 bb[8];
            float sxb[8];
#pragma unroll
            for (int ms = 0; ms < kAhead; ++ms) {
                bb[ms] = load_b(S, ms);
                sxb[ms] = S.xs[wm * 128 + ms * 16 + li];
            }
            // Every 16-token block is computed: in this launch every tile has
            // more than 128 rows, so the waves of the first token half (wm = 0)
            // always run 8 blocks, and the barrier of each K step waits for
            // them; the second half's blocks past the tile cost no time
            // (those waves sit on other SIMDs) and their rows are never kept.
            // The last product of block ms is scaled under block ms+1's first
            // MFMA, so no scaling waits on the MFMA just issued. Per block:
            // MFMA 0, (scale factors, scaling of the previous block's product
            // 3), MFMA 1, scaling of 0, MFMA 2, of 1, MFMA 3, of 2.
            f32x4 pend;
            float f_pend = 0.f;
#pragma unroll
            for (int ms = 0; ms < 8; ++ms) {
                if (ms + kAhead < 8) {
                    bb[ms + kAhead] = load_b(S, ms + kAhead);
                    sxb[ms + kAhead] = S.xs[wm * 128 + (ms + kAhead) * 16 + li];
                }
                f32x4 p[4];
                p[0] = mfma_fp8(__builtin_bit_cast(i32x8, a[0]), __builtin_bit_cast(i32x8, bb[ms]));
                const float f_lo = wsc_of(0) * sxb[ms], f_hi = wsc_of(2) * sxb[ms];
                if (ms > 0) {
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4)
                        acc[3][ms - 1][r4] = __builtin_fmaf(pend[r4], f_pend, acc[3][ms - 1][r4]);
                }
#pragma unroll
                for (int s = 1; s < 4; ++s) {
                    p[s] = mfma_fp8(__builtin_bit_cast(i32x8, a[s]), __builtin_bit_cast(i32x8, bb[ms]));
                    const float f = s - 1 < 2 ? f_lo : f_hi;
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4)
                        acc[s - 1][ms][r4] = __builtin_fmaf(p[s - 1][r4], f, acc[s - 1][ms][r4]);
                }
                pend = p[3];
                f_pend = f_hi;
                if constexpr (kSwiGLU) {
                    if (ms + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (ms > 0)
                        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                    else
                        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) acc[3][7][r4] = __builtin_fmaf(pend[r4], f_pend, acc[3][7][r4]);
        };

        issue(0, st0);
        for (int j = 0; j < nk; j += 2) {
            wait_vmcnt<0>();
            barrier_only();
            if (j + 1 < nk) issue(j + 1, st1);
            compute(j, st0);
            wait_vmcnt<0>();
            barrier_only();
            if (j + 2 < nk) issue(j + 2, st0);
            if (j + 1 < nk) compute(j + 1, st1);
        }
        __syncthreads();  // the stages and wsc are reused by the next item

        // epilogue: lane holds D[n = q0(s) + 4*lk + r4][m = wm*128 + ms*16 + li]
        if (kSwiGLU) {
#pragma unroll
            for (int ms = 0; ms < 8; ++ms) {
                float mx = 0.f;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        acc[h][ms][r4] = silu_mul(acc[h][ms][r4], acc[2 + h][ms][r4]);
                        mx = fmaxf(mx, fabsf(acc[h][ms][r4]));
                    }
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                if (lk == 0) red[wn * kGTM + wm * 128 + ms * 16 + li] = mx;
            }
            __syncthreads();
            uint8_t* codes = reinterpret_cast<uint8_t*>(out);
#pragma unroll
            for (int ms = 0; ms < 8; ++ms) {
                const int m = wm * 128 + ms * 16 + li;
                if (ms < nms && m < tile.rows) {
                    float mx = red[m];
#pragma unroll
                    for (int v = 1; v < 4; ++v) mx = fmaxf(mx, red[v * kGTM + m]);
                    const float sc = block_scale(mx);
                    uint8_t* orow = codes + (size_t)(tile.row0 + m) * ldo;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int col = nb * 128 + 32 * wn + 16 * h + 4 * lk;
                        *reinterpret_cast<uint32_t*>(orow + col) = pack_e4m3x4(
                            clamp_e4m3(acc[h][ms][0] / sc), clamp_e4m3(acc[h][ms][1] / sc),
                            clamp_e4m3(acc[h][ms][2] / sc), clamp_e4m3(acc[h][ms][3] / sc));
                    }
                    if (wn == 0 && lk == 0) out_scale[(size_t)nb * max_rows + tile.row0 + m] = sc;
                }
            }
            __syncthreads();
        } else {
            uint16_t* y = reinterpret_cast<uint16_t*>(out);
#pragma unroll
            for (int ms = 0; ms < 8; ++ms) {
                const int m = wm * 128 + ms * 16 + li;
                if (ms < nms && m < tile.rows) {
                    uint16_t* orow = y + (size_t)(tile.row0 + m) * ldo;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int col = nb * 256 + 64 * wn + 16 * s + 4 * lk;
                        *reinterpret_cast<uint2*>(orow + col) =
                            make_uint2(pack_bf16x2(acc[s][ms][0], acc[s][ms][1]),
                                       pack_bf16x2(acc[s][ms][2], acc[s][ms][3]));
                    }
                }
            }
        }
    }
}

// ============================================================================ fp32
// Plain VALU kernels for fp32 layers (small shapes): one thread per output.
__device__ __forceinline__ int group_of(const int32_t* offsets, int n_groups, int r) {
    int g = 0;
    while (g + 1 < n_groups && offsets[g + 1] <= r) ++g;
    return g;
}

__global__ void ffn_gemm1_f32_kernel(const float* __restrict__ X, const float* __restrict__ W,
                                     const float* __restrict__ Ws, int n_routed,
                                     const int32_t* __restrict__ offsets, int n_groups, int max_rows,
                                     int H, int I, float* __restrict__ A) {
    const long n = (long)min(offsets[n_groups], max_rows) * I;
    for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (long)gridDim.x * blockDim.x) {
        const int r = (int)(idx / I), i = (int)(idx % I);
        const int g = group_of(offsets, n_groups, r);
        const float* Wg = g < n_routed ? W + (size_t)g * 2 * I * H : Ws;
        const float* x = X + (size_t)r * H;
        float gs = 0.f, us = 0.f;
        for (int h = 0; h < H; ++h) {
            gs = __builtin_fmaf(x[h], Wg[(size_t)i * H + h], gs);
            us = __builtin_fmaf(x[h], Wg[(size_t)(I + i) * H + h], us);
        }
        A[idx] = silu_mul(gs, us);
    }
}

__global__ void ffn_gemm2_f32_kernel(const float* __restrict__ A, const float* __restrict__ W,
                                     const float* __restrict__ Ws, int n_routed,
                                     const int32_t* __restrict__ offsets, int n_groups, int max_rows,
                                     int H, int I, float* __restrict__ Y) {
    const long n = (long)min(offsets[n_groups], max_rows) * H;
    for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (long)gridDim.x * blockDim.x) {
        const int r = (int)(idx / H), h = (int)(idx % H);
        const int g = group_of(offsets, n_groups, r);
        const float* Wg = g < n_routed ? W + (size_t)g * H * I : Ws;
        const float* a = A + (size_t)r * I;
        float y = 0.f;
        for (int i = 0; i < I; ++i) y = __builtin_fmaf(a[i], Wg[(size_t)h * I + i], y);
        Y[idx] = y;
    }
}

struct FfnWs {
    void* a;        // intermediate activations A [max_rows][I]
    float* a_scale; // fp8 only: [I/128][max_rows] (K-major)
    size_t bytes;
};

FfnWs carve(const moe_expert_weights* w, int max_rows, void* base) {
    size_t off = 0;
    FfnWs r{};
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes, 256);
        return base ? (void*)((uint8_t*)base + o) : nullptr;
    };
    size_t eb = w->dt == MOE_F32 ? 4 : w->dt == MOE_BF16 ? 2 : 1;
    r.a = take((size_t)max_rows * w->I * eb);
    r.a_scale = w->dt == MOE_FP8_E4M3 ? (float*)take((size_t)max_rows * (w->I / kBK) * 4) : nullptr;
    r.bytes = off > 0 ? off : 256;
    return r;
}

// 8-wave bf16 workgroups when the groups are many and small (at most 32
// rows per group on average over the buffer bound, as in decode with all
// experts local): items stay plentiful at twice the width. Otherwise, or when
// H is not a multiple of 256 (the down GEMM's 256-row n-blocks), 4 waves.
bool bf16_wide(const moe_expert_weights* w, int max_rows, int n_groups) {
    return w->H % 256 == 0 && w->I % 128 == 0 && max_rows <= 32L * n_groups;
}

int persistent_grid(long bound, int per_cu) {
    const long cap = (long)device_info().cu_count * per_cu;
    long g = bound < cap ? bound : cap;
    return (int)(g > 0 ? g : 1);
}

// persistent grid rounded up to a multiple of the 8 XCDs
int persistent_grid_xcd(long bound, int per_cu) {
    const int g = persistent_grid(bound, per_cu);
    return (g + 7) / 8 * 8;
}

}  // namespace

size_t ffn_workspace_bytes(const moe_expert_weights* w, int max_rows) {
    return carve(w, max_rows, nullptr).bytes;
}

// Scratch of moe_expert_ffn_noalloc: the intermediate A (and its fp8 scales)
// in a file-scope device array, so that entry point calls no allocator. Each
// GPU holds its own copy for the life of the process. In host code the
// array's name only stands in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

moe_status ffn_noalloc_scratch(void** ptr) {
    static std::mutex mu;
    static std::vector<void*> per_device;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_error(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(mu);
    if ((int)per_device.size() <= dev) per_device.resize(dev + 1, nullptr);
    if (!per_device[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return set_error(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                             hipGetErrorString(e));
        per_device[dev] = p;
    }
    *ptr = per_device[dev];
    return MOE_OK;
}

moe_status launch_ffn_gate_up(const moe_expert_weights* w, const void* x_perm,
                              const float* x_perm_scale, const int32_t* offsets, int n_groups,
                              int max_rows, void* ws, hipStream_t st, const ActSrc& src) {
    if (src.row_slot && w->dt != MOE_FP8_E4M3)
        return set_error(MOE_ERR_UNSUPPORTED, "gate/up from token rows: fp8 only");
    FfnWs s = carve(w, max_rows, ws);
    const int H = w->H, I = w->I, E = w->E_local;
    if (w->dt == MOE_F32) {
        const int blocks = persistent_grid(((long)max_rows * I + 255) / 256, 8);
        hipLaunchKernelGGL(ffn_gemm1_f32_kernel, dim3(blocks), dim3(256), 0, st, (const float*)x_perm,
                           (const float*)w->w13, (const float*)w->ws13, E, offsets, n_groups, max_rows,
                           H, I, (float*)s.a);
        return check_launch("ffn_gemm1_f32_kernel");
    }
    if (w->dt == MOE_BF16) {
        const long tiles = (long)(max_rows + kBigTile - 1) / kBigTile + n_groups;
        if (bf16_wide(w, max_rows, n_groups)) {
            const int NB = I / (16 * 8);
            hipLaunchKernelGGL((ffn_gemm_bf16_kernel<true, kBigTile, 8>),
                               dim3(persistent_grid_xcd(tiles * NB, kBf16Occ / 2)), dim3(8 * 64), 0, st,
                               (const uint16_t*)x_perm, (const uint16_t*)w->w13, (const uint16_t*)w->ws13,
                               E, offsets, n_groups, max_rows, H, 2 * I, NB, (uint16_t*)s.a, I);
        } else {
            const int NB = I / (16 * 4);
            hipLaunchKernelGGL((ffn_gemm_bf16_kernel<true, kBigTile, 4>),
                               dim3(persistent_grid_xcd(tiles * NB, kBf16Occ)), dim3(4 * 64), 0, st,
                               (const uint16_t*)x_perm, (const uint16_t*)w->w13, (const uint16_t*)w->ws13,
                               E, offsets, n_groups, max_rows, H, 2 * I, NB, (uint16_t*)s.a, I);
        }
        return check_launch("ffn_gemm_bf16_kernel<gate_up>");
    }
    const int NB = I / 128;
    if (H / kBK <= kLMaxSteps) {  // LDS-ring kernels: the item's weight scales fit the step table
        // groups of at most 256 rows (one tile each), then the larger ones
        if (src.row_slot)
            hipLaunchKernelGGL((ffn_gemm_fp8_lds_kernel<true, true>),
                               dim3(persistent_grid_xcd((long)n_groups * NB, 1)), dim3(kLThreads), 0, st,
                               (const uint8_t*)x_perm, x_perm_scale, (const uint8_t*)w->w13,
                               w->w13_scale, (const uint8_t*)w->ws13, w->ws13_scale, E, offsets,
                               n_groups, max_rows, H, 2 * I, NB, s.a, s.a_scale, I, src);
        else
            hipLaunchKernelGGL((ffn_gemm_fp8_lds_kernel<true, false>),
                               dim3(persistent_grid_xcd((long)n_groups * NB, 1)), dim3(kLThreads), 0, st,
                               (const uint8_t*)x_perm, x_perm_scale, (const uint8_t*)w->w13,
                               w->w13_scale, (const uint8_t*)w->ws13, w->ws13_scale, E, offsets,
                               n_groups, max_rows, H, 2 * I, NB, s.a, s.a_scale, I, src);
        moe_status r = check_launch("ffn_gemm_fp8_lds_kernel<gate_up>");
        if (r || max_rows <= kLTM) return r;  // no group can exceed the buffer's rows
        const long tl = 2L * max_rows / kGTM + 1;  // tiles of groups above 256 rows
        if (src.row_slot)
            hipLaunchKernelGGL((ffn_gemm_fp8_big_kernel<true, true>), dim3(persistent_grid_xcd(tl * NB, 1)),
                               dim3(kLThreads), 0, st, (const uint8_t*)x_perm, x_perm_scale,
                               (const uint8_t*)w->w13, w->w13_scale, (const uint8_t*)w->ws13,
                               w->ws13_scale, E, offsets, n_groups, max_rows, H, 2 * I, NB, s.a,
                               s.a_scale, I, src);
        else
            hipLaunchKernelGGL((ffn_gemm_fp8_big_kernel<true, false>), dim3(persistent_grid_xcd(tl * NB, 1)),
                               dim3(kLThreads), 0, st, (const uint8_t*)x_perm, x_perm_scale,
                               (const uint8_t*)w->w13, w->w13_scale, (const uint8_t*)w->ws13,
                               w->ws13_scale, E, offsets, n_groups, max_rows, H, 2 * I, NB, s.a,
                               s.a_scale, I, src);
        return check_launch("ffn_gemm_fp8_big_kernel<gate_up>");
    }
    return set_error(MOE_ERR_UNSUPPORTED, "fp8 gate/up: H=%d exceeds %d", H, kLMaxSteps * kBK);
}

moe_status launch_ffn_down(const moe_expert_weights* w, const int32_t* offsets, int n_groups,
                           int max_rows, void* y_perm, void* ws, hipStream_t st) {
    FfnWs s = carve(w, max_rows, ws);
    const int H = w->H, I = w->I, E = w->E_local;
    if (w->dt == MOE_F32) {
        const int blocks = persistent_grid(((long)max_rows * H + 255) / 256, 8);
        hipLaunchKernelGGL(ffn_gemm2_f32_kernel, dim3(blocks), dim3(256), 0, st, (const float*)s.a,
                           (const float*)w->w2, (const float*)w->ws2, E, offsets, n_groups, max_rows,
                           H, I, (float*)y_perm);
        return check_launch("ffn_gemm2_f32_kernel");
    }
    if (w->dt == MOE_BF16) {
        const long tiles = (long)(max_rows + kBigTile - 1) / kBigTile + n_groups;
        if (bf16_wide(w, max_rows, n_groups)) {
            const int NB = H / (32 * 8);
            hipLaunchKernelGGL((ffn_gemm_bf16_kernel<false, kBigTile, 8>),
                               dim3(persistent_grid_xcd(tiles * NB, kBf16Occ / 2)), dim3(8 * 64), 0, st,
                               (const uint16_t*)s.a, (const uint16_t*)w->w2, (const uint16_t*)w->ws2, E,
                               offsets, n_groups, max_rows, I, H, NB, (uint16_t*)y_perm, H);
        } else {
            const int NB = H / (32 * 4);
            hipLaunchKernelGGL((ffn_gemm_bf16_kernel<false, kBigTile, 4>),
                               dim3(persistent_grid_xcd(tiles * NB, kBf16Occ)), dim3(4 * 64), 0, st,
                               (const uint16_t*)s.a, (const uint16_t*)w->w2, (const uint16_t*)w->ws2, E,
                               offsets, n_groups, max_rows, I, H, NB, (uint16_t*)y_perm, H);
        }
        return check_launch("ffn_gemm_bf16_kernel<down>");
    }
    const int NB = H / 256;
    if (I / kBK <= kLMaxSteps) {
        hipLaunchKernelGGL((ffn_gemm_fp8_lds_kernel<false, false>), dim3(persistent_grid_xcd((long)n_groups * NB, 1)),
                           dim3(kLThreads), 0, st, (const uint8_t*)s.a, s.a_scale, (const uint8_t*)w->w2,
                           w->w2_scale, (const uint8_t*)w->ws2, w->ws2_scale, E, offsets, n_groups,
                           max_rows, I, H, NB, y_perm, nullptr, H, ActSrc{nullptr, 0, 0, 0, 0});
        moe_status r = check_launch("ffn_gemm_fp8_lds_kernel<down>");
        if (r || max_rows <= kLTM) return r;
        const long tl = 2L * max_rows / kGTM + 1;
        hipLaunchKernelGGL((ffn_gemm_fp8_big_kernel<false, false>), dim3(persistent_grid_xcd(tl * NB, 1)),
                           dim3(kLThreads), 0, st, (const uint8_t*)s.a, s.a_scale, (const uint8_t*)w->w2,
                           w->w2_scale, (const uint8_t*)w->ws2, w->ws2_scale, E, offsets, n_groups,
                           max_rows, I, H, NB, y_perm, nullptr, H, ActSrc{nullptr, 0, 0, 0, 0});
        return check_launch("ffn_gemm_fp8_big_kernel<down>");
    }
    return set_error(MOE_ERR_UNSUPPORTED, "fp8 down: I=%d exceeds %d", I, kLMaxSteps * kBK);
}

}  // namespace moe
