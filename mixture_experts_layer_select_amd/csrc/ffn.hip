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
#include "moe_internal.h"

#include <mutex>
#include <type_traits>
#include <vector>

namespace moe {
namespace {

constexpr int kBigTile = 64;  // rows per m-tile of the bf16 kernels (128 measured slower)
#ifndef MOE_BF16_OCC
#define MOE_BF16_OCC 2
#endif
constexpr int kBf16Occ = MOE_BF16_OCC;  // waves per SIMD the bf16 GEMMs are compiled for
constexpr int kBK = 128;     // K per step

// m-tiles: group g's rows [offsets[g], offsets[g+1]) split into tiles of at
// most bm rows (the kernel's tile height); tiles are numbered group after
// group. Every workgroup builds the exclusive prefix of tiles per group in LDS
// once (n_groups <= 1025) and maps a work item to (group, first row, rows) by
// binary search. Rows at or past max_rows are dropped, so inconsistent offsets
// cannot push a row index outside the caller's buffers.
constexpr int kMaxGroups = 1025;

struct MTile {
    int group, row0, rows;
};

__device__ __forceinline__ int clamp_row(int r, int max_rows) {
    return r < 0 ? 0 : (r > max_rows ? max_rows : r);
}

struct TileMap {
    int start[kMaxGroups + 1];  // start[g] = first tile of group g; start[n_groups] = total
    int part[256];
};

// all threads of the block must call; returns the total number of tiles of
// bm rows. Only groups whose row count m satisfies lo < m <= hi get tiles
// (the others get none), so two kernels can split the groups between them.
__device__ int build_tile_map(TileMap& tm, const int32_t* __restrict__ offsets, int n_groups,
                              int max_rows, int bm, int lo = 0, int hi = 0x7fffffff) {
    // every thread of the workgroup calls this (it holds barriers); the first
    // 256 do the work, so any workgroup size >= 256 is fine
    const bool act = threadIdx.x < 256;
    const int per = (n_groups + 255) / 256;
    const int g0 = threadIdx.x * per;
    int local[5];  // per <= 5 since n_groups <= 1025 (+ slack)
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const int g = g0 + i;
        int nt = 0;
        if (act && i < per && g < n_groups) {
            const int m = clamp_row(offsets[g + 1], max_rows) - clamp_row(offsets[g], max_rows);
            nt = m > lo && m <= hi ? (m + bm - 1) / bm : 0;
        }
        local[i] = nt;
        sum += nt;
    }
    if (act) tm.part[threadIdx.x] = sum;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // inclusive Hillis-Steele scan
        const int v = act && threadIdx.x >= off ? tm.part[threadIdx.x - off] : 0;
        __syncthreads();
        if (act) tm.part[threadIdx.x] += v;
        __syncthreads();
    }
    if (act) {
        int run = tm.part[threadIdx.x] - sum;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int g = g0 + i;
            if (i < per && g < n_groups) tm.start[g] = run;
            run += local[i];
        }
        if (threadIdx.x == 255) tm.start[n_groups] = tm.part[255];
    }
    __syncthreads();
    return tm.start[n_groups];
}

__device__ __forceinline__ int group_of(const TileMap& tm, int n_groups, int mt) {
    int lo = 0, hi = n_groups - 1;  // last g with start[g] <= mt
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tm.start[mid] <= mt) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The nt = ceil(m / bm) tiles of a group with m rows split it evenly: tile t
// holds rows [floor(t m / nt), floor((t + 1) m / nt)), between 1 and bm rows.
// Tiles of one group then carry the same work, so the workgroups that share
// an n-block's weights through L2 (item_at) stay in step.
__device__ __forceinline__ MTile make_tile(const TileMap& tm, const int32_t* __restrict__ offsets,
                                           int max_rows, int g, int mt, int bm) {
    MTile t;
    const int r0 = clamp_row(offsets[g], max_rows);
    const int m = clamp_row(offsets[g + 1], max_rows) - r0;
    const int nt = tm.start[g + 1] - tm.start[g];
    const int i = mt - tm.start[g];
    const int a = (int)((long)i * m / nt);
    const int b = (int)((long)(i + 1) * m / nt);
    // the same for every lane: keep it in scalar registers
    t.group = __builtin_amdgcn_readfirstlane(g);
    t.row0 = __builtin_amdgcn_readfirstlane(r0 + a);
    t.rows = __builtin_amdgcn_readfirstlane(b - a);
    return t;
}

__device__ __forceinline__ MTile tile_at(const TileMap& tm, const int32_t* __restrict__ offsets,
                                         int n_groups, int max_rows, int mt, int bm) {
    return make_tile(tm, offsets, max_rows, group_of(tm, n_groups, mt), mt, bm);
}

// Item -> (M tile, n-block) with the M tiles of one n-block of a group
// consecutive: workgroups that run side by side on one XCD then read that
// n-block's weights once from HBM and share them through the XCD's L2. A
// group owns items [start[g]*NB, start[g+1]*NB) in this order as well.
// With panel > 0 a group's items go in panels of `panel` m-tiles (the last
// panel may be shorter): all n-blocks of a panel, its m-tiles fastest. The
// workgroups of one XCD then run a few m-tiles x several n-blocks at once, so
// each K step's activation slice and weight slice are both shared through L2.
__device__ __forceinline__ MTile item_at(const TileMap& tm, const int32_t* __restrict__ offsets,
                                         int n_groups, int max_rows, int item, int NB, int bm,
                                         int& nb, int panel = 0) {
    const int g = group_of(tm, n_groups, item / NB);
    const int t0 = tm.start[g];
    const int tg = tm.start[g + 1] - t0;
    const int local = item - t0 * NB;
    if (panel <= 0 || tg <= panel) {
        nb = __builtin_amdgcn_readfirstlane(local / tg);
        return make_tile(tm, offsets, max_rows, g, t0 + local % tg, bm);
    }
    const int full = tg / panel;
    const int pi = min(local / (panel * NB), full);
    const int ph = pi < full ? panel : tg - full * panel;
    const int idx = local - pi * panel * NB;
    nb = __builtin_amdgcn_readfirstlane(idx / ph);
    return make_tile(tm, offsets, max_rows, g, t0 + pi * panel + idx % ph, bm);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }


__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_fp8(i32x8 a, i32x8 b) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    // format 0 = e4m3 for both operands; E8M0 scale 127 = 1.0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}

// ============================================================================ bf16
// SwiGLU (GEMM-1): W = w13 [G][2I][K=H]; an item covers 64 intermediate columns:
//   wave w owns gate rows n0+16w.. and up rows I+n0+16w.. (n0 = nb*64)
//   out = A [rows][I] bf16 = silu(gate) * up
// Down (GEMM-2): W = w2 [G][H][K=I]; an item covers 128 output columns:
//   wave w owns rows n0+32w.. and n0+32w+16.. (n0 = nb*128); out = y [rows][H]
//
// Items are (m-tile of <= 64 rows, n-block); the 64 x 128 activation tile of
// a K step is shared through LDS by the 4 waves, and each wave reuses its
// weight registers for all m-subtiles, so an expert's weights cross HBM once
// per 64 rows. Pipeline per K step (128): a wave first issues the activation
// loads of step j+1 (4 x 16 B per lane, only for tile rows it owns), then the
// weight loads of step j+2 into a 3-deep register ring (8 x 16 B per lane),
// computes step j, waits for the activations only (the 8 weight loads may
// stay in flight: vmcnt 8), stores them to the other LDS buffer and meets the
// other waves at a bare barrier (no memory fence, which would drain the ring).
// Weight load c of a step reads 64 contiguous bytes of each of the wave's 16
// rows: MFMA c takes k = 32c + 8lk + [0, 8) from lane (li, lk), for the
// weights and the activations alike.
constexpr int kLdsRowBf16 = kBK * 2 + 16;  // bytes per staged activation row (16 B pad)

// s_waitcnt with only the vector-memory counter limited to N (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt, lgkmcnt at max)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// this wave's LDS accesses done (lgkmcnt 0), other counters free
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
// a workgroup barrier without the release/acquire fences of __syncthreads()
__device__ __forceinline__ void barrier_only() {
    wait_lds();
    __builtin_amdgcn_s_barrier();
}

// kW waves per workgroup: 4, or 8 (an item covers twice the weight rows and
// the activation tile, staged by waves 0..3, is shared by twice as many
// waves, so activations are re-read from L2 half as often; the launcher takes
// it when groups are many and small, where there are items enough for it)
template <bool kSwiGLU, int kTM, int kW>
__global__ __launch_bounds__(kW * 64) __attribute__((amdgpu_waves_per_eu(kBf16Occ, kBf16Occ))) void ffn_gemm_bf16_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, const uint16_t* __restrict__ Ws,
    int n_routed, const int32_t* __restrict__ offsets, int n_groups, int max_rows, int K, int Nw,
    int NB, uint16_t* __restrict__ out, int ldo) {
    constexpr int kSub = kTM / 16;    // m-subtiles per tile
    constexpr int kOwn = kTM / 64;    // 16-row pieces of the tile each wave stages
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][kTM * kLdsRowBf16];
    __shared__ TileMap tm;

    const int lane = threadIdx.x & 63;
    // left per-lane: making it wave-uniform measured 10% slower on a 512-token, 32-expert share
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15;
    const int lk = lane >> 4;
    const int nk = K / kBK;
    const int n_items = build_tile_map(tm, offsets, n_groups, max_rows, kTM) * NB;

    // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin
    // (blockIdx % 8); each XCD walks a contiguous slice of the items, so the
    // n-blocks of one m-tile (same activations) share that XCD's L2. If the
    // dealing differs only locality suffers. The grid is a multiple of 8.
    const int xcd = blockIdx.x & 7;
    const int per_xcd = gridDim.x >> 3;
    const int i_lo = (int)((long)n_items * xcd / 8);
    const int i_hi = (int)((long)n_items * (xcd + 1) / 8);

    // per-item addressing: the tile, its weight and activation descriptors and
    // this lane's offsets into them
    struct Ctx {
        MTile tile;
        int nb;
        __amdgpu_buffer_rsrc_t wr, xr;
        uint32_t wa, wb;
        uint32_t xoff[kOwn];
    };
    const int xrow0 = 16 * wave + li;  // activation staging: wave w owns tile rows 16(w + 4q) + [0, 16)
    auto ctx_of = [&](int it) {
        Ctx c;
        c.tile = item_at(tm, offsets, n_groups, max_rows, it, NB, kTM, c.nb);
        const uint16_t* Wg = c.tile.group < n_routed ? W + (size_t)c.tile.group * Nw * K : Ws;
        int ra, rb;
        if (kSwiGLU) {
            ra = c.nb * 16 * kW + 16 * wave + li;
            rb = ra + Nw / 2;
        } else {
            ra = c.nb * 32 * kW + 32 * wave + li;
            rb = ra + 16;
        }
        // buffer loads: 32-bit lane offsets against a scalar descriptor, so no
        // 64-bit VGPR address temporaries, which the register allocator would
        // otherwise carve out of the weight ring (forcing a wait for the ring's
        // loads before the address is written)
        c.wa = ((uint32_t)ra * K + 8 * lk) * 2;
        c.wb = ((uint32_t)rb * K + 8 * lk) * 2;
        c.wr = buffer_rsrc(Wg, clamp_bytes((size_t)Nw * K * 2));
        c.xr = buffer_rsrc(X + (size_t)c.tile.row0 * K, clamp_bytes((size_t)c.tile.rows * K * 2));
#pragma unroll
        for (int q = 0; q < kOwn; ++q) {
            const int xrow = xrow0 + 64 * q;
            const int xrr = xrow < c.tile.rows ? xrow : c.tile.rows - 1;
            c.xoff[q] = ((uint32_t)xrr * K + 8 * lk) * 2;
        }
        return c;
    };

    u32x4 ring[2][2][4];  // weights of steps j (slot j & 1) and j + 1
    u32x4 xr[kOwn][4];
    auto load_w = [&](const Ctx& c, int kc, auto slot_c) {
        constexpr int st = decltype(slot_c)::value;
        kc = kc < nk ? kc : nk - 1;
        const uint32_t ko = (uint32_t)kc * kBK * 2;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            ring[st][0][cc] = buffer_load16(c.wr, c.wa + 64 * cc, ko);
            ring[st][1][cc] = buffer_load16(c.wr, c.wb + 64 * cc, ko);
        }
    };
    auto load_x = [&](const Ctx& c, int kc) {
        kc = kc < nk ? kc : nk - 1;
        const uint32_t ko = (uint32_t)kc * kBK * 2;
#pragma unroll
        for (int q = 0; q < kOwn; ++q)
            if (16 * (wave + 4 * q) < c.tile.rows) {  // rows of this wave inside the tile
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) xr[q][cc] = buffer_load16(c.xr, c.xoff[q] + 64 * cc, ko);
            }
    };
    // unconditional: a wave whose rows lie past the tile stores whatever its
    // registers hold, which no MFMA result that is kept depends on. A
    // guarded store lets the compiler sink the loads into the guarded
    // block, behind the weight loads, and then wait for all of them there.
    auto store_x = [&](int buf) {
#pragma unroll
        for (int q = 0; q < kOwn; ++q) {
            uint8_t* d = &xs[buf][(xrow0 + 64 * q) * kLdsRowBf16];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) *reinterpret_cast<u32x4*>(d + 64 * cc + 16 * lk) = xr[q][cc];
        }
    };
    // waves 0..3 stage the activation tile; waves past them issue only their
    // 8 weight loads a step, so vmcnt(8) does not wait for those either
    const bool stager = kW == 4 || wave < 4;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    // Across items: the last K step of an item issues the next item's step 0
    // (into weight slot 0 and LDS buffer 0 when nk is even), so a workgroup's
    // next item starts with its first operands landed instead of waiting a
    // full memory latency.
    const bool chain = (nk & 1) == 0;
    bool primed = false;  // this item's step 0 was issued by the previous one

    for (int item = i_lo + (blockIdx.x >> 3); item < i_hi; item += per_xcd) {
        const Ctx cur_c = ctx_of(item);
        const bool has_next = chain && item + per_xcd < i_hi;
        const Ctx nxt_c = has_next ? ctx_of(item + per_xcd) : cur_c;
        const MTile tile = cur_c.tile;
        const int nb = cur_c.nb;
        const int nms = (tile.rows + 15) >> 4;

        f32x4 acc_a[kSub], acc_b[kSub];
#pragma unroll
        for (int i = 0; i < kSub; ++i) {
            acc_a[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc_b[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        auto compute = [&](int buf, auto slot_c) {
            constexpr int st = decltype(slot_c)::value;
#pragma unroll
            for (int ms = 0; ms < kSub; ++ms) {
                if (ms < nms) {
                    const uint8_t* row = &xs[buf][(ms * 16 + li) * kLdsRowBf16 + 16 * lk];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const u32x4 b = *reinterpret_cast<const u32x4*>(row + 64 * c);
                        acc_a[ms] = mfma_bf16(ring[st][0][c], b, acc_a[ms]);
                        acc_b[ms] = mfma_bf16(ring[st][1][c], b, acc_b[ms]);
                    }
                }
            }
        };
        // one K step: activations of j+1 first, then weights of j+1 (a 2-deep
        // ring measured faster than 3-deep at two workgroups per CU), compute
        // j, wait for the activations only (the 8 weight loads stay in flight),
        // stage them, barrier. The last step loads the next item's step 0.
        auto step = [&](int j, auto cur, auto nxt) {
            const bool to_next = has_next && j + 1 >= nk;
            const Ctx& lc = to_next ? nxt_c : cur_c;
            const int lk_step = to_next ? 0 : j + 1;
            if (stager) load_x(lc, lk_step);
            load_w(lc, lk_step, nxt);
            __builtin_amdgcn_sched_barrier(0);
            compute(j & 1, cur);
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<8>();
            if (stager) store_x((j + 1) & 1);
            barrier_only();
        };

        if (!primed) {  // prologue: activations and weights of step 0
            if (stager) load_x(cur_c, 0);
            load_w(cur_c, 0, S0{});
            wait_vmcnt<8>();  // the activations (issued first) have landed
            if (stager) store_x(0);
            barrier_only();
        }
        for (int j = 0;; j += 2) {
            step(j, S0{}, S1{});
            if (j + 1 >= nk) break;
            step(j + 1, S1{}, S0{});
            if (j + 2 >= nk) break;
        }
        primed = has_next;
        if (!has_next) wait_vmcnt<0>();  // the clamped tail loads land before registers are reused

        // epilogue: lane holds D[n = base + 4*lk + r][m = ms*16 + li]
#pragma unroll
        for (int ms = 0; ms < kSub; ++ms) {
            const int m = ms * 16 + li;
            if (ms < nms && m < tile.rows) {
                uint16_t* orow = out + (size_t)(tile.row0 + m) * ldo;
                if (kSwiGLU) {
                    const int col = nb * 16 * kW + 16 * wave + 4 * lk;
                    float a0 = silu_mul(acc_a[ms][0], acc_b[ms][0]);
                    float a1 = silu_mul(acc_a[ms][1], acc_b[ms][1]);
                    float a2 = silu_mul(acc_a[ms][2], acc_b[ms][2]);
                    float a3 = silu_mul(acc_a[ms][3], acc_b[ms][3]);
                    *reinterpret_cast<uint2*>(orow + col) =
                        make_uint2(pack_bf16x2(a0, a1), pack_bf16x2(a2, a3));
                } else {
                    const int col = nb * 32 * kW + 32 * wave + 4 * lk;
                    *reinterpret_cast<uint2*>(orow + col) =
                        make_uint2(pack_bf16x2(acc_a[ms][0], acc_a[ms][1]),
                                   pack_bf16x2(acc_a[ms][2], acc_a[ms][3]));
                    *reinterpret_cast<uint2*>(orow + col + 16) =
                        make_uint2(pack_bf16x2(acc_b[ms][0], acc_b[ms][1]),
                                   pack_bf16x2(acc_b[ms][2], acc_b[ms][3]));
                }
            }
        }
    }
}

// ============================================================================ fp8, LDS ring
// Tiles of 256 tokens x 256 weight rows, 8 waves; wave w owns 32 weight rows
// and all 256 tokens, i.e. 2 x 16 blocks of 16x16 accumulators (128 fp32 per
// lane). Weight rows are private to a wave, so they stream from global memory
// straight into a 3-slot register ring (MFMA A operand); the activation tile
// of each K step (128), shared by all waves, arrives by direct global->LDS
// loads (buffer_load_dwordx4 ... lds) into a 3-stage ring, each stage its own
// __shared__ object so the compiler can tell the stage being filled from the
// one being read. Steps j+1 and j+2 are in flight while step j computes.
// Every wave issues the same 5 + NX loads per step (2 weight fragments x 2
// halves, 1 scale piece, NX = 1, 2 or 4 activation pieces of 8 rows by the
// tile's height), so one vmcnt value is exact for all.
// An expert with up to 256 rows streams each weight byte once; larger ones
// run their M tiles of one n-block side by side (item_at) and share it
// through L2.
//   SwiGLU: the item covers intermediate columns nb*128 + [0,128); wave w
//     owns gate rows nb*128 + 16w + [0,16) (s = 0) and the up rows I + the
//     same (s = 1).
//   Down: wave w owns w2 rows nb*256 + 32w + 16s + [0,16).
// Lane (li, lk) holds the 32 codes at bytes 16lk + [0,16) and 64 + 16lk +
// [0,16) of a row's 128-byte step, for weights and activations alike. LDS
// activation rows are 128 bytes; chunk c of row r sits at physical chunk
// c ^ ((r >> 1) & 7), which makes the 16-row operand reads conflict-free.
// Activation scales are K-major ([K/128][max_rows]): one step's scales of a
// tile are one contiguous run.
constexpr int kLTM = 256;         // tokens per tile
constexpr int kLWaves = 8;
constexpr int kLThreads = kLWaves * 64;
constexpr int kLMaxSteps = 128;   // K <= 16384

struct XStage {
    uint8_t x[kLTM * kBK];  // 32 KB
    float xs[2 * kLTM];     // scales of the step: [0,256) used, the rest takes the
                            // duplicate scale loads of waves 4..7
};

// direct global->LDS loads through a buffer descriptor: a 32-bit lane offset
// plus a uniform offset in a scalar register, no 64-bit address per lane
__device__ __forceinline__ void lds_buf16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                          void* l) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)l, 16, voff,
                                             soff, 0, 0);
}
__device__ __forceinline__ void lds_buf4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                         void* l) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)l, 4, voff,
                                             soff, 0, 0);
}
__device__ __forceinline__ int swz(int r, int c) { return (c ^ ((r >> 1) & 7)) * 16; }


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
    __shared__ float wsc[2][kLMaxSteps];  // weight block scales of the item: [block][k step]
    __shared__ float red[kSwiGLU ? kLWaves * kLTM : 1];  // SwiGLU row amax per wave

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15;
    const int lk = lane >> 4;
    const int nk = K / kBK;
    const int n_items = build_tile_map(tm, offsets, n_groups, max_rows, kLTM, 0, kLTM) * NB;
    const int xcd = blockIdx.x & 7;
    const int per_xcd = gridDim.x >> 3;
    const int i_lo = (int)((long)n_items * xcd / 8);
    const int i_hi = (int)((long)n_items * (xcd + 1) / 8);

    for (int item = i_lo + (blockIdx.x >> 3); item < i_hi; item += per_xcd) {
        int nb_v;
        const MTile tile_v = item_at(tm, offsets, n_groups, max_rows, item, NB, kLTM, nb_v);
        // the item is the same for every lane: scalar registers, scalar buffer
        // descriptors and scalar branches on the tile's height
        const int nb = __builtin_amdgcn_readfirstlane(nb_v);
        const MTile tile{__builtin_amdgcn_readfirstlane(tile_v.group),
                         __builtin_amdgcn_readfirstlane(tile_v.row0),
                         __builtin_amdgcn_readfirstlane(tile_v.rows)};
        const bool routed = tile.group < n_routed;
        const uint8_t* Wg = routed ? W + (size_t)tile.group * Nw * K : Wsh;
        const float* Sg = routed ? Wsc + (size_t)tile.group * (Nw / kBK) * nk : Wsh_sc;
        // the two 128-row weight blocks of the item
        const int blk0 = kSwiGLU ? nb : 2 * nb;
        const int blk1 = kSwiGLU ? Nw / 2 / kBK + nb : 2 * nb + 1;
        for (int i = threadIdx.x; i < 2 * nk; i += kLThreads) {
            const int h = i / nk, kc = i % nk;
            wsc[h][kc] = Sg[(size_t)(h ? blk1 : blk0) * nk + kc];
        }
        // Every load goes through a buffer descriptor of the item (scalar) with
        // a 32-bit lane offset fixed for the item and the K step's offset in a
        // scalar register, so the loop computes no per-lane addresses.
        // This wave's weight fragments (A operand):
        uint32_t woff[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int row = kSwiGLU ? s * (Nw / 2) + nb * 128 + 16 * wave + li
                                    : nb * 256 + 32 * wave + 16 * s + li;
            woff[s] = (uint32_t)row * K + 16 * lk;
        }
        const int wblk = kSwiGLU ? 0 : (wave >> 2);  // SwiGLU: s selects the block
        // activation pieces p = 8i + wave hold LDS rows 8p + [0,8); lane: row
        // 8p + lane/8 (clamped to the tile), physical chunk lane%8
        // Activation rows: rows of the tile in x_perm (offsets from the tile's
        // first row), or their tokens' rows in a token buffer (offsets from
        // its start).
        constexpr bool gather = kGather;
        auto src_row = [&](int rr) -> int {
            if (!gather) return rr;
            const int slot = src.row_slot[tile.row0 + rr];
            return slot < src.S ? slot / src.k : slot - src.S;
        };
        uint32_t xoff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (i * 8 + wave) * 8 + (lane >> 3);
            const int rr = r < tile.rows ? r : tile.rows - 1;
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            xoff[i] = (uint32_t)src_row(rr) * K + c * 16;
        }
        // scales: wave w loads rows 64(w%4) + lane (clamped) into xs[64w + lane]
        const int sr = 64 * (wave & 3) + lane;
        const uint32_t soff = (uint32_t)src_row(sr < tile.rows ? sr : tile.rows - 1);
        const int s_ld = gather ? src.s_ld : max_rows;
        const int nms = (tile.rows + 15) >> 4;
        const __amdgpu_buffer_rsrc_t wr_d = buffer_rsrc(Wg, clamp_bytes((size_t)Nw * K));
        const __amdgpu_buffer_rsrc_t xr_d =
            gather ? buffer_rsrc(X, clamp_bytes((size_t)src.rows * K))
                   : buffer_rsrc(X + (size_t)tile.row0 * K, clamp_bytes((size_t)tile.rows * K));
        const __amdgpu_buffer_rsrc_t sr_d =
            gather ? buffer_rsrc(Xs, clamp_bytes(((size_t)(nk - 1) * s_ld + src.rows) * 4))
                   : buffer_rsrc(Xs + tile.row0,
                                 clamp_bytes(((size_t)(nk - 1) * max_rows + tile.rows) * 4));

        u32x8 wr[3][2];
        auto issue = [&](int kc, auto slot_c, XStage& S, auto nx_c) {
            constexpr int sl = decltype(slot_c)::value;
            constexpr int NX = decltype(nx_c)::value;
            kc = kc < nk ? kc : nk - 1;
            const uint32_t ko = (uint32_t)kc * kBK;
#pragma unroll
            for (int i = 0; i < NX; ++i) lds_buf16(xr_d, xoff[i], ko, &S.x[(i * 8 + wave) * 1024]);
            lds_buf4(sr_d, soff * 4, (uint32_t)kc * s_ld * 4, &S.xs[64 * wave]);
#pragma unroll
            for (int s = 0; s < 2; ++s)
                wr[sl][s] = __builtin_shufflevector(buffer_load16(wr_d, woff[s], ko),
                                                    buffer_load16(wr_d, woff[s] + 64, ko), 0, 1, 2, 3,
                                                    4, 5, 6, 7);
        };

        f32x4 acc[2][16];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int ms = 0; ms < 16; ++ms) acc[s][ms] = f32x4{0.f, 0.f, 0.f, 0.f};

        // row 16ms + li of the activation tile: the swizzle ((16ms + li) >> 1) & 7
        // does not depend on ms, so the two 16-byte reads are a per-lane offset
        // plus the immediate ms * 2048
        const int bo0 = li * kBK + ((lk ^ ((li >> 1) & 7)) << 4);
        const int bo1 = li * kBK + (((lk + 4) ^ ((li >> 1) & 7)) << 4);
        auto load_b = [&](const XStage& S, int ms) {
            const uint8_t* base = &S.x[ms * 16 * kBK];
            return __builtin_shufflevector(*reinterpret_cast<const u32x4*>(base + bo0),
                                           *reinterpret_cast<const u32x4*>(base + bo1),
                                           0, 1, 2, 3, 4, 5, 6, 7);
        };
        // token blocks in pairs (a block past the tile's rows computes on the
        // clamped duplicate rows and is never stored); the scheduling barriers
        // keep the compiler from hoisting every B fragment above the
        // 128 accumulators
        auto compute = [&](int kc, auto slot_c, const XStage& S) {
            constexpr int sl = decltype(slot_c)::value;
            // constant first index: the compiler keeps the table apart from the
            // ring (a computed row makes it wait for every load in flight)
            const float g0 = wsc[0][kc], g1 = wsc[1][kc];
            float sw[2];
            sw[0] = kSwiGLU ? g0 : (wblk ? g1 : g0);
            sw[1] = kSwiGLU ? g1 : sw[0];
#pragma unroll
            for (int ms = 0; ms < 16; ms += 2) {
                if (ms < nms) {
                    const u32x8 b0 = load_b(S, ms);
                    const u32x8 b1 = load_b(S, ms + 1);
                    const float sx0 = S.xs[ms * 16 + li];
                    const float sx1 = S.xs[ms * 16 + 16 + li];
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const f32x4 p0 = mfma_fp8(__builtin_bit_cast(i32x8, wr[sl][s]),
                                                  __builtin_bit_cast(i32x8, b0));
                        const f32x4 p1 = mfma_fp8(__builtin_bit_cast(i32x8, wr[sl][s]),
                                                  __builtin_bit_cast(i32x8, b1));
                        const float f0 = sw[s] * sx0, f1 = sw[s] * sx1;
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) {
                            acc[s][ms][r4] = __builtin_fmaf(p0[r4], f0, acc[s][ms][r4]);
                            acc[s][ms + 1][r4] = __builtin_fmaf(p1[r4], f1, acc[s][ms + 1][r4]);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        using S2 = std::integral_constant<int, 2>;

        // A single top-tested loop with guarded steps: exits from the middle of
        // the body make the compiler's wait analysis drain the ring (vmcnt 0)
        // before the first LDS read after the back edge. The analysis also
        // loses track of the ring at the loop header and drains it before the
        // first step of each iteration. Gate/up (56 K steps at R1 size) runs
        // twelve steps per iteration, down (16) six: a longer body makes the
        // drains rarer, but its last iteration issues (clamped, unused) loads
        // for every step past the end.
        // The activation pieces a wave loads per step: 32 pieces of 8 rows cover
        // 256 rows, so a tile of at most 64 (128) rows needs 8 (16) of them,
        // one (two) per wave. Each variant issues the same 5 + NX loads per
        // step in every wave, so its waits stay exact.
        auto run = [&](auto nx_c) {
            constexpr int NX = decltype(nx_c)::value;
            issue(0, S0{}, st0, nx_c);
            issue(1, S1{}, st1, nx_c);
            if constexpr (kSwiGLU) {
                for (int j = 0; j < nk; j += 12) {
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 2, S2{}, st2, nx_c);
                    compute(j, S0{}, st0);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 3, S0{}, st0, nx_c);
                    if (j + 1 < nk) compute(j + 1, S1{}, st1);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 4, S1{}, st1, nx_c);
                    if (j + 2 < nk) compute(j + 2, S2{}, st2);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 5, S2{}, st2, nx_c);
                    if (j + 3 < nk) compute(j + 3, S0{}, st0);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 6, S0{}, st0, nx_c);
                    if (j + 4 < nk) compute(j + 4, S1{}, st1);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 7, S1{}, st1, nx_c);
                    if (j + 5 < nk) compute(j + 5, S2{}, st2);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 8, S2{}, st2, nx_c);
                    if (j + 6 < nk) compute(j + 6, S0{}, st0);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 9, S0{}, st0, nx_c);
                    if (j + 7 < nk) compute(j + 7, S1{}, st1);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 10, S1{}, st1, nx_c);
                    if (j + 8 < nk) compute(j + 8, S2{}, st2);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 11, S2{}, st2, nx_c);
                    if (j + 9 < nk) compute(j + 9, S0{}, st0);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 12, S0{}, st0, nx_c);
                    if (j + 10 < nk) compute(j + 10, S1{}, st1);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 13, S1{}, st1, nx_c);
                    if (j + 11 < nk) compute(j + 11, S2{}, st2);
                }
            } else {
                for (int j = 0; j < nk; j += 6) {
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 2, S2{}, st2, nx_c);
                    compute(j, S0{}, st0);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 3, S0{}, st0, nx_c);
                    if (j + 1 < nk) compute(j + 1, S1{}, st1);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 4, S1{}, st1, nx_c);
                    if (j + 2 < nk) compute(j + 2, S2{}, st2);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 5, S2{}, st2, nx_c);
                    if (j + 3 < nk) compute(j + 3, S0{}, st0);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 6, S0{}, st0, nx_c);
                    if (j + 4 < nk) compute(j + 4, S1{}, st1);
                    wait_vmcnt<5 + NX>();
                    barrier_only();
                    issue(j + 7, S1{}, st1, nx_c);
                    if (j + 5 < nk) compute(j + 5, S2{}, st2);
                }
            }
            wait_vmcnt<0>();
        };
        using X1 = std::integral_constant<int, 1>;
        using X2 = std::integral_constant<int, 2>;
        using X4 = std::integral_constant<int, 4>;
        const int rows_u = __builtin_amdgcn_readfirstlane(tile.rows);
        if (rows_u <= 64)
            run(X1{});
        else if (rows_u <= 128)
            run(X2{});
        else
            run(X4{});
        __syncthreads();  // the ring and wsc are reused below and by the next item

        // epilogue: lane holds D[n = 16-row block s, row 4*lk + r4][m = ms*16 + li]
        // (the token index is made opaque per item: hoisted out of the item loop,
        // its 16 per-block copies would be spilled)
        int li_e = li;
        asm volatile("" : "+v"(li_e));
        if (kSwiGLU) {
#pragma unroll
            for (int ms = 0; ms < 16; ++ms) {
                float mx = 0.f;
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    acc[0][ms][r4] = silu_mul(acc[0][ms][r4], acc[1][ms][r4]);
                    mx = fmaxf(mx, fabsf(acc[0][ms][r4]));
                }
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                if (lk == 0) red[wave * kLTM + ms * 16 + li_e] = mx;
            }
            __syncthreads();
            uint8_t* codes = reinterpret_cast<uint8_t*>(out);
#pragma unroll
            for (int ms = 0; ms < 16; ++ms) {
                const int m = ms * 16 + li_e;
                if (ms < nms && m < tile.rows) {
                    float mx = red[m];
#pragma unroll
                    for (int v = 1; v < kLWaves; ++v) mx = fmaxf(mx, red[v * kLTM + m]);
                    const float sc = block_scale(mx);
                    uint8_t* orow = codes + (size_t)(tile.row0 + m) * ldo;
                    const int col = nb * 128 + 16 * wave + 4 * lk;
                    *reinterpret_cast<uint32_t*>(orow + col) = pack_e4m3x4(
                        clamp_e4m3(acc[0][ms][0] / sc), clamp_e4m3(acc[0][ms][1] / sc),
                        clamp_e4m3(acc[0][ms][2] / sc), clamp_e4m3(acc[0][ms][3] / sc));
                    if (wave == 0 && lk == 0) out_scale[(size_t)nb * max_rows + tile.row0 + m] = sc;
                }
            }
            __syncthreads();
        } else {
            uint16_t* y = reinterpret_cast<uint16_t*>(out);
#pragma unroll
            for (int ms = 0; ms < 16; ++ms) {
                const int m = ms * 16 + li_e;
                if (ms < nms && m < tile.rows) {
                    uint16_t* orow = y + (size_t)(tile.row0 + m) * ldo;
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const int col = nb * 256 + 32 * wave + 16 * s + 4 * lk;
                        *reinterpret_cast<uint2*>(orow + col) =
                            make_uint2(pack_bf16x2(acc[s][ms][0], acc[s][ms][1]),
                                       pack_bf16x2(acc[s][ms][2], acc[s][ms][3]));
                    }
                }
            }
        }
    }
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
            u32x8 bb[8];
            float sxb[8];
            bb[0] = load_b(S, 0);
            sxb[0] = S.xs[wm * 128 + li];
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
                if (ms + 1 < 8) {
                    bb[ms + 1] = load_b(S, ms + 1);
                    sxb[ms + 1] = S.xs[wm * 128 + (ms + 1) * 16 + li];
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
        if (r) return r;
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
        if (r) return r;
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
