// Device code of the grouped expert GEMMs (tile maps, the bf16 GEMM and the
// fp8 GEMM for groups of at most 256 rows, as functions of a workgroup index
// with their LDS passed in), shared by the GEMM kernels and the fused
// small-batch layer. Internal to libmoe.so; ffn.hip describes the design.
#pragma once

#include "moe_internal.h"

#include <type_traits>

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
// The GEMM of workgroup `bid` of `nblk` (a multiple of 8, dealt to the XCDs
// round-robin), with its LDS passed in: the activation double buffer xs and
// the tile map.
template <bool kSwiGLU, int kTM, int kW>
__device__ __forceinline__ void ffn_gemm_bf16_body(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, const uint16_t* __restrict__ Ws,
    int n_routed, const int32_t* __restrict__ offsets, int n_groups, int max_rows, int K, int Nw,
    int NB, uint16_t* __restrict__ out, int ldo, uint8_t (&xs)[2][kTM * kLdsRowBf16], TileMap& tm,
    unsigned bid, unsigned nblk) {
    constexpr int kSub = kTM / 16;    // m-subtiles per tile
    constexpr int kOwn = kTM / 64;    // 16-row pieces of the tile each wave stages

    const int lane = threadIdx.x & 63;
    // left per-lane: making it wave-uniform measured 10% slower on a 512-token, 32-expert share
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15;
    const int lk = lane >> 4;
    const int nk = K / kBK;
    const int n_items = build_tile_map(tm, offsets, n_groups, max_rows, kTM) * NB;

    // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin
    // (workgroup index % 8); each XCD walks a contiguous slice of the items, so the
    // n-blocks of one m-tile (same activations) share that XCD's L2. If the
    // dealing differs only locality suffers. The grid is a multiple of 8.
    const int xcd = bid & 7;
    const int per_xcd = nblk >> 3;
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

    for (int item = i_lo + (bid >> 3); item < i_hi; item += per_xcd) {
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


// The GEMM of workgroup `bid` of `nblk` (a multiple of 8), with its LDS passed
// in: the three activation stages (distinct objects, so the compiler tells
// the stage being filled from the one being read), the tile map, the weight
// block scales of the item [block][k step] and, for SwiGLU, the row amax per
// wave (kLWaves * kLTM floats).
template <bool kSwiGLU, bool kGather>
__device__ __forceinline__ void ffn_gemm_fp8_lds_body(
    const uint8_t* __restrict__ X, const float* __restrict__ Xs, const uint8_t* __restrict__ W,
    const float* __restrict__ Wsc, const uint8_t* __restrict__ Wsh, const float* __restrict__ Wsh_sc,
    int n_routed, const int32_t* __restrict__ offsets, int n_groups, int max_rows, int K, int Nw,
    int NB, void* __restrict__ out, float* __restrict__ out_scale, int ldo, ActSrc src, XStage& st0,
    XStage& st1, XStage& st2, TileMap& tm, float (&wsc)[2][kLMaxSteps], float* red, unsigned bid,
    unsigned nblk) {

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15;
    const int lk = lane >> 4;
    const int nk = K / kBK;
    const int n_items = build_tile_map(tm, offsets, n_groups, max_rows, kLTM, 0, kLTM) * NB;
    const int xcd = bid & 7;
    const int per_xcd = nblk >> 3;
    const int i_lo = (int)((long)n_items * xcd / 8);
    const int i_hi = (int)((long)n_items * (xcd + 1) / 8);

    for (int item = i_lo + (bid >> 3); item < i_hi; item += per_xcd) {
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

}  // namespace
}  // namespace moe
