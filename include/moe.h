/*
 * moe.h -- C ABI of libmoe.so: one DeepSeek-R1-style mixture-of-experts layer
 * on one MI355X (gfx950), as hand-written HIP kernels.
 *
 * The layer, as the sources state it:
 *   [Moreh-EP]   Moreh, "DeepSeek inference at 21K output tokens/s on AMD
 *                Instinct MI300X GPUs with expert parallelism":
 *                Overview (a lightweight gating network picks a few experts
 *                per token), Parallelization (R1: 256 routed experts, 8 active
 *                per token, one always-on shared expert; 32 experts per GPU at
 *                EP=8), Inter-GPU load balancing (activation counts, balanced
 *                sets of 32, remapped gating), Library optimization (fused MoE
 *                kernel; horizontal fusion of the shared expert's GEMMs),
 *                HIP Graphs (tensor sizes kept static for graph capture).
 *   [SGLang-H20] "Deploying DeepSeek-R1 efficiently on H20-96G together with
 *                SGLang": Prefill solutions (MoE fp8 b_scale handling, down
 *                projection input layout), SwapAB GEMM (variable M per expert
 *                needs small M tiles).
 *
 * Conventions shared by every call:
 *  - All tensors are caller-allocated device memory, row-major, densely
 *    packed. The library never allocates or frees device memory; scratch
 *    space is a caller-provided workspace whose size a *_workspace_size query
 *    returns.
 *  - Device calls only enqueue work on `stream` (a hipStream_t, NULL = the
 *    default stream): no host synchronisation, no device-to-host copies, so a
 *    sequence of calls can be captured into a HIP graph. Per-expert row counts
 *    stay on the device; buffers are sized by the static bound T*k (+T).
 *  - bf16 is IEEE bfloat16; fp8 is OCP e4m3fn (max 448). Expert weights are
 *    K-contiguous: w13 [E][2I][H] with rows 0..I-1 the gate projection and
 *    I..2I-1 the up projection, w2 [E][H][I]. fp8 weights carry one fp32
 *    scale per 128x128 block ([E][2I/128][H/128], [E][H/128][I/128]); fp8
 *    activations one fp32 scale per 1x128 block of a row.
 *  - Errors are reported synchronously by the return value; argument checks
 *    happen before anything is enqueued. Faults inside kernels surface at the
 *    caller's next synchronisation. Data values (NaN/Inf) are not checked.
 *  - T == 0 is a successful no-op.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int moe_status;
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG 1  /* null pointer, negative size, k > E, ...      */
#define MOE_ERR_UNSUPPORTED 2  /* a size or dtype combination not built       */
#define MOE_ERR_HIP 3          /* a HIP runtime call or kernel launch failed  */
#define MOE_ERR_WORKSPACE 4    /* workspace null or smaller than required     */

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;
typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_scoring;

/* Gating ([Moreh-EP] Overview, Parallelization; remapped order after the
 * load balancer, Inter-GPU load balancing).
 *   logits[t,e] = sum_h x[t,h] * w_router[e,h] (+ bias[e])
 * accumulated in fp32 in a fixed order (64 partial sums; partial j takes the
 * 8-element chunks h with floor(h/8) mod 64 == j in ascending h with fused
 * multiply-adds from +0; partials combined p[j] += p[j+s] for s = 32..1; then
 * one add of the bias), so the result is reproducible bit for bit.
 * topk_ids[t,:] = the k experts with the largest logits, ordered by (logit
 * descending, expert index ascending). topk_w = softmax or sigmoid of the
 * picked logits, renormalised to sum 1 over the k picks when `renormalize`
 * (softmax without it is normalised over all E).
 *   x [T,H], w_router [E,H]: dt = MOE_F32 or MOE_BF16 (both the same dt)
 *   bias [E] fp32 or NULL; logits [T,E] fp32 (out); topk_ids [T,k] int32 (out);
 *   topk_w [T,k] fp32 (out).
 * Limits: 1 <= k <= E <= 256 (MOE_ERR_UNSUPPORTED above), H >= 1. */
moe_status moe_route(const void* x, const void* w_router, const float* bias, moe_dtype dt,
                     int T, int H, int E, int k, moe_scoring scoring, int renormalize,
                     float* logits, int32_t* topk_ids, float* topk_w, void* stream);

/* Gating for large token batches: the same topk_ids and topk_w as moe_route
 * (bit for bit), without computing every fixed-order logit. Approximate logits
 * and sum_h |x_h w_eh| come from bf16 MFMAs over 64-deep stages added in fp32;
 * a rigorous bound (valid for any internal MFMA summation order with 16 or
 * more significant bits per addition, and for flushed denormals) on the distance
 * between an approximate logit and the fixed-order one leaves, per token, the
 * experts whose bound interval reaches the k-th largest lower bound. Only those
 * get their fixed-order logit (the selection rule of moe_route is then applied
 * to them, every other expert counting as -inf); the rest cannot be picked.
 *   x [T,H], w_router [E,H] bf16; bias [E] fp32 or NULL; topk_ids [T,k] int32
 *   (out), topk_w [T,k] fp32 (out); workspace: device memory of at least
 *   moe_route_select_workspace_size(T, E) bytes, caller-owned, 256-byte
 *   aligned; its contents on return are unspecified.
 * Limits: bf16 only; H % 32 == 0 and H <= 8192; 1 <= k <= E <= 256; softmax
 * scoring only with renormalize (the unrenormalised softmax needs every
 * logit): MOE_ERR_UNSUPPORTED otherwise, MOE_ERR_WORKSPACE if ws_bytes is too
 * small. Faster than moe_route for thousands of tokens; slower for a decode
 * batch (the MFMA pass has one workgroup per 64 tokens). */
size_t moe_route_select_workspace_size(int T, int E);
moe_status moe_route_select(const void* x, const void* w_router, const float* bias, moe_dtype dt,
                            int T, int H, int E, int k, moe_scoring scoring, int renormalize,
                            int32_t* topk_ids, float* topk_w, void* workspace, size_t ws_bytes,
                            void* stream);

/* Token -> expert grouping ([Moreh-EP] Library optimization: the fused MoE
 * kernel consumes tokens grouped per expert; Inter-GPU load balancing: the
 * per-expert activation counts). Slots s = t*k + j whose id lies in
 * [expert_base, expert_base + E_local) are local; they become rows ordered by
 * (expert, slot). Group E_local is the shared expert ([Moreh-EP]
 * Parallelization: runs on every token): with include_shared it holds the T
 * tokens in order after the routed rows.
 *   expert_counts [E_local+1] (out), expert_offsets [E_local+2] (out,
 *   exclusive scan of the counts; R = offsets[E_local] routed rows),
 *   row_to_slot [T*k+T] (out; shared rows hold T*k+t, unused rows -1),
 *   slot_to_row [T*k] (out; -1 = not local),
 *   x_perm [T*k+T, H] (out): x[token(row)] as a bit copy (perm_dt == x_dt)
 *   or, for perm_dt = MOE_FP8_E4M3 with bf16 x, e4m3 codes with
 *   x_perm_scale [H/128, T*k+T] fp32 (out, K-major: block b of row r at
 *   b*(T*k+T) + r): per 1x128 block s = amax/448 (1 for
 *   an all-zero block), code = e4m3(clamp(v/s, +-448)), fp32 division, round to
 *   nearest even. x and x_perm may both be NULL (maps and counts only).
 *   Rows of x_perm past the used ones are unspecified.
 * ids outside the local range (including negative ones) are simply not local.
 * Limits: 1 <= E_local <= 256; T*k+T < 2^31; fp8 needs H % 128 == 0.
 * workspace: moe_permute_workspace_size(T, k, E_local) bytes. */
size_t moe_permute_workspace_size(int T, int k, int E_local);
moe_status moe_permute(const int32_t* topk_ids, int T, int k, int expert_base, int E_local,
                       int include_shared, const void* x, moe_dtype x_dt, int H, moe_dtype perm_dt,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_to_slot,
                       int32_t* slot_to_row, void* x_perm, float* x_perm_scale,
                       void* workspace, size_t ws_bytes, void* stream);

/* Expert weights of one GPU's share: E_local routed experts plus an optional
 * shared expert (ws13/ws2, NULL when there is none), all in `dt`. The scale
 * pointers are used for MOE_FP8_E4M3 only. For MOE_F32 and MOE_BF16 the
 * activations are in the same dt; for MOE_FP8_E4M3 they are e4m3 + scales. */
typedef struct moe_expert_weights {
    moe_dtype dt;
    int E_local, H, I;
    const void* w13;
    const float* w13_scale;
    const void* w2;
    const float* w2_scale;
    const void* ws13;
    const float* ws13_scale;
    const void* ws2;
    const float* ws2_scale;
} moe_expert_weights;

/* Expert FFNs as grouped GEMMs with a device-resident, variable row count
 * per group ([SGLang-H20] SwapAB GEMM: variable M per expert; [Moreh-EP]
 * Library optimization: the shared expert joins the same launch, horizontal
 * fusion). For the rows of group g (rows [offsets[g], offsets[g+1])):
 *   [G|U] = x_perm w13_g^T,  A = silu(G) * U,  y_perm = A w2_g^T
 * groups 0..E_local-1 use the routed experts, group E_local (n_groups ==
 * E_local+1) the shared expert. fp32 accumulation. bf16: A is rounded to bf16
 * between the GEMMs. fp8: A is quantised per 1x128 block exactly like x_perm
 * (fp32 scale amax/448, round to nearest even), and block scales are applied
 * to each 128-deep partial product.
 *   x_perm [max_rows, H] (+ x_perm_scale [H/128, max_rows] for fp8, K-major
 *   as moe_permute writes it when max_rows = T*k+T),
 *   expert_offsets [n_groups+1] (device; as written by moe_permute),
 *   y_perm [max_rows, H] (out): bf16 (fp32 for dt = MOE_F32).
 * max_rows bounds offsets[n_groups] (T*k+T for the maps of moe_permute).
 * Limits: bf16 needs H % 128 == 0 and I % 128 == 0; fp8 needs H % 256 == 0,
 * I % 128 == 0 and H, I <= 16384 (the per-item table of weight block
 * scales); E_local <= 1024; n_groups in {E_local, E_local+1} (the
 * latter needs the shared weights).
 * workspace: moe_expert_ffn_workspace_size(w, max_rows) bytes. */
size_t moe_expert_ffn_workspace_size(const moe_expert_weights* w, int max_rows);
moe_status moe_expert_ffn(const moe_expert_weights* w, const void* x_perm,
                          const float* x_perm_scale, const int32_t* expert_offsets, int n_groups,
                          int max_rows, void* y_perm, void* workspace, size_t ws_bytes,
                          void* stream);

/* moe_expert_ffn as its two steps, one kernel each, for callers that time or
 * schedule them separately. gate_up computes A = silu(x_perm w13^T gate) *
 * (x_perm w13^T up) into the workspace (bf16, or e4m3 + 1x128 scales);
 * down reads A from the same workspace (written by the preceding gate_up on
 * the same stream with the same offsets) and writes y_perm. Arguments,
 * limits and workspace size as for moe_expert_ffn. */
moe_status moe_expert_ffn_gate_up(const moe_expert_weights* w, const void* x_perm,
                                  const float* x_perm_scale, const int32_t* expert_offsets,
                                  int n_groups, int max_rows, void* workspace, size_t ws_bytes,
                                  void* stream);
moe_status moe_expert_ffn_down(const moe_expert_weights* w, const int32_t* expert_offsets,
                               int n_groups, int max_rows, void* y_perm, void* workspace,
                               size_t ws_bytes, void* stream);

/* moe_expert_ffn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the intermediate A (and its fp8 scales) lives in a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends, instead of a caller workspace. Arguments, results and limits
 * as for moe_expert_ffn; the call allocates and frees nothing.
 *   Limit: moe_expert_ffn_workspace_size(w, max_rows) must not exceed
 *   MOE_NOALLOC_SCRATCH_BYTES (else MOE_ERR_WORKSPACE and nothing is
 *   enqueued); e.g. bf16 at I = 2048 allows 16384 rows, fp8 about 31700.
 *   Calls that overlap on one GPU (other streams, other threads) share the
 *   array and race: serialise them. Nothing in it needs clearing: every row
 *   of A that the down projection reads is written by the gate/up step of
 *   the same call. The first call on a device looks the array's address up
 *   (hipGetSymbolAddress), so make one outside graph capture. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_expert_ffn_noalloc(const moe_expert_weights* w, const void* x_perm,
                                  const float* x_perm_scale, const int32_t* expert_offsets,
                                  int n_groups, int max_rows, void* y_perm, void* stream);

/* fp8 gate/up without a permuted copy of the activations ([Moreh-EP] Library
 * optimization: the fused MoE kernel reads each expert's tokens itself):
 * moe_quantize_tokens quantises every token once, and
 * moe_expert_ffn_gate_up_tokens reads permuted row r's activations from its
 * token's row, token = slot < T*k ? slot / k : slot - T*k with
 * slot = row_to_slot[r] (moe_permute's map, which may then run with x_perm
 * NULL). The result in the workspace is bit for bit the one moe_expert_ffn_gate_up
 * computes from the x_perm moe_permute would write; moe_expert_ffn_down
 * follows as usual.
 *   moe_quantize_tokens: x [T, H] bf16 -> codes [T, H] e4m3 and scales
 *   [H/128, T] fp32 (out, K-major), per 1x128 block exactly as moe_permute's
 *   fp8 x_perm. Limits: H % 128 == 0, T*H < 2^31.
 *   moe_expert_ffn_gate_up_tokens: x_tokens, x_tokens_scale as written by
 *   moe_quantize_tokens; row_to_slot [max_rows] (device; rows below
 *   offsets[n_groups] must hold slots in [0, T*k+T)); other arguments, limits
 *   and workspace as for moe_expert_ffn_gate_up with dt = MOE_FP8_E4M3 only;
 *   T*H < 2^31. A slot outside that range reads another token's row or
 *   zeros, never memory outside the token buffers. */
moe_status moe_quantize_tokens(const void* x, moe_dtype x_dt, int T, int H, void* codes,
                               float* scales, void* stream);
moe_status moe_expert_ffn_gate_up_tokens(const moe_expert_weights* w, const void* x_tokens,
                                         const float* x_tokens_scale, int T, int k,
                                         const int32_t* row_to_slot, const int32_t* expert_offsets,
                                         int n_groups, int max_rows, void* workspace,
                                         size_t ws_bytes, void* stream);

/* The whole layer for a small batch in one persistent launch ([Moreh-EP]
 * Library optimization: a fused MoE kernel for small batches; Use of HIP
 * Graphs: static sizes, capturable): the gating of moe_route, the permutation
 * of moe_permute (all E experts local, the shared expert as group E when the
 * weights hold one), the expert FFN of moe_expert_ffn (fp8: activations
 * quantised per token and read through the permutation, as
 * moe_quantize_tokens + moe_expert_ffn_gate_up_tokens) and moe_combine, as
 * phases of one kernel separated by grid-wide barriers. Results are bit for
 * bit those of the separate calls on the same inputs.
 *   x [T,H] bf16, w_router [E,H] bf16, bias [E] fp32 or NULL, w: E_local == E
 *   experts in bf16 or fp8 (+ optional shared expert); topk_ids [T,k] int32,
 *   topk_w [T,k] fp32 and out [T,H] bf16 (out).
 *   workspace: moe_layer_fused_workspace_size(w, T, E, k) bytes of device
 *   memory; its first 256 bytes (the barrier words) must be zero before the
 *   first call, and every completed call leaves them zero. The other contents
 *   on return are unspecified.
 * Limits: 1 <= T <= 256, 1 <= k <= 8, k <= E <= 256, H % 256 == 0,
 * I % 128 == 0 (fp8: H, I <= 16384). The grid is one workgroup per CU and
 * its phases wait for each other: the device must hold the whole grid at
 * once (nothing else running on it). A barrier that waits too long (about
 * a second) sets the third 32-bit workspace word (bytes 8..11) nonzero and lets the
 * kernel finish; its outputs are then invalid and the first 256 bytes must
 * be zeroed again. */
size_t moe_layer_fused_workspace_size(const moe_expert_weights* w, int T, int E, int k);
moe_status moe_layer_fused(const void* x, const void* w_router, const float* bias, int T, int E,
                           int k, moe_scoring scoring, int renormalize,
                           const moe_expert_weights* w, int32_t* topk_ids, float* topk_w,
                           void* out, void* workspace, size_t ws_bytes, void* stream);

/* Routing-weighted combine back to token order ([Moreh-EP] Overview:
 * dispatch/combine; the local half of it).
 *   out[t] = sum_{j: slot_to_row[t*k+j] >= 0} topk_w[t,j] * y_perm[slot_to_row[t*k+j]]
 *            + y_perm[expert_offsets[shared_group] + t]   (if shared_group >= 0)
 * summed in fp32 in slot order, then rounded to nearest even.
 *   y_perm [.., H] in y_dt (MOE_BF16 or MOE_F32), out [T,H] in out_dt
 *   (MOE_BF16 or MOE_F32). */
moe_status moe_combine(const void* y_perm, moe_dtype y_dt, const int32_t* slot_to_row,
                       const float* topk_w, int T, int k, int H, const int32_t* expert_offsets,
                       int shared_group, void* out, moe_dtype out_dt, void* stream);

/* Host-only balanced partition of E experts into G sets of E/G with balanced
 * activation totals ([Moreh-EP] Inter-GPU load balancing: a balanced number
 * partitioning variant). LPT under the set-size limit (experts by count
 * descending, id ascending, each to the least-loaded non-full set, lower set
 * on ties), then best-improvement swaps out of the heaviest set (the swap of
 * a in the heaviest set g* with b in set h that minimises max(L_g* - d,
 * L_h + d) < L_g*, d = c_a - c_b > 0; ties to the smallest h, a, b) until no
 * swap improves (at most 10*E swaps). All pointers are host memory:
 * counts [E] (>= 0), new_to_old [E] (out; set g is new ids g*E/G.., old ids
 * ascending), old_to_new [E] (out), group_loads [G] (out). */
moe_status moe_balanced_partition(const int64_t* counts, int E, int G, int32_t* new_to_old,
                                  int32_t* old_to_new, int64_t* group_loads);

/* Gather whole rows: dst[i] = src[index[i]] for i < n_rows, each row
 * row_bytes long (a multiple of 4). Applies the balanced partition's expert
 * order to router rows, router bias and expert weights ([Moreh-EP]
 * Inter-GPU load balancing: reorder the experts, remap the gating).
 * index [n_rows] int32 is device memory with values in [0, n_src_rows). */
moe_status moe_gather_rows(const void* src, int n_src_rows, void* dst, const int32_t* index,
                           int n_rows, size_t row_bytes, void* stream);

/* Online rebalancing: the measurements the partition works from, kept on the
 * device across steps ([Moreh-EP] Inter-GPU load balancing: re-measure the
 * activation frequencies periodically and derive a new expert order;
 * [SGLang-H20] Expert Affinity EPLB: track top-k co-activation in an expert
 * affinity matrix).
 *
 * moe_count_accumulate: acc[i] += counts[i] for i < n (counts as written by
 * moe_permute). counts [n] int32 and acc [n] int64 are device memory; acc is
 * never cleared by the library.
 *
 * moe_coactivation: adds one step's top-k picks to an [E][E] int64 histogram
 * in device memory. For every token, each pick with 0 <= id < E adds 1 to
 * hist[id][id]; each pair of its picks i < j with valid, distinct ids adds 1
 * to hist[a][b] and to hist[b][a]; other ids are ignored. Integer atomics:
 * the result does not depend on the order of the additions. topk_ids [T,k]
 * int32 device memory. Limits: 1 <= E <= 1024, 1 <= k <= 256, T <= 2^24. */
moe_status moe_count_accumulate(const int32_t* counts, int n, int64_t* acc, void* stream);
moe_status moe_coactivation(const int32_t* topk_ids, int T, int k, int E, int64_t* hist,
                            void* stream);

/* Host-only affinity-aware partition ([SGLang-H20] Expert Affinity EPLB:
 * co-activated experts placed in the same set; the page gives no algorithm,
 * this is the reading). Starts from moe_balanced_partition, whose largest set
 * load is L; allows set loads up to cap = floor(L * (1000 + tol_permille) /
 * 1000); then repeatedly applies the swap of experts a < b in different sets
 * that keeps both loads <= cap and raises the total intra-set affinity
 * (sum over sets of aff[a][b] for a < b in the set) the most, the first such
 * (a, b) in ascending order on ties, until none raises it (at most 10*E
 * swaps). aff [E][E] int64 host memory, symmetric (the diagonal is unused);
 * other arguments as moe_balanced_partition, plus intra_affinity (out, the
 * final total). tol_permille >= 0. */
moe_status moe_affinity_partition(const int64_t* counts, const int64_t* aff, int E, int G,
                                  int tol_permille, int32_t* new_to_old, int32_t* old_to_new,
                                  int64_t* group_loads, int64_t* intra_affinity);

const char* moe_status_string(moe_status s);
/* detail of the last error on the calling thread ("" if none) */
const char* moe_last_error_message(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
