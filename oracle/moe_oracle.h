/*
 * CPU oracle for one DeepSeek-R1-style MoE layer -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct implementation of what the layer computes.
 * Only tests, the smoke check and the benchmark's CPU-baseline leg may load
 * it. It shares no code, header, table or helper with the GPU library.
 *
 * Sources (cited by page title and section):
 *   [Moreh-EP]  Moreh, "DeepSeek inference at 21K output tokens/s on AMD
 *               Instinct MI300X GPUs with expert parallelism" (ja/zh pages):
 *               Overview, Parallelization, Inter-GPU load balancing,
 *               Library optimization, HIP Graphs.
 *   [SGLang-H20] "Deploying DeepSeek-R1 efficiently on H20-96G together with
 *               SGLang: best practices": Prefill solutions (MoE b_scale),
 *               SwapAB GEMM, Expert Affinity EPLB.
 * The pages fix no precision, reduction order, score function or block
 * format; every such choice below is a stated reading, and the floating point
 * arithmetic of the expert FFN is done in fp64.
 *
 * Every function returns 0 on success and a negative value on a bad argument.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2 };
enum { ORC_SOFTMAX = 0, ORC_SIGMOID = 1 };

/* Gating logits l[t,e] = <x[t,:], wr[e,:]> (+ bias[e]) in the fixed fp32 order:
 * 64 partial sums, partial j accumulating with fmaf, from +0, over ascending h
 * with floor(h/8) mod 64 == j; then pairwise p[j] += p[j+s] for s = 32..1;
 * then one fp32 add of the bias. x [T,H], wr [E,H] in `dt` (F32 or BF16). */
int oracle_router_logits(const void* x, const void* wr, const float* bias, int dt,
                         int T, int H, int E, float* logits);

/* Top-k by (logit descending, expert index ascending) and combine weights
 * (softmax or sigmoid of the selected logits, renormalised over the k picks
 * when `renorm`), computed in fp64 and rounded to fp32. */
int oracle_select(const float* logits, int T, int E, int k, int scoring, int renorm,
                  int32_t* topk_ids, float* topk_w);

/* Histogram + stable permutation of (token, pick) slots onto local experts
 * [base, base+E_local). Rows are ordered by (expert, slot = t*k+j). Group
 * E_local is the shared expert: T rows in token order when `include_shared`.
 * counts[E_local+1], offsets[E_local+2] (exclusive scan),
 * row_to_slot[T*k+T] (shared rows hold T*k+t; unused rows -1),
 * slot_to_row[T*k] (-1 = not local). */
int oracle_permute(const int32_t* topk_ids, int T, int k, int base, int E_local,
                   int include_shared, int32_t* counts, int32_t* offsets,
                   int32_t* row_to_slot, int32_t* slot_to_row);

/* OCP fp8 e4m3fn (bias 7, no infinities, max 448). Encoding rounds to nearest,
 * ties to even, and saturates at +-448. */
uint8_t oracle_e4m3_encode(float v);
float oracle_e4m3_decode(uint8_t c);
/* round-to-nearest-even of a real (double) to bfloat16 bits */
uint16_t oracle_bf16_round(double v);
/* element-wise array forms of the three conversions above */
void oracle_e4m3_encode_n(const float* v, long n, uint8_t* out);
void oracle_e4m3_decode_n(const uint8_t* c, long n, float* out);
void oracle_bf16_round_n(const double* v, long n, uint16_t* out);

/* Per 1x128 block of each row: a = max|v|, s = a/448 (1 if a == 0),
 * code = e4m3(clamp(v/s, -448, 448)), all divisions in fp32. */
int oracle_quantize_1x128(const float* v, int rows, int cols, uint8_t* codes, float* scales);

/* x_perm[r] = x[token(r)] for r < n_rows: a bit copy (F32/BF16) or the 1x128
 * quantisation of the bf16 row (FP8: codes [n_rows,H], scales [n_rows,H/128]).
 * token(r) = s/k for a routed slot s < T*k, s - T*k for a shared row. */
int oracle_gather(const void* x, int x_dt, int T, int H, int k,
                  const int32_t* row_to_slot, int n_rows, int perm_dt,
                  void* x_perm, float* x_perm_scale);

/* Expert SwiGLU FFN for every row of every group g < n_groups, rows
 * [offsets[g], offsets[g+1]):  [G|U] = x w13^T,  A = silu(G)*U,  y = A w2^T.
 * w13[g] -> [2I,H] (rows 0..I-1 gate, I..2I-1 up), w2[g] -> [H,I];
 * FP8: scales [2I/128,H/128] and [H/128,I/128]; A is quantised 1x128 after
 * rounding to fp32. Accumulation in fp64; y_perm [offsets[n_groups], H] fp64.
 * Groups with no rows may pass null weight pointers. */
int oracle_expert_ffn(const void* const* w13, const float* const* w13_scale,
                      const void* const* w2, const float* const* w2_scale, int dt,
                      const void* x_perm, const float* x_perm_scale,
                      const int32_t* offsets, int n_groups, int H, int I,
                      int n_threads, double* y_perm);

/* out[t] = sum_j topk_w[t,j] * y_perm[slot_to_row[t*k+j]]  (slots with -1
 * skipped) + y_perm[shared_row0 + t] when shared_row0 >= 0; fp64 [T,H]. */
int oracle_combine(const double* y_perm, const int32_t* slot_to_row, const float* topk_w,
                   int T, int k, int H, int shared_row0, double* out);

/* Balanced partition of E experts into G groups of E/G (the load balancer of
 * [Moreh-EP] Inter-GPU load balancing). LPT: experts by (count desc, id asc)
 * each go to the least-loaded non-full group (ties -> lower group). Then
 * repeat: take the heaviest group g* (ties -> lowest index); among swaps of
 * a in g* with b in another group h with d = c_a - c_b > 0 and
 * max(L_g* - d, L_h + d) < L_g*, apply the one minimising that max (ties ->
 * smallest h, then a, then b); stop when none exists (or after 10*E swaps).
 * new_to_old[g*S+j] is the j-th smallest old id of group g. */
int oracle_balanced_partition(const int64_t* counts, int E, int G,
                              int32_t* new_to_old, int32_t* old_to_new, int64_t* group_loads);

/* Top-k co-activation histogram, accumulated ([SGLang-H20] Expert Affinity
 * EPLB: track which experts the top-k picks activate together). hist is
 * [E][E] row-major. For every token, each pick with 0 <= id < E adds 1 to
 * hist[id][id]; each pair of its picks i < j with valid, distinct ids adds 1
 * to hist[a][b] and to hist[b][a]. Ids outside [0, E) are ignored. */
int oracle_coactivation(const int32_t* ids, int T, int k, int E, int64_t* hist);

/* Affinity-aware balanced partition ([Moreh-EP] Inter-GPU load balancing for
 * the balanced start; [SGLang-H20] Expert Affinity EPLB for the adjustment,
 * whose steps the page does not give -- this is the reading): start from
 * oracle_balanced_partition, whose largest group load is L; allow loads up
 * to cap = floor(L * (1000 + tol_permille) / 1000); then, as long as one
 * exists, apply the swap of two experts a < b in different groups that keeps
 * both groups' loads <= cap and raises the total intra-group affinity
 * sum over groups, sum over pairs a < b in the group, of aff[a][b]
 * the most (the first such (a, b) in ascending order on ties), at most 10*E
 * swaps. aff is [E][E] and symmetric. Outputs as the balanced partition plus
 * *intra_affinity, the final total. */
int oracle_affinity_partition(const int64_t* counts, const int64_t* aff, int E, int G,
                              int tol_permille, int32_t* new_to_old, int32_t* old_to_new,
                              int64_t* group_loads, int64_t* intra_affinity);

#ifdef __cplusplus
}
#endif
#endif
