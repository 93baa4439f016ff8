/*
 * CPU oracle for one DeepSeek-R1-style MoE layer -- TEST INFRASTRUCTURE ONLY.
 * Plain loops in the order the definitions state; no blocking, no fusion.
 * Built with -ffp-contract=off so that the only fused multiply-adds are the
 * explicit fmaf calls of the gating logits. See moe_oracle.h for the sources.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ values */

static float bf16_bits_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float load_act(const void* p, int dt, long i) {
    if (dt == ORC_F32) return ((const float*)p)[i];
    return bf16_bits_to_float(((const uint16_t*)p)[i]);
}

float oracle_e4m3_decode(uint8_t c) {
    int sign = c >> 7, ex = (c >> 3) & 15, man = c & 7;
    double v;
    if (ex == 15 && man == 7) return NAN;               /* the only NaN codes */
    if (ex == 0) v = ldexp((double)man, -9);             /* subnormal: m * 2^-9 */
    else v = ldexp(1.0 + man / 8.0, ex - 7);             /* normal: 1.m * 2^(e-7) */
    return (float)(sign ? -v : v);
}

uint8_t oracle_e4m3_encode(float v) {
    /* round |v| to the e4m3 grid: quantum 2^(E-3) for binade E >= -6, 2^-9 below */
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (isnan(v)) return 0x7f;
    if (a >= 448.0) return sign | 0x7e;                  /* saturate to +-448 */
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                                         /* a = f 2^e, f in [0.5,1) */
    int E = e - 1;
    if (E < -6) E = -6;
    double quantum = ldexp(1.0, E - 3);
    double q = nearbyint(a / quantum);                    /* exact divide; RNE */
    double r = q * quantum;
    if (r == 0.0) return sign;
    if (r >= 448.0) return sign | 0x7e;
    frexp(r, &e);
    E = e - 1;
    if (E < -6) {                                          /* subnormal code */
        int m = (int)(r / ldexp(1.0, -9));
        return sign | (uint8_t)m;
    }
    int m = (int)((r / ldexp(1.0, E) - 1.0) * 8.0);
    return sign | (uint8_t)((E + 7) << 3) | (uint8_t)m;
}

uint16_t oracle_bf16_round(double v) {
    /* 8 significant bits; binades below 2^-126 share the quantum 2^-133 */
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return 0x7fc0;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    int E = e - 1;
    if (E < -126) E = -126;
    double quantum = ldexp(1.0, E - 7);
    double r = nearbyint(a / quantum) * quantum;
    if (r >= ldexp(1.0, 128)) return sign | 0x7f80;        /* overflow -> inf */
    float f = (float)r;                                    /* exact */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)((u >> 16) & 0x7fff);
}

void oracle_e4m3_encode_n(const float* v, long n, uint8_t* out) {
    for (long i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_e4m3_decode_n(const uint8_t* c, long n, float* out) {
    for (long i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}

void oracle_bf16_round_n(const double* v, long n, uint16_t* out) {
    for (long i = 0; i < n; ++i) out[i] = oracle_bf16_round(v[i]);
}

/* ------------------------------------------------------------------ gating */

int oracle_router_logits(const void* x, const void* wr, const float* bias, int dt,
                         int T, int H, int E, float* logits) {
    if (T < 0 || H <= 0 || E <= 0 || !logits || (T > 0 && (!x || !wr))) return -1;
    if (dt != ORC_F32 && dt != ORC_BF16) return -1;
#pragma omp parallel for schedule(static)
    for (long te = 0; te < (long)T * E; ++te) {
        long t = te / E, e = te % E;
        float p[64];
        for (int j = 0; j < 64; ++j) p[j] = 0.0f;
        for (int h = 0; h < H; ++h) {
            int j = (h / 8) % 64;
            p[j] = fmaf(load_act(x, dt, t * H + h), load_act(wr, dt, e * H + h), p[j]);
        }
        for (int s = 32; s >= 1; s /= 2)
            for (int j = 0; j < s; ++j) p[j] = p[j] + p[j + s];
        float l = p[0];
        if (bias) l = l + bias[e];
        logits[te] = l;
    }
    return 0;
}

int oracle_select(const float* logits, int T, int E, int k, int scoring, int renorm,
                  int32_t* topk_ids, float* topk_w) {
    if (T < 0 || E <= 0 || k <= 0 || k > E || k > 512 || (T > 0 && (!logits || !topk_ids || !topk_w)))
        return -1;
    if (scoring != ORC_SOFTMAX && scoring != ORC_SIGMOID) return -1;
    char* taken = (char*)malloc((size_t)E);
    if (!taken) return -2;
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (long)t * E;
        memset(taken, 0, (size_t)E);
        /* k rounds: the largest untaken logit, lower index first on equality */
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;   /* strict: keeps the lower index */
            }
            taken[best] = 1;
            topk_ids[(long)t * k + j] = best;
        }
        double v[512], den = 0.0;
        const int32_t* id = topk_ids + (long)t * k;
        if (scoring == ORC_SOFTMAX) {
            double lmax = l[id[0]];
            for (int j = 0; j < k; ++j) v[j] = exp((double)l[id[j]] - lmax);
            if (renorm) {
                for (int j = 0; j < k; ++j) den += v[j];
            } else {
                for (int e = 0; e < E; ++e) den += exp((double)l[e] - lmax);
            }
        } else {
            for (int j = 0; j < k; ++j) v[j] = 1.0 / (1.0 + exp(-(double)l[id[j]]));
            if (renorm) {
                for (int j = 0; j < k; ++j) den += v[j];
            } else {
                den = 1.0;
            }
        }
        for (int j = 0; j < k; ++j) topk_w[(long)t * k + j] = (float)(v[j] / den);
    }
    free(taken);
    return 0;
}

/* ------------------------------------------------------------- permutation */

int oracle_permute(const int32_t* topk_ids, int T, int k, int base, int E_local,
                   int include_shared, int32_t* counts, int32_t* offsets,
                   int32_t* row_to_slot, int32_t* slot_to_row) {
    if (T < 0 || k <= 0 || E_local <= 0 || !counts || !offsets) return -1;
    if (T > 0 && (!topk_ids || !row_to_slot || !slot_to_row)) return -1;
    long S = (long)T * k, cap = S + T;
    for (int g = 0; g <= E_local; ++g) counts[g] = 0;
    for (long s = 0; s < S; ++s) {
        int e = topk_ids[s] - base;
        if (e >= 0 && e < E_local) counts[e]++;
    }
    counts[E_local] = include_shared ? T : 0;
    offsets[0] = 0;
    for (int g = 0; g <= E_local; ++g) offsets[g + 1] = offsets[g] + counts[g];
    for (long r = 0; r < cap; ++r) row_to_slot[r] = -1;
    for (long s = 0; s < S; ++s) slot_to_row[s] = -1;
    /* rows in (expert, slot) order: a stable sort of the slots by expert */
    long r = 0;
    for (int e = 0; e < E_local; ++e)
        for (long s = 0; s < S; ++s)
            if (topk_ids[s] - base == e) {
                row_to_slot[r] = (int32_t)s;
                slot_to_row[s] = (int32_t)r;
                ++r;
            }
    if (include_shared)
        for (int t = 0; t < T; ++t) row_to_slot[r + t] = (int32_t)(S + t);
    return 0;
}

/* ---------------------------------------------------------- fp8 activations */

static void quantize_block(const float* v, int n, uint8_t* codes, float* scale) {
    float a = 0.0f;
    for (int i = 0; i < n; ++i) a = fmaxf(a, fabsf(v[i]));
    float s = (a == 0.0f) ? 1.0f : a / 448.0f;
    for (int i = 0; i < n; ++i) {
        float q = v[i] / s;
        if (q > 448.0f) q = 448.0f;
        if (q < -448.0f) q = -448.0f;
        codes[i] = oracle_e4m3_encode(q);
    }
    *scale = s;
}

int oracle_quantize_1x128(const float* v, int rows, int cols, uint8_t* codes, float* scales) {
    if (rows < 0 || cols <= 0 || cols % 128 || (rows > 0 && (!v || !codes || !scales))) return -1;
    int nb = cols / 128;
    for (long r = 0; r < rows; ++r)
        for (int b = 0; b < nb; ++b)
            quantize_block(v + r * cols + b * 128, 128, codes + r * cols + b * 128,
                           scales + r * nb + b);
    return 0;
}

int oracle_gather(const void* x, int x_dt, int T, int H, int k,
                  const int32_t* row_to_slot, int n_rows, int perm_dt,
                  void* x_perm, float* x_perm_scale) {
    if (T < 0 || H <= 0 || k <= 0 || n_rows < 0) return -1;
    if (n_rows > 0 && (!x || !row_to_slot || !x_perm)) return -1;
    if (perm_dt == ORC_FP8 && (H % 128 || x_dt != ORC_BF16 || (n_rows > 0 && !x_perm_scale)))
        return -1;
    if (perm_dt != ORC_FP8 && perm_dt != x_dt) return -1;
    long S = (long)T * k;
    float* row = (float*)malloc(sizeof(float) * (size_t)H);
    if (!row) return -2;
    for (long r = 0; r < n_rows; ++r) {
        long s = row_to_slot[r];
        if (s < 0 || s >= S + T) { free(row); return -1; }
        long t = s < S ? s / k : s - S;
        if (perm_dt == ORC_F32) {
            memcpy((float*)x_perm + r * H, (const float*)x + t * H, sizeof(float) * (size_t)H);
        } else if (perm_dt == ORC_BF16) {
            memcpy((uint16_t*)x_perm + r * H, (const uint16_t*)x + t * H, 2 * (size_t)H);
        } else {
            for (int h = 0; h < H; ++h) row[h] = load_act(x, ORC_BF16, t * H + h);
            oracle_quantize_1x128(row, 1, H, (uint8_t*)x_perm + r * H, x_perm_scale + r * (H / 128));
        }
    }
    free(row);
    return 0;
}

/* -------------------------------------------------------------- expert FFN */

/* dequantised weight element (i, h) of a [N, K] matrix in `dt` */
static double wval(const void* w, const float* sc, int dt, int K, long i, long h) {
    if (dt == ORC_F32) return ((const float*)w)[i * K + h];
    if (dt == ORC_BF16) return bf16_bits_to_float(((const uint16_t*)w)[i * K + h]);
    return (double)oracle_e4m3_decode(((const uint8_t*)w)[i * K + h]) *
           (double)sc[(i / 128) * (K / 128) + h / 128];
}

static double xval(const void* x, const float* sc, int dt, int H, long r, long h) {
    if (dt == ORC_F32) return ((const float*)x)[r * H + h];
    if (dt == ORC_BF16) return bf16_bits_to_float(((const uint16_t*)x)[r * H + h]);
    return (double)oracle_e4m3_decode(((const uint8_t*)x)[r * H + h]) *
           (double)sc[r * (H / 128) + h / 128];
}

int oracle_expert_ffn(const void* const* w13, const float* const* w13_scale,
                      const void* const* w2, const float* const* w2_scale, int dt,
                      const void* x_perm, const float* x_perm_scale,
                      const int32_t* offsets, int n_groups, int H, int I,
                      int n_threads, double* y_perm) {
    if (n_groups <= 0 || H <= 0 || I <= 0 || !offsets || !w13 || !w2) return -1;
    if (dt != ORC_F32 && dt != ORC_BF16 && dt != ORC_FP8) return -1;
    if (dt == ORC_FP8 && (H % 128 || I % 128 || !w13_scale || !w2_scale || !x_perm_scale)) return -1;
    long n_rows = offsets[n_groups];
    if (offsets[0] != 0) return -1;
    if (n_rows > 0 && (!x_perm || !y_perm)) return -1;
    for (int g = 0; g < n_groups; ++g) {
        if (offsets[g + 1] < offsets[g]) return -1;
        if (offsets[g + 1] > offsets[g] && (!w13[g] || !w2[g] ||
            (dt == ORC_FP8 && (!w13_scale[g] || !w2_scale[g]))))
            return -1;
    }
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
#else
    (void)n_threads;
#endif
    double* w13d = (double*)malloc(sizeof(double) * (size_t)2 * I * H);
    double* w2d = (double*)malloc(sizeof(double) * (size_t)H * I);
    if (!w13d || !w2d) { free(w13d); free(w2d); return -2; }
    for (int g = 0; g < n_groups; ++g) {
        long r0 = offsets[g], m = offsets[g + 1] - offsets[g];
        if (m == 0) continue;
        const float* s13 = dt == ORC_FP8 ? w13_scale[g] : 0;
        const float* s2 = dt == ORC_FP8 ? w2_scale[g] : 0;
        double* xd = (double*)malloc(sizeof(double) * (size_t)m * H);
        double* a = (double*)malloc(sizeof(double) * (size_t)m * I);
        if (!xd || !a) { free(xd); free(a); free(w13d); free(w2d); return -2; }
        /* dequantised operands: w = code * block scale, x = code * row-block scale */
#pragma omp parallel for schedule(static) num_threads(n_threads)
        for (long i = 0; i < 2L * I; ++i)
            for (long h = 0; h < H; ++h) w13d[i * H + h] = wval(w13[g], s13, dt, H, i, h);
#pragma omp parallel for schedule(static) num_threads(n_threads)
        for (long h = 0; h < H; ++h)
            for (long i = 0; i < I; ++i) w2d[h * I + i] = wval(w2[g], s2, dt, I, h, i);
        for (long r = 0; r < m; ++r)
            for (long h = 0; h < H; ++h) xd[r * H + h] = xval(x_perm, x_perm_scale, dt, H, r0 + r, h);
        /* gate/up projection and SwiGLU: a = silu(x.w_gate) * (x.w_up) */
#pragma omp parallel for schedule(static) num_threads(n_threads)
        for (long ri = 0; ri < m * I; ++ri) {
            long r = ri / I, i = ri % I;
            double gs = 0.0, us = 0.0;
            for (long h = 0; h < H; ++h) {
                gs += xd[r * H + h] * w13d[i * H + h];
                us += xd[r * H + h] * w13d[(I + i) * H + h];
            }
            a[ri] = gs / (1.0 + exp(-gs)) * us;
        }
        if (dt == ORC_FP8) {
            /* the intermediate enters the down projection as 1x128 e4m3 blocks,
             * quantised from its fp32 rounding */
            float* af = (float*)malloc(sizeof(float) * (size_t)I);
            uint8_t* ac = (uint8_t*)malloc((size_t)I);
            float* as = (float*)malloc(sizeof(float) * (size_t)(I / 128));
            if (!af || !ac || !as) { free(af); free(ac); free(as); free(xd); free(a); free(w13d); free(w2d); return -2; }
            for (long r = 0; r < m; ++r) {
                for (long i = 0; i < I; ++i) af[i] = (float)a[r * I + i];
                oracle_quantize_1x128(af, 1, I, ac, as);
                for (long i = 0; i < I; ++i)
                    a[r * I + i] = (double)oracle_e4m3_decode(ac[i]) * (double)as[i / 128];
            }
            free(af);
            free(ac);
            free(as);
        }
        /* down projection */
#pragma omp parallel for schedule(static) num_threads(n_threads)
        for (long rh = 0; rh < m * H; ++rh) {
            long r = rh / H, h = rh % H;
            double ys = 0.0;
            for (long i = 0; i < I; ++i) ys += a[r * I + i] * w2d[h * I + i];
            y_perm[(r0 + r) * H + h] = ys;
        }
        free(xd);
        free(a);
    }
    free(w13d);
    free(w2d);
    return 0;
}

/* ------------------------------------------------------------------ combine */

int oracle_combine(const double* y_perm, const int32_t* slot_to_row, const float* topk_w,
                   int T, int k, int H, int shared_row0, double* out) {
    if (T < 0 || k <= 0 || H <= 0) return -1;
    if (T > 0 && (!y_perm || !slot_to_row || !topk_w || !out)) return -1;
    for (long t = 0; t < T; ++t)
        for (long h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                long r = slot_to_row[t * k + j];
                if (r >= 0) acc += (double)topk_w[t * k + j] * y_perm[r * H + h];
            }
            if (shared_row0 >= 0) acc += y_perm[(shared_row0 + t) * H + h];
            out[t * H + h] = acc;
        }
    return 0;
}

/* ------------------------------------------------------- balanced partition */

int oracle_balanced_partition(const int64_t* counts, int E, int G,
                              int32_t* new_to_old, int32_t* old_to_new, int64_t* group_loads) {
    if (!counts || E <= 0 || G <= 0 || E % G || !new_to_old || !old_to_new || !group_loads) return -1;
    int S = E / G;
    int* order = (int*)malloc(sizeof(int) * (size_t)E);
    int* grp = (int*)malloc(sizeof(int) * (size_t)E);
    int* size = (int*)calloc((size_t)G, sizeof(int));
    int64_t* L = (int64_t*)calloc((size_t)G, sizeof(int64_t));
    if (!order || !grp || !size || !L) return -2;
    for (int e = 0; e < E; ++e) {
        if (counts[e] < 0) return -1;
        order[e] = e;
    }
    /* insertion sort by (count desc, id asc) */
    for (int i = 1; i < E; ++i) {
        int v = order[i], j = i - 1;
        while (j >= 0 && (counts[order[j]] < counts[v] ||
                          (counts[order[j]] == counts[v] && order[j] > v))) {
            order[j + 1] = order[j];
            --j;
        }
        order[j + 1] = v;
    }
    /* LPT with the cardinality limit */
    for (int i = 0; i < E; ++i) {
        int e = order[i], best = -1;
        for (int g = 0; g < G; ++g)
            if (size[g] < S && (best < 0 || L[g] < L[best])) best = g;
        grp[e] = best;
        size[best]++;
        L[best] += counts[e];
    }
    /* swap refinement on the heaviest group */
    for (int it = 0; it < 10 * E; ++it) {
        int gs = 0;
        for (int g = 1; g < G; ++g)
            if (L[g] > L[gs]) gs = g;
        int64_t best_max = L[gs];
        int bh = -1, ba = -1, bb = -1;
        for (int h = 0; h < G; ++h) {
            if (h == gs) continue;
            for (int a = 0; a < E; ++a) {
                if (grp[a] != gs) continue;
                for (int b = 0; b < E; ++b) {
                    if (grp[b] != h) continue;
                    int64_t d = counts[a] - counts[b];
                    if (d <= 0) continue;
                    int64_t m1 = L[gs] - d, m2 = L[h] + d;
                    int64_t mx = m1 > m2 ? m1 : m2;
                    if (mx < best_max) {
                        best_max = mx;
                        bh = h;
                        ba = a;
                        bb = b;
                    }
                }
            }
        }
        if (bh < 0) break;
        int64_t d = counts[ba] - counts[bb];
        grp[ba] = bh;
        grp[bb] = gs;
        L[gs] -= d;
        L[bh] += d;
    }
    for (int g = 0; g < G; ++g) {
        int j = 0;
        for (int e = 0; e < E; ++e)
            if (grp[e] == g) new_to_old[g * S + j++] = e;
        group_loads[g] = L[g];
    }
    for (int n = 0; n < E; ++n) old_to_new[new_to_old[n]] = n;
    free(order);
    free(grp);
    free(size);
    free(L);
    return 0;
}

/* ------------------------------------------------------- co-activation */

int oracle_coactivation(const int32_t* ids, int T, int k, int E, int64_t* hist) {
    if (T < 0 || k < 1 || E < 1 || (T > 0 && !ids) || !hist) return -1;
    for (int t = 0; t < T; ++t) {
        const int32_t* p = ids + (size_t)t * k;
        for (int i = 0; i < k; ++i) {
            int a = p[i];
            if (a < 0 || a >= E) continue;
            hist[(size_t)a * E + a] += 1;
            for (int j = i + 1; j < k; ++j) {
                int b = p[j];
                if (b < 0 || b >= E || b == a) continue;
                hist[(size_t)a * E + b] += 1;
                hist[(size_t)b * E + a] += 1;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------- affinity partition */

/* sum of aff[e][c] over the members c of group g other than e */
static int64_t aff_to_group(const int64_t* aff, const int* grp, int E, int e, int g) {
    int64_t s = 0;
    for (int c = 0; c < E; ++c)
        if (c != e && grp[c] == g) s += aff[(size_t)e * E + c];
    return s;
}

int oracle_affinity_partition(const int64_t* counts, const int64_t* aff, int E, int G,
                              int tol_permille, int32_t* new_to_old, int32_t* old_to_new,
                              int64_t* group_loads, int64_t* intra_affinity) {
    if (!aff || !intra_affinity || tol_permille < 0) return -1;
    int rc = oracle_balanced_partition(counts, E, G, new_to_old, old_to_new, group_loads);
    if (rc) return rc;
    int S = E / G;
    int* grp = (int*)malloc(sizeof(int) * (size_t)E);
    int64_t* L = (int64_t*)malloc(sizeof(int64_t) * (size_t)G);
    if (!grp || !L) return -2;
    int64_t Lmax = 0;
    for (int g = 0; g < G; ++g) {
        L[g] = group_loads[g];
        if (L[g] > Lmax) Lmax = L[g];
        for (int j = 0; j < S; ++j) grp[new_to_old[g * S + j]] = g;
    }
    int64_t cap = Lmax * (1000 + tol_permille) / 1000;
    for (int it = 0; it < 10 * E; ++it) {
        int64_t best = 0;
        int ba = -1, bb = -1;
        for (int a = 0; a < E; ++a) {
            for (int b = a + 1; b < E; ++b) {
                int p = grp[a], q = grp[b];
                if (p == q) continue;
                int64_t lp = L[p] - counts[a] + counts[b];
                int64_t lq = L[q] - counts[b] + counts[a];
                if (lp > cap || lq > cap) continue;
                /* a moves to q, b moves to p; the pair (a, b) is split before and after */
                int64_t gain = aff_to_group(aff, grp, E, a, q) - aff[(size_t)a * E + b] +
                               aff_to_group(aff, grp, E, b, p) - aff[(size_t)b * E + a] -
                               aff_to_group(aff, grp, E, a, p) - aff_to_group(aff, grp, E, b, q);
                if (gain > best) {
                    best = gain;
                    ba = a;
                    bb = b;
                }
            }
        }
        if (ba < 0) break;
        int p = grp[ba], q = grp[bb];
        L[p] += counts[bb] - counts[ba];
        L[q] += counts[ba] - counts[bb];
        grp[ba] = q;
        grp[bb] = p;
    }
    int64_t total = 0;
    for (int a = 0; a < E; ++a)
        for (int b = a + 1; b < E; ++b)
            if (grp[a] == grp[b]) total += aff[(size_t)a * E + b];
    *intra_affinity = total;
    for (int g = 0; g < G; ++g) {
        int j = 0;
        for (int e = 0; e < E; ++e)
            if (grp[e] == g) new_to_old[g * S + j++] = e;
        group_loads[g] = L[g];
    }
    for (int n = 0; n < E; ++n) old_to_new[new_to_old[n]] = n;
    free(grp);
    free(L);
    return 0;
}
