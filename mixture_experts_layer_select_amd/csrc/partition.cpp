// Balanced expert partition on the host ([Moreh-EP] Inter-GPU load
// balancing: measure each expert's activation frequency, group the experts
// into equal-size sets whose totals are as even as possible -- a balanced
// number partitioning variant -- then reorder so each set is contiguous).
//
// LPT under the set-size limit, then best-improvement swaps out of the
// heaviest set. Sets are kept as sorted member lists and the swap search
// walks only the heaviest set against each other set, O(G * S^2) per swap.
#include <algorithm>
#include <numeric>
#include <vector>

#include "moe_internal.h"

namespace moe {

moe_status balanced_partition(const int64_t* counts, int E, int G, int32_t* new_to_old,
                              int32_t* old_to_new, int64_t* group_loads) {
    const int S = E / G;
    std::vector<int> order(E);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return counts[a] > counts[b]; });  // ties keep id order

    std::vector<std::vector<int>> members(G);
    std::vector<int64_t> load(G, 0);
    for (int e : order) {
        int best = -1;
        for (int g = 0; g < G; ++g)
            if ((int)members[g].size() < S && (best < 0 || load[g] < load[best])) best = g;
        members[best].push_back(e);
        load[best] += counts[e];
    }
    for (auto& m : members) std::sort(m.begin(), m.end());

    for (int it = 0; it < 10 * E; ++it) {
        int gs = (int)(std::max_element(load.begin(), load.end()) - load.begin());  // first max
        int64_t best_max = load[gs];
        int bh = -1, ia = -1, ib = -1;
        for (int h = 0; h < G; ++h) {
            if (h == gs) continue;
            for (int i = 0; i < S; ++i) {
                const int64_t ca = counts[members[gs][i]];
                for (int j = 0; j < S; ++j) {
                    const int64_t d = ca - counts[members[h][j]];
                    if (d <= 0) continue;
                    const int64_t mx = std::max(load[gs] - d, load[h] + d);
                    if (mx < best_max) {  // strict: the first (h, a, b) in ascending order wins ties
                        best_max = mx;
                        bh = h;
                        ia = i;
                        ib = j;
                    }
                }
            }
        }
        if (bh < 0) break;
        const int a = members[gs][ia], b = members[bh][ib];
        const int64_t d = counts[a] - counts[b];
        members[gs][ia] = b;
        members[bh][ib] = a;
        std::sort(members[gs].begin(), members[gs].end());
        std::sort(members[bh].begin(), members[bh].end());
        load[gs] -= d;
        load[bh] += d;
    }
    for (int g = 0; g < G; ++g) {
        for (int j = 0; j < S; ++j) new_to_old[g * S + j] = members[g][j];
        group_loads[g] = load[g];
    }
    for (int n = 0; n < E; ++n) old_to_new[new_to_old[n]] = n;
    return MOE_OK;
}

// Affinity-aware adjustment ([SGLang-H20] Expert Affinity EPLB: co-activated
// experts in the same set; the steps are this library's reading): from the
// balanced partition, best-gain swaps that keep both sets within the load
// cap. W[e][g] = sum of aff[e][c] over the members c of set g (e's own term
// included when e is in g), kept up to date in O(E) per swap, so a swap's
// gain is four table reads and two matrix reads instead of four sums.
moe_status affinity_partition(const int64_t* counts, const int64_t* aff, int E, int G,
                              int tol_permille, int32_t* new_to_old, int32_t* old_to_new,
                              int64_t* group_loads, int64_t* intra_affinity) {
    moe_status st = balanced_partition(counts, E, G, new_to_old, old_to_new, group_loads);
    if (st != MOE_OK) return st;
    const int S = E / G;
    std::vector<int> grp(E);
    std::vector<int64_t> load(group_loads, group_loads + G);
    for (int g = 0; g < G; ++g)
        for (int j = 0; j < S; ++j) grp[new_to_old[g * S + j]] = g;
    const int64_t cap = *std::max_element(load.begin(), load.end()) * (1000 + tol_permille) / 1000;
    auto A = [&](int a, int b) { return aff[(size_t)a * E + b]; };
    std::vector<int64_t> W((size_t)E * G, 0);
    for (int e = 0; e < E; ++e)
        for (int c = 0; c < E; ++c) W[(size_t)e * G + grp[c]] += A(e, c);

    for (int it = 0; it < 10 * E; ++it) {
        int64_t best = 0;
        int ba = -1, bb = -1;
        for (int a = 0; a < E; ++a) {
            const int p = grp[a];
            const int64_t* Wa = &W[(size_t)a * G];
            for (int b = a + 1; b < E; ++b) {
                const int q = grp[b];
                if (p == q) continue;
                if (load[p] - counts[a] + counts[b] > cap || load[q] - counts[b] + counts[a] > cap)
                    continue;
                const int64_t* Wb = &W[(size_t)b * G];
                // a joins q \ {b}, b joins p \ {a}; each leaves its own set
                const int64_t gain = (Wa[q] - A(a, b)) + (Wb[p] - A(b, a)) - (Wa[p] - A(a, a)) -
                                     (Wb[q] - A(b, b));
                if (gain > best) {  // strict: the first (a, b) in ascending order wins ties
                    best = gain;
                    ba = a;
                    bb = b;
                }
            }
        }
        if (ba < 0) break;
        const int p = grp[ba], q = grp[bb];
        for (int c = 0; c < E; ++c) {
            W[(size_t)c * G + p] += A(c, bb) - A(c, ba);
            W[(size_t)c * G + q] += A(c, ba) - A(c, bb);
        }
        load[p] += counts[bb] - counts[ba];
        load[q] += counts[ba] - counts[bb];
        grp[ba] = q;
        grp[bb] = p;
    }
    int64_t total = 0;
    for (int a = 0; a < E; ++a)
        for (int b = a + 1; b < E; ++b)
            if (grp[a] == grp[b]) total += A(a, b);
    *intra_affinity = total;
    std::vector<int> fill(G, 0);
    for (int e = 0; e < E; ++e) new_to_old[grp[e] * S + fill[grp[e]]++] = e;  // ascending per set
    for (int g = 0; g < G; ++g) group_loads[g] = load[g];
    for (int n = 0; n < E; ++n) old_to_new[new_to_old[n]] = n;
    return MOE_OK;
}

}  // namespace moe
