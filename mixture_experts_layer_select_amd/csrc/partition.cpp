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

}  // namespace moe
