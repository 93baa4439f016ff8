"""Oracle pins for the expert-affinity step ([SGLang-H20] Expert Affinity
EPLB: top-k co-activation tracked into an affinity matrix, highly
co-activated experts grouped together; [Moreh-EP] Inter-GPU load balancing:
the balanced grouping it starts from). The page gives no algorithm for the
adjustment; the oracle's reading (swaps under a load cap) is pinned here by
properties a wrong implementation breaks: a planted block structure it must
recover, the load cap, local optimality checked by brute force over every
swap, and the reduction to the plain balanced partition."""
import numpy as np
import pytest

import oracle


def _topk_ids(rng, T, k, E):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def test_coactivation_is_onehot_gram_matrix():
    rng = np.random.default_rng(3)
    T, k, E = 200, 6, 20
    ids = _topk_ids(rng, T, k, E)
    M = np.zeros((T, E), np.int64)
    M[np.repeat(np.arange(T), k), ids.ravel()] = 1
    assert np.array_equal(oracle.coactivation(ids, E), M.T @ M)


def test_coactivation_accumulates_and_ignores_foreign_ids():
    ids = np.array([[0, 1, 2], [1, 2, 5], [0, -1, 3]], np.int32)
    h = oracle.coactivation(ids, 4)
    want = np.array([[2, 1, 1, 1],
                     [1, 2, 2, 0],
                     [1, 2, 2, 0],
                     [1, 0, 0, 1]], np.int64)
    assert np.array_equal(h, want)
    assert np.array_equal(oracle.coactivation(ids, 4, hist=h), 2 * want)


def test_coactivation_duplicate_picks_count_on_the_diagonal_only():
    h = oracle.coactivation(np.array([[0, 0, 3]], np.int32), 4)
    assert h[0, 0] == 2 and h[3, 3] == 1 and h[0, 3] == 2 and h[3, 0] == 2 and h[0, 1] == 0


def _intra(aff, n2o, G):
    S = len(n2o) // G
    tot = 0
    for g in range(G):
        m = n2o[g * S:(g + 1) * S]
        for i in range(S):
            for j in range(i + 1, S):
                tot += aff[m[i], m[j]]
    return tot


def _check_result(counts, aff, G, tol, n2o, o2n, loads, intra):
    E = len(counts)
    S = E // G
    assert sorted(n2o.tolist()) == list(range(E))
    assert np.array_equal(o2n[n2o], np.arange(E))
    grp = np.empty(E, int)
    for g in range(G):
        assert list(n2o[g * S:(g + 1) * S]) == sorted(n2o[g * S:(g + 1) * S])
        grp[n2o[g * S:(g + 1) * S]] = g
        assert loads[g] == counts[n2o[g * S:(g + 1) * S]].sum()
    _, _, base_loads = oracle.balanced_partition(counts, G)
    cap = int(base_loads.max()) * (1000 + tol) // 1000
    assert loads.max() <= cap
    assert intra == _intra(aff, n2o, G)
    # local optimality: no swap keeps both loads within the cap and raises the total
    for a in range(E):
        for b in range(a + 1, E):
            p, q = grp[a], grp[b]
            if p == q:
                continue
            if loads[p] - counts[a] + counts[b] > cap or loads[q] - counts[b] + counts[a] > cap:
                continue
            g2 = grp.copy()
            g2[a], g2[b] = q, p
            tot2 = sum(aff[x, y] for x in range(E) for y in range(x + 1, E) if g2[x] == g2[y])
            assert tot2 <= intra, (a, b)


def test_affinity_partition_recovers_planted_blocks():
    E, G = 8, 2
    counts = np.full(E, 10, np.int64)
    aff = np.ones((E, E), np.int64)
    aff[:4, :4] = 50
    aff[4:, 4:] = 50
    np.fill_diagonal(aff, 0)
    n2o, o2n, loads, intra = oracle.affinity_partition(counts, aff, G, 0)
    groups = {tuple(n2o[:4].tolist()), tuple(n2o[4:].tolist())}  # group order is free
    assert groups == {(0, 1, 2, 3), (4, 5, 6, 7)}
    assert loads.tolist() == [40, 40] and intra == 2 * 6 * 50
    # the balanced start alone interleaves them (LPT deals equal counts in id order)
    b_n2o, _, _ = oracle.balanced_partition(counts, G)
    assert b_n2o.tolist() == [0, 2, 4, 6, 1, 3, 5, 7]
    _check_result(counts, aff, G, 0, n2o, o2n, loads, intra)


@pytest.mark.parametrize("seed,E,G,tol", [(0, 12, 3, 0), (1, 16, 4, 20), (2, 16, 2, 50), (3, 24, 4, 10)])
def test_affinity_partition_properties(seed, E, G, tol):
    rng = np.random.default_rng(seed)
    counts = rng.zipf(1.3, E).clip(max=500).astype(np.int64) * 10 + rng.integers(0, 10, E)
    ids = _topk_ids(rng, 300, 4, E)
    aff = oracle.coactivation(ids, E)
    np.fill_diagonal(aff, 0)
    n2o, o2n, loads, intra = oracle.affinity_partition(counts, aff, G, tol)
    _check_result(counts, aff, G, tol, n2o, o2n, loads, intra)
    b_n2o, _, _ = oracle.balanced_partition(counts, G)
    assert intra >= _intra(aff, b_n2o, G)


def test_affinity_partition_without_affinity_is_the_balanced_partition():
    rng = np.random.default_rng(7)
    counts = rng.integers(1, 1000, 32).astype(np.int64)
    n2o, o2n, loads, intra = oracle.affinity_partition(counts, np.zeros((32, 32), np.int64), 4, 0)
    b = oracle.balanced_partition(counts, 4)
    assert np.array_equal(n2o, b[0]) and np.array_equal(loads, b[2]) and intra == 0
