"""Online rebalancing on the device (Moreh EP report, Inter-GPU load
balancing: activation frequencies re-measured over time and the experts
re-partitioned; SGLang H20 report, Expert Affinity EPLB: top-k co-activation
tracked into an affinity matrix and co-activated experts grouped).

Through the C ABI: per-step activation counts accumulated on the device
(moe_count_accumulate), the co-activation histogram (moe_coactivation), the
host affinity partition and the remap of the gating. Counts, histogram and
partition are integers and must equal the oracle's bit for bit."""
import time

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _clustered_ids(rng, T, k, E, n_clusters, foreign=0.0):
    """Picks mostly from one expert block per token (structure for the
    histogram to show); a fraction of picks replaced by ids outside [0, E)."""
    blk = E // n_clusters
    c = rng.integers(n_clusters, size=T)
    own = np.argsort(rng.random((T, blk)), axis=1)[:, : k - 2] + (c * blk)[:, None]
    other = rng.integers(0, E, size=(T, 2))
    ids = np.concatenate([own, other], axis=1).astype(np.int32)
    if foreign:
        mask = rng.random(ids.shape) < foreign
        ids[mask] = rng.choice(np.array([-1, E, E + 7, -300], np.int32), mask.sum())
    return ids


@pytest.mark.parametrize("T,k,E,foreign", [(4096, 8, 256, 0.0), (256, 8, 256, 0.02),
                                           (1, 1, 1, 0.0), (777, 16, 1024, 0.05),
                                           (300, 3, 5, 0.1)])
def test_coactivation_matches_oracle(T, k, E, foreign):
    import mixture_experts_layer_select_amd as L
    say(f"coactivation T={T} k={k} E={E} foreign={foreign}")
    rng = np.random.default_rng(T + k + E)
    if k >= 3 and E >= k:
        ids = _clustered_ids(rng, T, k, E, max(1, min(8, E // k)), foreign)
    else:
        ids = rng.integers(-1, E + 1, (T, k)).astype(np.int32)
    ids_d = torch.from_numpy(ids).to(DEV)
    hist = torch.zeros((E, E), dtype=torch.int64, device=DEV)
    L.moe_coactivation(ids_d, T, k, E, hist)
    L.moe_coactivation(ids_d[: T // 2], T // 2, k, E, hist)  # accumulates onto the first call
    torch.cuda.synchronize()
    ref = oracle.coactivation(ids, E)
    ref = oracle.coactivation(ids[: T // 2], E, hist=ref)
    assert np.array_equal(hist.cpu().numpy(), ref)


def test_count_accumulate_matches_sum():
    import mixture_experts_layer_select_amd as L
    rng = np.random.default_rng(9)
    n = 70001  # several blocks and a ragged tail
    acc0 = rng.integers(0, 2 ** 40, n).astype(np.int64)
    steps = [rng.integers(0, 2 ** 31 - 1, n).astype(np.int32) for _ in range(3)]
    acc = torch.from_numpy(acc0).to(DEV)
    for c in steps:
        L.moe_count_accumulate(torch.from_numpy(c).to(DEV), n, acc)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc0 + sum(c.astype(np.int64) for c in steps))


def _route(L, cfg, x, w, b):
    T = x.shape[0]
    logits = torch.empty((T, cfg.E), dtype=torch.float32, device=DEV)
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device=DEV)
    tw = torch.empty((T, cfg.k), dtype=torch.float32, device=DEV)
    L.moe_route(x, w, b, L.BF16, T, cfg.H, cfg.E, cfg.k, L.SIGMOID, True, logits, ids, tw)
    return ids


def test_online_rebalance_flow_zipf13():
    """Eight steps of 1024 calibration tokens: gating, the permute's
    per-expert counts accumulated on the device, the co-activation histogram,
    then the affinity partition of 256 experts into 8 sets and the remapped
    gating."""
    import mixture_experts_layer_select_amd as L
    cfg = mi.CONFIGS[5]
    G, S, E, k = cfg.extra["groups"], cfg.E // cfg.extra["groups"], cfg.E, cfg.k
    wr = mi.router_weight(cfg, device=DEV)
    bias = mi.router_bias(cfg, device=DEV)
    xc = mi.calibration_tokens(cfg, device=DEV)
    step_T = 1024
    acc = torch.zeros(E, dtype=torch.int64, device=DEV)
    hist = torch.zeros((E, E), dtype=torch.int64, device=DEV)
    cnt = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    off = torch.empty(E + 2, dtype=torch.int32, device=DEV)
    r2s = torch.empty(step_T * k + step_T, dtype=torch.int32, device=DEV)
    s2r = torch.empty(step_T * k, dtype=torch.int32, device=DEV)
    n = L.moe_permute_workspace_size(step_T, k, E)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    for s in range(xc.shape[0] // step_T):
        say(f"  step {s}: {step_T} tokens")
        ids = _route(L, cfg, xc[s * step_T:(s + 1) * step_T], wr, bias)
        L.moe_permute(ids, step_T, k, 0, E, False, None, L.BF16, 0, L.BF16, cnt, off, r2s, s2r,
                      None, None, ws, n)
        L.moe_count_accumulate(cnt, E, acc)
        L.moe_coactivation(ids, step_T, k, E, hist)
    torch.cuda.synchronize()
    _, ref_ids, _ = oracle.route(xc.cpu(), wr.cpu(), bias.cpu(), k, oracle.SIGMOID, True)
    ref_counts = np.bincount(ref_ids.ravel(), minlength=E).astype(np.int64)
    ref_hist = oracle.coactivation(ref_ids, E)
    assert np.array_equal(acc.cpu().numpy(), ref_counts)
    assert np.array_equal(hist.cpu().numpy(), ref_hist)

    tol = 20  # permille over the balanced partition's largest set
    n2o = torch.empty(E, dtype=torch.int32)
    o2n = torch.empty(E, dtype=torch.int32)
    loads = torch.empty(G, dtype=torch.int64)
    intra = torch.zeros(1, dtype=torch.int64)
    t0 = time.perf_counter()
    L.moe_affinity_partition(acc.cpu(), hist.cpu(), E, G, tol, n2o, o2n, loads, intra)
    host_ms = (time.perf_counter() - t0) * 1e3
    r_n2o, r_o2n, r_loads, r_intra = oracle.affinity_partition(ref_counts, ref_hist, G, tol)
    assert np.array_equal(n2o.numpy(), r_n2o) and np.array_equal(o2n.numpy(), r_o2n)
    assert np.array_equal(loads.numpy(), r_loads) and int(intra[0]) == r_intra
    b_n2o, _, b_loads = oracle.balanced_partition(ref_counts, G)
    b_intra = sum(int(ref_hist[np.ix_(g, g)].sum() - np.trace(ref_hist[np.ix_(g, g)])) // 2
                  for g in b_n2o.reshape(G, S))
    mean = ref_counts.sum() / G
    say(f"  affinity partition {host_ms:.1f} ms on the host: intra-set co-activation "
        f"{b_intra} -> {r_intra}, max/mean load {b_loads.max() / mean:.4f} -> "
        f"{r_loads.max() / mean:.4f}")
    assert r_intra >= b_intra
    assert r_loads.max() <= b_loads.max() * (1000 + tol) // 1000

    # the gating in the new numbering picks the same experts
    n2o_d = n2o.to(DEV)
    wr2, b2 = torch.empty_like(wr), torch.empty_like(bias)
    L.moe_gather_rows(wr, E, wr2, n2o_d, E, cfg.H * 2)
    L.moe_gather_rows(bias, E, b2, n2o_d, E, 4)
    x = mi.tokens(cfg, device=DEV)
    ids_new = _route(L, cfg, x, wr2, b2)
    torch.cuda.synchronize()
    _, ref_old, _ = oracle.route(x.cpu(), wr.cpu(), bias.cpu(), k, oracle.SIGMOID, True)
    assert np.array_equal(ids_new.cpu().numpy(), r_o2n[ref_old])


def test_coactivation_time_r1_batches():
    """Cost of tracking co-activation per step at the R1 batch sizes (printed;
    the bench reports it beside the layer step)."""
    import mixture_experts_layer_select_amd as L
    rng = np.random.default_rng(1)
    for T in (256, 4096):
        ids = torch.from_numpy(_clustered_ids(rng, T, 8, 256, 8)).to(DEV)
        hist = torch.zeros((256, 256), dtype=torch.int64, device=DEV)
        for _ in range(3):
            L.moe_coactivation(ids, T, 8, 256, hist)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(20):
            L.moe_coactivation(ids, T, 8, 256, hist)
        b.record()
        torch.cuda.synchronize()
        say(f"  coactivation T={T}: {a.elapsed_time(b) / 20 * 1e3:.1f} us per call")
        assert int(hist.trace()) == 23 * T * 8
