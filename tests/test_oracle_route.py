"""Pins of the oracle's gating step: logits, top-k selection and weights.

The Moreh EP report (Overview) has a lightweight gating network pick a small
subset of experts per token; Parallelization fixes 8 of 256 for R1. The pages
fix no precision, order, score function or tie rule: the oracle's readings are
a fixed fp32 reduction order, selection on the logit with ties to the lower
expert index, and softmax/sigmoid weights renormalised over the picks.
"""
import json
import os

import numpy as np
import pytest
import torch

import moe_inputs as mi

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _dense(spec, H, dtype):
    if spec == "ones":
        a = np.ones(H, np.float32)
    else:
        a = np.zeros(H, np.float32)
        for h, v in spec:
            a[h] = v
    if dtype == "bf16":
        bits = a.view(np.uint32)
        assert np.all(bits & 0xFFFF == 0), "golden values must be bf16-exact"
        return (bits >> 16).astype(np.uint16)[None]
    return a[None]


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLD, "router_order.json")))["cases"],
                         ids=lambda c: c["name"])
def test_router_order_golden(orc, case):
    H = case["H"]
    x = _dense(case["x"], H, case["dtype"])
    w = _dense(case["w"], H, case["dtype"])
    b = None if case["bias"] is None else np.array([case["bias"]], np.float32)
    l = orc.router_logits(x, w, b)
    assert l.shape == (1, 1)
    assert l[0, 0] == np.float32(case["expected"])


def test_router_logits_exact_on_integer_data(orc):
    """Small integers: every product and partial sum is exact, so the logit is the integer dot."""
    rng = np.random.default_rng(0)
    T, H, E = 5, 1000, 7
    xi = rng.integers(-8, 9, (T, H))
    wi = rng.integers(-8, 9, (E, H))
    bias = rng.integers(-50, 50, E).astype(np.float32)
    x = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(wi.astype(np.float32)).to(torch.bfloat16)
    l = orc.router_logits(x, w, bias)
    assert np.array_equal(l, (xi @ wi.T + bias).astype(np.float32))


def test_router_logits_error_bound(orc):
    """|l - exact| <= gamma_n * sum|x w| with n = terms per partial + tree depth + bias add."""
    cfg = mi.scaled(mi.CONFIGS[2], T=24, E=32)
    x = mi.tokens(cfg)
    wr = mi.router_weight(cfg)
    b = mi.router_bias(cfg)
    l = orc.router_logits(x, wr, b)
    xd, wd = x.double().numpy(), wr.double().numpy()
    exact = xd @ wd.T + b.double().numpy()
    n = cfg.H // 512 * 8 + 6 + 1
    u = 2.0 ** -24
    bound = n * u / (1 - n * u) * (np.abs(xd) @ np.abs(wd).T + np.abs(b.double().numpy()))
    err = np.abs(l.astype(np.float64) - exact)
    assert np.all(err <= bound)
    assert err.max() > 0  # fp32 rounding is really happening


def _brute_select(l, k):
    T, E = l.shape
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -l[t].astype(np.float64)))  # logit desc, index asc
        ids[t] = order[:k]
    return ids


@pytest.mark.parametrize("E,k", [(16, 2), (256, 8), (5, 5), (1, 1)])
def test_select_matches_stable_sort(orc, E, k):
    rng = np.random.default_rng(E * 31 + k)
    l = rng.standard_normal((40, E)).astype(np.float32)
    l[:, : E // 2] = np.round(l[:, : E // 2] * 4) / 4  # many exact ties
    ids, w = orc.select(l, k, orc.SIGMOID, True)
    assert np.array_equal(ids, _brute_select(l, k))
    # k distinct ids in range, logits non-increasing along the picks
    for t in range(40):
        assert len(set(ids[t])) == k and ids[t].min() >= 0 and ids[t].max() < E
        assert np.all(np.diff(l[t, ids[t]]) <= 0)


def test_select_matches_torch_topk_without_ties(orc):
    l = torch.randn(64, 256, generator=torch.Generator().manual_seed(5))
    ids, _ = orc.select(l.numpy(), 8, orc.SOFTMAX, True)
    v, i = torch.topk(l, 8, dim=1)
    assert np.array_equal(ids, i.numpy().astype(np.int32))


def test_duplicated_router_rows_tie_to_lower_index(orc):
    cfg = mi.CONFIGS[1]
    x = mi.tokens(cfg)
    wr = mi.router_weight(cfg).clone()
    wr[9] = wr[3]   # expert 9 duplicates expert 3: equal logits for every token
    wr[12] = wr[3]
    l, ids, w = orc.route(x, wr, None, 3, orc.SOFTMAX, True)
    assert np.array_equal(l[:, 3], l[:, 9])
    for t in range(cfg.T):
        picked = list(ids[t])
        if 9 in picked:
            assert 3 in picked and picked.index(3) < picked.index(9)
        if 12 in picked:
            assert 9 in picked
    assert np.array_equal(ids, _brute_select(l, 3))


def test_weights_closed_forms(orc):
    rng = np.random.default_rng(2)
    l = (rng.standard_normal((50, 32)) * 3).astype(np.float32)
    k = 4
    # softmax renormalised == full softmax restricted to the picks and rescaled
    ids, w = orc.select(l, k, orc.SOFTMAX, True)
    ld = l.astype(np.float64)
    full = np.exp(ld - ld.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, ids.astype(np.int64), 1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=0, atol=1e-7)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) <= 1e-6)
    # softmax without renormalisation == full softmax at the picks
    _, w0 = orc.select(l, k, orc.SOFTMAX, False)
    assert np.allclose(w0, sel, rtol=0, atol=1e-7)
    # sigmoid: proportional to 1/(1+e^-l); unnormalised equals the scores
    ids, w = orc.select(l, k, orc.SIGMOID, True)
    s = 1 / (1 + np.exp(-np.take_along_axis(ld, ids.astype(np.int64), 1)))
    assert np.allclose(w, s / s.sum(1, keepdims=True), rtol=0, atol=1e-7)
    _, w1 = orc.select(l, k, orc.SIGMOID, False)
    assert np.allclose(w1, s, rtol=0, atol=1e-7)
    # k == E with renormalised softmax is the plain softmax
    ids, w = orc.select(l, 32, orc.SOFTMAX, True)
    assert np.allclose(np.take_along_axis(full, ids.astype(np.int64), 1), w, atol=1e-7)


def test_zipf_bias_skews_routing(orc):
    """The synthetic bias gives the R1 decode batch the spread of hit experts
    the workload recipe targets (about half the experts hit at T=256)."""
    cfg = mi.scaled(mi.CONFIGS[2], T=256, E=256)
    x = mi.tokens(cfg)[:, :1024].contiguous()
    sub = mi.scaled(cfg, H=1024)
    wr = mi.router_weight(cfg)[:, :1024].contiguous()
    b = mi.router_bias(cfg) * np.sqrt(1024 / 7168)
    _, ids, _ = orc.route(x, wr, b, 8, orc.SIGMOID, True)
    hit = len(np.unique(ids))
    assert 90 <= hit <= 180
    counts = np.bincount(ids.ravel(), minlength=256)
    assert counts.max() >= 4 * np.median(counts[counts > 0])
