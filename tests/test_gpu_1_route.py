"""GPU gating (moe_route) against the oracle: logits, ids bit-exact; weights
within 1e-6. The Moreh EP report (Overview, Parallelization) has the gate
pick 8 of 256 experts per token; the fixed reduction order makes the pick
reproducible bit for bit."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _route_gpu(x, wr, bias, k, scoring, renorm):
    import mixture_experts_layer_select_amd as L
    T, H = x.shape
    E = wr.shape[0]
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    dt = L.F32 if x.dtype == torch.float32 else L.BF16
    L.moe_route(x, wr, bias, dt, T, H, E, k, scoring, renorm, logits, ids, w)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


def _check(x, wr, bias, k, scoring, renorm, rows=None):
    say(f"route T={x.shape[0]} H={x.shape[1]} E={wr.shape[0]} k={k} scoring={scoring} renorm={renorm}")
    gl, gi, gw = _route_gpu(x, wr, bias, k, scoring, renorm)
    xs = x.cpu() if rows is None else x[rows].cpu()
    ol, oi, ow = oracle.route(xs, wr.cpu(), None if bias is None else bias.cpu(), k, scoring, renorm)
    if rows is not None:
        gl, gi, gw = gl[rows], gi[rows], gw[rows]
    assert np.array_equal(gl.view(np.uint32), ol.view(np.uint32)), \
        f"logits differ at {np.argwhere(gl != ol)[:5]}"
    assert np.array_equal(gi, oi)
    assert np.abs(gw - ow).max() <= 1e-6
    return gi


def test_route_tiny_fp32_softmax():
    cfg = mi.CONFIGS[1]
    _check(mi.tokens(cfg, device=DEV), mi.router_weight(cfg, device=DEV), None, cfg.k,
           oracle.SOFTMAX, True)


def test_route_r1_decode_full_size():
    cfg = mi.CONFIGS[2]
    ids = _check(mi.tokens(cfg, device=DEV), mi.router_weight(cfg, device=DEV),
                 mi.router_bias(cfg, device=DEV), cfg.k, oracle.SIGMOID, True)
    hit = len(np.unique(ids))
    say(f"  experts hit: {hit}")
    assert 90 <= hit <= 200


@pytest.mark.parametrize("T,H,E,k,scoring,renorm,bias", [
    (37, 200, 50, 5, oracle.SOFTMAX, True, False),    # ragged H (not a multiple of 8), ragged T, E
    (37, 200, 50, 5, oracle.SOFTMAX, False, True),
    (19, 1032, 64, 7, oracle.SIGMOID, False, True),
    (5, 64, 1, 1, oracle.SIGMOID, True, False),        # one expert
    (33, 512, 16, 16, oracle.SOFTMAX, True, False),    # k == E
    (1, 7168, 256, 256, oracle.SIGMOID, True, True),   # k == E == 256
])
def test_route_shapes(T, H, E, k, scoring, renorm, bias):
    cfg = mi.scaled(mi.CONFIGS[2], T=T, H=H, E=E, zipf_s=1.1 if bias else None)
    x = mi.tokens(cfg, device=DEV)
    wr = mi.router_weight(cfg, device=DEV)
    b = mi.router_bias(cfg, device=DEV) if bias else None
    _check(x, wr, b, k, scoring, renorm)


def test_route_exact_ties_pick_lower_index():
    cfg = mi.scaled(mi.CONFIGS[2], T=64, H=1024, E=64)
    x = mi.tokens(cfg, device=DEV)
    wr = mi.router_weight(cfg, device=DEV)
    for dup, src in [(40, 3), (41, 3), (63, 0), (10, 9)]:
        wr[dup] = wr[src]
    gi = _check(x, wr, None, 8, oracle.SIGMOID, True)
    for t in range(64):
        row = list(gi[t])
        for dup, src in [(40, 3), (41, 3), (63, 0), (10, 9)]:
            if dup in row:
                assert src in row and row.index(src) < row.index(dup)


def test_route_large_batch_sampled():
    cfg = mi.CONFIGS[4]
    x = mi.tokens(cfg, device=DEV)
    rows = np.sort(np.random.default_rng(0).choice(cfg.T, 384, replace=False))
    _check(x, mi.router_weight(cfg, device=DEV), mi.router_bias(cfg, device=DEV), cfg.k,
           oracle.SIGMOID, True, rows=rows)
