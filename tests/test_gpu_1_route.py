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


# Batches of up to 64 bf16 tokens (H % 8 == 0, H <= 8192) take the row
# kernels: one wave per expert and one or two tokens, the whole rows in
# registers. Same fixed-order logits bit for bit.
@pytest.mark.parametrize("T,H,E,k", [
    (1, 7168, 256, 8), (2, 7168, 256, 8), (3, 7168, 256, 8), (4, 7168, 256, 8),
    (5, 7168, 256, 8), (16, 7168, 256, 8), (31, 7168, 256, 8), (32, 7168, 256, 8),
    (64, 7168, 256, 8), (65, 7168, 256, 8),  # the last row-kernel batch, the first tile one
    (7, 8192, 64, 6),     # 16 steps, all with data
    (9, 4104, 36, 4),     # 9 steps, the last one ragged; E not a multiple of 4
    (2, 520, 3, 2),       # 2 steps; fewer experts than a workgroup's waves
])
def test_route_small_batch_rows(T, H, E, k):
    cfg = mi.scaled(mi.CONFIGS[2], T=T, H=H, E=E, zipf_s=1.1)
    _check(mi.tokens(cfg, device=DEV), mi.router_weight(cfg, device=DEV),
           mi.router_bias(cfg, device=DEV), k, oracle.SIGMOID, True)


def test_route_small_batch_rows_match_tile_kernel_on_extreme_values():
    # 32 tokens take the row kernel, 40 the 8 x 8 tile kernel: the first 32
    # tokens' logits must agree bit for bit, also with denormal inputs, huge
    # rows and exact zeros, where the oracle's numpy arithmetic might not flush
    # the way the GPU does
    cfg = mi.scaled(mi.CONFIGS[2], T=40, H=7168, E=256, zipf_s=1.1)
    x = mi.tokens(cfg, device=DEV)
    wr = mi.router_weight(cfg, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(5)
    tiny = torch.full((40, 7168), 1e-39, dtype=torch.float32)
    mask = torch.rand((40, 7168), generator=g) < 0.1
    x = torch.where(mask.to(DEV), tiny.to(DEV), x.float()).to(torch.bfloat16)
    x[3] = 0.0
    x[4, 100:] = 0.0
    wr = wr.clone()
    wr[::16] *= 1000.0
    wr[7] = (wr[7].float() * 1e-38).to(torch.bfloat16)
    b = mi.router_bias(cfg, device=DEV)
    l40, i40, w40 = _route_gpu(x, wr, b, 8, oracle.SIGMOID, True)
    l32, i32, w32 = _route_gpu(x[:32].contiguous(), wr, b, 8, oracle.SIGMOID, True)
    assert np.array_equal(l32.view(np.uint32), l40[:32].view(np.uint32))
    assert np.array_equal(i32, i40[:32])
    assert np.array_equal(w32.view(np.uint32), w40[:32].view(np.uint32))
