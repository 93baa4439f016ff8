"""The whole layer for a small batch in one persistent launch
(moe_layer_fused; Moreh EP report, Library optimization: a fused MoE kernel
for small batch sizes; Use of HIP Graphs). On the R1 decode shape (H = 7168,
256 routed experts of intermediate 2048, top-8 by sigmoid score with the
Zipf-skewed router, one shared expert), in bf16 and fp8, at T = 1, 16, 37, 64,
65, 129 and 256 tokens (ragged batches on both sides of the router's row/tile
switch at 64): routing ids and weights, and the output, bit for bit those of the
separate calls (route, permute, expert FFN, combine); the output against the
oracle on every token; the barrier words back at zero; graph replays equal to
eager calls."""
import gc

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_util import DEV, oracle_rows, out_f64, rel_err, say

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp8": 3e-2}


@pytest.fixture(scope="module", params=["bf16", "fp8"])
def r1_layer(request):
    import mixture_experts_layer_select_amd as L
    fmt = request.param
    cfg = mi.CONFIGS[2] if fmt == "bf16" else mi.CONFIGS[4]
    say(f"fused layer {fmt}: drawing 256 experts + shared")
    st = mi.stacked_expert_weights(cfg, range(cfg.E), device=DEV)
    sh = mi.shared_weights(cfg, device=DEV)
    router = dict(w=mi.router_weight(cfg, device=DEV), bias=mi.router_bias(cfg, device=DEV),
                  scoring=L.SIGMOID, renormalize=True)
    layer = L.MoELayer(cfg.fmt, cfg.H, cfg.I, cfg.k, st["w13"], st["w2"], st["w13_scale"], st["w2_scale"],
                       shared=sh, router=router)
    yield fmt, cfg, layer, st, sh
    del layer, st, sh
    gc.collect()
    torch.cuda.empty_cache()


def _barrier_words(layer, T):
    return layer.fused_workspace(T)[:12].view(torch.int32).cpu().tolist()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [1, 16, 37, 64, 65, 129, 256])
def test_fused_layer_matches_separate_calls_and_oracle(r1_layer, T):
    fmt, cfg, layer, st, sh = r1_layer
    x = mi.tokens(cfg, T=T, device=DEV, tensor=20)
    b = layer.forward(x)
    torch.cuda.synchronize()
    ids_s, w_s, out_s = b.topk_ids.clone(), b.topk_w.clone(), b.out.clone()
    b = layer.forward_fused(x)
    torch.cuda.synchronize()
    count, gen, err = _barrier_words(layer, T)
    assert err == 0 and count == 0, f"barrier words {count} {gen} {err}"
    assert torch.equal(b.topk_ids, ids_s)
    assert torch.equal(b.topk_w.view(torch.int32), w_s.view(torch.int32))
    assert torch.equal(b.out.view(torch.int16), out_s.view(torch.int16)), "fused output differs"
    _, ref_ids, ref_w = oracle.route(x.cpu(), layer.router["w"].cpu(), layer.router["bias"].cpu(), cfg.k,
                                     oracle.SIGMOID, True)
    assert np.array_equal(b.topk_ids.cpu().numpy(), ref_ids)
    assert np.abs(b.topk_w.cpu().numpy() - ref_w).max() <= 1e-6
    ref = oracle_rows(x.cpu(), ref_ids, ref_w, st, sh, cfg.k, cfg.E, 0, fmt)
    e = rel_err(out_f64(b.out), ref)
    say(f"  {fmt} T={T}: bit-identical to the separate calls, every token vs oracle {e:.3e}, "
        f"{gen} barriers so far")
    assert e <= TOL[fmt]


@pytest.mark.timeout(300)
def test_fused_layer_graph_replays(r1_layer):
    """Captured once, replayed on new tokens written into the same buffer:
    every replay equals an eager call on those tokens."""
    fmt, cfg, layer, st, sh = r1_layer
    T = 48
    x = mi.tokens(cfg, T=T, device=DEV, tensor=21)
    layer.forward_fused(x)  # eager warm-up: buffers and workspace outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            b = layer.forward_fused(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        x.copy_(mi.tokens(cfg, T=T, device=DEV, tensor=30 + rep))
        g.replay()
        torch.cuda.synchronize()
        got_ids, got_out = b.topk_ids.clone(), b.out.clone()
        layer.forward_fused(x)
        torch.cuda.synchronize()
        assert torch.equal(got_ids, b.topk_ids) and torch.equal(got_out.view(torch.int16), b.out.view(torch.int16))
    assert _barrier_words(layer, T)[2] == 0
    say(f"  {fmt}: 3 graph replays equal to eager calls")
