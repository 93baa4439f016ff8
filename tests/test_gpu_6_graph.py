"""The whole layer captured in a HIP graph ([Moreh-EP] Use of HIP Graphs:
the decode step is launch-bound, so the pages replay captured launches).
Every step of the path is deterministic (fixed reduction orders, no
atomics in any sum), so each replay must equal an eager run on the same
tokens bit for bit. Three replays with new tokens copied in before each,
with eager work and synchronisations between them."""
import pytest
import torch

import moe_inputs as mi
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,T", [("bf16", 48), ("fp8", 48), ("bf16", 4096)])
def test_layer_graph_replays_match_eager(fmt, T):
    # T = 4096 routes through moe_route_select (the layer's large-batch gating)
    import mixture_experts_layer_select_amd as L
    base = mi.CONFIGS[2] if fmt == "bf16" else mi.CONFIGS[4]
    cfg = mi.scaled(base, T=T, H=512, E=24, I=256, k=4, cid=160)
    say(f"graph replay {fmt} T={cfg.T} H={cfg.H} E={cfg.E} I={cfg.I} k={cfg.k}")
    st = mi.stacked_expert_weights(cfg, range(cfg.E), device=DEV)
    sh = mi.shared_weights(cfg, device=DEV)
    r = dict(w=mi.router_weight(cfg, device=DEV), bias=mi.router_bias(cfg, device=DEV),
             scoring=L.SIGMOID, renormalize=True)
    layer = L.MoELayer(cfg.fmt, cfg.H, cfg.I, cfg.k, st["w13"], st["w2"], st["w13_scale"],
                       st["w2_scale"], shared=sh, router=r)
    x = mi.tokens(cfg, device=DEV)
    batches = [mi.normal(tuple(x.shape), cfg.x_std, 9100 + i, DEV, x.dtype) for i in range(3)]

    assert layer.uses_route_select(T) == (T >= layer.ROUTE_SELECT_MIN_T)
    layer.forward(x)  # eager warm-up: buffers and one-time library set-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            b = layer.forward(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for i, xi in enumerate(batches):
        x.copy_(xi)
        g.replay()
        torch.cuda.synchronize()
        got_out, got_ids = b.out.clone(), b.topk_ids.clone()
        layer.forward(x)  # eager on the same tokens, same buffers
        torch.cuda.synchronize()
        assert torch.equal(got_ids, b.topk_ids), f"replay {i}: routing differs"
        assert torch.equal(got_out, b.out), f"replay {i}: output differs"
        assert torch.count_nonzero(got_out).item() > 0
