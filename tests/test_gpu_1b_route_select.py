"""GPU gating through moe_route_select (approximate MFMA logits, a rigorous
bound, fixed-order logits for the remaining candidates only) against
moe_route, which computes every fixed-order logit: ids and weights bit for bit,
on the R1 shapes (decode batch, the 16384-token batch, the 8192-token
calibration batch), ragged shapes, exact ties and k == E; and against the
oracle on sampled tokens of the large batch. The Moreh EP report (Overview,
Parallelization) has the gate pick 8 of 256 experts per token."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _route(x, wr, bias, k, scoring, renorm):
    import mixture_experts_layer_select_amd as L
    T, H = x.shape
    E = wr.shape[0]
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    L.moe_route(x, wr, bias, L.BF16, T, H, E, k, scoring, renorm, logits, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def _select(x, wr, bias, k, scoring, renorm, ws_bytes=None):
    import mixture_experts_layer_select_amd as L
    T, H = x.shape
    E = wr.shape[0]
    need = L.moe_route_select_workspace_size(T, E)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    ids = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    L.moe_route_select(x, wr, bias, L.BF16, T, H, E, k, scoring, renorm, ids, w, ws,
                       need if ws_bytes is None else ws_bytes)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def _same_as_route(x, wr, bias, k, scoring, renorm):
    say(f"route_select T={x.shape[0]} H={x.shape[1]} E={wr.shape[0]} k={k} scoring={scoring} renorm={renorm}")
    ri, rw = _route(x, wr, bias, k, scoring, renorm)
    si, sw = _select(x, wr, bias, k, scoring, renorm)
    assert np.array_equal(si, ri), f"ids differ at tokens {np.nonzero((si != ri).any(axis=1))[0][:5]}"
    assert np.array_equal(sw.view(np.uint32), rw.view(np.uint32))
    return si, sw


def test_route_select_large_batch_all_tokens_and_oracle_sample():
    cfg = mi.CONFIGS[4]
    x = mi.tokens(cfg, device=DEV)
    wr = mi.router_weight(cfg, device=DEV)
    b = mi.router_bias(cfg, device=DEV)
    si, sw = _same_as_route(x, wr, b, cfg.k, oracle.SIGMOID, True)
    rows = np.sort(np.random.default_rng(1).choice(cfg.T, 256, replace=False))
    _, oi, ow = oracle.route(x[rows].cpu(), wr.cpu(), b.cpu(), cfg.k, oracle.SIGMOID, True)
    assert np.array_equal(si[rows], oi)
    assert np.abs(sw[rows] - ow).max() <= 1e-6


def test_route_select_decode_batch():
    cfg = mi.CONFIGS[2]
    _same_as_route(mi.tokens(cfg, device=DEV), mi.router_weight(cfg, device=DEV),
                   mi.router_bias(cfg, device=DEV), cfg.k, oracle.SIGMOID, True)


def test_route_select_calibration_batch():
    cfg = mi.scaled(mi.CONFIGS[5], T=8192)
    _same_as_route(mi.tokens(cfg, device=DEV), mi.router_weight(cfg, device=DEV),
                   mi.router_bias(cfg, device=DEV), cfg.k, oracle.SIGMOID, True)


@pytest.mark.parametrize("T,H,E,k,scoring,renorm,bias", [
    (37, 224, 50, 5, oracle.SOFTMAX, True, False),     # ragged T and E
    (19, 1024, 64, 7, oracle.SIGMOID, False, True),
    (5, 64, 1, 1, oracle.SIGMOID, True, False),         # one expert
    (33, 512, 16, 16, oracle.SOFTMAX, True, False),     # k == E
    (1, 7168, 256, 256, oracle.SIGMOID, True, True),    # k == E == 256
    (77, 7168, 256, 8, oracle.SIGMOID, True, True),     # ragged T at R1 width
    (130, 8192, 200, 6, oracle.SIGMOID, False, True),   # largest H, E not a multiple of 64
])
def test_route_select_shapes(T, H, E, k, scoring, renorm, bias):
    cfg = mi.scaled(mi.CONFIGS[2], T=T, H=H, E=E, zipf_s=1.1 if bias else None)
    x = mi.tokens(cfg, device=DEV)
    wr = mi.router_weight(cfg, device=DEV)
    b = mi.router_bias(cfg, device=DEV) if bias else None
    _same_as_route(x, wr, b, k, scoring, renorm)


def test_route_select_exact_ties_pick_lower_index():
    cfg = mi.scaled(mi.CONFIGS[2], T=64, H=1024, E=64)
    x = mi.tokens(cfg, device=DEV)
    wr = mi.router_weight(cfg, device=DEV)
    for dup, src in [(40, 3), (41, 3), (63, 0), (10, 9)]:
        wr[dup] = wr[src]
    si, _ = _same_as_route(x, wr, None, 8, oracle.SIGMOID, True)
    for t in range(64):
        row = list(si[t])
        for dup, src in [(40, 3), (41, 3), (63, 0), (10, 9)]:
            if dup in row:
                assert src in row and row.index(src) < row.index(dup)


def test_route_select_rejects_what_it_does_not_cover():
    import mixture_experts_layer_select_amd as L
    cfg = mi.scaled(mi.CONFIGS[2], T=8, H=1024, E=32)
    x = mi.tokens(cfg, device=DEV)
    wr = mi.router_weight(cfg, device=DEV)
    ids = torch.empty((8, 4), dtype=torch.int32, device=DEV)
    w = torch.empty((8, 4), dtype=torch.float32, device=DEV)
    ws = torch.empty(L.moe_route_select_workspace_size(8, 32), dtype=torch.uint8, device=DEV)
    cases = [
        (dict(dt=L.F32), "MOE_ERR_UNSUPPORTED"),
        (dict(H=1000), "MOE_ERR_UNSUPPORTED"),
        (dict(scoring=L.SOFTMAX, renorm=False), "MOE_ERR_UNSUPPORTED"),
        (dict(ws_bytes=ws.numel() - 1), "MOE_ERR_WORKSPACE"),
    ]
    for over, status in cases:
        a = dict(dt=L.BF16, H=1024, scoring=L.SIGMOID, renorm=True, ws_bytes=ws.numel())
        a.update(over)
        with pytest.raises(L.MoEError) as e:
            L.moe_route_select(x, wr, None, a["dt"], 8, a["H"], 32, 4, a["scoring"], a["renorm"], ids, w,
                               ws, a["ws_bytes"])
        assert e.value.status == status


def test_route_select_denormal_inputs_and_large_weights():
    """Denormal bf16 activations and weights next to router rows scaled up to
    |w| of about 20: the bound covers a flushed tiny input times a large
    weight, so the selection still matches moe_route (and the oracle's ids)
    bit for bit, with close logit races among the scaled rows."""
    T, H, E, k = 600, 1024, 64, 6
    g = torch.Generator(device=DEV)
    g.manual_seed(4242)
    x = torch.randn((T, H), generator=g, device=DEV)
    wr = torch.randn((E, H), generator=g, device=DEV) * 0.006
    # a tenth of the activations become bf16 denormals (+-1..127 x 2^-133)
    tiny = torch.randint(1, 128, (T, H), generator=g, device=DEV).float() * 2.0 ** -133
    sign = torch.where(torch.rand((T, H), generator=g, device=DEV) < 0.5, -1.0, 1.0)
    mask = torch.rand((T, H), generator=g, device=DEV) < 0.1
    x = torch.where(mask, tiny * sign, x).to(torch.bfloat16)
    # eight experts with large weights (|w| up to ~20), a few denormal weights
    wr[::8] *= 1000.0
    wmask = torch.rand((E, H), generator=g, device=DEV) < 0.05
    wr = torch.where(wmask, torch.full_like(wr, 3.0 * 2.0 ** -130), wr).to(torch.bfloat16)
    xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
    assert ((xb & 0x7f80) == 0).sum() > T * H // 20  # denormals really are there
    si, sw = _same_as_route(x, wr, None, k, oracle.SIGMOID, True)
    _, oi, _ = oracle.route(x.cpu(), wr.cpu(), None, k, oracle.SIGMOID, True)
    assert np.array_equal(si, oi)
