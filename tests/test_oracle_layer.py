"""Pins of the oracle's whole layer against the dense-masked definition.

The layer (Moreh EP report, Overview and Parallelization): each token is sent
to the k experts its gate picks, and an always-on shared expert runs on every
token. The plain definition is out[t] = sum_e [e in TopK_t] w_te FFN_e(x_t)
+ FFN_shared(x_t); the sparse route/permute/FFN/combine pipeline must equal
it. Here every expert is applied to every token with fp64 torch matmuls and
the non-picked ones are masked out.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi


def _f64(a):
    import oracle
    a = oracle.as_np(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(oracle.bf16_to_f32(a).astype(np.float64))
    return torch.from_numpy(a.astype(np.float64))


def _deq(orc, d, key):
    if d.get(key + "_scale") is None:
        return _f64(d[key])
    codes = orc.as_np(d[key])
    s = orc.as_np(d[key + "_scale"]).astype(np.float64)
    v = orc.e4m3_decode(codes).astype(np.float64)
    return torch.from_numpy(v * np.kron(s, np.ones((128, 128))))


def _swiglu_mlp(x64, w13, w2, I, quant=None):
    g = x64 @ w13[:I].T
    u = x64 @ w13[I:].T
    a = g / (1 + torch.exp(-g)) * u
    if quant is not None:
        a = quant(a)
    return a @ w2.T


def _dense_layer(orc, x, ids, w, experts, shared, I, fp8=False):
    T = x.shape[0]
    if fp8:
        codes, sc = orc.quantize_1x128(orc.bf16_to_f32(orc.as_np(x)))
        x64 = torch.from_numpy(orc.e4m3_decode(codes).astype(np.float64) * np.repeat(sc, 128, 1))

        def quant(a):
            c, s = orc.quantize_1x128(a.numpy().astype(np.float32))
            return torch.from_numpy(orc.e4m3_decode(c).astype(np.float64) * np.repeat(s, 128, 1))
    else:
        x64 = _f64(x)
        quant = None
    out = torch.zeros((T, x64.shape[1]), dtype=torch.float64)
    for e, d in enumerate(experts):
        y = _swiglu_mlp(x64, _deq(orc, d, "w13"), _deq(orc, d, "w2"), I, quant)
        mask = torch.from_numpy((ids == e).astype(np.float64) * w.astype(np.float64)).sum(1, keepdim=True)
        out += mask * y
    if shared is not None:
        out += _swiglu_mlp(x64, _deq(orc, shared, "w13"), _deq(orc, shared, "w2"), I, quant)
    return out.numpy()


def test_tiny_fp32_layer_equals_dense_definition(orc):
    cfg = mi.CONFIGS[1]
    x, wr = mi.tokens(cfg), mi.router_weight(cfg)
    experts = [mi.expert_weights(cfg, e) for e in range(cfg.E)]
    res = orc.moe_layer(x, cfg.k, experts, None, wr=wr, scoring=orc.SOFTMAX)
    ref = _dense_layer(orc, x, res["topk_ids"], res["topk_w"], experts, None, cfg.I)
    assert np.allclose(res["out64"], ref, rtol=1e-12, atol=1e-18)
    assert res["out"].dtype == np.float32
    assert np.array_equal(res["out"], res["out64"].astype(np.float32))


def test_bf16_layer_with_shared_expert_equals_dense_definition(orc):
    cfg = mi.scaled(mi.CONFIGS[2], T=19, H=256, E=8, I=128, k=3)
    x, wr, b = mi.tokens(cfg), mi.router_weight(cfg), mi.router_bias(cfg)
    experts = [mi.expert_weights(cfg, e) for e in range(cfg.E)]
    shared = mi.shared_weights(cfg)
    res = orc.moe_layer(x, cfg.k, experts, shared, wr=wr, bias=b, scoring=orc.SIGMOID)
    ref = _dense_layer(orc, x, res["topk_ids"], res["topk_w"], experts, shared, cfg.I)
    assert np.allclose(res["out64"], ref, rtol=1e-12, atol=1e-15)
    assert np.array_equal(res["out"], orc.bf16_round(res["out64"]))


def test_one_expert_top1_is_a_plain_swiglu_mlp(orc):
    cfg = mi.scaled(mi.CONFIGS[2], T=7, H=128, E=1, I=64, k=1)
    x, wr = mi.tokens(cfg), mi.router_weight(cfg)
    d = mi.expert_weights(cfg, 0)
    res = orc.moe_layer(x, 1, [d], None, wr=wr, scoring=orc.SIGMOID)
    assert np.all(res["topk_ids"] == 0) and np.all(res["topk_w"] == 1.0)
    ref = torch.nn.functional.silu(_f64(x) @ _f64(d["w13"])[:64].T) * (_f64(x) @ _f64(d["w13"])[64:].T)
    ref = torch.matmul(ref, _f64(d["w2"]).T).numpy()
    assert np.allclose(res["out64"], ref, rtol=1e-12, atol=1e-15)


def test_fp8_layer_equals_dense_definition_with_the_same_quantisation(orc):
    cfg = mi.scaled(mi.CONFIGS[4], T=13, H=256, E=4, I=256, k=2)
    x, wr, b = mi.tokens(cfg), mi.router_weight(cfg), mi.router_bias(cfg)
    experts = [mi.expert_weights(cfg, e) for e in range(cfg.E)]
    shared = mi.shared_weights(cfg)
    res = orc.moe_layer(x, cfg.k, experts, shared, wr=wr, bias=b, scoring=orc.SIGMOID, fmt=orc.FP8)
    ref = _dense_layer(orc, x, res["topk_ids"], res["topk_w"], experts, shared, cfg.I, fp8=True)
    assert np.allclose(res["out64"], ref, rtol=1e-9, atol=1e-12)


def test_fp8_layer_stays_within_quantisation_error_of_bf16(orc):
    cfg = mi.scaled(mi.CONFIGS[4], T=16, H=512, E=4, I=256, k=2)
    x, wr, b = mi.tokens(cfg), mi.router_weight(cfg), mi.router_bias(cfg)
    bf = [mi.expert_weights(cfg, e, fmt="bf16") for e in range(cfg.E)]
    f8 = [mi.expert_weights(cfg, e, fmt="fp8") for e in range(cfg.E)]
    sb, s8 = mi.shared_weights(cfg, fmt="bf16"), mi.shared_weights(cfg, fmt="fp8")
    rb = orc.moe_layer(x, 2, bf, sb, wr=wr, bias=b)
    r8 = orc.moe_layer(x, 2, f8, s8, wr=wr, bias=b, fmt=orc.FP8)
    assert np.array_equal(rb["topk_ids"], r8["topk_ids"])
    rel = np.abs(r8["out64"] - rb["out64"]).max() / np.abs(rb["out64"]).max()
    # e4m3 keeps 3 mantissa bits: a few percent of the output's range, not more
    assert 1e-3 < rel < 0.1


def test_ep_share_partial_combine(orc):
    """One GPU's expert share: only local picks contribute; non-local slots map to -1."""
    cfg = mi.scaled(mi.CONFIGS[3], H=128, I=128, extra=dict(global_T=64), E_local=4, E=16)
    ids, w, recv = mi.ep_share_routing(cfg)
    x = mi.ep_share_tokens(cfg, len(recv))
    experts = [mi.expert_weights(cfg, e) for e in range(cfg.E_local)]
    res = orc.moe_layer(x, cfg.k, experts, None, topk_ids=ids, topk_w=w, E_local=4, fmt=orc.FP8)
    idn = ids.numpy()
    assert np.all((idn < 4).any(1))                        # every received token has a local pick
    assert np.array_equal(res["slot_to_row"] >= 0, (idn < 4).ravel())
    ref = _dense_layer(orc, x, idn, w.numpy(), experts, None, cfg.I, fp8=True)
    assert np.allclose(res["out64"], ref, rtol=1e-9, atol=1e-12)
