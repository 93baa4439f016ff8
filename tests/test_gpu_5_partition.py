"""The load-balancing flow of the Moreh EP report (Inter-GPU load balancing):
measure each expert's activation count on a calibration batch, split the 256
experts into 8 balanced sets of 32, reorder them so each set is contiguous,
let the gating emit ids in the new order, and run one GPU's set.

GPU side through the C ABI (moe_route, moe_permute histogram,
moe_balanced_partition, moe_gather_rows, the FFN of the heaviest set); the
oracle checks every step: routing and counts bit-exact, the partition
bit-exact, the remapped routing equal to the old routing mapped through the
permutation, and the set's outputs within 1e-2."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_util import DEV, oracle_rows, out_f64, rel_err, say

pytestmark = pytest.mark.gpu


def _route(L, cfg, x, w, b):
    T = x.shape[0]
    logits = torch.empty((T, cfg.E), dtype=torch.float32, device=DEV)
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device=DEV)
    tw = torch.empty((T, cfg.k), dtype=torch.float32, device=DEV)
    L.moe_route(x, w, b, L.BF16, T, cfg.H, cfg.E, cfg.k, L.SIGMOID, True, logits, ids, tw)
    return ids, tw


def _counts(L, cfg, ids):
    T = ids.shape[0]
    cnt = torch.empty(cfg.E + 1, dtype=torch.int32, device=DEV)
    off = torch.empty(cfg.E + 2, dtype=torch.int32, device=DEV)
    r2s = torch.empty(T * cfg.k + T, dtype=torch.int32, device=DEV)
    s2r = torch.empty(T * cfg.k, dtype=torch.int32, device=DEV)
    n = L.moe_permute_workspace_size(T, cfg.k, cfg.E)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    L.moe_permute(ids, T, cfg.k, 0, cfg.E, False, None, L.BF16, 0, L.BF16, cnt, off, r2s, s2r, None,
                  None, ws, n)
    return cnt[: cfg.E].cpu().to(torch.int64)


@pytest.mark.timeout(600)
def test_balanced_partition_flow_zipf13():
    import mixture_experts_layer_select_amd as L
    cfg = mi.CONFIGS[5]
    G, S = cfg.extra["groups"], cfg.E // cfg.extra["groups"]
    wr = mi.router_weight(cfg, device=DEV)
    bias = mi.router_bias(cfg, device=DEV)

    say("c5 calibration: 8192 tokens")
    xc = mi.calibration_tokens(cfg, device=DEV)
    ids_c, _ = _route(L, cfg, xc, wr, bias)
    counts = _counts(L, cfg, ids_c)
    torch.cuda.synchronize()
    _, ref_ids_c, _ = oracle.route(xc.cpu(), wr.cpu(), bias.cpu(), cfg.k, oracle.SIGMOID, True)
    assert np.array_equal(ids_c.cpu().numpy(), ref_ids_c)
    assert np.array_equal(counts.numpy(), np.bincount(ref_ids_c.ravel(), minlength=cfg.E))

    n2o = torch.empty(cfg.E, dtype=torch.int32)
    o2n = torch.empty(cfg.E, dtype=torch.int32)
    loads = torch.empty(G, dtype=torch.int64)
    L.moe_balanced_partition(counts, cfg.E, G, n2o, o2n, loads)
    r_n2o, r_o2n, r_loads = oracle.balanced_partition(counts.numpy(), G)
    assert np.array_equal(n2o.numpy(), r_n2o) and np.array_equal(loads.numpy(), r_loads)
    mean = counts.sum().item() / G
    contiguous = counts.view(G, S).sum(1)
    say(f"  calibration max/mean: contiguous {contiguous.max().item() / mean:.3f}, "
        f"balanced {loads.max().item() / mean:.3f}")
    assert contiguous.max().item() / mean > 1.3       # skewed popularity really is imbalanced
    assert loads.max().item() / mean < 1.05           # "within 5%" after the partition

    # remap the router rows and the bias to the new expert order
    n2o_d = n2o.to(DEV)
    wr2 = torch.empty_like(wr)
    b2 = torch.empty_like(bias)
    L.moe_gather_rows(wr, cfg.E, wr2, n2o_d, cfg.E, cfg.H * 2)
    L.moe_gather_rows(bias, cfg.E, b2, n2o_d, cfg.E, 4)
    torch.cuda.synchronize()
    assert torch.equal(wr2, wr[n2o_d.long()]) and torch.equal(b2, bias[n2o_d.long()])

    say("c5 evaluation: 512 tokens with the remapped gating")
    x = mi.tokens(cfg, device=DEV)
    ids_new, w_new = _route(L, cfg, x, wr2, b2)
    torch.cuda.synchronize()
    _, ref_old, ref_w = oracle.route(x.cpu(), wr.cpu(), bias.cpu(), cfg.k, oracle.SIGMOID, True)
    got = ids_new.cpu().numpy()
    assert np.array_equal(got, r_o2n[ref_old])       # the same experts, in the new numbering
    assert np.abs(w_new.cpu().numpy() - ref_w).max() <= 1e-6

    ev = np.bincount(got.ravel(), minlength=cfg.E).reshape(G, S).sum(1)
    ev_old = np.bincount(ref_old.ravel(), minlength=cfg.E).reshape(G, S).sum(1)
    heavy = int(ev.argmax())
    say(f"  eval max/mean: contiguous {ev_old.max() / ev_old.mean():.3f}, "
        f"balanced {ev.max() / ev.mean():.3f}; heaviest set {heavy} with {ev[heavy]} rows")

    # a larger held-out batch separates the partition's quality from the
    # sampling noise of 512 tokens (a set's load varies by a few percent there)
    xh = mi.tokens(cfg, T=4096, device=DEV, tensor=mi.XHELD)
    ids_h, _ = _route(L, cfg, xh, wr2, b2)
    ids_h_old, _ = _route(L, cfg, xh, wr, bias)
    torch.cuda.synchronize()
    hv = np.bincount(ids_h.cpu().numpy().ravel(), minlength=cfg.E).reshape(G, S).sum(1)
    hv_old = np.bincount(ids_h_old.cpu().numpy().ravel(), minlength=cfg.E).reshape(G, S).sum(1)
    say(f"  held-out 4096 tokens max/mean: contiguous {hv_old.max() / hv_old.mean():.3f}, "
        f"balanced {hv.max() / hv.mean():.3f}")
    assert hv_old.max() / hv_old.mean() > 1.3
    assert hv.max() / hv.mean() < 1.05  # "within 5%" on a batch large enough to see it

    # one GPU's share: the heaviest set's 32 experts, in the new order
    old_ids = n2o[heavy * S:(heavy + 1) * S].tolist()
    st = mi.stacked_expert_weights(cfg, old_ids, device=DEV)
    layer = L.MoELayer("bf16", cfg.H, cfg.I, cfg.k, st["w13"], st["w2"], expert_base=heavy * S)
    b = layer.forward(x, topk_ids=ids_new, topk_w=w_new)
    torch.cuda.synchronize()
    p = oracle.permute(got, heavy * S, S, False)
    assert np.array_equal(b.counts.cpu().numpy(), p["counts"])
    assert np.array_equal(b.row_to_slot.cpu().numpy(), p["row_to_slot"])
    local_tokens = np.nonzero(((got >= heavy * S) & (got < (heavy + 1) * S)).any(1))[0]
    rows = local_tokens  # every token with a pick in this set
    ref = oracle_rows(x[torch.from_numpy(rows).to(DEV)].cpu(), got[rows],
                      w_new.cpu().numpy()[rows], st, None, cfg.k, S, heavy * S, "bf16")
    e = rel_err(out_f64(b.out[torch.from_numpy(rows).to(DEV)]), ref)
    say(f"  heaviest set: all {len(rows)} local tokens compared, max rel err {e:.3e}")
    assert e <= 1e-2
    # tokens without a pick in this set get an exact zero row
    others = np.setdiff1d(np.arange(cfg.T), local_tokens)
    if len(others):
        assert torch.count_nonzero(b.out[torch.from_numpy(others).to(DEV)]).item() == 0
