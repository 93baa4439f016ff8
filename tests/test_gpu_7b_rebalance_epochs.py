"""Continuous rebalancing over several epochs (Moreh EP report, Inter-GPU
load balancing: activation frequencies are measured again from time to time
and the permutation regenerated). The token distribution drifts between
epochs (each epoch's tokens lean toward a different set of 16 experts), so
the partition has to change.

Per epoch, through the C ABI: gating with the serving copy of the router (in
the current expert numbering), per-step counts accumulated on the device,
the balanced partition on the host library, then the remap of the serving
router rows, bias, fp8 expert weights and their 128x128 block scales
(moe_gather_rows), and the permutation composed with the previous ones.
Checked every epoch against the oracle, which only ever sees the original
numbering: ids equal the oracle's mapped into the current numbering, counts
and partition bit-exact, every remapped tensor equal to the original one
indexed through the composed permutation, and the heaviest set's layer
output (every token with a pick in it) within the fp8 tolerance."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_util import DEV, oracle_rows, out_f64, rel_err, say

pytestmark = pytest.mark.gpu

EPOCHS, STEPS, STEP_T, EVAL_T = 3, 4, 1024, 512


def _drifted_tokens(cfg, wr, epoch, T, tensor):
    """N(0,1) tokens plus a shift along the sum of 16 seeded router rows: those
    experts' logits rise by about one noise standard deviation."""
    g = torch.Generator(device="cpu")
    g.manual_seed(mi.seed(cfg.cid, 40 + epoch))
    pref = torch.randperm(cfg.E, generator=g)[:16]
    d = wr[pref.to(DEV)].float().sum(dim=0)
    x = mi.normal((T, cfg.H), 1.0, mi.seed(cfg.cid, tensor, epoch), DEV, torch.float32)
    return (x + 4.0 * d / d.norm()).to(torch.bfloat16)


def _route(L, cfg, x, w, b):
    T = x.shape[0]
    logits = torch.empty((T, cfg.E), dtype=torch.float32, device=DEV)
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device=DEV)
    tw = torch.empty((T, cfg.k), dtype=torch.float32, device=DEV)
    L.moe_route(x, w, b, L.BF16, T, cfg.H, cfg.E, cfg.k, L.SIGMOID, True, logits, ids, tw)
    return ids, tw


def _gather(L, src, idx_d):
    """dst[i] = src[idx[i]] over the first dimension, through the library."""
    dst = torch.empty_like(src)
    n = src.shape[0]
    L.moe_gather_rows(src, n, dst, idx_d, n, src[0].numel() * src.element_size())
    return dst


@pytest.mark.timeout(900)
def test_rebalance_three_epochs_remap_fp8_experts():
    import mixture_experts_layer_select_amd as L
    cfg = mi.CONFIGS[5]
    cfgw = mi.scaled(cfg, fmt="fp8")
    E, G, k, H, I = cfg.E, cfg.extra["groups"], cfg.k, cfg.H, cfg.I
    S = E // G
    wr = mi.router_weight(cfg, device=DEV)
    bias = mi.router_bias(cfg, device=DEV)
    say("drawing 256 fp8 experts (original numbering)")
    W = mi.stacked_expert_weights(cfgw, range(E), device=DEV)
    names = ("w13", "w13_scale", "w2", "w2_scale")
    serve = dict(wr=wr.clone(), b=bias.clone(), **{n: W[n].clone() for n in names})
    n2o_tot = np.arange(E, dtype=np.int64)  # current id -> original id
    wr_c, b_c = wr.cpu(), bias.cpu()
    cnt = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    off = torch.empty(E + 2, dtype=torch.int32, device=DEV)
    r2s = torch.empty(STEP_T * k + STEP_T, dtype=torch.int32, device=DEV)
    s2r = torch.empty(STEP_T * k, dtype=torch.int32, device=DEV)
    nws = L.moe_permute_workspace_size(STEP_T, k, E)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    for epoch in range(EPOCHS):
        o2n_tot = np.argsort(n2o_tot)
        xc = _drifted_tokens(cfg, wr, epoch, STEPS * STEP_T, 11)
        acc = torch.zeros(E, dtype=torch.int64, device=DEV)
        ids_all = []
        for s in range(STEPS):
            ids, _ = _route(L, cfg, xc[s * STEP_T:(s + 1) * STEP_T], serve["wr"], serve["b"])
            L.moe_permute(ids, STEP_T, k, 0, E, False, None, L.BF16, 0, L.BF16, cnt, off, r2s, s2r,
                          None, None, ws, nws)
            L.moe_count_accumulate(cnt, E, acc)
            ids_all.append(ids)
        torch.cuda.synchronize()
        got = torch.cat(ids_all).cpu().numpy()
        _, ref_orig, _ = oracle.route(xc.cpu(), wr_c, b_c, k, oracle.SIGMOID, True)
        assert np.array_equal(got, o2n_tot[ref_orig]), f"epoch {epoch}: gating in the current numbering"
        counts = acc.cpu()
        assert np.array_equal(counts.numpy(), np.bincount(got.ravel(), minlength=E))
        mean = counts.sum().item() / G
        before = counts.view(G, S).sum(1).max().item() / mean

        n2o = torch.empty(E, dtype=torch.int32)
        o2n = torch.empty(E, dtype=torch.int32)
        loads = torch.empty(G, dtype=torch.int64)
        L.moe_balanced_partition(counts, E, G, n2o, o2n, loads)
        r_n2o, r_o2n, r_loads = oracle.balanced_partition(counts.numpy(), G)
        assert np.array_equal(n2o.numpy(), r_n2o) and np.array_equal(loads.numpy(), r_loads)
        after = loads.max().item() / mean
        moved = int((r_n2o != np.arange(E)).sum())

        # remap every serving tensor through the library, compose the maps
        n2o_d = n2o.to(DEV)
        serve = {n: _gather(L, t, n2o_d) for n, t in serve.items()}
        n2o_tot = n2o_tot[r_n2o]
        o2n_tot = np.argsort(n2o_tot)
        idx = torch.from_numpy(n2o_tot).to(DEV)
        torch.cuda.synchronize()
        assert torch.equal(serve["wr"], wr[idx]) and torch.equal(serve["b"], bias[idx])
        for n in names:
            assert torch.equal(serve[n], W[n][idx]), f"epoch {epoch}: remapped {n}"

        # held-out tokens of the same epoch through the new numbering
        xe = _drifted_tokens(cfg, wr, epoch, EVAL_T, 12)
        ids_e, w_e = _route(L, cfg, xe, serve["wr"], serve["b"])
        torch.cuda.synchronize()
        ide = ids_e.cpu().numpy()
        _, ref_e, ref_we = oracle.route(xe.cpu(), wr_c, b_c, k, oracle.SIGMOID, True)
        assert np.array_equal(ide, o2n_tot[ref_e])
        assert np.abs(w_e.cpu().numpy() - ref_we).max() <= 1e-6
        ev = np.bincount(ide.ravel(), minlength=E).reshape(G, S).sum(1)
        h = int(ev.argmax())
        layer = L.MoELayer("fp8", H, I, k, serve["w13"][h * S:(h + 1) * S],
                           serve["w2"][h * S:(h + 1) * S], serve["w13_scale"][h * S:(h + 1) * S],
                           serve["w2_scale"][h * S:(h + 1) * S], expert_base=h * S)
        b = layer.forward(xe, topk_ids=ids_e, topk_w=w_e)
        torch.cuda.synchronize()
        local = np.nonzero(((ide >= h * S) & (ide < (h + 1) * S)).any(1))[0]
        orig = torch.from_numpy(n2o_tot[h * S:(h + 1) * S]).to(DEV)
        st_orig = {n: W[n][orig] for n in names}  # the set's experts from the original draw
        ref = oracle_rows(xe[torch.from_numpy(local).to(DEV)].cpu(), ide[local], w_e.cpu().numpy()[local],
                          st_orig, None, k, S, h * S, "fp8")
        e = rel_err(out_f64(b.out[torch.from_numpy(local).to(DEV)]), ref)
        say(f"  epoch {epoch}: {moved} experts moved; calibration max/mean {before:.3f} -> {after:.3f}; "
            f"held-out max/mean {ev.max() / ev.mean():.3f}; heaviest set {h}: {len(local)} tokens, "
            f"rel err {e:.3e}")
        assert after < 1.05
        assert e <= 3e-2
        del layer, b
