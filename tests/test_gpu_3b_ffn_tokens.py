"""fp8 gate/up from token rows (moe_quantize_tokens + moe_expert_ffn_gate_up_tokens)
against the oracle's 1x128 quantisation (codes and scales bit for bit) and
against the materialised path (moe_permute's fp8 x_perm + moe_expert_ffn_gate_up):
the intermediate A and its scales, then y_perm after moe_expert_ffn_down, bit for
bit, on groups on both sides of 256 rows (both kernels), with and without the
shared group and for an expert-parallel share. The Moreh EP report (Library
optimization) has the fused MoE kernel read each expert's tokens itself."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _ids(T, k, E, seed, s):
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, E + 1) ** s
    p /= p.sum()
    out = np.empty((T, k), np.int32)
    for t in range(T):
        out[t] = rng.choice(E, k, replace=False, p=p)
    return out


@pytest.mark.parametrize("T,H", [(37, 512), (300, 7168)])
def test_quantize_tokens_matches_oracle(T, H):
    import mixture_experts_layer_select_amd as L
    say(f"[quantize tokens] T={T} H={H}")
    x = mi.normal((T, H), 1.0, 900 + T, DEV, torch.bfloat16)
    x[3, :128] = 0  # an all-zero block: scale 1
    codes = torch.full((T, H), 0x55, dtype=torch.uint8, device=DEV)
    scales = torch.full((H // 128, T), float("nan"), dtype=torch.float32, device=DEV)
    L.moe_quantize_tokens(x, L.BF16, T, H, codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_1x128(x.float().cpu().numpy())
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy().T.view(np.uint32), rs.astype(np.float32).view(np.uint32))


def _layer_parts(H, I, E_local, base, E, T, k, shared, seed, s):
    import mixture_experts_layer_select_amd as L
    cfg = mi.scaled(mi.CONFIGS[4], H=H, I=I, cid=400 + seed)
    st = mi.stacked_expert_weights(cfg, range(E_local), device=DEV)
    sh = mi.shared_weights(cfg, device=DEV) if shared else None
    shd = sh or {}
    w = L.make_weights(L.FP8_E4M3, E_local, H, I, st["w13"], st["w2"], st["w13_scale"], st["w2_scale"],
                       shd.get("w13"), shd.get("w2"), shd.get("w13_scale"), shd.get("w2_scale"))
    ids = torch.from_numpy(_ids(T, k, E, seed, s)).to(DEV)
    x = mi.normal((T, H), 1.0, 950 + seed, DEV, torch.bfloat16)
    return w, ids, x


def _compare(H, I, E_local, base, E, T, k, shared, seed, s=1.2):
    import mixture_experts_layer_select_amd as L
    w, ids, x = _layer_parts(H, I, E_local, base, E, T, k, shared, seed, s)
    cap = T * k + T
    n_groups = E_local + (1 if shared else 0)
    i32 = dict(dtype=torch.int32, device=DEV)
    counts = torch.empty(E_local + 1, **i32)
    offsets = torch.empty(E_local + 2, **i32)
    r2s = torch.empty(cap, **i32)
    s2r = torch.empty(T * k, **i32)
    xp = torch.empty((cap, H), dtype=torch.uint8, device=DEV)
    xs = torch.empty((H // 128, cap), dtype=torch.float32, device=DEV)
    wsp_n = L.moe_permute_workspace_size(T, k, E_local)
    wsp = torch.empty(wsp_n, dtype=torch.uint8, device=DEV)
    L.moe_permute(ids, T, k, base, E_local, shared, x, L.BF16, H, L.FP8_E4M3, counts, offsets, r2s, s2r,
                  xp, xs, wsp, wsp_n)
    xt = torch.empty((T, H), dtype=torch.uint8, device=DEV)
    xts = torch.empty((H // 128, T), dtype=torch.float32, device=DEV)
    L.moe_quantize_tokens(x, L.BF16, T, H, xt, xts)
    ws_n = L.moe_expert_ffn_workspace_size(w, cap)
    ws1 = torch.zeros(ws_n, dtype=torch.uint8, device=DEV)
    ws2 = torch.zeros(ws_n, dtype=torch.uint8, device=DEV)
    L.moe_expert_ffn_gate_up(w, xp, xs, offsets, n_groups, cap, ws1, ws_n)
    L.moe_expert_ffn_gate_up_tokens(w, xt, xts, T, k, r2s, offsets, n_groups, cap, ws2, ws_n)
    y1 = torch.zeros((cap, H), dtype=torch.bfloat16, device=DEV)
    y2 = torch.zeros((cap, H), dtype=torch.bfloat16, device=DEV)
    L.moe_expert_ffn_down(w, offsets, n_groups, cap, y1, ws1, ws_n)
    L.moe_expert_ffn_down(w, offsets, n_groups, cap, y2, ws2, ws_n)
    torch.cuda.synchronize()
    off = offsets.cpu().numpy()
    R = int(off[n_groups])
    sizes = np.diff(off[: n_groups + 1])
    say(f"  rows {R}, largest group {sizes.max()}, groups above 256 rows {(sizes > 256).sum()}")
    # the materialised rows are their tokens' codes and scales
    slot = r2s[:R].cpu().numpy().astype(np.int64)
    tok = np.where(slot < T * k, slot // k, slot - T * k)
    assert np.array_equal(xp[:R].cpu().numpy(), xt.cpu().numpy()[tok]), "x_perm rows differ"
    assert np.array_equal(xs[:, :R].cpu().numpy(), xts.cpu().numpy()[:, tok]), "x_perm scales differ"
    # workspace: A codes [cap][I], then (256-aligned) A scales [I/128][cap]
    so = (cap * I + 255) // 256 * 256
    a1, a2 = ws1[: cap * I].view(cap, I)[:R].cpu(), ws2[: cap * I].view(cap, I)[:R].cpu()
    assert torch.equal(a1, a2), "A codes differ"
    s1 = ws1[so: so + cap * (I // 128) * 4].view(torch.int32).view(I // 128, cap)[:, :R].cpu()
    s2 = ws2[so: so + cap * (I // 128) * 4].view(torch.int32).view(I // 128, cap)[:, :R].cpu()
    assert torch.equal(s1, s2), "A scales differ"
    assert torch.equal(y1[:R].view(torch.int16).cpu(), y2[:R].view(torch.int16).cpu()), "y_perm differs"
    return sizes


def test_gate_up_tokens_r1_shape_both_kernels():
    """R1 widths, 8 experts + shared, skewed so that the first groups exceed
    256 rows (large-group kernel) while the tail stays below (small-group)."""
    sizes = _compare(7168, 2048, 8, 0, 8, 400, 4, True, seed=1, s=1.5)
    assert (sizes[:-1] > 256).any() and (sizes[:-1] <= 256).any()


def test_gate_up_tokens_ragged_no_shared():
    _compare(512, 256, 40, 0, 40, 333, 6, False, seed=2)


def test_gate_up_tokens_expert_parallel_share():
    """Experts [16, 48) of 64 are local: slots outside them are not rows."""
    _compare(1024, 512, 32, 16, 64, 700, 8, True, seed=3, s=0.8)


def test_gate_up_tokens_rejects_non_fp8():
    import mixture_experts_layer_select_amd as L
    cfg = mi.scaled(mi.CONFIGS[2], H=256, I=128, cid=450)
    st = mi.stacked_expert_weights(cfg, range(2), device=DEV)
    w = L.make_weights(L.BF16, 2, 256, 128, st["w13"], st["w2"], None, None)
    ws_n = L.moe_expert_ffn_workspace_size(w, 12)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=DEV)
    r2s = torch.zeros(12, dtype=torch.int32, device=DEV)
    off = torch.zeros(4, dtype=torch.int32, device=DEV)
    x = torch.zeros((4, 256), dtype=torch.uint8, device=DEV)
    xs = torch.zeros((2, 4), dtype=torch.float32, device=DEV)
    with pytest.raises(L.MoEError) as e:
        L.moe_expert_ffn_gate_up_tokens(w, x, xs, 4, 2, r2s, off, 2, 12, ws, ws_n)
    assert e.value.status == "MOE_ERR_UNSUPPORTED"


def test_quantize_tokens_and_gate_up_tokens_empty_cases():
    """T = 0 is a no-op for both calls; rows routed elsewhere (an expert-parallel
    share that receives nothing) leave every group empty and A untouched."""
    import mixture_experts_layer_select_amd as L
    H, I, E_local, T, k = 256, 128, 4, 9, 2
    cfg = mi.scaled(mi.CONFIGS[4], H=H, I=I, cid=460)
    st = mi.stacked_expert_weights(cfg, range(E_local), device=DEV)
    w = L.make_weights(L.FP8_E4M3, E_local, H, I, st["w13"], st["w2"], st["w13_scale"], st["w2_scale"])
    codes = torch.zeros((1, H), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((H // 128, 1), dtype=torch.float32, device=DEV)
    L.moe_quantize_tokens(codes, L.BF16, 0, H, codes, scales)  # T = 0: nothing is read or written
    ids = torch.full((T, k), 40, dtype=torch.int32, device=DEV)  # outside the local experts
    cap = T * k + T
    i32 = dict(dtype=torch.int32, device=DEV)
    counts, offsets = torch.empty(E_local + 1, **i32), torch.empty(E_local + 2, **i32)
    r2s, s2r = torch.empty(cap, **i32), torch.empty(T * k, **i32)
    wsp_n = L.moe_permute_workspace_size(T, k, E_local)
    wsp = torch.empty(wsp_n, dtype=torch.uint8, device=DEV)
    L.moe_permute(ids, T, k, 0, E_local, False, None, L.BF16, H, L.FP8_E4M3, counts, offsets, r2s, s2r,
                  None, None, wsp, wsp_n)
    x = mi.normal((T, H), 1.0, 461, DEV, torch.bfloat16)
    xt = torch.empty((T, H), dtype=torch.uint8, device=DEV)
    xts = torch.empty((H // 128, T), dtype=torch.float32, device=DEV)
    L.moe_quantize_tokens(x, L.BF16, T, H, xt, xts)
    ws_n = L.moe_expert_ffn_workspace_size(w, cap)
    ws = torch.full((ws_n,), 0xA5, dtype=torch.uint8, device=DEV)
    L.moe_expert_ffn_gate_up_tokens(w, xt, xts, T, k, r2s, offsets, E_local, cap, ws, ws_n)
    torch.cuda.synchronize()
    assert int(offsets[E_local].item()) == 0
    assert bool((ws == 0xA5).all())
