"""moe_expert_ffn_noalloc (the intermediate in the library's static device
scratch, no caller workspace, nothing allocated) against moe_expert_ffn with
a caller workspace: y_perm bit for bit on two calls in a row, the second one
smaller, for bf16 and fp8; a size beyond the static scratch is refused."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _case(L, fmt, H, I, sizes, shared, seed):
    base = {"bf16": mi.CONFIGS[2], "fp8": mi.CONFIGS[4]}[fmt]
    cfg = mi.scaled(base, H=H, I=I, cid=700 + seed)
    E_local = len(sizes) - (1 if shared else 0)
    st = mi.stacked_expert_weights(cfg, range(E_local), device=DEV)
    sh = mi.shared_weights(cfg, device=DEV) if shared else None
    shd = sh or {}
    dt = {"bf16": L.BF16, "fp8": L.FP8_E4M3}[fmt]
    w = L.make_weights(dt, E_local, H, I, st["w13"], st["w2"], st["w13_scale"], st["w2_scale"],
                       shd.get("w13"), shd.get("w2"), shd.get("w13_scale"), shd.get("w2_scale"))
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(offsets[-1])
    max_rows = R + 3
    x = mi.normal((max_rows, H), 1.0, 880 + seed, DEV, torch.bfloat16)
    if fmt == "fp8":
        codes, scales = oracle.quantize_1x128(x.float().cpu().numpy())
        xp = torch.from_numpy(codes).to(DEV)
        xs = torch.from_numpy(np.ascontiguousarray(scales.T)).to(DEV)
    else:
        xp, xs = x, None
    return w, xp, xs, torch.from_numpy(offsets).to(DEV), len(sizes), max_rows, R


def _both(L, w, xp, xs, off, n_groups, max_rows, R, H):
    y_ref = torch.full((max_rows, H), 3.0, dtype=torch.bfloat16, device=DEV)
    y_na = torch.full((max_rows, H), 5.0, dtype=torch.bfloat16, device=DEV)
    n = L.moe_expert_ffn_workspace_size(w, max_rows)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    L.moe_expert_ffn(w, xp, xs, off, n_groups, max_rows, y_ref, ws, n)
    L.moe_expert_ffn_noalloc(w, xp, xs, off, n_groups, max_rows, y_na)
    torch.cuda.synchronize()
    return y_ref[:R], y_na[:R]


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_noalloc_matches_workspace_entry_point_two_calls(fmt):
    import mixture_experts_layer_select_amd as L
    H, I = 512, 256
    # first call: groups on both sides of the fp8 launches' 256-row split,
    # a shared group; second call: fewer, smaller groups
    calls = [([0, 300, 17, 64, 1, 130, 40], True, 1), ([5, 0, 33, 2], False, 2)]
    for sizes, shared, seed in calls:
        say(f"[noalloc {fmt}] sizes={sizes} shared={shared}")
        w, xp, xs, off, ng, max_rows, R = _case(L, fmt, H, I, sizes, shared, seed)
        ref, got = _both(L, w, xp, xs, off, ng, max_rows, R, H)
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16)), "differs from moe_expert_ffn"
        assert torch.isfinite(got.float()).all()


def test_noalloc_r1_decode_shape():
    """The R1 decode buffer bound (T*k + T = 2304 rows at H = 7168, I = 2048)
    fits the static scratch: 126 routed groups of a few rows + shared."""
    import mixture_experts_layer_select_amd as L
    rng = np.random.default_rng(4)
    sizes = list(rng.integers(0, 9, 40)) + [256]
    w, xp, xs, off, ng, max_rows, R = _case(L, "bf16", 7168, 2048, sizes, True, 3)
    assert L.moe_expert_ffn_workspace_size(w, 2304) <= L.NOALLOC_SCRATCH_BYTES
    ref, got = _both(L, w, xp, xs, off, ng, max_rows, R, 7168)
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16))


def test_noalloc_refuses_rows_beyond_the_scratch():
    import mixture_experts_layer_select_amd as L
    w, xp, xs, off, ng, max_rows, R = _case(L, "bf16", 512, 256, [4, 4], False, 5)
    big = L.NOALLOC_SCRATCH_BYTES // (256 * 2) + 64
    y = torch.empty((8, 512), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(L.MoEError) as ei:
        L.moe_expert_ffn_noalloc(w, xp, xs, off, ng, big, y)
    assert ei.value.status == "MOE_ERR_WORKSPACE"
