"""GPU token->expert grouping (moe_permute) against the oracle: counts,
offsets and both maps bit-exact, x_perm bit-exact (bf16 copies, e4m3 codes and
their scales). The Moreh EP report (Library optimization) feeds a fused MoE
kernel with tokens grouped per expert; Inter-GPU load balancing counts each
expert's activations."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _ids(T, k, E, seed, s=1.2, lo=0):
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, E + 1) ** s
    p /= p.sum()
    out = np.empty((T, k), np.int32)
    for t in range(T):
        out[t] = rng.choice(E, k, replace=False, p=p) + lo
    return out


def _permute_gpu(ids, x, base, E_local, shared, fp8):
    import mixture_experts_layer_select_amd as L
    T, k = ids.shape
    cap = T * k + T
    i32 = dict(dtype=torch.int32, device=DEV)
    counts = torch.full((E_local + 1,), -7, **i32)
    offsets = torch.full((E_local + 2,), -7, **i32)
    r2s = torch.full((cap,), -7, **i32)
    s2r = torch.full((T * k,), -7, **i32)
    H = x.shape[1] if x is not None else 0
    xp = xs = None
    if x is not None:
        xp = torch.zeros((cap, H), dtype=torch.uint8 if fp8 else x.dtype, device=DEV)
        # scales are K-major: [H/128][cap]
        xs = torch.zeros((H // 128, cap), dtype=torch.float32, device=DEV) if fp8 else None
    ws_n = L.moe_permute_workspace_size(T, k, E_local)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=DEV)
    xdt = L.BF16 if x is None or x.dtype == torch.bfloat16 else L.F32
    L.moe_permute(torch.from_numpy(ids).to(DEV), T, k, base, E_local, shared, x, xdt, H,
                  L.FP8_E4M3 if fp8 else xdt, counts, offsets, r2s, s2r, xp, xs, ws, ws_n)
    torch.cuda.synchronize()
    return counts, offsets, r2s, s2r, xp, xs


def _check(ids, x, base, E_local, shared, fp8=False, sample_rows=None):
    T, k = ids.shape
    say(f"permute T={T} k={k} base={base} E_local={E_local} shared={shared} fp8={fp8}")
    counts, offsets, r2s, s2r, xp, xs = _permute_gpu(ids, x, base, E_local, shared, fp8)
    ref = oracle.permute(ids, base, E_local, shared)
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(offsets.cpu().numpy(), ref["offsets"])
    assert np.array_equal(s2r.cpu().numpy(), ref["slot_to_row"])
    assert np.array_equal(r2s.cpu().numpy(), ref["row_to_slot"])
    if x is None:
        return ref
    n = int(ref["offsets"][-1])
    rows = np.arange(n) if sample_rows is None else np.sort(
        np.random.default_rng(1).choice(n, min(n, sample_rows), replace=False))
    r2s_ref = ref["row_to_slot"][rows]
    xp_ref, xs_ref = oracle.gather(x.cpu(), k, r2s_ref, len(rows),
                                   oracle.FP8 if fp8 else oracle.dt_of(x.cpu()))
    got = oracle.as_np(xp[torch.from_numpy(rows).to(DEV)].cpu())
    assert np.array_equal(got, xp_ref)
    if fp8:
        gs = xs[:, torch.from_numpy(rows).to(DEV)].t().contiguous().cpu().numpy()
        assert np.array_equal(gs.view(np.uint32), xs_ref.view(np.uint32))
    return ref


def test_permute_decode_batch_with_shared_bf16():
    cfg = mi.CONFIGS[2]
    ids = _ids(256, 8, 256, 0)
    _check(ids, mi.tokens(cfg, device=DEV), 0, 256, True)


def test_permute_ep_share_fp8():
    cfg = mi.CONFIGS[3]
    ids, w, recv = mi.ep_share_routing(cfg)
    x = mi.ep_share_tokens(cfg, len(recv), device=DEV)
    ref = _check(ids.numpy(), x, 0, 32, False, fp8=True)
    say(f"  received tokens {len(recv)}, local rows {ref['offsets'][32]}")
    assert 3000 < ref["offsets"][32] < 5200


def test_permute_large_batch_fp8_sampled_rows():
    cfg = mi.CONFIGS[4]
    ids = _ids(cfg.T, 8, 256, 4, s=1.1)
    _check(ids, mi.tokens(cfg, device=DEV), 0, 256, True, fp8=True, sample_rows=3000)


@pytest.mark.parametrize("T,k,E,base,E_local,shared", [
    (1, 1, 1, 0, 1, True),
    (1, 8, 256, 0, 256, False),
    (129, 8, 256, 64, 32, False),    # a middle share of the experts
    (300, 8, 256, 224, 32, True),    # the last share
    (500, 3, 20, 5, 7, True),
])
def test_permute_edges_bf16(T, k, E, base, E_local, shared):
    cfg = mi.scaled(mi.CONFIGS[2], T=T, H=384)
    ids = _ids(T, k, E, T + base)
    _check(ids, mi.tokens(cfg, device=DEV), base, E_local, shared)


def test_permute_foreign_and_negative_ids_maps_only():
    ids = _ids(200, 8, 256, 9)
    ids[::7, 2] = -1
    ids[::5, 0] = 1000
    _check(ids, None, 0, 256, True)


def test_permute_fp32_rows():
    cfg = mi.CONFIGS[1]
    ids = _ids(cfg.T, cfg.k, cfg.E, 3)
    _check(ids, mi.tokens(cfg, device=DEV), 0, cfg.E, False)
