"""moe_combine on its own against the oracle's combine (fp64), on ragged shapes
and every kernel path: bf16 with k <= 8 (scalar pick indices), bf16 with k > 8
and columns not a multiple of 8, and fp32. Picks that are not local (row -1)
contribute nothing, with and without the shared row. With one-hot weights on a
local pick and no shared row the output is the picked row, bit for bit. The
Moreh EP report (Overview) sums each token's expert outputs weighted by its
routing scores; this is the GPU-local half of that combine."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, rel_err, say

pytestmark = pytest.mark.gpu


def _case(T, k, H, frac_local, shared, seed):
    """Seeded maps and values: a random injective map of the local slots onto
    rows [0, R), -1 for the others; the shared rows follow at R."""
    rng = np.random.default_rng(seed)
    S = T * k
    local = rng.random(S) < frac_local
    R = int(local.sum())
    s2r = np.full(S, -1, np.int32)
    s2r[local] = rng.permutation(R).astype(np.int32)
    n_rows = max(R + (T if shared else 0), 1)
    y = rng.standard_normal((n_rows, H)).astype(np.float32)
    w = rng.uniform(0.0, 1.0, (T, k)).astype(np.float32)
    return s2r, y, w, R


def _combine_gpu(y_dev, y_dt, s2r, w, T, k, H, shared_row0, out_dt):
    import mixture_experts_layer_select_amd as L
    offsets = torch.tensor([shared_row0 if shared_row0 >= 0 else 0], dtype=torch.int32, device=DEV)
    out = torch.full((T, H), float("nan"), device=DEV,
                     dtype=torch.bfloat16 if out_dt == L.BF16 else torch.float32)
    L.moe_combine(y_dev, y_dt, torch.from_numpy(s2r).to(DEV), torch.from_numpy(w).to(DEV), T, k, H,
                  offsets, 0 if shared_row0 >= 0 else -1, out, out_dt)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("T,k,H,shared", [
    (37, 8, 7168, True), (37, 8, 7168, False), (29, 3, 264, True), (29, 1, 8, False),
    (2688, 8, 7168, False), (23, 9, 7168, True), (23, 9, 36, False), (17, 2, 1032, True),
])
def test_combine_bf16_matches_oracle(T, k, H, shared):
    import mixture_experts_layer_select_amd as L
    say(f"[combine bf16] T={T} k={k} H={H} shared={shared}")
    s2r, y, w, R = _case(T, k, H, 0.4, shared, 100 + T + k + H)
    y_dev = torch.from_numpy(y).to(DEV).to(torch.bfloat16)
    y64 = y_dev.float().cpu().numpy().astype(np.float64)
    got = _combine_gpu(y_dev, L.BF16, s2r, w, T, k, H, R if shared else -1, L.BF16)
    ref = oracle.combine(y64, s2r, w, k, R if shared else -1)
    got64 = got.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got64).all()
    # tokens without any local pick and no shared row are exactly zero
    if not shared:
        empty = (s2r.reshape(T, k) < 0).all(axis=1)
        assert (got64[empty] == 0).all()
    # one fp32 sum of at most k + 1 terms, then one bf16 rounding (half an ulp
    # is 2^-9 of the value): at most about 2e-3 of max|out|, with margin
    assert rel_err(got64, ref) <= 4e-3


@pytest.mark.parametrize("T,k,H", [(31, 8, 7168), (19, 4, 264), (13, 9, 7168)])
def test_combine_one_hot_returns_the_row(T, k, H):
    import mixture_experts_layer_select_amd as L
    say(f"[combine one-hot] T={T} k={k} H={H}")
    s2r, y, _, _ = _case(T, k, H, 0.5, False, 7 + T)
    rng = np.random.default_rng(11 + T)
    w = np.zeros((T, k), np.float32)
    picked = np.full(T, -1)
    for t in range(T):
        loc = np.nonzero(s2r[t * k:(t + 1) * k] >= 0)[0]
        if len(loc):
            j = int(rng.choice(loc))
            w[t, j] = 1.0
            picked[t] = s2r[t * k + j]
    y_dev = torch.from_numpy(y).to(DEV).to(torch.bfloat16)
    got = _combine_gpu(y_dev, L.BF16, s2r, w, T, k, H, -1, L.BF16).view(torch.int16).cpu().numpy()
    ybits = y_dev.view(torch.int16).cpu().numpy()
    for t in range(T):
        if picked[t] >= 0:
            assert np.array_equal(got[t], ybits[picked[t]]), t
        else:
            assert (got[t] == 0).all(), t


@pytest.mark.parametrize("T,k,H,shared", [(21, 2, 64, False), (21, 8, 1024, True)])
def test_combine_fp32_matches_oracle(T, k, H, shared):
    import mixture_experts_layer_select_amd as L
    say(f"[combine fp32] T={T} k={k} H={H} shared={shared}")
    s2r, y, w, R = _case(T, k, H, 0.6, shared, 300 + T)
    y_dev = torch.from_numpy(y).to(DEV)
    got = _combine_gpu(y_dev, L.F32, s2r, w, T, k, H, R if shared else -1, L.F32)
    ref = oracle.combine(y.astype(np.float64), s2r, w, k, R if shared else -1)
    assert rel_err(got.cpu().numpy(), ref) <= 1e-5
