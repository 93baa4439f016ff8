"""Pins of the oracle's token->expert grouping (histogram, stable permutation,
gather) -- the step that feeds the fused MoE GEMMs (Moreh EP report, Library
optimization: fused MoE kernel; Inter-GPU load balancing: per-expert activation
frequency). Rows are ordered by (local expert, slot t*k+j); the pages leave the
order inside an expert open, the reading here is stable by slot.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi


def _ids(T, k, E, seed, skew=False):
    rng = np.random.default_rng(seed)
    p = None
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        p /= p.sum()
    return np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,k,E,base,E_local,shared", [
    (16, 2, 16, 0, 16, False),
    (100, 8, 256, 0, 256, True),
    (300, 8, 256, 64, 32, False),
    (1, 1, 1, 0, 1, True),
    (0, 8, 256, 0, 32, True),
])
def test_permute_against_bincount_and_stable_argsort(orc, T, k, E, base, E_local, shared):
    ids = _ids(T, k, E, T + E, skew=True) if T else np.zeros((0, k), np.int32)
    p = orc.permute(ids, base, E_local, shared)
    flat = ids.ravel().astype(np.int64) - base
    local = (flat >= 0) & (flat < E_local)
    counts = np.bincount(flat[local], minlength=E_local)
    assert np.array_equal(p["counts"][:E_local], counts)
    assert p["counts"][E_local] == (T if shared else 0)
    assert np.array_equal(p["offsets"], np.concatenate([[0], np.cumsum(p["counts"])]))
    R = int(local.sum())
    slots = np.nonzero(local)[0]
    order = slots[np.argsort(flat[local], kind="stable")]
    assert np.array_equal(p["row_to_slot"][:R], order)
    if shared:
        assert np.array_equal(p["row_to_slot"][R:R + T], T * k + np.arange(T))
    n = R + (T if shared else 0)
    assert np.all(p["row_to_slot"][n:] == -1)
    # permute then unpermute is the identity
    s2r = p["slot_to_row"]
    assert np.all(s2r[~local] == -1)
    assert np.array_equal(s2r[p["row_to_slot"][:R]], np.arange(R))
    assert np.array_equal(p["row_to_slot"][s2r[local]], np.nonzero(local)[0])


def test_gather_is_a_bit_copy_and_combine_one_hot_restores(orc):
    cfg = mi.scaled(mi.CONFIGS[2], T=37, H=256)
    x = mi.tokens(cfg)
    ids = _ids(37, 8, 64, 5)
    p = orc.permute(ids, 0, 64, True)
    n = int(p["offsets"][-1])
    xp, xs = orc.gather(x, 8, p["row_to_slot"], n, orc.BF16)
    assert xs is None
    xn = orc.as_np(x)
    for r in range(n):
        s = p["row_to_slot"][r]
        t = s // 8 if s < 37 * 8 else s - 37 * 8
        assert np.array_equal(xp[r], xn[t])
    # combine with weight 1 on one pick and no shared row returns x exactly
    w = np.zeros((37, 8), np.float32)
    w[:, 3] = 1.0
    y = orc.bf16_to_f32(xp).astype(np.float64)
    out = orc.combine(y, p["slot_to_row"], w, 8, -1)
    assert np.array_equal(orc.bf16_round(out), xn)
    # the shared rows alone (all routed weights 0) also return x exactly
    out = orc.combine(y, p["slot_to_row"], np.zeros_like(w), 8, int(p["offsets"][64]))
    assert np.array_equal(orc.bf16_round(out), xn)


def test_gather_fp8_quantises_each_row(orc):
    cfg = mi.scaled(mi.CONFIGS[4], T=9, H=384)
    x = mi.tokens(cfg)
    ids = _ids(9, 8, 32, 1)
    p = orc.permute(ids, 0, 32, True)
    n = int(p["offsets"][-1])
    xp, xs = orc.gather(x, 8, p["row_to_slot"], n, orc.FP8)
    codes, scales = orc.quantize_1x128(x.float())
    for r in range(n):
        s = p["row_to_slot"][r]
        t = s // 8 if s < 72 else s - 72
        assert np.array_equal(xp[r], codes[t]) and np.array_equal(xs[r], scales[t])


def test_combine_matches_weighted_sum(orc):
    rng = np.random.default_rng(9)
    T, k, H = 11, 3, 40
    ids = _ids(T, k, 6, 2)
    p = orc.permute(ids, 0, 4, True)   # experts 4 and 5 are not local
    n = int(p["offsets"][-1])
    y = rng.standard_normal((n, H))
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    out = orc.combine(y, p["slot_to_row"], w, k, int(p["offsets"][4]))
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            if ids[t, j] < 4:
                ref[t] += float(w[t, j]) * y[p["slot_to_row"][t * k + j]]
        ref[t] += y[int(p["offsets"][4]) + t]
    assert np.allclose(out, ref, rtol=1e-15, atol=1e-15)
