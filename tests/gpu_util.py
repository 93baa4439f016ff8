"""Shared helpers of the GPU parity tests (not a test module).

Inputs come from moe_inputs (drawn on the GPU), the reference values from the
CPU oracle fed with copies of the very same input bytes.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import moe_inputs as mi
import oracle

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def cpu_expert(st: dict, j: int) -> dict:
    """The j-th expert of a stacked weight dict, copied to the host."""
    d = dict(w13=st["w13"][j].cpu(), w2=st["w2"][j].cpu())
    if st.get("w13_scale") is not None:
        d["w13_scale"] = st["w13_scale"][j].cpu()
        d["w2_scale"] = st["w2_scale"][j].cpu()
    return d


def cpu_dict(d: dict | None) -> dict | None:
    if d is None:
        return None
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def oracle_rows(x_rows, ids_rows, w_rows, st, shared, k, E_local, base, fmt, n_threads=0):
    """Oracle layer output (fp64) for a handful of tokens, given their routing.
    Only the experts these tokens pick are copied to the host."""
    ids_rows = np.asarray(ids_rows)
    used = sorted({int(e) - base for e in ids_rows.ravel() if 0 <= int(e) - base < E_local})
    groups = [None] * E_local
    for e in used:
        groups[e] = cpu_expert(st, e)
    res = oracle.moe_layer(x_rows, k, groups, cpu_dict(shared), topk_ids=ids_rows,
                           topk_w=np.asarray(w_rows), base=base, E_local=E_local,
                           fmt=oracle.FP8 if fmt == "fp8" else None, n_threads=n_threads)
    return res["out64"]


def tile_cover_tokens(offsets, row_to_slot, T, k, n_groups, n_min, seed, tile=256):
    """Tokens whose rows reach every m-tile of every group, filled up with
    seeded random tokens to at least n_min.

    A group of m rows is split into nt = ceil(m / tile) tiles of even height
    (tile t holds rows [t*m/nt, (t+1)*m/nt)), as the grouped GEMMs split it;
    one random row of every tile is taken, and its token is slot // k for a
    routed slot, slot - T*k for a shared-group slot. Every output column of a
    chosen token's rows is compared, so every n-block of every tile is
    covered too."""
    offsets = np.asarray(offsets)
    row_to_slot = np.asarray(row_to_slot)
    rng = np.random.default_rng(seed)
    toks = set()
    for g in range(n_groups):
        a, b = int(offsets[g]), int(offsets[g + 1])
        m = b - a
        if m <= 0:
            continue
        nt = (m + tile - 1) // tile
        for t in range(nt):
            lo, hi = a + t * m // nt, a + (t + 1) * m // nt
            slot = int(row_to_slot[int(rng.integers(lo, hi))])
            toks.add(slot // k if slot < T * k else slot - T * k)
    rest = np.setdiff1d(np.arange(T), np.fromiter(toks, dtype=np.int64, count=len(toks)))
    need = max(0, n_min - len(toks))
    if need:
        toks.update(int(t) for t in rng.choice(rest, min(need, len(rest)), replace=False))
    return np.array(sorted(toks), dtype=np.int64)
