"""GPU grouped expert FFN (moe_expert_ffn) against the oracle on identical
permuted inputs: y_perm within the layer tolerance (1e-2 bf16, 3e-2 fp8,
1e-5 fp32) as max|gpu - oracle| / max|oracle|. Group sizes cover empty
groups, single rows, ragged 16-row and 64-row tails and several m-tiles
(the variable M per expert of the SGLang H20 report, SwapAB GEMM); the last
group is the shared expert (Moreh EP report, Library optimization)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from gpu_util import DEV, cpu_dict, cpu_expert, rel_err, say

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp8": 3e-2, "f32": 1e-5}


def _run(fmt, H, I, sizes, shared, seed=0):
    import mixture_experts_layer_select_amd as L
    say(f"ffn fmt={fmt} H={H} I={I} sizes={sizes} shared={shared}")
    base = {"f32": mi.CONFIGS[1], "bf16": mi.CONFIGS[2], "fp8": mi.CONFIGS[4]}[fmt]
    cfg = mi.scaled(base, H=H, I=I, cid=100 + seed)
    E_local = len(sizes) - (1 if shared else 0)
    st = mi.stacked_expert_weights(cfg, range(E_local), device=DEV)
    sh = mi.shared_weights(cfg, device=DEV) if shared else None
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(offsets[-1])
    max_rows = R + 5  # a little slack, like the T*k+T bound
    x = mi.normal((max_rows, H), 1.0, 777 + seed, DEV, cfg.act_dtype)
    if fmt == "fp8":
        codes, scales = oracle.quantize_1x128(x.float().cpu().numpy())
        xp = torch.from_numpy(codes).to(DEV)
        xs = torch.from_numpy(np.ascontiguousarray(scales.T)).to(DEV)  # K-major [H/128][max_rows]
    else:
        xp, xs = x, None
    dt = {"f32": L.F32, "bf16": L.BF16, "fp8": L.FP8_E4M3}[fmt]
    shd = sh or {}
    w = L.make_weights(dt, E_local, H, I, st["w13"], st["w2"], st["w13_scale"], st["w2_scale"],
                       shd.get("w13"), shd.get("w2"), shd.get("w13_scale"), shd.get("w2_scale"))
    ws_n = L.moe_expert_ffn_workspace_size(w, max_rows)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=DEV)
    y = torch.zeros((max_rows, H), dtype=torch.float32 if fmt == "f32" else torch.bfloat16,
                    device=DEV)
    off_d = torch.from_numpy(offsets).to(DEV)
    L.moe_expert_ffn(w, xp, xs, off_d, len(sizes), max_rows, y, ws, ws_n)
    torch.cuda.synchronize()
    groups = [cpu_expert(st, e) if sizes[e] else None for e in range(E_local)]
    if shared:
        groups.append(cpu_dict(sh))
    ref = oracle.expert_ffn(groups, xp[:R].cpu() if fmt == "fp8" else x[:R].cpu(),
                            None if xs is None else xs[:, :R].t().contiguous().cpu(), offsets, H, I)
    got = y[:R].float().cpu().numpy()
    for g in range(len(sizes)):
        a, b = offsets[g], offsets[g + 1]
        if b > a:
            e = rel_err(got[a:b], ref[a:b])
            assert e <= TOL[fmt], f"group {g} (rows {b - a}): rel err {e:.3e}"
    e = rel_err(got, ref)
    say(f"  max rel err {e:.3e}")
    return e


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_ffn_ragged_groups(fmt):
    _run(fmt, 512, 256, [0, 1, 17, 64, 65, 130, 16, 0, 200], shared=True)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_ffn_no_shared_many_small_groups(fmt):
    rng = np.random.default_rng(5)
    sizes = list(rng.integers(0, 9, 40))
    _run(fmt, 768, 384, sizes, shared=False, seed=1)


def test_ffn_bf16_wide_path_mixed_groups():
    """Many groups averaging a few rows (the launcher's 8-wave bf16 path: at
    most 32 rows per group over the buffer) with three multi-tile groups among
    them and the shared group last."""
    rng = np.random.default_rng(11)
    sizes = list(rng.integers(0, 7, 57))
    sizes[5], sizes[20], sizes[41] = 70, 150, 200
    assert sum(sizes) + 5 <= 32 * (len(sizes) + 1)
    _run("bf16", 512, 256, sizes + [33], shared=True, seed=6)


def test_ffn_fp32_tiny():
    _run("f32", 64, 32, [3, 0, 5, 1, 7], shared=True)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_ffn_r1_shape_one_expert_two_tiles(fmt):
    """H=7168, I=2048: one routed expert with 80 rows (a full 64-row tile and a
    16-row tail) plus a 3-row shared group."""
    _run(fmt, 7168, 2048, [80, 3], shared=True, seed=2)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_ffn_groups_across_the_tile_height(fmt):
    """Groups on both sides of 256 rows (the fp8 path runs groups of at most
    256 rows and larger ones in separate launches): 257 = one row over, 513 =
    two full tiles and a one-row tail split into three even tiles, 700, and a
    600-row shared group, between empty and tiny groups."""
    _run(fmt, 512, 256, [0, 257, 3, 513, 256, 700, 1, 0, 600], shared=True, seed=3)


def test_ffn_fp8_small_group_heights():
    """Small-group fp8 tiles on both sides of 64 and 128 rows (a tile loads one,
    two or four 8-row activation pieces per wave and K step by its height) and
    up to 256 rows, with K loops of exactly one unrolled body: H = 1536 gives
    12 gate/up steps, I = 768 six down steps."""
    _run("fp8", 1536, 768, [63, 64, 65, 127, 128, 129, 191, 193, 255, 256, 8], shared=True, seed=8)


def test_ffn_fp8_large_groups_in_panels():
    """Groups of 6 and 9 256-row tiles (the large-group launch orders a
    group's items in panels of 4 m-tiles: one full panel and a 2-tile
    remainder, two full panels and a 1-tile one), a 5-tile group and small
    groups between them."""
    _run("fp8", 512, 256, [1300, 7, 2100, 0, 1180, 40], shared=True, seed=7)


def test_ffn_fp8_r1_shape_large_group():
    """H=7168, I=2048 with one 300-row expert (two tiles of 150) and a 40-row
    one: the full-size K loops of both fp8 launches."""
    _run("fp8", 7168, 2048, [300, 40], shared=False, seed=4)


@pytest.mark.timeout(600)
def test_ffn_fp8_r1_shape_large_group_all_panels():
    """H=7168, I=2048, every row compared: a 2400-row expert is 10 even tiles
    of 240 rows, run by the large-group launch in two full panels of 4 m-tiles
    and a 2-tile remainder panel, with the full 56-step (gate/up) and 16-step
    (down) K loops; a 513-row expert (3 tiles, one short panel), small
    experts for the small-group launch, and a 300-row shared group (2
    tiles)."""
    _run("fp8", 7168, 2048, [2400, 0, 7, 513, 1, 120, 300], shared=True, seed=9)


@pytest.mark.timeout(600)
def test_ffn_bf16_r1_shape_wide_many_groups():
    """H=7168, I=2048, every row compared: 120 routed experts of 0 to 6 rows
    with three multi-tile ones among them (70, 150, 230 rows) and a 33-row
    shared group. At most 32 rows per group over the buffer bound, so the
    8-wave bf16 launch runs it (the decode shape's path)."""
    rng = np.random.default_rng(21)
    sizes = list(rng.integers(0, 7, 120))
    sizes[7], sizes[60], sizes[111] = 70, 150, 230
    assert sum(sizes) + 33 + 5 <= 32 * (len(sizes) + 1)
    _run("bf16", 7168, 2048, sizes + [33], shared=True, seed=10)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_ffn_every_group_empty(fmt):
    """No group has a row: the launches find no work and write nothing."""
    import mixture_experts_layer_select_amd as L
    H, I, E_local, max_rows = 512, 256, 6, 9
    cfg = mi.scaled({"bf16": mi.CONFIGS[2], "fp8": mi.CONFIGS[4]}[fmt], H=H, I=I, cid=150)
    st = mi.stacked_expert_weights(cfg, range(E_local), device=DEV)
    dt = {"bf16": L.BF16, "fp8": L.FP8_E4M3}[fmt]
    w = L.make_weights(dt, E_local, H, I, st["w13"], st["w2"], st["w13_scale"], st["w2_scale"])
    if fmt == "fp8":
        xp = torch.zeros((max_rows, H), dtype=torch.uint8, device=DEV)
        xs = torch.ones((H // 128, max_rows), dtype=torch.float32, device=DEV)
    else:
        xp, xs = torch.zeros((max_rows, H), dtype=torch.bfloat16, device=DEV), None
    ws_n = L.moe_expert_ffn_workspace_size(w, max_rows)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=DEV)
    y = torch.full((max_rows, H), 7.0, dtype=torch.bfloat16, device=DEV)
    off = torch.zeros(E_local + 1, dtype=torch.int32, device=DEV)
    L.moe_expert_ffn(w, xp, xs, off, E_local, max_rows, y, ws, ws_n)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


@pytest.mark.parametrize("rows", [1, 5, 8, 9, 16])
def test_ffn_fp8_small_group_rows_do_not_depend_on_the_group_height(rows):
    """A row's result does not depend on how many rows its group has: two
    experts with the same weights, the first given `rows` rows (one 16-token
    block, one or two 8-row staging pieces) and the second the same rows plus
    more (17 or more rows: two blocks): gate/up codes and scales and the down
    output of those rows agree bit for bit, at the R1 shape."""
    import mixture_experts_layer_select_amd as L
    cfg = mi.CONFIGS[4]
    H, I = cfg.H, cfg.I
    st = mi.stacked_expert_weights(cfg, [3], device=DEV)
    w13 = st["w13"].repeat(2, 1, 1).contiguous()
    w2 = st["w2"].repeat(2, 1, 1).contiguous()
    s13 = st["w13_scale"].repeat(2, 1, 1).contiguous()
    s2 = st["w2_scale"].repeat(2, 1, 1).contiguous()
    w = L.make_weights(L.FP8_E4M3, 2, H, I, w13, w2, s13, s2)
    n2 = max(rows + 1, 17)
    x = mi.normal((n2, H), 1.0, 4242 + rows, DEV, torch.bfloat16)
    codes, scales = oracle.quantize_1x128(x.float().cpu().numpy())
    xc = torch.from_numpy(codes).to(DEV)
    xs = torch.from_numpy(scales).to(DEV)                       # [n2][H/128]
    R = rows + n2
    max_rows = R + 3
    xp = torch.zeros((max_rows, H), dtype=torch.uint8, device=DEV)
    xp[:rows] = xc[:rows]
    xp[rows:R] = xc
    xps = torch.ones((H // 128, max_rows), dtype=torch.float32, device=DEV)
    xps[:, :rows] = xs[:rows].t()
    xps[:, rows:R] = xs.t()
    off = torch.tensor([0, rows, R], dtype=torch.int32, device=DEV)
    ws_n = L.moe_expert_ffn_workspace_size(w, max_rows)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=DEV)
    y = torch.zeros((max_rows, H), dtype=torch.bfloat16, device=DEV)
    L.moe_expert_ffn(w, xp, xps, off, 2, max_rows, y, ws, ws_n)
    torch.cuda.synchronize()
    assert torch.equal(y[:rows].view(torch.int16), y[rows:2 * rows].view(torch.int16))
    # the intermediate: codes [max_rows][I] at the start of the workspace,
    # then its scales [I/128][max_rows]
    a = ws[:max_rows * I].view(max_rows, I)
    a_off = ((max_rows * I + 255) // 256) * 256
    a_sc = ws[a_off:a_off + max_rows * (I // 128) * 4].view(torch.float32).view(I // 128, max_rows)
    assert torch.equal(a[:rows], a[rows:2 * rows])
    assert torch.equal(a_sc[:, :rows].view(torch.int32), a_sc[:, rows:2 * rows].view(torch.int32))
    groups = [cpu_expert(st, 0), cpu_expert(st, 0)]
    ref = oracle.expert_ffn(groups, xp[:R].cpu(), xps[:, :R].t().contiguous().cpu(),
                            off.cpu().numpy(), H, I)
    e = rel_err(y[:R].float().cpu().numpy(), ref)
    say(f"  group of {rows} rows: bit-identical to the {n2}-row group, vs oracle {e:.3e}")
    assert e <= TOL["fp8"]
