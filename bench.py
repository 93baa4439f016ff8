"""Benchmark of one DeepSeek-R1-style MoE layer on one MI355X.

A step is one pass of the whole layer through the C ABI -- moe_route (or,
for batches of 4096 tokens and more, moe_route_select, which returns the same
ids and weights), moe_permute, moe_expert_ffn_gate_up, moe_expert_ffn_down,
moe_combine -- over one batch of synthetic tokens already resident in HBM. fp8
layers with a shared expert run moe_permute for the maps only, quantise each
token once (moe_quantize_tokens) and read the token rows in gate/up
(moe_expert_ffn_gate_up_tokens).

The headline workload is the largest single-GPU shape: the R1 layer on a
large batch in fp8 (16384 tokens, hidden 7168, 256 routed experts of
intermediate 2048, top-8 by sigmoid score with Zipf(1.1)-skewed popularity,
one shared expert; e4m3 weights with 128x128 block scales, activations
quantised per 1x128 block), MFMA-bound. The R1 decode layer in bf16 (256
tokens, same experts, HBM-bound) is measured in the same process afterwards
and reported under "decode" in the same line (--decode-config 0 skips it).
Other workloads (--config 2, 3, 5) can be measured on their own.

Printed: one JSON line with tokens/s, the roofline of the dominant kernel
(the gate/up grouped GEMM: algorithmic flops or bytes per launch over its
average duration, timed with HIP events on the launch stream inside the
timed region) and the CPU oracle's throughput on a bounded sample of the
headline workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at 1 GPU + % of HBM/MFMA roofline (R1-shaped)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, choices=[2, 3, 4, 5])
    ap.add_argument("--decode-config", type=int, default=2, choices=[0, 2, 3, 5],
                    help="second workload timed in the same process after the first and "
                         "reported under 'decode' (0 = none)")
    ap.add_argument("--also-configs", default="3,5",
                    help="further workloads timed in the same process after the first two and "
                         "reported under 'also' (comma list of 3 and 5; 'none' = skip)")
    ap.add_argument("--cpu-sample", type=int, default=256,
                    help="tokens of the workload the CPU oracle runs end to end (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--fused-T", default="1,16,64,256",
                    help="batch sizes at which the one-launch layer (moe_layer_fused) is timed against "
                         "the five-launch path on the same weights ('none' = skip)")
    ap.add_argument("--fused-only", action="store_true",
                    help="only the small-batch comparison on the --config layer (for kernel traces); "
                         "prints its JSON record instead of the benchmark line")
    ap.add_argument("--graph", action="store_true",
                    help="after the eager timed steps, capture one step in a HIP graph and also "
                         "report the replay time (graph_ms_per_step)")
    return ap.parse_args()


def build_layer(cid: int, dev: str):
    import torch
    import moe_inputs as mi
    import mixture_experts_layer_select_amd as L

    cfg = mi.CONFIGS[cid]
    info = {}
    topk = None
    if cid == 3:
        ids, w, recv = mi.ep_share_routing(cfg, device=dev)
        x = mi.ep_share_tokens(cfg, len(recv), device=dev)
        st = mi.stacked_expert_weights(cfg, range(cfg.E_local), device=dev)
        layer = L.MoELayer(cfg.fmt, cfg.H, cfg.I, cfg.k, st["w13"], st["w2"], st["w13_scale"],
                           st["w2_scale"], shared=None, router=None)
        topk = (ids, w)
        info["T_recv"] = len(recv)
        return cfg, layer, x, st, None, topk, info
    if cid == 5:
        return build_partition_layer(cfg, dev)
    st = mi.stacked_expert_weights(cfg, range(cfg.E), device=dev)
    sh = mi.shared_weights(cfg, device=dev) if cfg.shared else None
    router = dict(w=mi.router_weight(cfg, device=dev), bias=mi.router_bias(cfg, device=dev),
                  scoring=L.SIGMOID, renormalize=True)
    layer = L.MoELayer(cfg.fmt, cfg.H, cfg.I, cfg.k, st["w13"], st["w2"], st["w13_scale"],
                       st["w2_scale"], shared=sh, router=router)
    x = mi.tokens(cfg, device=dev)
    return cfg, layer, x, st, sh, topk, info


def build_partition_layer(cfg, dev):
    """Calibrate expert counts, partition 256 experts into 8 balanced sets of
    32, remap the router, and build the heaviest set's layer."""
    import numpy as np
    import torch
    import moe_inputs as mi
    import mixture_experts_layer_select_amd as L

    G = cfg.extra["groups"]
    S = cfg.E // G
    wr = mi.router_weight(cfg, device=dev)
    bias = mi.router_bias(cfg, device=dev)

    def counts_of(x, w, b):
        T = x.shape[0]
        logits = torch.empty((T, cfg.E), dtype=torch.float32, device=dev)
        ids = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
        tw = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
        L.moe_route(x, w, b, L.BF16, T, cfg.H, cfg.E, cfg.k, L.SIGMOID, True, logits, ids, tw)
        cnt = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
        off = torch.empty(cfg.E + 2, dtype=torch.int32, device=dev)
        r2s = torch.empty(T * cfg.k + T, dtype=torch.int32, device=dev)
        s2r = torch.empty(T * cfg.k, dtype=torch.int32, device=dev)
        n = L.moe_permute_workspace_size(T, cfg.k, cfg.E)
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
        L.moe_permute(ids, T, cfg.k, 0, cfg.E, False, None, L.BF16, 0, L.BF16, cnt, off, r2s, s2r,
                      None, None, ws, n)
        return cnt[: cfg.E].cpu().to(torch.int64), ids, tw

    xc = mi.calibration_tokens(cfg, device=dev)
    counts, _, _ = counts_of(xc, wr, bias)
    n2o = torch.empty(cfg.E, dtype=torch.int32)
    o2n = torch.empty(cfg.E, dtype=torch.int32)
    loads = torch.empty(G, dtype=torch.int64)
    L.moe_balanced_partition(counts, cfg.E, G, n2o, o2n, loads)
    contiguous = counts.view(G, S).sum(1)
    mean = counts.sum().item() / G
    # remap the router rows and bias into the new expert order
    n2o_d = n2o.to(dev)
    wr2 = torch.empty_like(wr)
    L.moe_gather_rows(wr, cfg.E, wr2, n2o_d, cfg.E, cfg.H * 2)
    b2 = torch.empty_like(bias)
    L.moe_gather_rows(bias, cfg.E, b2, n2o_d, cfg.E, 4)
    x = mi.tokens(cfg, device=dev)
    ev_before, _, _ = counts_of(x, wr, bias)
    ev_after, ids, tw = counts_of(x, wr2, b2)
    g_before = ev_before.view(G, S).sum(1)
    g_after = ev_after.view(G, S).sum(1)
    heavy = int(torch.argmax(g_after).item())
    # a larger held-out batch: the set loads without the sampling noise of 512 tokens
    xh = mi.tokens(cfg, T=4096, device=dev, tensor=mi.XHELD)
    h_before = counts_of(xh, wr, bias)[0].view(G, S).sum(1)
    h_after = counts_of(xh, wr2, b2)[0].view(G, S).sum(1)
    old_ids = n2o[heavy * S:(heavy + 1) * S].tolist()
    st = mi.stacked_expert_weights(cfg, old_ids, device=dev)
    layer = L.MoELayer(cfg.fmt, cfg.H, cfg.I, cfg.k, st["w13"], st["w2"], shared=None, router=None,
                       expert_base=heavy * S)
    info = dict(
        calib_max_over_mean_contiguous=round(contiguous.max().item() / mean, 4),
        calib_max_over_mean_balanced=round(loads.max().item() / mean, 4),
        eval_max_over_mean_contiguous=round(g_before.max().item() / (ev_before.sum().item() / G), 4),
        eval_max_over_mean_balanced=round(g_after.max().item() / (ev_after.sum().item() / G), 4),
        heldout4096_max_over_mean_contiguous=round(h_before.max().item() / (h_before.sum().item() / G), 4),
        heldout4096_max_over_mean_balanced=round(h_after.max().item() / (h_after.sum().item() / G), 4),
        heaviest_group=heavy, heaviest_group_rows=int(g_after.max().item()),
        heaviest_group_rows_contiguous=int(g_before.max().item()),
        heaviest_group_hit_experts=int((ev_after.view(G, S)[heavy] > 0).sum().item()),
    )
    return cfg, layer, x, st, None, (ids, tw), info


def alg_bytes_gate_up(cfg, layer, counts, n_rows):
    """Algorithmic bytes of one gate/up launch: the w13 panels of every group
    with rows (once), the permuted activations read once, A written once."""
    wb = 1 if cfg.fmt == "fp8" else 2
    hit = int((counts[: layer.E_local] > 0).sum()) + (1 if layer.shared is not None else 0)
    w13 = 2 * cfg.I * cfg.H * wb + (2 * cfg.I // 128) * (cfg.H // 128) * 4 * (cfg.fmt == "fp8")
    xin = n_rows * cfg.H * wb + (n_rows * cfg.H // 128 * 4 if cfg.fmt == "fp8" else 0)
    aout = n_rows * cfg.I * wb + (n_rows * cfg.I // 128 * 4 if cfg.fmt == "fp8" else 0)
    return hit * w13 + xin + aout, hit


def layer_alg(cfg, layer, counts, T, n_rows):
    """Whole-layer algorithmic bytes and flops: weights (+scales) of the hit
    experts and the shared expert, router rows, x read once, out written once,
    routing ids/weights; flops 2*(2I*H + H*I) per routed or shared row."""
    wb = 1 if cfg.fmt == "fp8" else 2
    hit = int((counts[: layer.E_local] > 0).sum()) + (1 if layer.shared is not None else 0)
    per_expert = 3 * cfg.I * cfg.H * wb
    if cfg.fmt == "fp8":
        per_expert += ((2 * cfg.I // 128) * (cfg.H // 128) + (cfg.H // 128) * (cfg.I // 128)) * 4
    router = layer.router["w"].numel() * 2 if layer.router is not None else 0
    byt = hit * per_expert + router + 2 * T * cfg.H * 2 + T * cfg.k * 8
    flops = 2.0 * 3 * cfg.I * cfg.H * n_rows
    return byt, flops


def gemm_source_digest() -> str:
    """SHA-256 over the sources of the grouped GEMM kernels (device code, then
    kernels and launchers): a committed counter summary applies only to them."""
    import hashlib
    h = hashlib.sha256()
    for name in ("ffn_dev.h", "ffn.hip"):
        h.update(open(os.path.join(ROOT, "mixture_experts_layer_select_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def profiled_traffic(kernel_key: str, workload: str):
    """HBM bytes per launch from the committed counter summary of this kernel
    and workload (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known
    size), or None when there is none or the kernel source changed since."""
    import glob
    import hashlib
    digest = gemm_source_digest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            line = line.strip()
            if not (line.startswith("{") and "traffic_bytes" in line):
                continue
            try:
                rec = json.loads(line)
            except ValueError:
                continue
            if (rec.get("kernel") == kernel_key and rec.get("workload") == workload
                    and rec.get("gemm_sources_sha256") == digest):
                return int(rec["traffic_bytes"])
    return None


def step_traffic(fmt_key: str, workload: str):
    """HBM bytes of the timed gate/up step: the bf16 kernel, or the sum of the
    two fp8 launches (groups of at most 256 rows, then the larger ones)."""
    if fmt_key != "fp8":
        return profiled_traffic("gemm_bf16_kernel<true", workload)
    parts = [profiled_traffic(k, workload) for k in ("gemm_fp8_lds_kernel<true", "gemm_fp8_big_kernel<true")]
    return None if any(p is None for p in parts) else sum(parts)


def cpu_groups(st, sh, ids, base, E_local):
    """Host copies of the experts that the sampled tokens pick (+ shared)."""
    used = sorted({int(e) - base for e in ids.ravel() if 0 <= int(e) - base < E_local})
    groups = [None] * E_local
    for e in used:
        d = dict(w13=st["w13"][e].cpu(), w2=st["w2"][e].cpu())
        if st.get("w13_scale") is not None:
            d["w13_scale"] = st["w13_scale"][e].cpu()
            d["w2_scale"] = st["w2_scale"][e].cpu()
        groups[e] = d
    shared = None if sh is None else {k: (v.cpu() if v is not None else None) for k, v in sh.items()}
    return groups, shared


def cpu_baseline(cfg, layer, b, x, st, sh, topk, n_sample):
    """The oracle as it stands on a bounded sample: gating of every token of
    the batch (when the layer has a router) plus the rest of the layer for
    n_sample tokens; the per-token cost is scaled to tokens/s."""
    import numpy as np
    import torch
    import oracle

    T = x.shape[0]
    xc = x.cpu()
    t_route = 0.0
    if layer.router is not None:
        wr = layer.router["w"].cpu()
        bias = layer.router["bias"].cpu() if layer.router["bias"] is not None else None
        t0 = time.perf_counter()
        _, ids, w = oracle.route(xc, wr, bias, cfg.k, oracle.SIGMOID, True)
        t_route = time.perf_counter() - t0
    else:
        ids, w = topk[0].cpu().numpy(), topk[1].cpu().numpy()
    rows = np.sort(np.random.default_rng(0).choice(T, min(n_sample, T), replace=False))
    groups, shared = cpu_groups(st, sh, ids[rows], layer.expert_base, layer.E_local)
    # whole passes over the sample until about 10 s of CPU work have run, so
    # a small batch is timed over several passes rather than one short one
    passes, t_rest = 0, 0.0
    while passes == 0 or (t_rest < 10.0 and passes < 16):
        t0 = time.perf_counter()
        oracle.moe_layer(xc[torch.from_numpy(rows)], cfg.k, groups, shared, topk_ids=ids[rows],
                         topk_w=w[rows], base=layer.expert_base, E_local=layer.E_local,
                         fmt=oracle.FP8 if cfg.fmt == "fp8" else None)
        t_rest += time.perf_counter() - t0
        passes += 1
    per_token = t_route / T + t_rest / (passes * len(rows))
    threads = int(os.environ.get("OMP_NUM_THREADS", 0)) or os.cpu_count()
    return {"value": round(1.0 / per_token, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"gating of all {T} tokens ({t_route:.2f} s) + permute/FFN/combine of "
                      f"{len(rows)} seeded tokens x {passes} passes ({t_rest:.2f} s), fp64 FFN, "
                      f"scaled per token"}


def fused_sweep(cfg, layer, Ts, dev, reps=50, warm=5):
    """The layer at small batches: the five-launch path (route, permute, gate/up,
    down, combine) eagerly and replayed from a HIP graph, and the one-launch
    layer, on the same weights and tokens; mean ms per call from HIP events on
    the launch stream."""
    import torch
    import moe_inputs as mi
    stream = torch.cuda.current_stream()
    res = {}
    for T in Ts:
        if T > layer.FUSED_MAX_T:
            continue
        x = mi.tokens(cfg, T=T, device=dev, tensor=20)

        def timed(fn):
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps

        sep = timed(lambda: layer.forward(x))
        fused = timed(lambda: layer.forward_fused(x))
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                layer.forward(x)
        stream.wait_stream(side)
        graph = timed(g.replay)
        err = int(layer.fused_workspace(T)[8:12].view(torch.int32).item())
        res[str(T)] = {"five_launch_ms": round(sep, 4), "five_launch_graph_ms": round(graph, 4),
                       "fused_ms": round(fused, 4), "fused_barrier_error": err}
        log(f"[bench] T={T}: five launches {sep:.4f} ms (graph {graph:.4f}), one launch {fused:.4f} ms")
        del g
    return res


def measure(cid: int, args, dev: str, with_cpu: bool) -> dict:
    """Time one workload (warm-up, then args.steps whole-layer steps) and
    return its JSON fields."""
    import numpy as np
    import torch
    import mixture_experts_layer_select_amd as L

    log(f"[bench] building workload config {cid}")
    cfg, layer, x, st, sh, topk, info = build_layer(cid, dev)
    T = x.shape[0]
    b = layer.buffers(T, dev)
    stream = torch.cuda.current_stream()
    ids_in, w_in = (topk if topk is not None else (None, None))

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    def step(i=None):
        if ids_in is None:
            layer.route(x, b)
        layer.permute(x, b, ids_in)
        if i is not None:
            ev[i][0].record(stream)
        layer.gate_up(b)
        if i is not None:
            ev[i][1].record(stream)
        layer.down(b)
        layer.combine(b, w_in)

    log(f"[bench] c{cid}: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] c{cid}: timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    value = T / (ms / 1e3)
    k_ms = float(np.mean([a.elapsed_time(z) for a, z in ev]))
    log(f"[bench] c{cid}: {ms:.4f} ms/step, gate/up {k_ms:.4f} ms")

    graph_ms = None
    if args.graph:
        # one step captured on a side stream (the eager steps above did every
        # one-time set-up), then warm-up and timed replays
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                step()
        stream.wait_stream(side)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - g0) * 1e3 / args.steps
        log(f"[bench] graph replay {graph_ms:.4f} ms/step")

    # online rebalancing: what tracking one step costs on the device (the
    # permute's counts accumulated, the step's picks added to the
    # co-activation histogram), and the host re-partition from the result
    ids_all = b.topk_ids if ids_in is None else ids_in
    acc = torch.zeros(layer.E_local, dtype=torch.int64, device=dev)
    hist = torch.zeros((cfg.E, cfg.E), dtype=torch.int64, device=dev)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_track = 50
    for i in range(n_track + 5):
        if i == 5:
            r0.record(stream)
        L.moe_count_accumulate(b.counts, layer.E_local, acc)
        L.moe_coactivation(ids_all, T, cfg.k, cfg.E, hist)
    r1.record(stream)
    torch.cuda.synchronize()
    track_us = r0.elapsed_time(r1) / n_track * 1e3
    hist_h = hist.cpu()
    G = 8
    n2o, o2n = torch.empty(cfg.E, dtype=torch.int32), torch.empty(cfg.E, dtype=torch.int32)
    loads, intra = torch.empty(G, dtype=torch.int64), torch.zeros(1, dtype=torch.int64)
    h0 = time.perf_counter()
    L.moe_affinity_partition(torch.diagonal(hist_h).contiguous(), hist_h, cfg.E, G, 20, n2o, o2n,
                             loads, intra)
    part_ms = (time.perf_counter() - h0) * 1e3
    log(f"[bench] rebalance tracking {track_us:.2f} us/step, host affinity partition "
        f"{part_ms:.2f} ms")

    counts = b.counts.cpu().numpy()
    n_rows = int(b.offsets[-1].item())
    gbytes, hit = alg_bytes_gate_up(cfg, layer, counts, n_rows)
    gflops = 2.0 * n_rows * 2 * cfg.I * cfg.H
    lbytes, lflops = layer_alg(cfg, layer, counts, T, n_rows)
    fmt_key = "fp8" if cfg.fmt == "fp8" else "bf16"
    # the gate/up step is bound by whichever of its bytes and its flops takes
    # longer at peak; the fp8 step is two launches (groups of at most 256 rows,
    # then the larger ones), timed together
    mfma_bound = gflops / (MFMA_PEAK_TFLOPS[fmt_key] * 1e12) > gbytes / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        achieved, peak, unit = gflops / (k_ms / 1e3) / 1e12, MFMA_PEAK_TFLOPS[fmt_key], "TFLOP/s"
    else:
        achieved, peak, unit = gbytes / (k_ms / 1e3) / 1e9, HBM_PEAK_GBS, "GB/s"
    kname = ("ffn_gemm_fp8_lds_kernel<gate_up>+ffn_gemm_fp8_big_kernel<gate_up>" if fmt_key == "fp8"
             else "ffn_gemm_bf16_kernel<gate_up>")
    t_roof = max(lbytes / (HBM_PEAK_GBS * 1e9), lflops / (MFMA_PEAK_TFLOPS[fmt_key] * 1e12))
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8_e4m3", "f32": "f32"}[cfg.fmt], "data": "synthetic",
        "config": {"workload": f"c{cfg.cid} {cfg.name}", "tokens": T, "hidden": cfg.H,
                   "experts": cfg.E, "local_experts": layer.E_local, "top_k": cfg.k,
                   "intermediate": cfg.I, "shared_expert": layer.shared is not None,
                   "experts_hit": hit - (1 if layer.shared is not None else 0),
                   "rows": n_rows, **info},
        "roofline": {"kernel": kname, "bound": "mfma" if mfma_bound else "hbm",
                     "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4),
                     "traffic": step_traffic(fmt_key, f"c{cfg.cid}"),
                     "bytes_per_launch": int(gbytes), "flops_per_launch": gflops,
                     "avg_launch_ms": round(k_ms, 4)},
        "layer_roofline": {"bytes": int(lbytes), "flops": lflops,
                           "t_roof_ms": round(t_roof * 1e3, 4),
                           "frac": round(t_roof * 1e3 / ms, 4),
                           "hbm_GBs": round(lbytes / (ms / 1e3) / 1e9, 1),
                           "tflops": round(lflops / (ms / 1e3) / 1e12, 2)},
        "cpu_baseline": None,
        "rebalance": {"track_us_per_step": round(track_us, 2),
                      "track_frac_of_step": round(track_us / 1e3 / ms, 5),
                      "affinity_partition_host_ms": round(part_ms, 3),
                      "partition": f"E={cfg.E} into {G} sets, load cap +2%"},
    }
    Ts = [int(t) for t in args.fused_T.split(",") if t.strip() and t.strip() != "none"]
    if Ts and layer.router is not None and layer.E_local == cfg.E and cfg.k <= 8:
        line["fused_small_batch"] = {"layer": f"c{cfg.cid} weights, {cfg.fmt}",
                                     **fused_sweep(cfg, layer, Ts, dev)}
    if graph_ms is not None:
        line["graph_ms_per_step"] = round(graph_ms, 4)
        line["graph_tokens_per_s"] = round(T / (graph_ms / 1e3), 2)
    if with_cpu and args.cpu_sample > 0:
        log(f"[bench] cpu oracle baseline on {args.cpu_sample} tokens")
        line["cpu_baseline"] = cpu_baseline(cfg, layer, b, x, st, sh, topk, args.cpu_sample)
    del layer, st, sh, b, x, hist, acc
    return line


def dict_args(args, **changes):
    """A copy of the parsed arguments with some fields replaced."""
    a = argparse.Namespace(**vars(args))
    for key, v in changes.items():
        setattr(a, key, v)
    return a


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the layer runs on one "
              "GPU's share and uses no collectives.", file=sys.stderr)
        sys.exit(2)
    import gc
    import torch

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.fused_only:
        cfg, layer, x, st, sh, topk, info = build_layer(args.config, dev)
        Ts = [int(t) for t in args.fused_T.split(",") if t.strip() and t.strip() != "none"]
        print(json.dumps({"fused_small_batch": {"layer": f"c{cfg.cid} weights, {cfg.fmt}",
                                                **fused_sweep(cfg, layer, Ts, dev)}}), flush=True)
        return
    line = measure(args.config, args, dev, with_cpu=True)
    if args.decode_config and args.decode_config != args.config:
        gc.collect()
        torch.cuda.empty_cache()
        d = measure(args.decode_config, args, dev, with_cpu=False)
        line["decode"] = {key: d[key] for key in ("value", "unit", "ms_per_step", "dtype", "config",
                                                  "roofline", "layer_roofline", "fused_small_batch")
                          if key in d}
    also = [int(c) for c in args.also_configs.split(",") if c.strip() and c.strip() != "none"]
    for cid in also:
        if cid in (args.config, args.decode_config) or cid not in (2, 3, 5):
            continue
        gc.collect()
        torch.cuda.empty_cache()
        a = measure(cid, dict_args(args, fused_T="none"), dev, with_cpu=False)
        line.setdefault("also", {})[a["config"]["workload"]] = {
            key: a[key] for key in ("value", "unit", "ms_per_step", "dtype", "config", "roofline",
                                    "layer_roofline") if key in a}
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 1 GiB read + 1 GiB written by one copy kernel")
        del src, dst
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
