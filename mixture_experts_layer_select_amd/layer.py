"""One MoE layer on one GPU: buffers plus the four C-ABI calls in order.

route -> permute -> expert FFN -> combine ([Moreh-EP] Overview and
Parallelization: gating picks k experts per token, the expert FFNs run on the
tokens routed to them, an always-on shared expert runs on every token, and
the results are combined with the routing weights). This module only
allocates device buffers (torch) and passes pointers to libmoe.so; all
arithmetic happens in the library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L


@dataclass
class LayerBuffers:
    T: int
    logits: Optional[torch.Tensor]
    topk_ids: torch.Tensor
    topk_w: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    row_to_slot: torch.Tensor
    slot_to_row: torch.Tensor
    x_perm: Optional[torch.Tensor]  # None when fp8 gate/up reads the token rows
    x_perm_scale: Optional[torch.Tensor]
    y_perm: torch.Tensor
    out: torch.Tensor
    ws_perm: torch.Tensor
    ws_ffn: torch.Tensor
    ws_route: Optional[torch.Tensor] = None  # moe_route_select's workspace (large batches)
    x_tok: Optional[torch.Tensor] = None  # fp8 token codes [T, H] (moe_quantize_tokens)
    x_tok_scale: Optional[torch.Tensor] = None  # their scales [H/128, T]


class MoELayer:
    """Weights of one GPU's expert share (+ optional shared expert and router).

    fmt: "f32", "bf16" or "fp8". Expert weights are device tensors
    w13 [E_local, 2I, H], w2 [E_local, H, I] (uint8 e4m3 codes for fp8, with
    w13_scale [E_local, 2I/128, H/128], w2_scale [E_local, H/128, I/128]).
    router: dict(w=[E, H], bias=[E] or None, scoring, renormalize) or None
    when the routing is handed in (expert-parallel share).
    """

    def __init__(self, fmt: str, H: int, I: int, k: int, w13, w2, w13_scale=None, w2_scale=None,
                 shared: Optional[dict] = None, router: Optional[dict] = None, expert_base: int = 0):
        self.fmt = fmt
        self.H, self.I, self.k = H, I, k
        self.E_local = w13.shape[0]
        self.expert_base = expert_base
        self.dt = {"f32": L.F32, "bf16": L.BF16, "fp8": L.FP8_E4M3}[fmt]
        self.act_dt = L.F32 if fmt == "f32" else L.BF16
        self.w13, self.w2, self.w13_scale, self.w2_scale = w13, w2, w13_scale, w2_scale
        self.shared = shared
        self.router = router
        sh = shared or {}
        self.weights = L.make_weights(self.dt, self.E_local, H, I, w13, w2, w13_scale, w2_scale,
                                      sh.get("w13"), sh.get("w2"), sh.get("w13_scale"),
                                      sh.get("w2_scale"))
        self.n_groups = self.E_local + (1 if shared is not None else 0)
        self._bufs = {}

    # fp8 layers with a shared expert quantise each token once and let gate/up
    # read its token's row (moe_quantize_tokens + moe_expert_ffn_gate_up_tokens)
    # instead of copying every routed row into x_perm; the result is the same
    # bit for bit. Without a shared group moe_permute quantises each routed row
    # straight from x in one pass, and gate/up on the contiguous rows is faster
    # than the gathered reads.
    FP8_FROM_TOKENS = True

    def uses_tokens(self) -> bool:
        return self.fmt == "fp8" and self.FP8_FROM_TOKENS and self.shared is not None

    # Batches of at least this many tokens route through moe_route_select
    # (same ids and weights as moe_route; faster once the MFMA pass has a few
    # thousand tokens, slower for a decode batch). The logits buffer is then
    # left unfilled.
    ROUTE_SELECT_MIN_T = 4096

    def uses_route_select(self, T: int) -> bool:
        r = self.router
        if r is None or self.act_dt != L.BF16 or T < self.ROUTE_SELECT_MIN_T:
            return False
        E = r["w"].shape[0]
        return (self.H % 32 == 0 and self.H <= 8192 and E <= 256
                and (r["scoring"] == L.SIGMOID or r.get("renormalize", True)))

    # ------------------------------------------------------------------ buffers
    def buffers(self, T: int, device=None) -> LayerBuffers:
        if T in self._bufs:
            return self._bufs[T]
        device = device or self.w13.device
        k, H = self.k, self.H
        cap = T * k + T
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        act = torch.float32 if self.fmt == "f32" else torch.bfloat16
        E = self.router["w"].shape[0] if self.router is not None else 0
        xdt = torch.uint8 if self.fmt == "fp8" else act
        ws_p = L.moe_permute_workspace_size(T, k, self.E_local)
        ws_f = L.moe_expert_ffn_workspace_size(self.weights, cap)
        b = LayerBuffers(
            T=T,
            logits=torch.empty((T, E), **f32) if E else None,
            topk_ids=torch.empty((T, k), **i32),
            topk_w=torch.empty((T, k), **f32),
            counts=torch.empty(self.E_local + 1, **i32),
            offsets=torch.empty(self.E_local + 2, **i32),
            row_to_slot=torch.empty(cap, **i32),
            slot_to_row=torch.empty(T * k, **i32),
            x_perm=None if self.uses_tokens() else torch.empty((cap, H), dtype=xdt, device=device),
            x_perm_scale=(torch.empty((H // 128, cap), **f32)
                          if self.fmt == "fp8" and not self.uses_tokens() else None),
            y_perm=torch.empty((cap, H), dtype=act, device=device),
            out=torch.empty((T, H), dtype=act, device=device),
            ws_perm=torch.empty(max(ws_p, 1), dtype=torch.uint8, device=device),
            ws_ffn=torch.empty(max(ws_f, 1), dtype=torch.uint8, device=device),
        )
        if self.uses_tokens():
            b.x_tok = torch.empty((T, H), dtype=torch.uint8, device=device)
            b.x_tok_scale = torch.empty((H // 128, T), **f32)
        if self.uses_route_select(T):
            b.ws_route = torch.empty(L.moe_route_select_workspace_size(T, E), dtype=torch.uint8,
                                     device=device)
        self._bufs[T] = b
        return b

    # ------------------------------------------------------------------ steps
    def route(self, x: torch.Tensor, b: LayerBuffers, stream=None):
        r = self.router
        T, H = x.shape
        E = r["w"].shape[0]
        if b.ws_route is not None:
            L.moe_route_select(x, r["w"], r.get("bias"), self.act_dt, T, H, E, self.k, r["scoring"],
                               r.get("renormalize", True), b.topk_ids, b.topk_w, b.ws_route,
                               b.ws_route.numel(), stream)
        else:
            L.moe_route(x, r["w"], r.get("bias"), self.act_dt, T, H, E, self.k, r["scoring"],
                        r.get("renormalize", True), b.logits, b.topk_ids, b.topk_w, stream)

    def permute(self, x: torch.Tensor, b: LayerBuffers, topk_ids=None, stream=None):
        T = x.shape[0]
        ids = b.topk_ids if topk_ids is None else topk_ids
        L.moe_permute(ids, T, self.k, self.expert_base, self.E_local, self.shared is not None, x,
                      self.act_dt, self.H, self.dt if self.fmt == "fp8" else self.act_dt, b.counts,
                      b.offsets, b.row_to_slot, b.slot_to_row, b.x_perm, b.x_perm_scale, b.ws_perm,
                      b.ws_perm.numel(), stream)
        if self.uses_tokens():
            L.moe_quantize_tokens(x, self.act_dt, T, self.H, b.x_tok, b.x_tok_scale, stream)

    def gate_up(self, b: LayerBuffers, stream=None):
        cap = b.T * self.k + b.T
        if self.uses_tokens():
            L.moe_expert_ffn_gate_up_tokens(self.weights, b.x_tok, b.x_tok_scale, b.T, self.k,
                                            b.row_to_slot, b.offsets, self.n_groups, cap, b.ws_ffn,
                                            b.ws_ffn.numel(), stream)
        else:
            L.moe_expert_ffn_gate_up(self.weights, b.x_perm, b.x_perm_scale, b.offsets,
                                     self.n_groups, cap, b.ws_ffn, b.ws_ffn.numel(), stream)

    def down(self, b: LayerBuffers, stream=None):
        cap = b.T * self.k + b.T
        L.moe_expert_ffn_down(self.weights, b.offsets, self.n_groups, cap, b.y_perm, b.ws_ffn,
                              b.ws_ffn.numel(), stream)

    def ffn(self, b: LayerBuffers, stream=None):
        self.gate_up(b, stream)
        self.down(b, stream)

    def combine(self, b: LayerBuffers, topk_w=None, stream=None):
        w = b.topk_w if topk_w is None else topk_w
        L.moe_combine(b.y_perm, self.act_dt, b.slot_to_row, w, b.T, self.k, self.H, b.offsets,
                      self.E_local if self.shared is not None else -1, b.out, self.act_dt, stream)

    def check_inputs(self, x: torch.Tensor, topk_ids=None, topk_w=None):
        """x must be [T, H] in the layer's activation dtype on the weights'
        device; given routing must be int32 ids and fp32 weights [T, k]."""
        act = torch.float32 if self.fmt == "f32" else torch.bfloat16
        dev = self.w13.device
        L.expect(x, "x", (act,), dev)
        if x.dim() != 2 or x.shape[1] != self.H:
            raise ValueError(f"x: shape {tuple(x.shape)}, expected [T, {self.H}]")
        if (topk_ids is None) != (topk_w is None):
            raise ValueError("routing must be given as both topk_ids and topk_w, or neither")
        if topk_ids is None and self.router is None:
            raise ValueError("the layer has no router: pass topk_ids and topk_w")
        for t, name, dt in ((topk_ids, "topk_ids", torch.int32), (topk_w, "topk_w", torch.float32)):
            if t is not None:
                L.expect(t, name, (dt,), dev)
                if tuple(t.shape) != (x.shape[0], self.k):
                    raise ValueError(f"{name}: shape {tuple(t.shape)}, expected [{x.shape[0]}, {self.k}]")

    # the one-launch layer (moe_layer_fused) takes batches up to this size
    FUSED_MAX_T = 256

    def fused_workspace(self, T: int) -> torch.Tensor:
        """The fused layer's workspace for T tokens, zeroed once at allocation
        (its barrier words must start at zero; every call leaves them so)."""
        key = ("fused", T)
        if key not in self._bufs:
            E = self.router["w"].shape[0]
            n = L.moe_layer_fused_workspace_size(self.weights, T, E, self.k)
            self._bufs[key] = torch.zeros(max(n, 256), dtype=torch.uint8, device=self.w13.device)
        return self._bufs[key]

    def forward_fused(self, x: torch.Tensor, stream=None) -> LayerBuffers:
        """The whole layer in one launch (routing by this layer's router, all
        experts local): the same ids, weights and output as forward()."""
        self.check_inputs(x)
        T = x.shape[0]
        b = self.buffers(T, x.device)
        ws = self.fused_workspace(T)
        r = self.router
        L.moe_layer_fused(x, r["w"], r.get("bias"), T, r["w"].shape[0], self.k, r["scoring"],
                          r.get("renormalize", True), self.weights, b.topk_ids, b.topk_w, b.out, ws,
                          ws.numel(), stream)
        return b

    def forward(self, x: torch.Tensor, topk_ids=None, topk_w=None, stream=None) -> LayerBuffers:
        """The whole layer. Routing comes from the router unless given."""
        self.check_inputs(x, topk_ids, topk_w)
        b = self.buffers(x.shape[0], x.device)
        if topk_ids is None:
            self.route(x, b, stream)
        self.permute(x, b, topk_ids, stream)
        self.ffn(b, stream)
        self.combine(b, topk_w, stream)
        return b
