"""Seeded synthetic inputs for the DeepSeek-R1-style MoE layer workloads.

This module is the only code shared by the CPU oracle tests and the GPU path.
It draws tensors and nothing else: it computes no step of the layer (no
router logits, no selection, no permutation, no expert FFN, no combine).
Two preparation steps that a serving stack performs offline, before the
layer ever runs, also live here because they define the *inputs*:

* expert weights in fp8 are the bf16 draws cast to e4m3 with one fp32 scale
  per 128x128 block (torch's own cast does the rounding), and
* the router bias that skews expert popularity toward a Zipf law.

Workloads (sizes follow the R1 shape of the Moreh EP report, "Parallelization"
section: 256 routed experts, 8 active per token, one always-on shared expert,
32 experts per GPU under EP=8):

  c1  tiny fp32 layer: T=16, H=64, E=16, top-2, I=32, softmax router
  c2  R1 decode layer, bf16: T=256, H=7168, E=256, top-8 sigmoid, I=2048, shared
  c3  one GPU's EP share, fp8: 32 local experts, routing of a 4096-token global
      batch given (uniform), ~2710 received tokens, no router, no shared
  c4  large batch, fp8: T=16384 through the c2 layer
  c5  partition case, bf16: Zipf(1.3) popularity, 8192 calibration tokens,
      512 evaluation tokens, 8 groups of 32 experts

Every tensor is drawn with its own ``torch.Generator`` seeded from
(config, tensor id, index); draws happen on the device that will use them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

# tensor ids used in seeds
X, WR, RANK, W13, W2, WS13, WS2, ROUTING, XCAL, XHELD = 1, 2, 3, 4, 5, 6, 7, 8, 9, 10

BLOCK = 128          # fp8 block edge (weights 128x128, activations 1x128)
E4M3_MAX = 448.0     # largest finite OCP e4m3fn value


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    T: int                  # tokens through the layer (received tokens for c3)
    H: int                  # hidden size
    E: int                  # routed experts (global)
    k: int                  # experts per token
    I: int                  # expert intermediate size
    fmt: str                # "f32", "bf16" or "fp8" (expert weights / path)
    scoring: str = "sigmoid"
    renormalize: bool = True
    shared: bool = False    # one always-on shared expert of intermediate I
    zipf_s: Optional[float] = None
    x_std: float = 1.0
    w_std: float = 0.006
    E_local: Optional[int] = None
    expert_base: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def act_dtype(self):
        return torch.float32 if self.fmt == "f32" else torch.bfloat16


CONFIGS = {
    1: Config(1, "tiny-f32", T=16, H=64, E=16, k=2, I=32, fmt="f32",
              scoring="softmax", x_std=0.02, w_std=0.02),
    2: Config(2, "r1-decode-bf16", T=256, H=7168, E=256, k=8, I=2048, fmt="bf16",
              shared=True, zipf_s=1.1),
    3: Config(3, "r1-ep-share-fp8", T=0, H=7168, E=256, k=8, I=2048, fmt="fp8",
              E_local=32, extra=dict(global_T=4096)),
    4: Config(4, "r1-large-batch-fp8", T=16384, H=7168, E=256, k=8, I=2048, fmt="fp8",
              shared=True, zipf_s=1.1),
    5: Config(5, "r1-partition-bf16", T=512, H=7168, E=256, k=8, I=2048, fmt="bf16",
              zipf_s=1.3, E_local=32, extra=dict(calib_T=8192, groups=8)),
}


def scaled(cfg: Config, **changes) -> Config:
    """A config with some sizes changed (smaller parity cases of the same recipe)."""
    d = dict(cfg.__dict__)
    d.update(changes)
    return Config(**d)


def seed(cid: int, tensor: int, index: int = 0) -> int:
    return cid * 1_000_000 + tensor * 10_000 + index


def _gen(s: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(s)
    return g


def normal(shape, std: float, s: int, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    """N(0, std) draw in fp32, rounded to ``dtype``."""
    t = torch.randn(shape, generator=_gen(s, device), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


# ----------------------------------------------------------------------------
# router inputs
# ----------------------------------------------------------------------------
def zipf_lambda(H: int, w_std: float) -> float:
    """Scale that puts the bias on the Gumbel scale of the Gaussian router noise.

    The router noise per logit has std ``w_std*sqrt(H)`` for unit activations;
    a Gumbel variable has std pi/sqrt(6), so Gaussian noise plus ``lambda*ln p``
    approximates sampling experts with probabilities ``p`` without replacement.
    """
    return w_std * math.sqrt(H) / (math.pi / math.sqrt(6.0))


def zipf_bias(cfg: Config, device="cpu") -> torch.Tensor:
    """b_e = lambda * ln p_{rank(e)},  p_r proportional to r^-s,  rank a seeded permutation."""
    E, s = cfg.E, cfg.zipf_s
    r = torch.arange(1, E + 1, dtype=torch.float64)
    p = r.pow(-s)
    p = p / p.sum()
    rank = torch.randperm(E, generator=_gen(seed(cfg.cid, RANK), "cpu"))
    b = zipf_lambda(cfg.H, cfg.w_std) * torch.log(p[rank])
    return b.to(torch.float32).to(device)


def tokens(cfg: Config, T: Optional[int] = None, device="cpu", tensor: int = X) -> torch.Tensor:
    T = cfg.T if T is None else T
    return normal((T, cfg.H), cfg.x_std, seed(cfg.cid, tensor), device, cfg.act_dtype)


def router_weight(cfg: Config, device="cpu") -> torch.Tensor:
    """Router rows [E, H]; fp32 in the tiny config, bf16 otherwise (never fp8)."""
    return normal((cfg.E, cfg.H), cfg.w_std, seed(cfg.cid, WR), device, cfg.act_dtype)


def router_bias(cfg: Config, device="cpu") -> Optional[torch.Tensor]:
    return zipf_bias(cfg, device) if cfg.zipf_s is not None else None


# ----------------------------------------------------------------------------
# expert weights
# ----------------------------------------------------------------------------
def fp8_blocks(w: torch.Tensor):
    """Cast a weight matrix [N, K] to e4m3 codes with one fp32 scale per 128x128 block.

    scale = amax(block)/448 (1 for an all-zero block); codes = e4m3(w/scale)
    saturated to +-448 and rounded to nearest-even by torch's cast.
    Returns (codes uint8 [N, K], scales fp32 [N/128, K/128]).
    """
    N, K = w.shape
    assert N % BLOCK == 0 and K % BLOCK == 0
    wf = w.to(torch.float32).view(N // BLOCK, BLOCK, K // BLOCK, BLOCK)
    amax = wf.abs().amax(dim=(1, 3))
    sc = amax / E4M3_MAX
    sc = torch.where(amax == 0, torch.ones_like(sc), sc)
    q = (wf / sc[:, None, :, None]).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.view(N, K).view(torch.uint8), sc.contiguous()


def _matrix(cfg: Config, shape, s: int, device, fmt: str):
    w = normal(shape, cfg.w_std, s, device, cfg.act_dtype)
    if fmt == "fp8":
        return fp8_blocks(w)
    return w, None


def expert_weights(cfg: Config, e: int, device="cpu", fmt: Optional[str] = None):
    """Weights of routed expert ``e`` (its global, original id).

    w13 [2I, H]: rows 0..I-1 are the gate projection, rows I..2I-1 the up projection.
    w2  [H, I]: the down projection. Both K-contiguous.
    """
    fmt = fmt or cfg.fmt
    w13, s13 = _matrix(cfg, (2 * cfg.I, cfg.H), seed(cfg.cid, W13, e), device, fmt)
    w2, s2 = _matrix(cfg, (cfg.H, cfg.I), seed(cfg.cid, W2, e), device, fmt)
    return dict(w13=w13, w13_scale=s13, w2=w2, w2_scale=s2)


def shared_weights(cfg: Config, device="cpu", fmt: Optional[str] = None):
    fmt = fmt or cfg.fmt
    w13, s13 = _matrix(cfg, (2 * cfg.I, cfg.H), seed(cfg.cid, WS13), device, fmt)
    w2, s2 = _matrix(cfg, (cfg.H, cfg.I), seed(cfg.cid, WS2), device, fmt)
    return dict(w13=w13, w13_scale=s13, w2=w2, w2_scale=s2)


def stacked_expert_weights(cfg: Config, ids, device="cpu", fmt: Optional[str] = None):
    """Experts ``ids`` (original ids, in that order) stacked into contiguous
    [n, 2I, H] / [n, H, I] tensors (plus [n, 2I/128, H/128] / [n, H/128, I/128]
    scales for fp8), filled one expert at a time."""
    fmt = fmt or cfg.fmt
    ids = list(ids)
    n = len(ids)
    wdt = torch.uint8 if fmt == "fp8" else cfg.act_dtype
    w13 = torch.empty((n, 2 * cfg.I, cfg.H), dtype=wdt, device=device)
    w2 = torch.empty((n, cfg.H, cfg.I), dtype=wdt, device=device)
    s13 = s2 = None
    if fmt == "fp8":
        s13 = torch.empty((n, 2 * cfg.I // BLOCK, cfg.H // BLOCK), dtype=torch.float32, device=device)
        s2 = torch.empty((n, cfg.H // BLOCK, cfg.I // BLOCK), dtype=torch.float32, device=device)
    for j, e in enumerate(ids):
        d = expert_weights(cfg, e, device, fmt)
        w13[j].copy_(d["w13"])
        w2[j].copy_(d["w2"])
        if fmt == "fp8":
            s13[j].copy_(d["w13_scale"])
            s2[j].copy_(d["w2_scale"])
        del d
    return dict(w13=w13, w13_scale=s13, w2=w2, w2_scale=s2)


# ----------------------------------------------------------------------------
# c3: routing handed over by the other GPUs' routers
# ----------------------------------------------------------------------------
def ep_share_routing(cfg: Config, device="cpu"):
    """Routing of a global batch that a GPU owning experts [base, base+E_local) receives.

    Each of ``global_T`` tokens picks k distinct experts of E uniformly
    (seeded sampling without replacement) with positive combine weights
    sigmoid(N(0,1)) scaled to sum to one per token. Only tokens with at least
    one local expert are received. Returns (topk_ids [T_recv, k] int32 with
    global ids, topk_w [T_recv, k] fp32, token indices in the global batch).
    """
    gT = cfg.extra["global_T"]
    g = _gen(seed(cfg.cid, ROUTING), "cpu")
    ids = torch.rand((gT, cfg.E), generator=g).argsort(dim=1)[:, : cfg.k].to(torch.int32)
    raw = torch.sigmoid(torch.randn((gT, cfg.k), generator=g, dtype=torch.float64))
    w = (raw / raw.sum(dim=1, keepdim=True)).to(torch.float32)
    lo, hi = cfg.expert_base, cfg.expert_base + cfg.E_local
    recv = ((ids >= lo) & (ids < hi)).any(dim=1).nonzero().flatten()
    return ids[recv].contiguous().to(device), w[recv].contiguous().to(device), recv


def ep_share_tokens(cfg: Config, T_recv: int, device="cpu") -> torch.Tensor:
    return normal((T_recv, cfg.H), cfg.x_std, seed(cfg.cid, X), device, cfg.act_dtype)


def calibration_tokens(cfg: Config, device="cpu") -> torch.Tensor:
    return tokens(cfg, cfg.extra["calib_T"], device, tensor=XCAL)
