"""CPU oracle for one DeepSeek-R1-style MoE layer -- TEST INFRASTRUCTURE ONLY.

A ctypes front end over ``libmoe_oracle.so`` (plain C, see moe_oracle.h for
the definitions and sources). Only tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. It shares no code with the GPU
library and imports nothing from it.

Arrays are numpy (torch CPU tensors are accepted and viewed as numpy):
bf16 data travels as uint16 bit patterns, fp8 as uint8 e4m3fn codes.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

F32, BF16, FP8 = 0, 1, 2
SOFTMAX, SIGMOID = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

_p = C.c_void_p
_i = C.c_int


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        L.oracle_router_logits.argtypes = [_p, _p, _p, _i, _i, _i, _i, _p]
        L.oracle_select.argtypes = [_p, _i, _i, _i, _i, _i, _p, _p]
        L.oracle_permute.argtypes = [_p, _i, _i, _i, _i, _i, _p, _p, _p, _p]
        L.oracle_e4m3_encode.argtypes = [C.c_float]
        L.oracle_e4m3_encode.restype = C.c_uint8
        L.oracle_e4m3_decode.argtypes = [C.c_uint8]
        L.oracle_e4m3_decode.restype = C.c_float
        L.oracle_bf16_round.argtypes = [C.c_double]
        L.oracle_bf16_round.restype = C.c_uint16
        L.oracle_e4m3_encode_n.argtypes = [_p, C.c_long, _p]
        L.oracle_e4m3_decode_n.argtypes = [_p, C.c_long, _p]
        L.oracle_bf16_round_n.argtypes = [_p, C.c_long, _p]
        L.oracle_quantize_1x128.argtypes = [_p, _i, _i, _p, _p]
        L.oracle_gather.argtypes = [_p, _i, _i, _i, _i, _p, _i, _i, _p, _p]
        L.oracle_expert_ffn.argtypes = [_p, _p, _p, _p, _i, _p, _p, _p, _i, _i, _i, _i, _p]
        L.oracle_combine.argtypes = [_p, _p, _p, _i, _i, _i, _i, _p]
        L.oracle_balanced_partition.argtypes = [_p, _i, _i, _p, _p, _p]
        L.oracle_coactivation.argtypes = [_p, _i, _i, _i, _p]
        L.oracle_affinity_partition.argtypes = [_p, _p, _i, _i, _i, _p, _p, _p, _p]
        _lib = L
    return _lib


# ----------------------------------------------------------------------------
# array plumbing
# ----------------------------------------------------------------------------
def as_np(a):
    """numpy view of a CPU array/tensor; bf16 -> uint16 bits, fp8 -> uint8 codes."""
    if isinstance(a, np.ndarray):
        return a
    import torch
    t = a.detach()
    if t.device.type != "cpu":
        t = t.cpu()
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def dt_of(a) -> int:
    a = as_np(a)
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return FP8
    raise TypeError(f"unsupported oracle dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    a = as_np(a)
    if dtype is not None and a.dtype != dtype:
        a = a.astype(dtype)
    return np.ascontiguousarray(a)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (rc={rc})")


# ----------------------------------------------------------------------------
# steps
# ----------------------------------------------------------------------------
def router_logits(x, wr, bias=None) -> np.ndarray:
    x, wr = _c(x), _c(wr)
    assert x.dtype == wr.dtype
    T, H = x.shape
    E = wr.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), np.float32)
    _check(lib().oracle_router_logits(_ptr(x), _ptr(wr), _ptr(b), dt_of(x), T, H, E, _ptr(out)),
           "oracle_router_logits")
    return out


def select(logits, k: int, scoring: int, renorm: bool = True):
    l = _c(logits, np.float32)
    T, E = l.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _check(lib().oracle_select(_ptr(l), T, E, k, scoring, int(renorm), _ptr(ids), _ptr(w)),
           "oracle_select")
    return ids, w


def route(x, wr, bias, k: int, scoring: int, renorm: bool = True):
    logits = router_logits(x, wr, bias)
    ids, w = select(logits, k, scoring, renorm)
    return logits, ids, w


def permute(topk_ids, base: int, E_local: int, include_shared: bool):
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E_local + 1, np.int32)
    offsets = np.empty(E_local + 2, np.int32)
    r2s = np.empty(T * k + T, np.int32)
    s2r = np.empty(T * k, np.int32)
    _check(lib().oracle_permute(_ptr(ids), T, k, base, E_local, int(include_shared), _ptr(counts),
                                _ptr(offsets), _ptr(r2s), _ptr(s2r)), "oracle_permute")
    return dict(counts=counts, offsets=offsets, row_to_slot=r2s, slot_to_row=s2r)


def e4m3_encode(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e4m3_encode_n(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_decode(c) -> np.ndarray:
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float32)
    lib().oracle_e4m3_decode_n(_ptr(c), c.size, _ptr(out))
    return out


def bf16_round(v) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_bf16_round_n(_ptr(v), v.size, _ptr(out))
    return out


def bf16_to_f32(u) -> np.ndarray:
    return (_c(u, np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_1x128(v):
    v = _c(v, np.float32)
    rows, cols = v.shape
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty((rows, cols // 128), np.float32)
    _check(lib().oracle_quantize_1x128(_ptr(v), rows, cols, _ptr(codes), _ptr(scales)),
           "oracle_quantize_1x128")
    return codes, scales


def gather(x, k: int, row_to_slot, n_rows: int, perm_dt: int):
    x = _c(x)
    T, H = x.shape
    r2s = _c(row_to_slot, np.int32)
    if perm_dt == FP8:
        xp = np.empty((n_rows, H), np.uint8)
        xs = np.empty((n_rows, H // 128), np.float32)
    else:
        xp = np.empty((n_rows, H), x.dtype)
        xs = None
    _check(lib().oracle_gather(_ptr(x), dt_of(x), T, H, k, _ptr(r2s), n_rows, perm_dt, _ptr(xp),
                               _ptr(xs)), "oracle_gather")
    return xp, xs


def expert_ffn(groups, x_perm, x_perm_scale, offsets, H: int, I: int, n_threads: int = 0):
    """groups: one entry per group, a dict(w13, w13_scale, w2, w2_scale) or None
    (only for groups without rows). Returns y_perm [offsets[-1], H] fp64."""
    offsets = _c(offsets, np.int32)
    n_groups = len(offsets) - 1
    assert len(groups) == n_groups
    keep = []
    w13p = (C.c_void_p * n_groups)()
    w13s = (C.c_void_p * n_groups)()
    w2p = (C.c_void_p * n_groups)()
    w2s = (C.c_void_p * n_groups)()
    dt = None
    for g, d in enumerate(groups):
        if d is None:
            continue
        a13, a2 = _c(d["w13"]), _c(d["w2"])
        s13 = None if d.get("w13_scale") is None else _c(d["w13_scale"], np.float32)
        s2 = None if d.get("w2_scale") is None else _c(d["w2_scale"], np.float32)
        keep += [a13, a2, s13, s2]
        w13p[g], w2p[g] = _ptr(a13), _ptr(a2)
        w13s[g], w2s[g] = _ptr(s13), _ptr(s2)
        dt = dt_of(a13)
    if dt is None:
        dt = dt_of(x_perm)
    xp = _c(x_perm)
    xs = None if x_perm_scale is None else _c(x_perm_scale, np.float32)
    y = np.zeros((int(offsets[-1]), H), np.float64)
    _check(lib().oracle_expert_ffn(w13p, w13s, w2p, w2s, dt, _ptr(xp), _ptr(xs), _ptr(offsets),
                                   n_groups, H, I, n_threads, _ptr(y)), "oracle_expert_ffn")
    return y


def combine(y_perm, slot_to_row, topk_w, k: int, shared_row0: int = -1):
    y = _c(y_perm, np.float64)
    s2r = _c(slot_to_row, np.int32)
    w = _c(topk_w, np.float32)
    T = w.shape[0]
    H = y.shape[1]
    out = np.empty((T, H), np.float64)
    _check(lib().oracle_combine(_ptr(y), _ptr(s2r), _ptr(w), T, k, H, shared_row0, _ptr(out)),
           "oracle_combine")
    return out


def balanced_partition(counts, G: int):
    c = _c(counts, np.int64)
    E = c.shape[0]
    n2o = np.empty(E, np.int32)
    o2n = np.empty(E, np.int32)
    loads = np.empty(G, np.int64)
    _check(lib().oracle_balanced_partition(_ptr(c), E, G, _ptr(n2o), _ptr(o2n), _ptr(loads)),
           "oracle_balanced_partition")
    return n2o, o2n, loads


def coactivation(ids, E: int, hist=None):
    """Top-k co-activation histogram [E][E] int64, added to ``hist`` when given."""
    a = _c(ids, np.int32)
    T, k = a.shape
    h = np.zeros((E, E), np.int64) if hist is None else _c(hist, np.int64).copy()
    _check(lib().oracle_coactivation(_ptr(a), T, k, E, _ptr(h)), "oracle_coactivation")
    return h


def affinity_partition(counts, aff, G: int, tol_permille: int):
    """Balanced partition, then affinity-raising swaps under the load cap."""
    c = _c(counts, np.int64)
    A = _c(aff, np.int64)
    E = c.shape[0]
    n2o = np.empty(E, np.int32)
    o2n = np.empty(E, np.int32)
    loads = np.empty(G, np.int64)
    intra = np.zeros(1, np.int64)
    _check(lib().oracle_affinity_partition(_ptr(c), _ptr(A), E, G, tol_permille, _ptr(n2o),
                                           _ptr(o2n), _ptr(loads), _ptr(intra)),
           "oracle_affinity_partition")
    return n2o, o2n, loads, int(intra[0])


def to_output(out64, dt: int):
    """Final rounding of the combined rows: fp32 (F32 layers) or bf16 bits."""
    if dt == F32:
        return out64.astype(np.float32)
    return bf16_round(out64)


# ----------------------------------------------------------------------------
# the whole layer
# ----------------------------------------------------------------------------
def moe_layer(x, k: int, groups, shared=None, *, wr=None, bias=None, scoring=SIGMOID,
              renorm=True, topk_ids=None, topk_w=None, base=0, E_local=None, fmt=None,
              n_threads: int = 0):
    """route -> permute -> gather(+quantise) -> expert FFN -> combine.

    ``groups``: per local expert a weight dict (or None if it gets no rows);
    ``shared``: the shared expert's weight dict or None. Routing comes from
    the router (wr, bias) or is given (topk_ids, topk_w). Returns every
    intermediate plus ``out64`` (fp64) and ``out`` (rounded like the layer's
    output: fp32 for fp32 layers, bf16 bits otherwise).
    """
    x = _c(x)
    xdt = dt_of(x)
    fmt = xdt if fmt is None else fmt
    res = {}
    if topk_ids is None:
        res["logits"], topk_ids, topk_w = route(x, wr, bias, k, scoring, renorm)
    res["topk_ids"], res["topk_w"] = _c(topk_ids, np.int32), _c(topk_w, np.float32)
    E_local = len(groups) if E_local is None else E_local
    p = permute(res["topk_ids"], base, E_local, shared is not None)
    res.update(p)
    n_rows = int(p["offsets"][-1])
    xp, xs = gather(x, k, p["row_to_slot"], n_rows, fmt)
    res["x_perm"], res["x_perm_scale"] = xp, xs
    gl = list(groups) + [shared]
    H = x.shape[1]
    I = None
    for d in gl:
        if d is not None:
            I = as_np(d["w2"]).shape[1]
            break
    y = expert_ffn(gl, xp, xs, p["offsets"], H, I, n_threads) if I is not None else \
        np.zeros((n_rows, H))
    res["y_perm"] = y
    R = int(p["offsets"][E_local])
    out64 = combine(y, p["slot_to_row"], res["topk_w"], k, R if shared is not None else -1)
    res["out64"] = out64
    res["out"] = to_output(out64, F32 if xdt == F32 else BF16)
    return res
