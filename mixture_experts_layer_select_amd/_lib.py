"""ctypes binding of libmoe.so: the C-ABI entry points under the same names.

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, status codes become exceptions. Every step of
the layer runs in the library's HIP kernels. There is no fallback: if the
library has not been built this module raises on first use.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH selects another build of the same library (A/B comparisons)
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(_HERE, "libmoe.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
SOFTMAX, SIGMOID = 0, 1
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = 0, 1, 2, 3, 4

EXPORTS = [
    "moe_route", "moe_route_select_workspace_size", "moe_route_select", "moe_permute_workspace_size", "moe_permute", "moe_expert_ffn_workspace_size",
    "moe_expert_ffn", "moe_expert_ffn_gate_up", "moe_expert_ffn_down", "moe_expert_ffn_noalloc",
    "moe_quantize_tokens",
    "moe_expert_ffn_gate_up_tokens", "moe_layer_fused_workspace_size", "moe_layer_fused", "moe_combine",
    "moe_balanced_partition", "moe_gather_rows",
    "moe_count_accumulate", "moe_coactivation", "moe_affinity_partition",
    "moe_status_string", "moe_last_error_message",
]


class MoEError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


class moe_expert_weights(C.Structure):
    _fields_ = [
        ("dt", C.c_int), ("E_local", C.c_int), ("H", C.c_int), ("I", C.c_int),
        ("w13", C.c_void_p), ("w13_scale", C.c_void_p), ("w2", C.c_void_p), ("w2_scale", C.c_void_p),
        ("ws13", C.c_void_p), ("ws13_scale", C.c_void_p), ("ws2", C.c_void_p), ("ws2_scale", C.c_void_p),
    ]


_lib = None


def lib() -> C.CDLL:
    """Load libmoe.so (built by mixture_experts_layer_select_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m mixture_experts_layer_select_amd.build` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        p, i, sz = C.c_void_p, C.c_int, C.c_size_t
        L.moe_route.argtypes = [p, p, p, i, i, i, i, i, i, i, p, p, p, p]
        L.moe_route_select_workspace_size.argtypes = [i, i]
        L.moe_route_select_workspace_size.restype = sz
        L.moe_route_select.argtypes = [p, p, p, i, i, i, i, i, i, i, p, p, p, sz, p]
        L.moe_permute_workspace_size.argtypes = [i, i, i]
        L.moe_permute_workspace_size.restype = sz
        L.moe_permute.argtypes = [p, i, i, i, i, i, p, i, i, i, p, p, p, p, p, p, p, sz, p]
        L.moe_expert_ffn_workspace_size.argtypes = [C.POINTER(moe_expert_weights), i]
        L.moe_expert_ffn_workspace_size.restype = sz
        L.moe_expert_ffn.argtypes = [C.POINTER(moe_expert_weights), p, p, p, i, i, p, p, sz, p]
        L.moe_expert_ffn_gate_up.argtypes = [C.POINTER(moe_expert_weights), p, p, p, i, i, p, sz, p]
        L.moe_expert_ffn_down.argtypes = [C.POINTER(moe_expert_weights), p, i, i, p, p, sz, p]
        L.moe_expert_ffn_noalloc.argtypes = [C.POINTER(moe_expert_weights), p, p, p, i, i, p, p]
        L.moe_quantize_tokens.argtypes = [p, i, i, i, p, p, p]
        L.moe_expert_ffn_gate_up_tokens.argtypes = [C.POINTER(moe_expert_weights), p, p, i, i, p, p, i, i,
                                                    p, sz, p]
        L.moe_layer_fused_workspace_size.argtypes = [C.POINTER(moe_expert_weights), i, i, i]
        L.moe_layer_fused_workspace_size.restype = sz
        L.moe_layer_fused.argtypes = [p, p, p, i, i, i, i, i, C.POINTER(moe_expert_weights), p, p, p, p,
                                      sz, p]
        L.moe_combine.argtypes = [p, i, p, p, i, i, i, p, i, p, i, p]
        L.moe_balanced_partition.argtypes = [p, i, i, p, p, p]
        L.moe_gather_rows.argtypes = [p, i, p, p, i, sz, p]
        L.moe_count_accumulate.argtypes = [p, i, p, p]
        L.moe_coactivation.argtypes = [p, i, i, i, p, p]
        L.moe_affinity_partition.argtypes = [p, p, i, i, i, p, p, p, p]
        L.moe_status_string.argtypes = [i]
        L.moe_status_string.restype = C.c_char_p
        L.moe_last_error_message.restype = C.c_char_p
        for f in ("moe_route", "moe_route_select", "moe_permute", "moe_expert_ffn", "moe_expert_ffn_gate_up",
                  "moe_expert_ffn_down", "moe_expert_ffn_noalloc", "moe_quantize_tokens", "moe_expert_ffn_gate_up_tokens",
                  "moe_layer_fused", "moe_combine",
                  "moe_balanced_partition", "moe_gather_rows", "moe_count_accumulate",
                  "moe_coactivation", "moe_affinity_partition"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != OK:
        L = lib()
        raise MoEError(fn, L.moe_status_string(status).decode(), L.moe_last_error_message().decode())


def _ptr(t):
    """Raw pointer of a tensor (or an int address). The library reads every
    buffer as dense row-major memory, so a strided view is refused rather
    than read as raw memory."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError(f"tensor of shape {tuple(t.shape)} and strides {t.stride()} is not "
                         "contiguous: the library reads dense row-major buffers")
    return t.data_ptr()


def expect(t, name: str, dtypes, device=None):
    """Check a tensor argument's dtype (one of `dtypes`), contiguity and
    device before its pointer is handed to the library."""
    if t is None:
        return
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous (strides {t.stride()})")
    if device is not None and t.device != torch.device(device):
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"no MoE dtype for {t.dtype}")


# ----------------------------------------------------------------------------
# entry points (same names and argument order as include/moe.h)
# ----------------------------------------------------------------------------
def moe_route(x, w_router, bias, dt, T, H, E, k, scoring, renormalize, logits, topk_ids, topk_w,
              stream=None):
    _check("moe_route", lib().moe_route(_ptr(x), _ptr(w_router), _ptr(bias), dt, T, H, E, k, scoring,
                                        int(bool(renormalize)), _ptr(logits), _ptr(topk_ids),
                                        _ptr(topk_w), _stream(stream)))


def moe_route_select_workspace_size(T, E) -> int:
    return int(lib().moe_route_select_workspace_size(T, E))


def moe_route_select(x, w_router, bias, dt, T, H, E, k, scoring, renormalize, topk_ids, topk_w,
                     workspace, ws_bytes, stream=None):
    _check("moe_route_select", lib().moe_route_select(
        _ptr(x), _ptr(w_router), _ptr(bias), dt, T, H, E, k, scoring, int(bool(renormalize)),
        _ptr(topk_ids), _ptr(topk_w), _ptr(workspace), ws_bytes, _stream(stream)))


def moe_permute_workspace_size(T, k, E_local) -> int:
    return int(lib().moe_permute_workspace_size(T, k, E_local))


def moe_permute(topk_ids, T, k, expert_base, E_local, include_shared, x, x_dt, H, perm_dt,
                expert_counts, expert_offsets, row_to_slot, slot_to_row, x_perm, x_perm_scale,
                workspace, ws_bytes, stream=None):
    _check("moe_permute", lib().moe_permute(
        _ptr(topk_ids), T, k, expert_base, E_local, int(bool(include_shared)), _ptr(x), x_dt, H,
        perm_dt, _ptr(expert_counts), _ptr(expert_offsets), _ptr(row_to_slot), _ptr(slot_to_row),
        _ptr(x_perm), _ptr(x_perm_scale), _ptr(workspace), ws_bytes, _stream(stream)))


def make_weights(dt, E_local, H, I, w13, w2, w13_scale=None, w2_scale=None, ws13=None, ws2=None,
                 ws13_scale=None, ws2_scale=None) -> moe_expert_weights:
    w = moe_expert_weights(dt, E_local, H, I, _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale),
                           _ptr(ws13), _ptr(ws13_scale), _ptr(ws2), _ptr(ws2_scale))
    # the struct holds raw device pointers: keep the tensors alive with it, or
    # their memory could be handed to other tensors while the struct is in use
    w._tensors = (w13, w2, w13_scale, w2_scale, ws13, ws2, ws13_scale, ws2_scale)
    return w


def moe_expert_ffn_workspace_size(w: moe_expert_weights, max_rows: int) -> int:
    return int(lib().moe_expert_ffn_workspace_size(C.byref(w), max_rows))


def moe_expert_ffn(w: moe_expert_weights, x_perm, x_perm_scale, expert_offsets, n_groups, max_rows,
                   y_perm, workspace, ws_bytes, stream=None):
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        C.byref(w), _ptr(x_perm), _ptr(x_perm_scale), _ptr(expert_offsets), n_groups, max_rows,
        _ptr(y_perm), _ptr(workspace), ws_bytes, _stream(stream)))


def moe_expert_ffn_gate_up(w: moe_expert_weights, x_perm, x_perm_scale, expert_offsets, n_groups,
                           max_rows, workspace, ws_bytes, stream=None):
    _check("moe_expert_ffn_gate_up", lib().moe_expert_ffn_gate_up(
        C.byref(w), _ptr(x_perm), _ptr(x_perm_scale), _ptr(expert_offsets), n_groups, max_rows,
        _ptr(workspace), ws_bytes, _stream(stream)))


# size of the static device scratch behind moe_expert_ffn_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_expert_ffn_noalloc(w: moe_expert_weights, x_perm, x_perm_scale, expert_offsets, n_groups,
                           max_rows, y_perm, stream=None):
    _check("moe_expert_ffn_noalloc", lib().moe_expert_ffn_noalloc(
        C.byref(w), _ptr(x_perm), _ptr(x_perm_scale), _ptr(expert_offsets), n_groups, max_rows,
        _ptr(y_perm), _stream(stream)))


def moe_quantize_tokens(x, x_dt, T, H, codes, scales, stream=None):
    _check("moe_quantize_tokens", lib().moe_quantize_tokens(
        _ptr(x), x_dt, T, H, _ptr(codes), _ptr(scales), _stream(stream)))


def moe_expert_ffn_gate_up_tokens(w: moe_expert_weights, x_tokens, x_tokens_scale, T, k, row_to_slot,
                                  expert_offsets, n_groups, max_rows, workspace, ws_bytes, stream=None):
    _check("moe_expert_ffn_gate_up_tokens", lib().moe_expert_ffn_gate_up_tokens(
        C.byref(w), _ptr(x_tokens), _ptr(x_tokens_scale), T, k, _ptr(row_to_slot),
        _ptr(expert_offsets), n_groups, max_rows, _ptr(workspace), ws_bytes, _stream(stream)))


def moe_layer_fused_workspace_size(w: moe_expert_weights, T, E, k) -> int:
    return int(lib().moe_layer_fused_workspace_size(C.byref(w), T, E, k))


def moe_layer_fused(x, w_router, bias, T, E, k, scoring, renormalize, w: moe_expert_weights, topk_ids,
                    topk_w, out, workspace, ws_bytes, stream=None):
    _check("moe_layer_fused", lib().moe_layer_fused(
        _ptr(x), _ptr(w_router), _ptr(bias), T, E, k, scoring, int(bool(renormalize)), C.byref(w),
        _ptr(topk_ids), _ptr(topk_w), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))


def moe_expert_ffn_down(w: moe_expert_weights, expert_offsets, n_groups, max_rows, y_perm, workspace,
                        ws_bytes, stream=None):
    _check("moe_expert_ffn_down", lib().moe_expert_ffn_down(
        C.byref(w), _ptr(expert_offsets), n_groups, max_rows, _ptr(y_perm), _ptr(workspace),
        ws_bytes, _stream(stream)))


def moe_combine(y_perm, y_dt, slot_to_row, topk_w, T, k, H, expert_offsets, shared_group, out, out_dt,
                stream=None):
    _check("moe_combine", lib().moe_combine(
        _ptr(y_perm), y_dt, _ptr(slot_to_row), _ptr(topk_w), T, k, H, _ptr(expert_offsets),
        shared_group, _ptr(out), out_dt, _stream(stream)))


def moe_balanced_partition(counts, E, G, new_to_old, old_to_new, group_loads):
    """Host call: all arguments are CPU tensors (int64 counts/loads, int32 maps)."""
    for t in (counts, new_to_old, old_to_new, group_loads):
        assert t.device.type == "cpu" and t.is_contiguous()
    _check("moe_balanced_partition", lib().moe_balanced_partition(
        _ptr(counts), E, G, _ptr(new_to_old), _ptr(old_to_new), _ptr(group_loads)))


def moe_gather_rows(src, n_src_rows, dst, index, n_rows, row_bytes, stream=None):
    _check("moe_gather_rows", lib().moe_gather_rows(_ptr(src), n_src_rows, _ptr(dst), _ptr(index),
                                                    n_rows, row_bytes, _stream(stream)))


def moe_count_accumulate(counts, n, acc, stream=None):
    """acc[i] += counts[i] on the device (int32 counts, int64 acc)."""
    _check("moe_count_accumulate", lib().moe_count_accumulate(_ptr(counts), n, _ptr(acc),
                                                              _stream(stream)))


def moe_coactivation(topk_ids, T, k, E, hist, stream=None):
    """Adds one step's picks to the [E, E] int64 co-activation histogram."""
    _check("moe_coactivation", lib().moe_coactivation(_ptr(topk_ids), T, k, E, _ptr(hist),
                                                      _stream(stream)))


def moe_affinity_partition(counts, aff, E, G, tol_permille, new_to_old, old_to_new, group_loads,
                           intra_affinity):
    """Host call: CPU tensors (int64 counts/aff/loads/intra_affinity[1], int32 maps)."""
    for t in (counts, aff, new_to_old, old_to_new, group_loads, intra_affinity):
        assert t.device.type == "cpu" and t.is_contiguous()
    _check("moe_affinity_partition", lib().moe_affinity_partition(
        _ptr(counts), _ptr(aff), E, G, tol_permille, _ptr(new_to_old), _ptr(old_to_new),
        _ptr(group_loads), _ptr(intra_affinity)))
