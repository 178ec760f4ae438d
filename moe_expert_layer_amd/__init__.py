"""MI355X (gfx950) MoE expert layer, forward and backward: Python binding over the C ABI in
``include/moe_expert_layer.h``.

Every step of the layer runs in the HIP library (``libmoe_expert_layer.so``, built in-tree by
``moe_expert_layer_amd.build``).  This module only checks tensor shapes, allocates outputs and
workspaces with torch, and passes device pointers and the current HIP stream across the ABI.  If
the library is missing, every call raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "MoeError", "library", "lib_path", "F32", "BF16", "MXFP8",
    "workspace_size", "expert_forward", "expert_forward_mx", "expert_forward_train",
    "backward_workspace_size", "expert_backward", "route", "route_noalloc", "permute", "unpermute",
    "grouped_ffn_workspace_size", "grouped_ffn", "grouped_ffn_mx", "mx_quantize",
    "mx_fc1_epilogue_encode", "device_status", "chunk_counters",
    "intermediate_h", "quantized_x",
    "timing_enable", "timing_collect", "timing_reset",
]

F32, BF16, MXFP8 = 0, 1, 2
_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmoe_expert_layer.so")
_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


class MoeProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("F", ctypes.c_int64),
                ("E", ctypes.c_int64), ("k", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("head_m_size", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name


_SIGS = {
    "moe_workspace_size": [ctypes.POINTER(MoeProblem), ctypes.POINTER(ctypes.c_size_t)],
    "moe_expert_forward": [ctypes.POINTER(MoeProblem)] + [_P] * 8 + [ctypes.c_size_t, _P],
    "moe_expert_forward_mx": [ctypes.POINTER(MoeProblem)] + [_P] * 12 + [ctypes.c_size_t, _P],
    "moe_backward_workspace_size": [ctypes.POINTER(MoeProblem), ctypes.POINTER(ctypes.c_size_t)],
    "moe_expert_backward": [ctypes.POINTER(MoeProblem)] + [_P] * 14 + [ctypes.c_size_t, _P],
    "moe_expert_forward_train": [ctypes.POINTER(MoeProblem)] + [_P] * 9 + [ctypes.c_size_t, _P],
    "moe_route_workspace_size": [_I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
    "moe_route": [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_route_noalloc": [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P],
    "moe_permute": [ctypes.POINTER(MoeProblem), _P, _P, _P, _P, _P, _P],
    "moe_unpermute": [ctypes.POINTER(MoeProblem), _P, _P, _P, _P, _P],
    "moe_grouped_ffn_workspace_size": [ctypes.POINTER(MoeProblem), _I64, _I64,
                                       ctypes.POINTER(ctypes.c_size_t)],
    "moe_grouped_ffn": [ctypes.POINTER(MoeProblem), _P, _I64, _P, _P, _I64, _P, _P, _P, _P, _P,
                        ctypes.c_size_t, _P],
    "moe_grouped_ffn_mx": [ctypes.POINTER(MoeProblem), _P, _P, _I64, _P, _P, _I64, _P, _P, _P,
                           _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_mx_quantize": [_P, _I64, _I64, _P, _P, _P],
    "moe_mx_fc1_epilogue_encode": [_P, _I64, _I64, ctypes.c_int32, _P, _P, _P],
    "moe_router_topk": [_P, _I64, _I64, _I64, _P, _P, _P],
    "moe_query_device_status": [_P, _P, ctypes.POINTER(ctypes.c_int32)],
    "moe_chunk_counters": [ctypes.POINTER(MoeProblem), _P, ctypes.c_size_t, _I64,
                           ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_I64)],
    "moe_quantized_x_offsets": [ctypes.POINTER(MoeProblem), ctypes.POINTER(ctypes.c_size_t),
                                ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_int32)],
    "moe_intermediate_offsets": [ctypes.POINTER(MoeProblem), _I64, _I64,
                                 ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)],
    "moe_status_string": [ctypes.c_int],
    "moe_last_error": [],
    "moe_timing_enable": [ctypes.c_int],
    "moe_timing_collect": [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                           ctypes.POINTER(_I64), ctypes.c_int, ctypes.POINTER(ctypes.c_int)],
    "moe_timing_reset": [],
}


def library(path: str | None = None):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            p = path or lib_path
            if not os.path.exists(p):
                raise RuntimeError(f"HIP library {p} is missing: build it with "
                                   "`python -m moe_expert_layer_amd.build` (no CPU fallback exists)")
            lib = ctypes.CDLL(p)
            for name, args in _SIGS.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = ctypes.c_int
            lib.moe_status_string.restype = ctypes.c_char_p
            lib.moe_last_error.restype = ctypes.c_char_p
            _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        lib = library()
        raise MoeError(status, lib.moe_status_string(status).decode(), lib.moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16; MX uses the *_mx calls)")


FLAG_SEPARATE_PERMUTE = 1    # run the permute step as a kernel of its own (see the C header)
FLAG_QUANTIZE_X = 2          # MX problem with bfloat16 x, encoded by the library (see the C header)


def problem(T, H, F, E, k, dtype, head_m_size=0, flags=0) -> MoeProblem:
    return MoeProblem(int(T), int(H), int(F), int(E), int(k), int(dtype), int(head_m_size), int(flags), 0)


def workspace_size(prob: MoeProblem) -> int:
    n = ctypes.c_size_t()
    _check(library().moe_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
    return n.value


def _workspace(nbytes: int, device, workspace):
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _need(workspace, "workspace", torch.uint8, device=device)
    if workspace.numel() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes, has {workspace.numel()}")
    return workspace


# ---------------------------------------------------------------------------------------------- layer

def expert_forward(x, w_gate, w_up, w_down, expert_ids, probs, head_m_size: int = 0, out=None,
                   workspace=None, separate_permute: bool = False):
    """out[T,H] = sum_j probs[t,j] * FFN_{expert_ids[t,j]}(x[t]) for float32 or bfloat16 inputs."""
    dt = _dtype_code(x)
    T, H = x.shape
    E, _, F = w_gate.shape
    k = expert_ids.shape[1]
    dev = x.device
    _need(x, "x", x.dtype, (T, H))
    _need(w_gate, "w_gate", x.dtype, (E, H, F), dev)
    _need(w_up, "w_up", x.dtype, (E, H, F), dev)
    _need(w_down, "w_down", x.dtype, (E, F, H), dev)
    _need(expert_ids, "expert_ids", torch.int32, (T, k), dev)
    _need(probs, "probs", torch.float32, (T, k), dev)
    prob = problem(T, H, F, E, k, dt, head_m_size, FLAG_SEPARATE_PERMUTE if separate_permute else 0)
    ws = _workspace(workspace_size(prob), dev, workspace)
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=dev)
    _need(out, "out", x.dtype, (T, H), dev)
    _check(library().moe_expert_forward(ctypes.byref(prob), _ptr(x), _ptr(w_gate), _ptr(w_up),
                                        _ptr(w_down), _ptr(expert_ids), _ptr(probs), _ptr(out),
                                        _ptr(ws), ws.numel(), _stream(x)))
    return out


def backward_workspace_size(prob: MoeProblem) -> int:
    n = ctypes.c_size_t()
    _check(library().moe_backward_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
    return n.value


def expert_forward_train(x, w_gate, w_up, w_down, expert_ids, probs, out=None, saved_gu=None,
                        workspace=None):
    """expert_forward (bfloat16) that also returns g and u of every routed slot, bf16 [2, T*k, F],
    for expert_backward(..., saved_gu=...).  Returns (out, saved_gu)."""
    T, H = x.shape
    E, _, F = w_gate.shape
    k = expert_ids.shape[1]
    dev = x.device
    bf = torch.bfloat16
    _need(x, "x", bf, (T, H))
    _need(w_gate, "w_gate", bf, (E, H, F), dev)
    _need(w_up, "w_up", bf, (E, H, F), dev)
    _need(w_down, "w_down", bf, (E, F, H), dev)
    _need(expert_ids, "expert_ids", torch.int32, (T, k), dev)
    _need(probs, "probs", torch.float32, (T, k), dev)
    prob = problem(T, H, F, E, k, BF16)
    ws = _workspace(workspace_size(prob), dev, workspace)
    if out is None:
        out = torch.empty((T, H), dtype=bf, device=dev)
    if saved_gu is None:
        saved_gu = torch.empty((2, T * k, F), dtype=bf, device=dev)
    _need(out, "out", bf, (T, H), dev)
    _need(saved_gu, "saved_gu", bf, (2, T * k, F), dev)
    _check(library().moe_expert_forward_train(ctypes.byref(prob), _ptr(x), _ptr(w_gate), _ptr(w_up),
                                              _ptr(w_down), _ptr(expert_ids), _ptr(probs), _ptr(out),
                                              _ptr(saved_gu), _ptr(ws), ws.numel(), _stream(x)))
    return out, saved_gu


def expert_backward(x, w_gate, w_up, w_down, expert_ids, probs, dout, workspace=None,
                    saved_gu=None):
    """Gradients of sum(dout * out) for expert_forward's bfloat16 layer:
    (dx bf16 [T,H], dw_gate f32 [E,H,F], dw_up f32 [E,H,F], dw_down f32 [E,F,H], dprobs f32 [T,k]).
    saved_gu: g and u from expert_forward_train on the same inputs (skips their recomputation)."""
    T, H = x.shape
    E, _, F = w_gate.shape
    k = expert_ids.shape[1]
    dev = x.device
    bf = torch.bfloat16
    _need(x, "x", bf, (T, H))
    _need(w_gate, "w_gate", bf, (E, H, F), dev)
    _need(w_up, "w_up", bf, (E, H, F), dev)
    _need(w_down, "w_down", bf, (E, F, H), dev)
    _need(expert_ids, "expert_ids", torch.int32, (T, k), dev)
    _need(probs, "probs", torch.float32, (T, k), dev)
    _need(dout, "dout", bf, (T, H), dev)
    if saved_gu is not None:
        _need(saved_gu, "saved_gu", bf, (2, T * k, F), dev)
    prob = problem(T, H, F, E, k, BF16)
    ws = _workspace(backward_workspace_size(prob), dev, workspace)
    dx = torch.empty((T, H), dtype=bf, device=dev)
    dwg = torch.empty((E, H, F), dtype=torch.float32, device=dev)
    dwu = torch.empty((E, H, F), dtype=torch.float32, device=dev)
    dwd = torch.empty((E, F, H), dtype=torch.float32, device=dev)
    dprobs = torch.empty((T, k), dtype=torch.float32, device=dev)
    _check(library().moe_expert_backward(ctypes.byref(prob), _ptr(x), _ptr(w_gate), _ptr(w_up),
                                         _ptr(w_down), _ptr(expert_ids), _ptr(probs), _ptr(dout),
                                         _ptr(saved_gu), _ptr(dx), _ptr(dwg), _ptr(dwu), _ptr(dwd),
                                         _ptr(dprobs),
                                         _ptr(ws), ws.numel(), _stream(x)))
    return dx, dwg, dwu, dwd, dprobs


def expert_forward_mx(x, x_scale, w_gate, wg_scale, w_up, wu_scale, w_down, wd_scale, expert_ids,
                      probs, head_m_size: int = 0, out=None, workspace=None,
                      separate_permute: bool = False):
    """The same layer on OCP-MX E4M3 bytes (uint8 tensors) with E8M0 block scales; bf16 output.
    A bfloat16 x with x_scale None is encoded by the library on its way into the gather
    (MOE_FLAG_QUANTIZE_X)."""
    T, H = x.shape
    E, _, F = w_gate.shape
    k = expert_ids.shape[1]
    dev = x.device
    u8 = torch.uint8
    quantize_x = x.dtype == torch.bfloat16
    if quantize_x:
        if x_scale is not None:
            raise ValueError("a bfloat16 x is encoded by the library: pass x_scale=None")
        _need(x, "x", torch.bfloat16, (T, H))
    else:
        _need(x, "x", u8, (T, H))
        _need(x_scale, "x_scale", u8, (T, H // 32), dev)
    _need(w_gate, "w_gate", u8, (E, H, F), dev)
    _need(wg_scale, "wg_scale", u8, (E, H // 32, F), dev)
    _need(w_up, "w_up", u8, (E, H, F), dev)
    _need(wu_scale, "wu_scale", u8, (E, H // 32, F), dev)
    _need(w_down, "w_down", u8, (E, F, H), dev)
    _need(wd_scale, "wd_scale", u8, (E, F // 32, H), dev)
    _need(expert_ids, "expert_ids", torch.int32, (T, k), dev)
    _need(probs, "probs", torch.float32, (T, k), dev)
    flags = (FLAG_SEPARATE_PERMUTE if separate_permute else 0) | (FLAG_QUANTIZE_X if quantize_x else 0)
    prob = problem(T, H, F, E, k, MXFP8, head_m_size, flags)
    ws = _workspace(workspace_size(prob), dev, workspace)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H), dev)
    _check(library().moe_expert_forward_mx(
        ctypes.byref(prob), _ptr(x), _ptr(x_scale), _ptr(w_gate), _ptr(wg_scale), _ptr(w_up),
        _ptr(wu_scale), _ptr(w_down), _ptr(wd_scale), _ptr(expert_ids), _ptr(probs), _ptr(out),
        _ptr(ws), ws.numel(), _stream(x)))
    return out


# ---------------------------------------------------------------------------------------------- sub-steps

def route(expert_ids, E: int, workspace=None):
    """(counts[E], offsets[E+1], perm[M], pos[M], workspace) for int32 ids [T, k]."""
    _need(expert_ids, "expert_ids", torch.int32)
    T, k = expert_ids.shape
    dev = expert_ids.device
    n = ctypes.c_size_t()
    _check(library().moe_route_workspace_size(T, k, E, ctypes.byref(n)))
    ws = _workspace(n.value, dev, workspace)
    i32 = dict(dtype=torch.int32, device=dev)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    perm, pos = torch.empty(T * k, **i32), torch.empty(T * k, **i32)
    _check(library().moe_route(_ptr(expert_ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm),
                               _ptr(pos), _ptr(ws), ws.numel(), _stream(expert_ids)))
    return counts, offsets, perm, pos, ws


def route_noalloc(expert_ids, E: int, out=None):
    """moe_route without a workspace (the library's static per-GPU scratch): (counts[E],
    offsets[E+1], perm[M], pos[M]).  `out` may hold those four int32 tensors to write into."""
    _need(expert_ids, "expert_ids", torch.int32)
    T, k = expert_ids.shape
    dev = expert_ids.device
    i32 = dict(dtype=torch.int32, device=dev)
    if out is None:
        out = (torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(T * k, **i32),
               torch.empty(T * k, **i32))
    for t, n, name in zip(out, (E, E + 1, T * k, T * k), ("counts", "offsets", "perm", "pos")):
        _need(t, name, torch.int32, (n,), dev)
    counts, offsets, perm, pos = out
    _check(library().moe_route_noalloc(_ptr(expert_ids), T, k, E, _ptr(counts), _ptr(offsets),
                                       _ptr(perm), _ptr(pos), _stream(expert_ids)))
    return counts, offsets, perm, pos


def permute(x, pos, k: int, E: int | None = None, x_scale=None, F: int = 128, x_perm=None,
            x_perm_scale=None):
    """x_perm[pos[s]] = x[s // k].  x float32 / bfloat16, or uint8 MX codes with x_scale.  The
    outputs are allocated unless given."""
    T, H = x.shape
    mx = x.dtype == torch.uint8
    dt = MXFP8 if mx else _dtype_code(x)
    _need(x, "x")
    _need(pos, "pos", torch.int32, (T * k,), x.device)
    prob = problem(T, H, F, E if E is not None else k, k, dt)
    if x_perm is None:
        x_perm = torch.empty((T * k, H), dtype=x.dtype, device=x.device)
    _need(x_perm, "x_perm", x.dtype, (T * k, H), x.device)
    xs_perm = None
    if mx:
        _need(x_scale, "x_scale", torch.uint8, (T, H // 32), x.device)
        xs_perm = x_perm_scale
        if xs_perm is None:
            xs_perm = torch.empty((T * k, H // 32), dtype=torch.uint8, device=x.device)
        _need(xs_perm, "x_perm_scale", torch.uint8, (T * k, H // 32), x.device)
    _check(library().moe_permute(ctypes.byref(prob), _ptr(x), _ptr(x_scale), _ptr(pos),
                                 _ptr(x_perm), _ptr(xs_perm), _stream(x)))
    return (x_perm, xs_perm) if mx else x_perm


def unpermute(y_perm, pos, probs, F: int = 128, E: int | None = None, out=None):
    """out[t] = sum_j probs[t,j] * y_perm[pos[t*k+j]] (float32 or bfloat16 rows); out is allocated
    unless given."""
    T, k = probs.shape
    M, H = y_perm.shape
    dt = _dtype_code(y_perm)
    _need(y_perm, "y_perm")
    _need(pos, "pos", torch.int32, (T * k,), y_perm.device)
    _need(probs, "probs", torch.float32, (T, k), y_perm.device)
    if M != T * k:
        raise ValueError("y_perm must have T*k rows")
    prob = problem(T, H, F, E if E is not None else k, k, dt)
    if out is None:
        out = torch.empty((T, H), dtype=y_perm.dtype, device=y_perm.device)
    _need(out, "out", y_perm.dtype, (T, H), y_perm.device)
    _check(library().moe_unpermute(ctypes.byref(prob), _ptr(y_perm), _ptr(pos), _ptr(probs),
                                   _ptr(out), _stream(y_perm)))
    return out


def grouped_ffn_workspace_size(prob: MoeProblem, M: int, G: int) -> int:
    n = ctypes.c_size_t()
    _check(library().moe_grouped_ffn_workspace_size(ctypes.byref(prob), M, G, ctypes.byref(n)))
    return n.value


def grouped_ffn(rows, group_offsets, group_expert, w_gate, w_up, w_down, head_m_size: int = 0,
                workspace=None, out=None):
    """y[r] = FFN_{expert of r's group}(rows[r]) on rows already grouped (float32 / bfloat16)."""
    M, H = rows.shape
    E, _, F = w_gate.shape
    G = group_expert.shape[0]
    dev = rows.device
    dt = _dtype_code(rows)
    _need(rows, "rows", rows.dtype, (M, H))
    _need(group_offsets, "group_offsets", torch.int32, (G + 1,), dev)
    _need(group_expert, "group_expert", torch.int32, (G,), dev)
    for name, w, shp in (("w_gate", w_gate, (E, H, F)), ("w_up", w_up, (E, H, F)),
                         ("w_down", w_down, (E, F, H))):
        _need(w, name, rows.dtype, shp, dev)
    prob = problem(0, H, F, E, 1, dt, head_m_size)
    n = ctypes.c_size_t()
    _check(library().moe_grouped_ffn_workspace_size(ctypes.byref(prob), M, G, ctypes.byref(n)))
    ws = _workspace(n.value, dev, workspace)
    if out is None:
        out = torch.empty((M, H), dtype=rows.dtype, device=dev)
    _check(library().moe_grouped_ffn(ctypes.byref(prob), _ptr(rows), M, _ptr(group_offsets),
                                     _ptr(group_expert), G, _ptr(w_gate), _ptr(w_up),
                                     _ptr(w_down), _ptr(out), _ptr(ws), ws.numel(), _stream(rows)))
    return out


def grouped_ffn_mx(rows, rows_scale, group_offsets, group_expert, w_gate, wg_scale, w_up,
                   wu_scale, w_down, wd_scale, head_m_size: int = 0, workspace=None, out=None):
    M, H = rows.shape
    E, _, F = w_gate.shape
    G = group_expert.shape[0]
    dev = rows.device
    prob = problem(0, H, F, E, 1, MXFP8, head_m_size)
    n = ctypes.c_size_t()
    _check(library().moe_grouped_ffn_workspace_size(ctypes.byref(prob), M, G, ctypes.byref(n)))
    ws = _workspace(n.value, dev, workspace)
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    _check(library().moe_grouped_ffn_mx(
        ctypes.byref(prob), _ptr(rows), _ptr(rows_scale), M, _ptr(group_offsets),
        _ptr(group_expert), G, _ptr(w_gate), _ptr(wg_scale), _ptr(w_up), _ptr(wu_scale),
        _ptr(w_down), _ptr(wd_scale), _ptr(out), _ptr(ws), ws.numel(), _stream(rows)))
    return out


def router_topk(logits, k: int):
    """Top-k gate: float32 logits [T, E] -> (expert_ids int32 [T, k], probs float32 [T, k])."""
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    probs = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(library().moe_router_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(probs), _stream(logits)))
    return ids, probs


def mx_quantize(v):
    """OCP-MX encode float32 [rows, cols] -> (codes uint8 [rows, cols], scales uint8 [rows, cols/32])."""
    _need(v, "v", torch.float32)
    rows, cols = v.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=v.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=v.device)
    _check(library().moe_mx_quantize(_ptr(v), rows, cols, _ptr(codes), _ptr(scales), _stream(v)))
    return codes, scales


def mx_fc1_epilogue_encode(v, large_tiles: bool = True):
    """The MX fc1 epilogue's encoder (the GEMM's own device code) on float32 v [rows, cols] in place
    of the SwiGLU output -> (codes uint8 [rows, cols], scales uint8 [rows, cols/32])."""
    _need(v, "v", torch.float32)
    rows, cols = v.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=v.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=v.device)
    _check(library().moe_mx_fc1_epilogue_encode(_ptr(v), rows, cols, 1 if large_tiles else 0,
                                                _ptr(codes), _ptr(scales), _stream(v)))
    return codes, scales


# ---------------------------------------------------------------------------------------------- status

def device_status(workspace) -> int:
    """Waits for the current stream, then returns the status word of the last call on `workspace`."""
    st = ctypes.c_int32()
    _check(library().moe_query_device_status(_ptr(workspace), _stream(workspace), ctypes.byref(st)))
    return int(st.value)


def chunk_counters(workspace, M: int, H: int, F: int, head_m_size: int, dtype: int = BF16):
    """(done, expected) int32 tensors (views into the workspace) of a chunked call's counters."""
    prob = problem(0, H, F, 1, 1, dtype, head_m_size)
    c, t, n = _P(), _P(), _I64()
    _check(library().moe_chunk_counters(ctypes.byref(prob), _ptr(workspace), workspace.numel(), M,
                                        ctypes.byref(c), ctypes.byref(t), ctypes.byref(n)))
    base = workspace.data_ptr()
    oc, ot = c.value - base, t.value - base
    nb = 4 * n.value
    return (workspace[oc:oc + nb].view(torch.int32), workspace[ot:ot + nb].view(torch.int32))


def quantized_x(workspace, T: int, H: int, F: int, E: int, k: int, head_m_size: int = 0,
                separate_permute: bool = False):
    """Views into `workspace` of the encoded x that a forward with a bfloat16 x left there:
    (codes uint8 [rows, H], scales uint8 [rows, H/32], permuted), in token order (rows = T,
    permuted False) or in the permuted row order (rows = T*k, permuted True)."""
    flags = FLAG_QUANTIZE_X | (FLAG_SEPARATE_PERMUTE if separate_permute else 0)
    prob = problem(T, H, F, E, k, MXFP8, head_m_size, flags)
    co, so, pm = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int32()
    _check(library().moe_quantized_x_offsets(ctypes.byref(prob), ctypes.byref(co), ctypes.byref(so),
                                             ctypes.byref(pm)))
    rows = T * k if pm.value else T
    return (workspace[co.value:co.value + rows * H].view(rows, H),
            workspace[so.value:so.value + rows * (H // 32)].view(rows, H // 32), bool(pm.value))


def intermediate_h(workspace, M: int, G: int, H: int, F: int, E: int, dtype: int,
                   head_m_size: int = 0):
    """Views into `workspace` of the SwiGLU output h [M, F] (and MX scales [M, F/32], else None)
    left there by the last grouped-FFN or forward call that used it."""
    prob = problem(0, H, F, E, 1, dtype, head_m_size)
    ho, so = ctypes.c_size_t(), ctypes.c_size_t()
    _check(library().moe_intermediate_offsets(ctypes.byref(prob), M, G, ctypes.byref(ho),
                                              ctypes.byref(so)))
    esz = {F32: 4, BF16: 2, MXFP8: 1}[dtype]
    h = workspace[ho.value:ho.value + M * F * esz]
    if dtype == MXFP8:
        return h.view(M, F), workspace[so.value:so.value + M * (F // 32)].view(M, F // 32)
    return h.view(torch.float32 if dtype == F32 else torch.bfloat16).view(M, F), None


def timing_enable(on: bool = True):
    _check(library().moe_timing_enable(1 if on else 0))


def timing_reset():
    _check(library().moe_timing_reset())


def timing_collect() -> dict:
    """{kernel name: (total ms, launches)} accumulated since the last reset."""
    lib = library()
    cap = 64
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_double * cap)()
    cnt = (_I64 * cap)()
    n = ctypes.c_int()
    _check(lib.moe_timing_collect(names, ms, cnt, cap, ctypes.byref(n)))
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(min(n.value, cap))}
