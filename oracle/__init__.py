"""CPU oracle for the MoE expert layer, forward and backward (ctypes wrapper around ``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the CPU-baseline leg of
the benchmark.  Nothing in the HIP library imports or calls it, and it imports nothing from the HIP
library's package.  All arithmetic lives in ``oracle.c`` (double precision); this module only moves
numpy arrays across the C boundary.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against things other than itself
(numpy's bincount / stable argsort, a numpy fp64 dense MLP, torch's float8_e4m3fn codec, closed
forms, hand-derived golden fixtures, brute-force per-token loops and invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

DTYPES = {"f32": 0, "bf16": 1, "mxfp8": 2}
_ESIZE = {"f32": 4, "bf16": 2, "mxfp8": 1}

GCC_CMD = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-o", _LIB, _SRC, "-lm"]


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (generic x86-64 code, so the library also runs on other hosts)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = list(GCC_CMD)
        cmd[cmd.index(_LIB)] = tmp
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
            lib.oracle_route.argtypes = [P, I64, I64, I64, P, P, P, P]
            lib.oracle_route.restype = I32
            lib.oracle_router.argtypes = [P, I64, I64, I64, P, P]
            lib.oracle_router.restype = None
            lib.oracle_permute.argtypes = [P, I64, P, I64, I64, P]
            lib.oracle_permute.restype = None
            lib.oracle_ffn_rows.argtypes = [I32, I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, P]
            lib.oracle_ffn_rows.restype = I32
            lib.oracle_forward.argtypes = ([I32] + [I64] * 5 + [P] * 10 + [I64] + [P] * 5)
            lib.oracle_forward.restype = I32
            lib.oracle_forward_tokens.argtypes = ([I32] + [I64] * 5 + [P] * 11 + [I64, P])
            lib.oracle_forward_tokens.restype = I32
            lib.oracle_backward.argtypes = [I32] + [I64] * 5 + [P] * 12
            lib.oracle_backward.restype = I32
            lib.oracle_backward_tokens.argtypes = [I32] + [I64] * 5 + [P] * 8 + [I64, P, P]
            lib.oracle_backward_tokens.restype = I32
            lib.oracle_wgrad_entries.argtypes = [I32] + [I64] * 5 + [P] * 7 + [I64] + [P] * 6
            lib.oracle_wgrad_entries.restype = I32
            lib.oracle_mx_quantize.argtypes = [P, I64, P, P]
            lib.oracle_mx_quantize.restype = None
            lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
            lib.oracle_e4m3_encode.restype = ctypes.c_uint8
            lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
            lib.oracle_e4m3_value.restype = ctypes.c_double
            lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
            lib.oracle_e8m0_value.restype = ctypes.c_double
            lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
            lib.oracle_bf16_value.restype = ctypes.c_double
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = I32
            _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype) if dtype is not None else np.ascontiguousarray(a)


class OracleError(RuntimeError):
    pass


def num_threads() -> int:
    return int(_load().oracle_num_threads())


# ---------------------------------------------------------------------------------------------- codecs

def bf16_value(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.oracle_bf16_value(int(v)) for v in b]).reshape(np.shape(bits))


def e4m3_value(code: int) -> float:
    return float(_load().oracle_e4m3_value(int(code)))


def e8m0_value(code: int) -> float:
    return float(_load().oracle_e8m0_value(int(code)))


def e4m3_encode(v: float) -> int:
    return int(_load().oracle_e4m3_encode(float(v)))


def mx_quantize(v) -> tuple[np.ndarray, np.ndarray]:
    """Encode the last axis of ``v`` (a multiple of 32) in OCP-MX E4M3 blocks of 32.
    Returns (codes uint8 same shape, scales uint8 with last axis / 32)."""
    v = _c(v, np.float64)
    n = v.shape[-1]
    if n % 32:
        raise ValueError("last axis must be a multiple of 32")
    nb = v.size // 32
    q = np.empty(v.shape, np.uint8)
    s = np.empty(v.shape[:-1] + (n // 32,), np.uint8)
    _load().oracle_mx_quantize(_p(v), nb, _p(q), _p(s))
    return q, s


def mx_decode(codes, scales) -> np.ndarray:
    """Value of each element: E4M3 code value times its block's E8M0 scale (last axis blocks of 32)."""
    lib = _load()
    t4 = np.array([lib.oracle_e4m3_value(i) for i in range(256)])
    t8 = np.array([lib.oracle_e8m0_value(i) for i in range(256)])
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    return t4[codes] * np.repeat(t8[scales], 32, axis=-1)


# ---------------------------------------------------------------------------------------------- route / permute

def route(expert_ids, E: int):
    """counts[E], offsets[E+1], perm[M], pos[M] (int32) for ids [T, k]."""
    ids = _c(expert_ids, np.int32)
    T, k = ids.shape
    M = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(M, np.int32)
    pos = np.empty(M, np.int32)
    rc = _load().oracle_route(_p(ids), T, k, E, _p(counts), _p(offsets), _p(perm), _p(pos))
    if rc != 0:
        raise OracleError("expert id out of range")
    return counts, offsets, perm, pos


def router(logits, k: int):
    """Top-k gate: (expert_ids int32 [T, k] in descending logit order, ties to the lower id;
    probs float64 [T, k] = softmax over the k selected logits) for float32 logits [T, E]."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), np.int32)
    probs = np.empty((T, k), np.float64)
    _load().oracle_router(_p(logits), T, E, k, _p(ids), _p(probs))
    return ids, probs


def permute(x, perm, k: int) -> np.ndarray:
    """Rows of ``x`` ([T, ...], any dtype) gathered as x_perm[p] = x[perm[p] // k]."""
    x = _c(x)
    perm = _c(perm, np.int32)
    M = perm.shape[0]
    out = np.empty((M,) + x.shape[1:], x.dtype)
    row_bytes = x[0].nbytes if x.shape[0] else 0
    _load().oracle_permute(_p(x), row_bytes, _p(perm), M, k, _p(out))
    return out


# ---------------------------------------------------------------------------------------------- FFN / layer

def _weights(inp):
    return (_c(inp.w_gate), _c(getattr(inp, "wg_scale", None)), _c(inp.w_up),
            _c(getattr(inp, "wu_scale", None)), _c(inp.w_down), _c(getattr(inp, "wd_scale", None)))


def ffn_rows(dtype: str, rows, row_expert, w_gate, w_up, w_down, rows_scale=None,
             wg_scale=None, wu_scale=None, wd_scale=None) -> np.ndarray:
    """fp64 SwiGLU expert FFN of each stored row through its own expert."""
    rows = _c(rows)
    n, H = rows.shape
    E, _, F = w_gate.shape
    row_expert = _c(row_expert, np.int32)
    y = np.empty((n, H), np.float64)
    args = [_c(w_gate), _c(wg_scale), _c(w_up), _c(wu_scale), _c(w_down), _c(wd_scale)]
    rs = _c(rows_scale)
    rc = _load().oracle_ffn_rows(DTYPES[dtype], n, H, F, E, _p(rows), _p(rs), _p(row_expert),
                                 *[_p(a) for a in args], _p(y))
    if rc != 0:
        raise OracleError("bad expert index")
    return y


def grouped_ffn(g, row_index=None) -> np.ndarray:
    """FFN of rows already grouped by (source, local expert) (``synth.GroupedInputs``).
    ``row_index`` restricts the computation to those rows (returned in that order)."""
    offs = np.asarray(g.group_offsets, np.int64)
    row_expert = np.repeat(np.asarray(g.group_expert, np.int32), np.diff(offs))
    rows = g.rows
    rows_scale = getattr(g, "rows_scale", None)
    if row_index is not None:
        row_index = np.asarray(row_index, np.int64)
        rows = rows[row_index]
        row_expert = row_expert[row_index]
        if rows_scale is not None:
            rows_scale = rows_scale[row_index]
    return ffn_rows(g.dtype, rows, row_expert, g.w_gate, g.w_up, g.w_down, rows_scale=rows_scale,
                    wg_scale=getattr(g, "wg_scale", None), wu_scale=getattr(g, "wu_scale", None),
                    wd_scale=getattr(g, "wd_scale", None))


def forward(inp, chunk: int = 0):
    """Whole layer over every token.  Returns (out fp64 [T,H], counts, offsets, perm, pos)."""
    T, H, F, E, k = inp.T, inp.H, inp.F, inp.E, inp.k
    M = T * k
    out = np.empty((T, H), np.float64)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(M, np.int32)
    pos = np.empty(M, np.int32)
    x = _c(inp.x)
    xs = _c(inp.x_scale)
    ws = _weights(inp)
    ids = _c(inp.expert_ids, np.int32)
    probs = _c(inp.probs, np.float32)
    rc = _load().oracle_forward(DTYPES[inp.dtype], T, H, F, E, k, _p(x), _p(xs),
                                *[_p(a) for a in ws], _p(ids), _p(probs), int(chunk), _p(out),
                                _p(counts), _p(offsets), _p(perm), _p(pos))
    if rc != 0:
        raise OracleError("oracle_forward rejected its inputs")
    return out, counts, offsets, perm, pos


def forward_tokens(inp, tokens) -> np.ndarray:
    """Per-token definition for the listed tokens: out[i] = sum_j p[t,j] FFN_{ids[t,j]}(x[t])."""
    tokens = _c(tokens, np.int32)
    out = np.empty((tokens.shape[0], inp.H), np.float64)
    x = _c(inp.x)
    xs = _c(inp.x_scale)
    ws = _weights(inp)
    ids = _c(inp.expert_ids, np.int32)
    probs = _c(inp.probs, np.float32)
    rc = _load().oracle_forward_tokens(DTYPES[inp.dtype], inp.T, inp.H, inp.F, inp.E, inp.k,
                                       _p(x), _p(xs), *[_p(a) for a in ws], _p(ids), _p(probs),
                                       _p(tokens), tokens.shape[0], _p(out))
    if rc != 0:
        raise OracleError("oracle_forward_tokens rejected its inputs")
    return out


# ---------------------------------------------------------------------------------------------- backward

def _bwd_args(inp, dout):
    if inp.dtype not in ("f32", "bf16"):
        raise ValueError("the backward oracle takes float32 or bfloat16 storage")
    dout = _c(dout)
    if dout.dtype != inp.x.dtype or dout.shape != (inp.T, inp.H):
        raise ValueError("dout must be [T, H] in the storage format of x")
    return (DTYPES[inp.dtype], inp.T, inp.H, inp.F, inp.E, inp.k, _c(inp.x), _c(inp.w_gate),
            _c(inp.w_up), _c(inp.w_down), _c(inp.expert_ids, np.int32), _c(inp.probs, np.float32),
            dout)


def backward(inp, dout):
    """Gradients of sum(dout * out) for the layer of ``inp`` (float32 / bfloat16 storage), all fp64:
    (dx [T,H], dw_gate [E,H,F], dw_up [E,H,F], dw_down [E,F,H], dprobs [T,k])."""
    a = _bwd_args(inp, dout)
    _, T, H, F, E, k = a[:6]
    dx = np.empty((T, H), np.float64)
    dwg = np.empty((E, H, F), np.float64)
    dwu = np.empty((E, H, F), np.float64)
    dwd = np.empty((E, F, H), np.float64)
    dprobs = np.empty((T, k), np.float64)
    rc = _load().oracle_backward(*a[:6], *[_p(v) for v in a[6:]], _p(dx), _p(dwg), _p(dwu),
                                 _p(dwd), _p(dprobs))
    if rc != 0:
        raise OracleError("oracle_backward rejected its inputs")
    return dx, dwg, dwu, dwd, dprobs


def backward_tokens(inp, dout, tokens):
    """(dx rows [n, H], dprobs rows [n, k]) of the listed tokens, fp64."""
    a = _bwd_args(inp, dout)
    tokens = _c(tokens, np.int32)
    n = tokens.shape[0]
    dx = np.empty((n, inp.H), np.float64)
    dprobs = np.empty((n, inp.k), np.float64)
    rc = _load().oracle_backward_tokens(*a[:6], *[_p(v) for v in a[6:]], _p(tokens), n, _p(dx),
                                        _p(dprobs))
    if rc != 0:
        raise OracleError("oracle_backward_tokens rejected its inputs")
    return dx, dprobs


def wgrad_entries(inp, dout, e, f, h):
    """Entries (dWg[e,h,f], dWu[e,h,f], dWd[e,f,h]) for index arrays e, f, h, fp64."""
    a = _bwd_args(inp, dout)
    e, f, h = (_c(np.atleast_1d(v), np.int32) for v in (e, f, h))
    n = e.shape[0]
    out = [np.empty(n, np.float64) for _ in range(3)]
    rc = _load().oracle_wgrad_entries(*a[:6], *[_p(v) for v in a[6:]], n, _p(e), _p(f), _p(h),
                                      *[_p(o) for o in out])
    if rc != 0:
        raise OracleError("oracle_wgrad_entries rejected its inputs")
    return tuple(out)


def row_inf_norm_rel(a, ref) -> float:
    """max over rows r of max |a_r - ref_r| / max |ref_r| (rows whose reference is all zero count
    their absolute error): the per-token form of inf_norm_rel, so that a wrong row with small
    outputs cannot hide under the largest row of the tensor."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    a = a.reshape(ref.shape[0], -1)
    ref = ref.reshape(ref.shape[0], -1)
    num = np.max(np.abs(a - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1.0), num)))


def inf_norm_rel(a, ref) -> float:
    """max |a - ref| / max |ref| over the whole tensor (the comparison metric for float outputs)."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(a - ref)) if ref.size else 0.0
    return float(num / den) if den > 0 else float(num)
