"""Seeded synthetic inputs for the MoE expert layer.

This module only *draws* inputs: activations, expert weights, router choices
(expert ids and their probabilities) and, for the one-EP-rank workload, the
received-row counts.  It holds none of the layer's own arithmetic (routing
counts, permutation, GEMMs, SwiGLU, combine); both the HIP library and the
CPU oracle consume the bytes produced here.

Storage formats handed to both sides:

* ``f32``   - float32 arrays.
* ``bf16``  - uint16 arrays holding bfloat16 bit patterns (round-to-nearest-even
  from the float32 draw, done once here).
* ``mxfp8`` - OCP-MX inputs: uint8 E4M3 element codes plus one uint8 E8M0 scale
  per 32 consecutive elements along the contraction axis.  The input encoder
  below follows the OCP Microscaling Formats v1.0 recipe (shared exponent
  floor(log2 amax) - 8, elements rounded to nearest-even and saturated to 448).

Recipe (fixed, so every run of every test sees the same bytes): a
``numpy.random.SeedSequence(seed)`` is split into child streams in a fixed order
(router, x, then one stream per (tensor, expert) for w_gate, w_up, w_down);
values are float32 standard normals, weights multiplied by 0.02 in float32.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "WORKLOADS", "LayerInputs", "GroupedInputs", "make_layer", "make_grouped",
    "make_workload", "make_dout", "to_bf16_bits", "bf16_bits_to_f32", "mx_encode_blocks",
]

# The five workloads: sizes, dtypes and routing structure (dims are the full sizes).
WORKLOADS = {
    "tiny_f32": dict(kind="layer", T=64, H=128, F=256, E=4, k=2, dtype="f32",
                     routing="normal_logits"),
    "mixtral_bf16": dict(kind="layer", T=4096, H=4096, F=14336, E=8, k=2, dtype="bf16",
                         routing="normal_logits", head_m_size=512),
    "ep_rank_bf16": dict(kind="grouped", rows=16384, H=4096, F=14336, E_local=2, sources=8,
                         zipf_s=1.2, dtype="bf16"),
    "finegrained_bf16": dict(kind="layer", T=8192, H=2048, F=768, E=128, k=8, dtype="bf16",
                             routing="zipf_gumbel", zipf_s=1.1, n_zero=8),
    "mxfp8": dict(kind="layer", T=16384, H=7168, F=2048, E=32, k=4, dtype="mxfp8",
                  routing="normal_logits", head_m_size=512),
}

_WORKERS = max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------- storage encoders

def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even (no NaN/Inf in inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def mx_encode_blocks(v: np.ndarray, axis: int) -> tuple[np.ndarray, np.ndarray]:
    """Encode float32 ``v`` as OCP-MX E4M3 with one E8M0 scale per 32 elements along ``axis``.

    Returns (codes uint8 with v's shape, scales uint8 with v.shape[axis] // 32 along ``axis``).
    Shared exponent: floor(log2(max|block|)) - 8, clamped to [-127, 127] (an all-zero block
    gets -127).  Elements: v / 2^e rounded to nearest-even on the E4M3 grid, saturated to +-448,
    sign kept (a negative value that rounds to zero encodes as 0x80).
    """
    v = np.asarray(v, dtype=np.float32)
    n = v.shape[axis]
    assert n % 32 == 0, "MX block axis must be a multiple of 32"
    vb = np.moveaxis(v, axis, -1)
    lead = vb.shape[:-1]
    vb = vb.reshape(lead + (n // 32, 32))
    amax = np.max(np.abs(vb), axis=-1)
    _, ex = np.frexp(amax)                      # amax = m * 2^ex, m in [0.5, 1)
    e = np.where(amax > 0, ex.astype(np.int32) - 1 - 8, -127)
    e = np.clip(e, -127, 127)
    scaled = np.ldexp(vb, (-e)[..., None]).astype(np.float32)   # exact power-of-two scaling
    a = np.abs(scaled)
    _, ea = np.frexp(a)
    ea = ea.astype(np.int32) - 1                # floor(log2 a) for a > 0
    qexp = np.where(a >= 2.0 ** -6, ea - 3, -9)  # grid spacing exponent (normals / subnormals)
    q = np.ldexp(np.rint(np.ldexp(a, -qexp)), qexp)
    q = np.minimum(q, 448.0).astype(np.float32)
    _, eq = np.frexp(q)
    eq = eq.astype(np.int32) - 1
    normal = q >= 2.0 ** -6
    exp_field = np.where(normal, eq + 7, 0)
    man_field = np.where(normal,
                         np.rint(np.ldexp(q, -eq) * 8.0 - 8.0),
                         np.rint(np.ldexp(q, 9)))
    code = (exp_field.astype(np.int32) << 3) | man_field.astype(np.int32)
    code = code | np.where(np.signbit(scaled), 0x80, 0)
    code = code.astype(np.uint8).reshape(lead + (n,))
    codes = np.ascontiguousarray(np.moveaxis(code, -1, axis))
    scales = np.ascontiguousarray(np.moveaxis((e + 127).astype(np.uint8), -1, axis))
    return codes, scales


# ----------------------------------------------------------------------------- containers

@dataclass
class LayerInputs:
    T: int
    H: int
    F: int
    E: int
    k: int
    dtype: str                      # "f32" | "bf16" | "mxfp8"
    x: np.ndarray                   # [T,H] f32 | uint16 bf16 bits | uint8 E4M3 codes
    w_gate: np.ndarray              # [E,H,F]
    w_up: np.ndarray                # [E,H,F]
    w_down: np.ndarray              # [E,F,H]
    expert_ids: np.ndarray          # [T,k] int32
    probs: np.ndarray               # [T,k] float32
    x_scale: np.ndarray | None = None    # [T,H/32]  (mxfp8)
    x_bf16: np.ndarray | None = None     # [T,H] bfloat16 bits of the x draw (mxfp8 workloads)
    wg_scale: np.ndarray | None = None   # [E,H/32,F]
    wu_scale: np.ndarray | None = None   # [E,H/32,F]
    wd_scale: np.ndarray | None = None   # [E,F/32,H]
    meta: dict = field(default_factory=dict)


@dataclass
class GroupedInputs:
    """Rows as one EP rank receives them: groups g = s * E_local + j (source-major), group g uses
    local expert j.  Only the grouped FFN applies to them."""
    H: int
    F: int
    E_local: int
    sources: int
    dtype: str
    rows: np.ndarray                # [M,H]
    group_offsets: np.ndarray       # [G+1] int32
    group_expert: np.ndarray        # [G] int32
    recv_counts: np.ndarray         # [sources, E_local] int64
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    rows_scale: np.ndarray | None = None   # mxfp8: [M, H/32]
    wg_scale: np.ndarray | None = None
    wu_scale: np.ndarray | None = None
    wd_scale: np.ndarray | None = None
    meta: dict = field(default_factory=dict)


# ----------------------------------------------------------------------------- draws

def _streams(seed: int, n: int) -> list[np.random.Generator]:
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal_f32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return v


def _store(v: np.ndarray, dtype: str, mx_axis: int | None):
    if dtype == "f32":
        return v, None
    if dtype == "bf16":
        return to_bf16_bits(v), None
    if dtype == "mxfp8":
        return mx_encode_blocks(v, mx_axis)
    raise ValueError(dtype)


def _logits(rng: np.random.Generator, T: int, E: int, routing: str, **kw) -> np.ndarray:
    """Router logits [T, E] (float64) of the named distribution."""
    if routing == "normal_logits":
        logits = rng.standard_normal((T, E))
    elif routing == "zipf_gumbel":
        s = float(kw.get("zipf_s", 1.1))
        n_zero = int(kw.get("n_zero", 0))
        rank_of = rng.permutation(E)                  # expert e has popularity rank rank_of[e] + 1
        w = (rank_of + 1.0) ** (-s)
        w[rank_of >= E - n_zero] = 0.0                # the n_zero least popular experts get nothing
        with np.errstate(divide="ignore"):
            logw = np.log(w)
        logits = logw[None, :] + rng.gumbel(size=(T, E))
    else:
        raise ValueError(routing)
    return logits


def _route(rng: np.random.Generator, T: int, E: int, k: int, routing: str, **kw):
    """Router draw: expert_ids = top-k of the logits (descending, ties -> lower id);
    probs = softmax over the k selected logits (fp64), stored as float32."""
    logits = _logits(rng, T, E, routing, **kw)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, order, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    probs = z / z.sum(axis=1, keepdims=True)
    return order.astype(np.int32), probs.astype(np.float32)


def make_layer(T: int, H: int, F: int, E: int, k: int, dtype: str = "bf16",
               routing: str = "normal_logits", seed: int = 0, x_std: float = 1.0,
               w_std: float = 0.02, **routing_kw) -> LayerInputs:
    if dtype == "mxfp8" and (H % 32 or F % 32):
        raise ValueError("mxfp8 needs H and F multiples of 32")
    st = _streams(seed, 2 + 3 * E)
    ids, probs = _route(st[0], T, E, k, routing, **routing_kw)
    x32 = _normal_f32(st[1], (T, H), x_std)
    x, xs = _store(x32, dtype, 1)
    # MX workloads also carry the same draw rounded to bfloat16: activations as a bf16 producer
    # hands them over, for the path that encodes x itself
    x_bf16 = to_bf16_bits(x32) if dtype == "mxfp8" else None
    del x32

    u8 = dtype == "mxfp8"
    edt = {"f32": np.float32, "bf16": np.uint16, "mxfp8": np.uint8}[dtype]
    mats = [np.empty((E, H, F), edt), np.empty((E, H, F), edt), np.empty((E, F, H), edt)]
    scl = ([np.empty((E, H // 32, F), np.uint8), np.empty((E, H // 32, F), np.uint8),
            np.empty((E, F // 32, H), np.uint8)] if u8 else [None, None, None])

    def one(job):
        which, e = job
        shape = (H, F) if which < 2 else (F, H)
        q, sc = _store(_normal_f32(st[2 + which * E + e], shape, w_std), dtype, 0)
        mats[which][e] = q
        if u8:
            scl[which][e] = sc

    jobs = [(w, e) for w in range(3) for e in range(E)]
    with ThreadPoolExecutor(_WORKERS) as ex:
        list(ex.map(one, jobs))
    return LayerInputs(T=T, H=H, F=F, E=E, k=k, dtype=dtype, x=x, w_gate=mats[0], w_up=mats[1],
                       w_down=mats[2], expert_ids=ids, probs=probs, x_scale=xs, x_bf16=x_bf16,
                       wg_scale=scl[0], wu_scale=scl[1], wd_scale=scl[2],
                       meta=dict(seed=seed, routing=routing, **routing_kw))


def make_grouped(rows: int, H: int, F: int, E_local: int = 2, sources: int = 8, zipf_s: float = 1.2,
                 dtype: str = "bf16", seed: int = 0, n_experts_global: int = 8) -> GroupedInputs:
    """One EP rank's share: for each source s a seeded permutation pi_s of the global experts gives the
    weight (pi_s(e) + 1)^-zipf_s to each local expert e; the 16 (source, expert) cells share ``rows``
    by a multinomial draw.  Rows are laid out source-major, as an AllToAllv would deliver them."""
    st = _streams(seed, 2 + 3 * E_local)
    rng = st[0]
    wts = np.zeros((sources, E_local))
    for s in range(sources):
        pi = rng.permutation(n_experts_global)
        wts[s] = (pi[:E_local] + 1.0) ** (-zipf_s)
    p = (wts / wts.sum()).ravel()
    counts = rng.multinomial(rows, p).reshape(sources, E_local)
    G = sources * E_local
    offs = np.zeros(G + 1, dtype=np.int64)
    offs[1:] = np.cumsum(counts.ravel())
    gexp = np.tile(np.arange(E_local, dtype=np.int32), sources)
    x, xs = _store(_normal_f32(st[1], (rows, H), 1.0), dtype, 1)

    def one(job):
        which, e = job
        shape = (H, F) if which < 2 else (F, H)
        return _store(_normal_f32(st[2 + which * E_local + e], shape, 0.02), dtype, 0)

    jobs = [(w, e) for w in range(3) for e in range(E_local)]
    with ThreadPoolExecutor(_WORKERS) as ex:
        res = list(ex.map(one, jobs))
    mats = [np.stack([r[0] for r in res[w * E_local:(w + 1) * E_local]]) for w in range(3)]
    scl = [np.stack([r[1] for r in res[w * E_local:(w + 1) * E_local]]) if dtype == "mxfp8"
           else None for w in range(3)]
    return GroupedInputs(H=H, F=F, E_local=E_local, sources=sources, dtype=dtype, rows=x,
                         group_offsets=offs.astype(np.int32), group_expert=gexp,
                         recv_counts=counts, w_gate=mats[0], w_up=mats[1], w_down=mats[2],
                         rows_scale=xs, wg_scale=scl[0], wu_scale=scl[1], wd_scale=scl[2],
                         meta=dict(seed=seed, zipf_s=zipf_s))


def make_dout(inp: LayerInputs, std: float = 1.0) -> np.ndarray:
    """Output gradient [T, H] for the backward of ``inp``'s layer, in x's storage format (float32 or
    bfloat16 bits): float32 normals times ``std`` from the stream after the layer's own streams."""
    if inp.dtype not in ("f32", "bf16"):
        raise ValueError("the backward takes float32 or bfloat16 storage")
    seed = inp.meta.get("seed", 0)
    rng = _streams(seed, 3 + 3 * inp.E)[-1]
    v, _ = _store(_normal_f32(rng, (inp.T, inp.H), std), inp.dtype, None)
    return v


def make_logits(T: int, E: int, routing: str = "normal_logits", seed: int = 0, **routing_kw) -> np.ndarray:
    """The router logits behind make_layer(T=T, E=E, routing=routing, seed=seed, ...), as float32
    (the same stream, so top-k of these gives that layer's expert_ids)."""
    st = _streams(seed, 2 + 3 * E)
    return _logits(st[0], T, E, routing, **routing_kw).astype(np.float32)


def make_workload(name: str, seed: int = 0, **override):
    """Build one of the five named workloads at full size (``override`` shrinks dims for tests)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    kind = cfg.pop("kind")
    cfg.pop("head_m_size", None)
    if kind == "grouped":
        return make_grouped(seed=seed, **cfg)
    return make_layer(seed=seed, **cfg)
