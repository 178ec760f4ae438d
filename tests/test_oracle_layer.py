"""Pins for the oracle's expert FFN and whole-layer forward.

The layer (page 'NPU Training Operators - MC2', section 执行路径, steps 6-10; operand set of
mc2_fused_expert on page 'MC2 通算融合', section 用法) is, per token t,
    out[t] = sum_j probs[t,j] * Wd[e]^T (silu(Wg[e]^T x_t) * (Wu[e]^T x_t)),  e = ids[t,j].
The tests below re-derive it by other routes: numpy fp64 matmuls with scipy's logistic function,
a closed form with diagonal weights (catches a swapped gate/up or a dropped term), brute-force
per-token loops (no routing or permutation at all), and invariances the definition implies.
Inputs are decoded here with torch's own bf16 / float8_e4m3fn codecs, not with the oracle's.
"""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import synth

RTOL = 1e-10     # oracle (double, ascending sums) vs numpy double matmuls (blocked sums)


def dec(a, dtype):
    """Storage -> float64 with library codecs (independent of the oracle's decoders)."""
    if dtype == "f32":
        return np.asarray(a, np.float64)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).double().numpy()
    raise ValueError(dtype)


def dec_mx(codes, scales, axis):
    v = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()
    sc = np.exp2(np.asarray(scales, np.float64) - 127)
    return v * np.repeat(sc, 32, axis=axis)


def weights64(inp):
    if inp.dtype == "mxfp8":
        return (dec_mx(inp.w_gate, inp.wg_scale, 1), dec_mx(inp.w_up, inp.wu_scale, 1),
                dec_mx(inp.w_down, inp.wd_scale, 1))
    return dec(inp.w_gate, inp.dtype), dec(inp.w_up, inp.dtype), dec(inp.w_down, inp.dtype)


def x64(inp):
    if inp.dtype == "mxfp8":
        return dec_mx(inp.x, inp.x_scale, 1)
    return dec(inp.x, inp.dtype)


def brute_force(inp):
    """Per-token loop straight from the definition; MX variant encodes h with the (separately
    pinned) oracle MX encoder and decodes it with torch's float8 codec."""
    X = x64(inp)
    Wg, Wu, Wd = weights64(inp)
    out = np.zeros((inp.T, inp.H))
    for t in range(inp.T):
        for j in range(inp.k):
            e = inp.expert_ids[t, j]
            g = X[t] @ Wg[e]
            u = X[t] @ Wu[e]
            h = g * expit(g) * u
            if inp.dtype == "mxfp8":
                q, s = oracle.mx_quantize(h[None, :])
                h = dec_mx(q, s, 1)[0]
            out[t] += float(inp.probs[t, j]) * (h @ Wd[e])
    return out


def test_dense_swiglu_special_case():
    """E = 1, k = 1, p = 1: the layer is a dense SwiGLU MLP."""
    inp = synth.make_layer(T=40, H=64, F=96, E=1, k=1, dtype="f32")
    inp.probs[:] = 1.0
    out, *_ = oracle.forward(inp)
    X = inp.x.astype(np.float64)
    Wg, Wu, Wd = (w[0].astype(np.float64) for w in (inp.w_gate, inp.w_up, inp.w_down))
    G = X @ Wg
    ref = (G * expit(G) * (X @ Wu)) @ Wd
    assert oracle.inf_norm_rel(out, ref) < RTOL


def test_closed_form_diagonal_weights():
    """Wg[e] = a_e I, Wu[e] = b_e I, Wd[e] = c_e I: out[t] = sum_j p_j c_e silu(a_e x) (b_e x)."""
    T, H, E, k = 32, 32, 3, 2
    inp = synth.make_layer(T=T, H=H, F=H, E=E, k=k, dtype="f32")
    a = [0.5, -1.5, 2.0]
    b = [1.25, 0.75, -0.5]
    c = [1.0, 2.0, 0.25]
    eye = np.eye(H, dtype=np.float32)
    inp.w_gate = np.stack([a[e] * eye for e in range(E)])
    inp.w_up = np.stack([b[e] * eye for e in range(E)])
    inp.w_down = np.stack([c[e] * eye for e in range(E)])
    out, *_ = oracle.forward(inp)
    X = inp.x.astype(np.float64)
    ref = np.zeros_like(X)
    for t in range(T):
        for j in range(k):
            e = inp.expert_ids[t, j]
            z = a[e] * X[t]
            ref[t] += float(inp.probs[t, j]) * c[e] * (z * expit(z)) * (b[e] * X[t])
    assert oracle.inf_norm_rel(out, ref) < RTOL
    # the gate/up roles are not symmetric: swapping them changes the result
    inp.w_gate, inp.w_up = inp.w_up, inp.w_gate
    swapped, *_ = oracle.forward(inp)
    assert oracle.inf_norm_rel(swapped, ref) > 1e-2


@pytest.mark.parametrize("dtype,T,H,F,E,k,routing,kw", [
    ("f32", 64, 128, 256, 4, 2, "normal_logits", {}),
    ("bf16", 96, 64, 160, 8, 2, "normal_logits", {}),
    ("bf16", 64, 64, 96, 32, 8, "zipf_gumbel", {"zipf_s": 1.1, "n_zero": 8}),
    ("mxfp8", 48, 64, 96, 6, 4, "normal_logits", {}),
])
def test_grouped_forward_equals_per_token_brute_force(dtype, T, H, F, E, k, routing, kw):
    inp = synth.make_layer(T=T, H=H, F=F, E=E, k=k, dtype=dtype, routing=routing, **kw)
    out, counts, *_ = oracle.forward(inp)
    ref = brute_force(inp)
    assert oracle.inf_norm_rel(out, ref) < RTOL
    tok = oracle.forward_tokens(inp, np.arange(T))
    assert oracle.inf_norm_rel(tok, ref) < RTOL
    sel = np.array([T - 1, 0, T // 2])
    assert np.array_equal(oracle.forward_tokens(inp, sel), tok[sel])


def test_mx_h_encoding_matters():
    """The MX variant encodes h before fc2; leaving that out moves the result measurably."""
    inp = synth.make_layer(T=32, H=64, F=128, E=4, k=2, dtype="mxfp8")
    out, *_ = oracle.forward(inp)
    X = x64(inp)
    Wg, Wu, Wd = weights64(inp)
    ref = np.zeros((inp.T, inp.H))
    for t in range(inp.T):
        for j in range(inp.k):
            e = inp.expert_ids[t, j]
            g = X[t] @ Wg[e]
            ref[t] += float(inp.probs[t, j]) * ((g * expit(g) * (X[t] @ Wu[e])) @ Wd[e])
    err = oracle.inf_norm_rel(out, ref)
    assert 1e-3 < err < 6e-2


@pytest.mark.parametrize("chunk", [1, 7, 64, 512, 100000])
def test_chunked_equals_unchunked(chunk):
    inp = synth.make_layer(T=80, H=64, F=96, E=5, k=3, dtype="bf16")
    ref, *_ = oracle.forward(inp, chunk=0)
    out, *_ = oracle.forward(inp, chunk=chunk)
    assert np.array_equal(out, ref)


def test_invariances():
    inp = synth.make_layer(T=60, H=64, F=96, E=6, k=2, dtype="bf16", seed=4)
    base, *_ = oracle.forward(inp)
    rng = np.random.default_rng(11)
    # token permutation permutes the output rows
    tp = rng.permutation(inp.T)
    inp2 = synth.make_layer(T=60, H=64, F=96, E=6, k=2, dtype="bf16", seed=4)
    inp2.x, inp2.expert_ids, inp2.probs = inp.x[tp], inp.expert_ids[tp], inp.probs[tp]
    out, *_ = oracle.forward(inp2)
    assert np.array_equal(out, base[tp])
    # relabelling experts (weights and ids together) changes nothing
    rel = rng.permutation(inp.E)                     # new label of old expert e is rel[e]
    inv = np.argsort(rel)
    inp3 = synth.make_layer(T=60, H=64, F=96, E=6, k=2, dtype="bf16", seed=4)
    inp3.w_gate, inp3.w_up, inp3.w_down = inp.w_gate[inv], inp.w_up[inv], inp.w_down[inv]
    inp3.expert_ids = rel[inp.expert_ids].astype(np.int32)
    out, *_ = oracle.forward(inp3)
    assert np.array_equal(out, base)
    # doubling the probabilities doubles the output (exact in binary floating point)
    inp4 = synth.make_layer(T=60, H=64, F=96, E=6, k=2, dtype="bf16", seed=4)
    inp4.probs = inp.probs * np.float32(2)
    out, *_ = oracle.forward(inp4)
    assert np.array_equal(out, 2 * base)


def test_grouped_rows_source_major():
    """One EP rank's received rows: group g = s * E_local + j uses local expert j
    (page 'NPU Training Operators - MC2', 执行路径 step 5: recv_counts taken source by source)."""
    g = synth.make_grouped(rows=300, H=64, F=96, E_local=2, sources=8, zipf_s=1.2)
    assert g.group_offsets[-1] == 300 and g.recv_counts.sum() == 300
    assert np.array_equal(np.diff(g.group_offsets), g.recv_counts.ravel())
    y = oracle.grouped_ffn(g)
    X = dec(g.rows, "bf16")
    Wg, Wu, Wd = dec(g.w_gate, "bf16"), dec(g.w_up, "bf16"), dec(g.w_down, "bf16")
    ref = np.zeros_like(y)
    for grp in range(16):
        e = grp % 2
        for r in range(g.group_offsets[grp], g.group_offsets[grp + 1]):
            G = X[r] @ Wg[e]
            ref[r] = (G * expit(G) * (X[r] @ Wu[e])) @ Wd[e]
    assert oracle.inf_norm_rel(y, ref) < RTOL
    sub = np.array([299, 0, 150])
    assert np.array_equal(oracle.grouped_ffn(g, sub), y[sub])


def test_row_inf_norm_rel_is_taken_per_row():
    """The per-token metric: each row's error against that row's own largest reference value (a
    zero row counts its absolute error), so a small row's 10% error is not hidden by a large row."""
    ref = np.array([[10.0, -1.0], [0.1, 0.05], [0.0, 0.0]])
    a = ref + np.array([[0.1, 0.0], [0.0, -0.01], [0.0, 0.002]])
    assert oracle.row_inf_norm_rel(a, ref) == pytest.approx(0.1)
    assert oracle.inf_norm_rel(a, ref) == pytest.approx(0.01)
    assert oracle.row_inf_norm_rel(ref, ref) == 0.0
    assert oracle.row_inf_norm_rel(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0
