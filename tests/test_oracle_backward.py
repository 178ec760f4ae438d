"""Pins for the oracle's backward of the layer (gradients of sum(dout * out)).

The backward follows from the chain rule on the forward definition (steps 6-10 of 执行路径 on the
page "NPU Training Operators - MC2"; its 验证项 list the fc1 / fc2 gradients among the checks).
Pinned here against things other than itself:
  * central finite differences of the forward oracle (no derivative code at all), on every
    coordinate of a tiny problem whose inputs sit on a grid so that the perturbed values are exact;
  * torch's fp64 autograd of the per-token definition (a library differentiating a plain loop);
  * Euler's theorem: out is homogeneous of degree 1 in w_down, in w_up and in probs, so
    <dW, W> = sum(dout * out) for each of them;
  * the token-list and single-entry forms against the whole backward; structural zeros.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _grid_layer(T, H, F, E, k, seed):
    """float32 layer whose values are multiples of 2^-8 (x, dout) or 2^-10 (weights), so that adding
    or subtracting 2^-12 is exact; probs multiples of 2^-8 in (0, 1)."""
    rng = np.random.default_rng(seed)
    x = (rng.integers(-384, 385, (T, H)) / 256).astype(np.float32)
    wg, wu = ((rng.integers(-200, 201, (2, E, H, F)) / 1024).astype(np.float32))
    wd = (rng.integers(-200, 201, (E, F, H)) / 1024).astype(np.float32)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    probs = (rng.integers(1, 256, (T, k)) / 256).astype(np.float32)
    dout = (rng.integers(-256, 257, (T, H)) / 256).astype(np.float32)
    inp = synth.LayerInputs(T=T, H=H, F=F, E=E, k=k, dtype="f32", x=x, w_gate=wg, w_up=wu,
                            w_down=wd, expert_ids=ids, probs=probs)
    return inp, dout


def _loss(inp, dout):
    out, *_ = oracle.forward(inp)
    return float(np.sum(dout.astype(np.float64) * out))


def _finite_differences(inp, dout, name, eps=2.0 ** -12):
    base = getattr(inp, name)
    fd = np.empty(base.shape, np.float64)
    for idx in np.ndindex(base.shape):
        saved = base[idx]
        base[idx] = saved + np.float32(eps)
        lp = _loss(inp, dout)
        base[idx] = saved - np.float32(eps)
        lm = _loss(inp, dout)
        base[idx] = saved
        fd[idx] = (lp - lm) / (2 * eps)
    return fd


def test_central_differences_of_the_forward():
    inp, dout = _grid_layer(T=5, H=6, F=10, E=3, k=2, seed=1)
    dx, dwg, dwu, dwd, dprobs = oracle.backward(inp, dout)
    for name, grad in (("x", dx), ("w_gate", dwg), ("w_up", dwu), ("w_down", dwd),
                       ("probs", dprobs)):
        fd = _finite_differences(inp, dout, name)
        scale = np.max(np.abs(grad))
        assert scale > 0
        # central differences: error ~ eps^2 * third derivative (~1e-7 of the scale here)
        np.testing.assert_allclose(fd, grad, rtol=0, atol=2e-6 * scale, err_msg=name)


def _torch_reference(inp, dout):
    """Per-token definition in fp64 torch, differentiated by autograd."""
    dec = (lambda a: synth.bf16_bits_to_f32(a)) if inp.dtype == "bf16" else (lambda a: a)
    t = lambda a: torch.tensor(np.asarray(dec(a), np.float64), requires_grad=True)
    x, wg, wu, wd = t(inp.x), t(inp.w_gate), t(inp.w_up), t(inp.w_down)
    probs = torch.tensor(inp.probs.astype(np.float64), requires_grad=True)
    rows = []
    for tok in range(inp.T):
        acc = torch.zeros(inp.H, dtype=torch.float64)
        for j in range(inp.k):
            e = int(inp.expert_ids[tok, j])
            g = x[tok] @ wg[e]
            u = x[tok] @ wu[e]
            acc = acc + probs[tok, j] * ((torch.nn.functional.silu(g) * u) @ wd[e])
        rows.append(acc)
    out = torch.stack(rows)
    loss = (torch.tensor(np.asarray(dec(dout), np.float64)) * out).sum()
    loss.backward()
    return [v.grad.numpy() for v in (x, wg, wu, wd, probs)]


@pytest.mark.parametrize("dtype,T,H,F,E,k,seed", [("bf16", 12, 16, 24, 4, 2, 3),
                                                  ("f32", 9, 8, 16, 5, 3, 4),
                                                  ("bf16", 7, 8, 8, 2, 1, 5)])
def test_torch_autograd_of_the_per_token_definition(dtype, T, H, F, E, k, seed):
    inp = synth.make_layer(T=T, H=H, F=F, E=E, k=k, dtype=dtype, seed=seed, w_std=0.3)
    dout = synth.make_dout(inp)
    ours = oracle.backward(inp, dout)
    ref = _torch_reference(inp, dout)
    for name, a, r in zip(("dx", "dwg", "dwu", "dwd", "dprobs"), ours, ref):
        np.testing.assert_allclose(a, r, rtol=0, atol=1e-12 * np.max(np.abs(r)), err_msg=name)


def test_euler_identities():
    inp = synth.make_layer(T=64, H=64, F=96, E=4, k=2, dtype="bf16", seed=6)
    dout = synth.make_dout(inp)
    out, *_ = oracle.forward(inp)
    L = float(np.sum(synth.bf16_bits_to_f32(dout).astype(np.float64) * out))
    dx, dwg, dwu, dwd, dprobs = oracle.backward(inp, dout)
    wu = synth.bf16_bits_to_f32(inp.w_up).astype(np.float64)
    wd = synth.bf16_bits_to_f32(inp.w_down).astype(np.float64)
    assert abs(L) > 0
    for lhs in (np.sum(dwd * wd), np.sum(dwu * wu), np.sum(dprobs * inp.probs.astype(np.float64))):
        assert abs(lhs - L) <= 1e-11 * abs(L)


def test_token_and_entry_forms_match_the_whole_backward():
    inp = synth.make_layer(T=40, H=32, F=48, E=5, k=2, dtype="bf16", seed=7)
    dout = synth.make_dout(inp)
    dx, dwg, dwu, dwd, dprobs = oracle.backward(inp, dout)
    tokens = np.array([0, 3, 17, 39])
    dxr, dpr = oracle.backward_tokens(inp, dout, tokens)
    np.testing.assert_allclose(dxr, dx[tokens], rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(dpr, dprobs[tokens], rtol=1e-13, atol=1e-300)
    rng = np.random.default_rng(0)
    e, f, h = rng.integers(0, 5, 30), rng.integers(0, 48, 30), rng.integers(0, 32, 30)
    g1, u1, d1 = oracle.wgrad_entries(inp, dout, e, f, h)
    np.testing.assert_allclose(g1, dwg[e, h, f], rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(u1, dwu[e, h, f], rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(d1, dwd[e, f, h], rtol=1e-13, atol=1e-300)


def test_structural_zeros():
    """An expert that receives no slot has zero weight gradients; a slot with probability 0 adds
    nothing to dx or to the weight gradients but still gets its dprobs."""
    inp = synth.make_layer(T=30, H=16, F=32, E=5, k=2, dtype="bf16", seed=8)
    ids = inp.expert_ids
    ids[ids == 4] = np.where(ids[ids == 4] == 4, 0, 0)
    ids[:, 1] = np.where(ids[:, 1] == ids[:, 0], (ids[:, 0] + 1) % 4, ids[:, 1])
    inp.expert_ids = ids
    dout = synth.make_dout(inp)
    dx, dwg, dwu, dwd, dprobs = oracle.backward(inp, dout)
    assert np.all(dwg[4] == 0) and np.all(dwu[4] == 0) and np.all(dwd[4] == 0)
    # zero probability for slot (t, 1): same dx and dW as the layer without that slot's term
    p0 = inp.probs.copy()
    p0[:, 1] = 0.0
    inp.probs = p0
    dx0, dwg0, dwu0, dwd0, dprobs0 = oracle.backward(inp, dout)
    inp1 = synth.LayerInputs(T=inp.T, H=inp.H, F=inp.F, E=inp.E, k=1, dtype="bf16", x=inp.x,
                             w_gate=inp.w_gate, w_up=inp.w_up, w_down=inp.w_down,
                             expert_ids=np.ascontiguousarray(ids[:, :1]),
                             probs=np.ascontiguousarray(p0[:, :1]))
    dx1, dwg1, dwu1, dwd1, _ = oracle.backward(inp1, dout)
    for a, b in ((dx0, dx1), (dwg0, dwg1), (dwu0, dwu1), (dwd0, dwd1)):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-300)
    assert np.all(dprobs0[:, 1] != 0)


def test_rejects_mx_and_bad_shapes():
    inp = synth.make_layer(T=4, H=32, F=32, E=2, k=1, dtype="mxfp8", seed=0)
    with pytest.raises(ValueError):
        oracle.backward(inp, np.zeros((4, 32), np.uint8))
    inp = synth.make_layer(T=4, H=8, F=8, E=2, k=1, dtype="bf16", seed=0)
    with pytest.raises(ValueError):
        oracle.backward(inp, np.zeros((3, 8), np.uint16))
