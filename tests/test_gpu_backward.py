"""Parity of the layer's backward (bf16) with the oracle's fp64 gradients.

Small layers are compared whole: dx, dw_gate, dw_up, dw_down and dprobs each within 2e-2 inf-norm
relative error (the bf16 bar; g, u, dg, du, probs * h and the per-slot dx rows are bf16 on the GPU,
the oracle keeps everything in double).  At the workloads' full sizes the oracle computes sampled
tokens (dx rows, dprobs) and sampled weight-gradient entries one by one; samples include the tokens
and the weight columns at tile edges.
"""
import numpy as np
import pytest
import torch

import moe_expert_layer_amd as mel
import oracle
import synth
from synth import device as dv

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    mel.library()
    oracle.build()


def _gpu_backward(inp, dout):
    d = dv.layer(inp)
    dd = dv.tensor(dout)
    res = mel.expert_backward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs, dd)
    torch.cuda.synchronize()
    return [dv.host(t) for t in res]


def _compare(gpu, ref, names=("dx", "dw_gate", "dw_up", "dw_down", "dprobs")):
    for name, a, r in zip(names, gpu, ref):
        err = oracle.inf_norm_rel(a, r)
        print(f"    {name}: inf-norm rel {err:.2e}", flush=True)
        assert np.all(np.isfinite(a)), name
        assert err <= TOL, (name, err)


CASES = [
    # T, H, F, E, k, routing kwargs: several row tiles with ragged tails, several column tiles
    (300, 256, 384, 6, 2, {}),
    # fine-grained shape: many experts, some empty (zero weight gradients), k = 4
    (200, 128, 256, 16, 4, dict(routing="zipf_gumbel", zipf_s=1.1, n_zero=3)),
    # one token, one expert slot
    (1, 128, 128, 2, 1, {}),
    # k = E: every token uses every expert
    (40, 128, 256, 3, 3, {}),
    # H and F multiples of 256: the weight gradients take the LDS-DMA kernel (ragged expert rows,
    # several row / column tiles)
    (300, 256, 512, 5, 2, {}),
    (260, 512, 256, 16, 4, dict(routing="zipf_gumbel", zipf_s=1.1, n_zero=4)),
    # the most experts the routing takes: one or no row per expert, every tile partial
    (128, 256, 256, 1023, 8, {}),
]


@pytest.mark.parametrize("T,H,F,E,k,kw", CASES)
def test_backward_matches_oracle(T, H, F, E, k, kw):
    print(f"[backward] T={T} H={H} F={F} E={E} k={k} {kw}", flush=True)
    inp = synth.make_layer(T=T, H=H, F=F, E=E, k=k, dtype="bf16", seed=T + E, **kw)
    dout = synth.make_dout(inp)
    gpu = _gpu_backward(inp, dout)
    ref = oracle.backward(inp, dout)
    _compare(gpu, ref)
    counts = np.bincount(inp.expert_ids.ravel(), minlength=E)
    for e in np.flatnonzero(counts == 0):
        assert np.all(gpu[1][e] == 0) and np.all(gpu[2][e] == 0) and np.all(gpu[3][e] == 0)


def test_backward_is_deterministic():
    inp = synth.make_layer(T=257, H=256, F=256, E=5, k=2, dtype="bf16", seed=11)
    dout = synth.make_dout(inp)
    a = _gpu_backward(inp, dout)
    b = _gpu_backward(inp, dout)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                              y.view(np.uint32) if y.dtype == np.float32 else y)


@pytest.mark.parametrize("H,F", [(128, 128), (256, 512)])
def test_backward_without_tokens_zeroes_the_weight_gradients(H, F):
    inp = synth.make_layer(T=4, H=H, F=F, E=3, k=1, dtype="bf16", seed=2)
    d = dv.layer(inp)
    x = d.x[:0]
    ids = d.expert_ids[:0]
    probs = d.probs[:0]
    dout = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    dx, dwg, dwu, dwd, dprobs = mel.expert_backward(x, d.w_gate, d.w_up, d.w_down, ids, probs, dout)
    torch.cuda.synchronize()
    assert dx.shape == (0, H) and dprobs.shape == (0, 1)
    for t in (dwg, dwu, dwd):
        assert torch.count_nonzero(t).item() == 0


def test_backward_one_busy_expert():
    """Every slot on expert 0: the later experts own no rows (their row range starts at the end of
    the permuted rows) and get zero weight gradients."""
    inp = synth.make_layer(T=200, H=256, F=256, E=4, k=1, dtype="bf16", seed=4)
    inp.expert_ids[:] = 0
    dout = synth.make_dout(inp)
    gpu = _gpu_backward(inp, dout)
    ref = oracle.backward(inp, dout)
    _compare(gpu, ref)
    for e in (1, 2, 3):
        assert np.all(gpu[1][e] == 0) and np.all(gpu[2][e] == 0) and np.all(gpu[3][e] == 0)


def test_backward_zero_probability_slot():
    """probs 0 on slot 1 of every token: dx and the weight gradients equal those of the k = 1 layer
    within the tolerance, dprobs of the zero slots is still <dout, y>."""
    inp = synth.make_layer(T=150, H=128, F=256, E=4, k=2, dtype="bf16", seed=5)
    inp.probs[:, 1] = 0.0
    dout = synth.make_dout(inp)
    gpu = _gpu_backward(inp, dout)
    ref = oracle.backward(inp, dout)
    _compare(gpu, ref)


def test_backward_rejects_other_dtypes():
    inp = synth.make_layer(T=8, H=128, F=128, E=2, k=1, dtype="f32", seed=0)
    d = dv.layer(inp)
    dout = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        mel.expert_backward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs, dout)


def _edge_columns(n, rng, n_random, tile=128):
    cols = {0, n - 1, tile - 1, tile, n - tile}
    cols.update(int(c) for c in rng.choice(n, size=n_random, replace=False))
    return np.array(sorted(c for c in cols if 0 <= c < n))


@pytest.mark.parametrize("name,n_tokens,n_entries", [("mixtral_bf16", 6, 24),
                                                     ("finegrained_bf16", 8, 32)])
def test_backward_full_size_sampled(name, n_tokens, n_entries):
    print(f"[backward-full] {name}: generating inputs", flush=True)
    inp = synth.make_workload(name)
    dout = synth.make_dout(inp)
    print(f"[backward-full] {name}: T={inp.T} H={inp.H} F={inp.F} E={inp.E} k={inp.k}", flush=True)
    dx, dwg, dwu, dwd, dprobs = _gpu_backward(inp, dout)
    rng = np.random.default_rng(0)
    counts, offsets, perm, pos = oracle.route(inp.expert_ids, inp.E)
    # tokens owning the first / last row of the largest experts, and random ones
    big = np.argsort(-counts)[:2]
    toks = {int(perm[offsets[e]]) // inp.k for e in big} | {int(perm[offsets[e + 1] - 1]) // inp.k for e in big}
    toks.update(int(t) for t in rng.choice(inp.T, size=n_tokens, replace=False))
    toks = np.array(sorted(toks), np.int32)
    print(f"[backward-full] {name}: oracle on {len(toks)} tokens", flush=True)
    ref_dx, ref_dp = oracle.backward_tokens(inp, dout, toks)
    _compare([dx[toks], dprobs[toks]], [ref_dx, ref_dp], names=("dx rows", "dprobs rows"))
    # weight-gradient entries: experts with rows, columns at tile edges and random
    live = np.flatnonzero(counts > 0)
    e = rng.choice(live, size=n_entries)
    f = rng.choice(_edge_columns(inp.F, rng, 8), size=n_entries)
    h = rng.choice(_edge_columns(inp.H, rng, 8), size=n_entries)
    print(f"[backward-full] {name}: oracle on {n_entries} weight-gradient entries", flush=True)
    rg, ru, rd = oracle.wgrad_entries(inp, dout, e, f, h)
    _compare([dwg[e, h, f], dwu[e, h, f], dwd[e, f, h]], [rg, ru, rd],
             names=("dw_gate entries", "dw_up entries", "dw_down entries"))
    empty = np.flatnonzero(counts == 0)
    for ee in empty:
        assert np.all(dwg[ee] == 0) and np.all(dwu[ee] == 0) and np.all(dwd[ee] == 0)


def test_backward_out_of_range_ids_skipped_and_flagged():
    """Slots whose expert id lies outside [0, E) are skipped (dprobs 0, nothing in dx or the weight
    gradients) and set the status word; every other gradient is that of the layer in which those
    slots carry probability 0 (and any valid id)."""
    inp = synth.make_layer(T=200, H=256, F=256, E=4, k=2, dtype="bf16", seed=12)
    bad = np.zeros(inp.expert_ids.shape, bool)
    bad[::7, 1] = True
    bad[3::11, 0] = True
    ids_bad = inp.expert_ids.copy()
    ids_bad[bad] = np.where(np.arange(bad.sum()) % 2 == 0, 4, -1)
    dout = synth.make_dout(inp)
    d = dv.layer(inp)
    ws = torch.empty(mel.backward_workspace_size(mel.problem(inp.T, inp.H, inp.F, inp.E, inp.k, mel.BF16)),
                     dtype=torch.uint8, device="cuda")
    res = mel.expert_backward(d.x, d.w_gate, d.w_up, d.w_down, dv.tensor(ids_bad), d.probs,
                              dv.tensor(dout), workspace=ws)
    assert mel.device_status(ws) == 4                 # MOE_ERR_EXPERT_ID_OUT_OF_RANGE
    gpu = [dv.host(t) for t in res]
    inp.probs = np.where(bad, np.float32(0.0), inp.probs).astype(np.float32)
    ref = oracle.backward(inp, dout)
    _compare(gpu[:4], ref[:4], names=("dx", "dw_gate", "dw_up", "dw_down"))
    assert np.all(gpu[4][bad] == 0)
    assert oracle.inf_norm_rel(gpu[4][~bad], ref[4][~bad]) <= TOL


@pytest.mark.parametrize("T,H,F,E,k", [(300, 384, 256, 6, 2), (300, 256, 512, 5, 2), (700, 512, 256, 8, 2)],
                         ids=["small_tiles", "large_tiles", "large_tiles_gathered"])
def test_saved_gate_up_values_are_those_recomputed(T, H, F, E, k):
    """expert_forward_train's output is bitwise expert_forward's; the backward on its saved g and u
    is bitwise the backward that recomputes them."""
    inp = synth.make_layer(T=T, H=H, F=F, E=E, k=k, dtype="bf16", seed=T + H)
    dout = dv.tensor(synth.make_dout(inp))
    d = dv.layer(inp)
    out = mel.expert_forward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs)
    out_t, saved = mel.expert_forward_train(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs)
    assert torch.equal(out, out_t)
    a = mel.expert_backward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs, dout)
    b = mel.expert_backward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs, dout,
                            saved_gu=saved)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_saved_gate_up_values_full_size():
    print("[backward-saved] mixtral_bf16: generating inputs", flush=True)
    inp = synth.make_workload("mixtral_bf16")
    d = dv.layer(inp)
    dout = dv.tensor(synth.make_dout(inp))
    out = mel.expert_forward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs)
    out_t, saved = mel.expert_forward_train(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs)
    assert torch.equal(out, out_t)
    a = mel.expert_backward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs, dout)
    b = mel.expert_backward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs, dout,
                            saved_gu=saved)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
