"""Parity of the router kernel (top-k gate) with the oracle: expert ids bit-exact, probabilities
within 1e-6 relative (float32 exp and division against the oracle's double; a few ulps)."""
import numpy as np
import pytest
import torch

import moe_expert_layer_amd as mel
import oracle
import synth

pytestmark = pytest.mark.gpu

PROB_RTOL = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _lib():
    mel.library()
    oracle.build()


def _check(logits, k):
    ids_ref, probs_ref = oracle.router(logits, k)
    ids, probs = mel.router_topk(torch.from_numpy(logits).cuda(), k)
    torch.cuda.synchronize()
    ids, probs = ids.cpu().numpy(), probs.cpu().numpy().astype(np.float64)
    assert np.array_equal(ids, ids_ref)
    np.testing.assert_allclose(probs, probs_ref, rtol=PROB_RTOL, atol=1e-30)
    return ids


@pytest.mark.parametrize("name", ["mixtral_bf16", "finegrained_bf16", "mxfp8", "tiny_f32"])
def test_workload_logits(name):
    """The logits behind each workload's routing (Mixtral E=8 k=2; fine-grained E=128 k=8 with
    -inf logits for the unused experts; MX E=32 k=4), at full token count."""
    w = dict(synth.WORKLOADS[name])
    kw = {key: w[key] for key in ("zipf_s", "n_zero") if key in w}
    logits = synth.make_logits(w["T"], w["E"], w.get("routing", "normal_logits"), seed=0, **kw)
    print(f"[router] {name}: T={w['T']} E={w['E']} k={w['k']}", flush=True)
    _check(logits, w["k"])


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 3, 3), (100, 64, 64), (33, 65, 5), (50, 100, 7),
                                   (20, 200, 16), (9, 1024, 64), (300, 511, 2), (0, 8, 2)])
def test_shapes_and_ties(T, E, k):
    """Ragged E across the 64-lane wave, k = E, k = 64, E = 1024, T = 0; half the rows on a coarse
    grid so that equal logits occur (taken in ascending id)."""
    rng = np.random.default_rng(T * 131 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[::2] = np.round(logits[::2] * 2) / 2
    _check(logits, k)


def test_signed_zeros_tie():
    """-0 and +0 are equal logits: the lower id goes first."""
    logits = np.zeros((8, 6), np.float32)
    logits[:, 1] = -0.0
    logits[:, 4] = 0.5
    ids = _check(logits, 3)
    assert np.all(ids == np.array([4, 0, 1]))


def test_minus_infinity_taken_last():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((64, 40)).astype(np.float32)
    logits[:, 3:37] = -np.inf
    ids = _check(logits, 8)
    assert np.all(ids[:, 6:] == np.array([3, 4]))


def test_feeds_the_layer():
    """Router output drives the forward: same result as the host-generated routing of that layer."""
    T, H, F, E, k = 300, 256, 128, 6, 2
    inp = synth.make_layer(T=T, H=H, F=F, E=E, k=k, dtype="bf16", seed=8)
    logits = synth.make_logits(T, E, seed=8)
    ids, probs = mel.router_topk(torch.from_numpy(logits).cuda(), k)
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    ref_ids, ref_probs = oracle.router(logits, k)
    assert np.array_equal(ids_h, ref_ids)
    inp.expert_ids = ids_h
    inp.probs = probs.cpu().numpy()
    ref, *_ = oracle.forward(inp)
    from synth import device as dv
    d = dv.layer(inp)
    out = mel.expert_forward(d.x, d.w_gate, d.w_up, d.w_down, ids, probs)
    assert oracle.inf_norm_rel(dv.host(out), ref) <= 2e-2


def test_rejects_bad_arguments():
    x = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    for k in (0, 9):
        with pytest.raises(mel.MoeError):
            mel.router_topk(x, k)
